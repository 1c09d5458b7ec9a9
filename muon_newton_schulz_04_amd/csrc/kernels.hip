// gfx950 (CDNA4) kernels of the Muon update.
//
//   momentum_kernel   buf' = mu buf + G, u = G + mu buf' | buf' | G, and one
//                     fixed-order sum of u^2 per work item        (HBM-bound)
//   normalize_kernel  X0 = u / (sqrt(sum u^2) + eps) written in the
//                     rows<=cols orientation as fp32 master + operand copy,
//                     zero-padded to 128-multiples                 (HBM-bound)
//   gemm_kernel<GRAM>   A = X X^T           upper-triangle tiles, mirrored
//   gemm_kernel<POLY>   B = b A + c A A     upper-triangle tiles, mirrored
//   gemm_kernel<UPDATE> X = a X + B X       (last step writes `out`)
//
// The three matrix-core kernels share one 128 x 128 output-tile engine:
// 4 waves of 64 lanes, each wave owning a 64 x 64 sub-tile made of 4 x 4
// v_mfma_f32_16x16x32_{f16,bf16} (bf16 sets; fp16 operands by default) or
// v_mfma_f32_16x16x4_f32 (fp32 sets) accumulators. Operands are staged through LDS as [row][k] tiles of
// 128 rows x 128 bytes (16-byte chunks XOR-swizzled against bank conflicts);
// the next k-slab is prefetched into registers while the current one is
// multiplied. Operands whose k index runs along memory rows (X in B X) are
// transposed in registers on their way into LDS.
//
// Every launch takes a schedule of work items; block b runs item b. The
// schedules keep one matrix's tiles on one XCD (block b runs on XCD b % 8).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.hpp"

namespace muon {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 bits

// float -> bfloat16 bits, round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, float v) {
    static_cast<float*>(p)[i] = v;
  }
  static __device__ __forceinline__ float round(float v) { return v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const void* p, int64_t i) {
    return bf2f(static_cast<const uint16_t*>(p)[i]);
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = f2bf(v);
  }
  static __device__ __forceinline__ float round(float v) { return bf2f(f2bf(v)); }
};

// Operand formats of the matrix products (X, A, B in the workspace).
enum OpFmt { OP_F32 = 0, OP_F16 = 1, OP_BF16 = 2 };
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

template <int OP> struct Op;
template <> struct Op<OP_F32> {
  static constexpr int bytes = 4;
  static __device__ __forceinline__ float load(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, float v) {
    static_cast<float*>(p)[i] = v;
  }
};
template <> struct Op<OP_F16> {
  static constexpr int bytes = 2;
  static __device__ __forceinline__ uint16_t bits(float v) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));  // RNE
  }
  static __device__ __forceinline__ float load(const void* p, int64_t i) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<const uint16_t*>(p)[i]));
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = bits(v);
  }
};
template <> struct Op<OP_BF16> {
  static constexpr int bytes = 2;
  static __device__ __forceinline__ uint16_t bits(float v) { return f2bf(v); }
  static __device__ __forceinline__ float load(const void* p, int64_t i) {
    return bf2f(static_cast<const uint16_t*>(p)[i]);
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = f2bf(v);
  }
};

// Fixed-order block sum over 256 threads (deterministic).
__device__ __forceinline__ float block_sum_256(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float s = (red[0] + red[1]) + (red[2] + red[3]);
  return s;
}

// StepArgs (kernel arguments) is declared in launch.hpp.

// u from the gradient and the already-updated buffer (same expression in
// both elementwise kernels so u is bitwise identical).
__device__ __forceinline__ float form_u(float g, float nb, const StepArgs& A) {
  if (!A.use_mom) return g;
  return A.nesterov ? __fmaf_rn(A.mu, nb, g) : nb;
}

// --------------------------------------------------------- momentum kernel

template <typename T>
__global__ __launch_bounds__(256) void momentum_kernel(StepArgs A) {
  const WorkItem it = A.items[blockIdx.x];
  if (it.mat < 0) return;
  const MatInfo M = A.mats[it.mat];
  const int32_t r0 = it.a, nr = it.b;
  float acc = 0.f;
  const T* g = static_cast<const T*>(M.grad);
  T* mb = static_cast<T*>(M.mom);
  constexpr int V = 16 / sizeof(T);  // elements per 16-byte vector
  if (M.vec_ok) {
    const int32_t vpr = M.cols / V;
    const int32_t nv = nr * vpr;
    for (int32_t v = threadIdx.x; v < nv; v += 256) {
      const int32_t r = r0 + v / vpr, cv = (v % vpr) * V;
      const int64_t off = int64_t(r) * M.ld + cv;
      uint4 gv = *reinterpret_cast<const uint4*>(g + off);
      const T* ge = reinterpret_cast<const T*>(&gv);
      if (A.use_mom) {
        uint4 bv = *reinterpret_cast<const uint4*>(mb + off);
        T* be = reinterpret_cast<T*>(&bv);
        uint4 ov;
        T* oe = reinterpret_cast<T*>(&ov);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const float gf = Elem<T>::load(ge, e);
          const float nb = Elem<T>::round(__fmaf_rn(A.mu, Elem<T>::load(be, e), gf));
          Elem<T>::store(oe, e, nb);
          const float u = form_u(gf, nb, A);
          acc = __fmaf_rn(u, u, acc);
        }
        *reinterpret_cast<uint4*>(mb + off) = ov;
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const float u = Elem<T>::load(ge, e);
          acc = __fmaf_rn(u, u, acc);
        }
      }
    }
  } else {
    const int32_t ne = nr * M.cols;
    for (int32_t e = threadIdx.x; e < ne; e += 256) {
      const int64_t off = int64_t(r0 + e / M.cols) * M.ld + (e % M.cols);
      const float gf = Elem<T>::load(g, off);
      float u = gf;
      if (A.use_mom) {
        const float nb = Elem<T>::round(__fmaf_rn(A.mu, Elem<T>::load(mb, off), gf));
        Elem<T>::store(mb, off, nb);
        u = form_u(gf, nb, A);
      }
      acc = __fmaf_rn(u, u, acc);
    }
  }
  __shared__ float red[4];
  const float s = block_sum_256(acc, red);
  if (threadIdx.x == 0) A.parts[it.c] = s;
}

// -------------------------------------------------------- normalize kernel
//
// Item {mat, ti, tj}: a 64 x 64 tile of X0 in the rows<=cols orientation
// (rows ti*64.., cols tj*64.. of the mp x np padded layout). The caller-side
// tile (transposed for tall matrices) is read into LDS, scaled, and written
// out row-major, zeros in the padding. With zero steps the scaled values go
// straight to `out` in the caller's layout.

template <typename T, int OP>
__global__ __launch_bounds__(256) void normalize_kernel(StepArgs A) {
  const WorkItem it = A.items[blockIdx.x];
  if (it.mat < 0) return;
  const MatInfo M = A.mats[it.mat];
  __shared__ float red[4];
  __shared__ float tile[64][65];

  // 1. scale from this matrix's partial sums, in slot order
  float s = 0.f;
  for (int32_t p = threadIdx.x; p < M.part_cnt; p += 256) s += A.parts[M.part_off + p];
  s = block_sum_256(s, red);
  const float scale = 1.0f / (sqrtf(s) + A.eps);

  // 2. caller-side tile: rows cr0.., cols cc0..
  const int32_t i0 = it.a * 64, j0 = it.b * 64;  // X0 (wide) coordinates
  const int32_t cr0 = M.tall ? j0 : i0, cc0 = M.tall ? i0 : j0;
  const T* g = static_cast<const T*>(M.grad);
  const T* mb = static_cast<const T*>(M.mom);
  for (int32_t e = threadIdx.x; e < 64 * 64; e += 256) {
    const int32_t r = e >> 6, cidx = e & 63;
    const int32_t cr = cr0 + r, cc = cc0 + cidx;
    float v = 0.f;
    if (cr < M.rows && cc < M.cols) {
      const int64_t off = int64_t(cr) * M.ld + cc;
      const float gf = Elem<T>::load(g, off);
      const float nb = A.use_mom ? Elem<T>::load(mb, off) : 0.f;
      v = form_u(gf, nb, A) * scale;
    }
    tile[r][cidx] = v;
  }
  __syncthreads();

  if (A.direct) {  // zero steps: X0 is the result, caller layout
    T* o = static_cast<T*>(M.out);
    for (int32_t e = threadIdx.x; e < 64 * 64; e += 256) {
      const int32_t r = e >> 6, cidx = e & 63;
      const int32_t cr = cr0 + r, cc = cc0 + cidx;
      if (cr < M.rows && cc < M.cols) Elem<T>::store(o, int64_t(cr) * M.ld + cc, tile[r][cidx]);
    }
    return;
  }
  // 3. X0 rows i0.., cols j0.. of the padded wide layout (row stride np)
  for (int32_t e = threadIdx.x; e < 64 * 64; e += 256) {
    const int32_t r = e >> 6, cidx = e & 63;
    const float v = M.tall ? tile[cidx][r] : tile[r][cidx];
    const int64_t off = int64_t(i0 + r) * M.np + (j0 + cidx);
    if constexpr (OP != OP_F32) {
      reinterpret_cast<float*>(A.ws + M.xm_off)[off] = v;
      Op<OP>::store(A.ws + M.xo_off[0], off, v);
    } else {
      reinterpret_cast<float*>(A.ws + M.xo_off[0])[off] = v;
    }
  }
}

// ------------------------------------------------------ matrix-core engine

enum GemmKind { GRAM = 0, POLY = 1, UPDATE = 2 };

constexpr int BM = 128;           // output tile (rows and cols)
constexpr int ROWB = 128;         // LDS bytes per tile row (one k-slab)

// byte offset of (row, 16-byte chunk) in an LDS operand tile
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * ROWB + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// Loads a 128-row x 128-byte slab of a row-major operand whose k index is
// contiguous (rows r0.., bytes k0b..): 4 x 16 bytes per thread.
__device__ __forceinline__ void load_rows(uint4 (&r)[4], const char* base, int64_t ld_bytes,
                                          int64_t k0b) {
  const int t = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = (t >> 3) + 32 * q, ch = t & 7;
    r[q] = *reinterpret_cast<const uint4*>(base + row * ld_bytes + k0b + ch * 16);
  }
}
__device__ __forceinline__ void store_rows(char* lds, const uint4 (&r)[4]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = (t >> 3) + 32 * q, ch = t & 7;
    *reinterpret_cast<uint4*>(lds + lds_off(row, ch)) = r[q];
  }
}

// Operand with k along memory rows (X[k][n], n contiguous): the slab is
// KS k-rows x 128 n-columns (KS = 64 bf16 or 32 fp32). Thread t loads a
// block of 4 k-rows x V columns (V = 8 bf16 / 4 fp32, 16 bytes) and later
// writes it transposed into the [n][k] LDS tile.
template <int ES>
__device__ __forceinline__ void load_cols(uint4 (&r)[4], const char* base, int64_t ld_bytes,
                                          int64_t k0) {
  constexpr int V = 16 / ES;
  constexpr int NG = 128 / V;  // column groups per slab (16 bf16, 32 fp32)
  const int t = threadIdx.x;
  const int kq = t / NG, ng = t % NG;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    r[q] = *reinterpret_cast<const uint4*>(base + (k0 + 4 * kq + q) * ld_bytes + ng * 16);
}
template <int ES>
__device__ __forceinline__ void store_cols(char* lds, const uint4 (&r)[4]) {
  constexpr int V = 16 / ES;
  constexpr int NG = 128 / V;
  const int t = threadIdx.x;
  const int kq = t / NG, ng = t % NG;
  if constexpr (ES == 2) {
    // k-quad kq covers 16-bit k = 4kq..4kq+3: 8 bytes inside chunk kq/2
    const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r[0]);
    const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r[1]);
    const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r[2]);
    const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r[3]);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      // columns 2d (low halves) and 2d+1 (high halves)
      uint2 lo, hi;
      lo.x = (w0[d] & 0xffffu) | (w1[d] << 16);
      lo.y = (w2[d] & 0xffffu) | (w3[d] << 16);
      hi.x = (w0[d] >> 16) | (w1[d] & 0xffff0000u);
      hi.y = (w2[d] >> 16) | (w3[d] & 0xffff0000u);
      const int n0 = ng * 8 + 2 * d;
      *reinterpret_cast<uint2*>(lds + lds_off(n0, kq >> 1) + (kq & 1) * 8) = lo;
      *reinterpret_cast<uint2*>(lds + lds_off(n0 + 1, kq >> 1) + (kq & 1) * 8) = hi;
    }
  } else {
    // k-quad kq covers fp32 k = 4kq..4kq+3: exactly chunk kq
    const float* f0 = reinterpret_cast<const float*>(&r[0]);
    const float* f1 = reinterpret_cast<const float*>(&r[1]);
    const float* f2 = reinterpret_cast<const float*>(&r[2]);
    const float* f3 = reinterpret_cast<const float*>(&r[3]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float4 v = make_float4(f0[e], f1[e], f2[e], f3[e]);
      *reinterpret_cast<float4*>(lds + lds_off(ng * 4 + e, kq)) = v;
    }
  }
}

// One k-slab (128 bytes of k per row) of MFMAs for this wave's 64 x 64.
template <int OP>
__device__ __forceinline__ void mma_slab(f32x4_t (&acc)[4][4], const char* sA, const char* sB,
                                         int wm, int wn) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int ch = half * 4 + lg;  // each lane group takes one 16-byte k chunk
    uint4 af[4], bfr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[i] = *reinterpret_cast<const uint4*>(sA + lds_off(wm * 64 + i * 16 + lr, ch));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bfr[j] = *reinterpret_cast<const uint4*>(sB + lds_off(wn * 64 + j * 16 + lr, ch));
    if constexpr (OP == OP_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, af[i]), __builtin_bit_cast(bf16x8_t, bfr[j]),
              acc[i][j], 0, 0, 0);
    } else if constexpr (OP == OP_F16) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              __builtin_bit_cast(f16x8_t, af[i]), __builtin_bit_cast(f16x8_t, bfr[j]),
              acc[i][j], 0, 0, 0);
    } else {
      // four k=4 MFMAs per 16-byte chunk; lane group g supplies k = 4(ch)+e
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                __uint_as_float((&af[i].x)[e]), __uint_as_float((&bfr[j].x)[e]), acc[i][j], 0,
                0, 0);
    }
  }
}

// Item {mat, ti, tj}. GRAM/POLY: C = Op Op^T on upper-triangle tiles (ti <=
// tj) mirrored into the lower triangle; UPDATE: X = a X + B X on all tiles.
template <typename T, int OP, int KIND>
__global__ __launch_bounds__(256) void gemm_kernel(StepArgs P) {
  const WorkItem it = P.items[blockIdx.x];
  if (it.mat < 0) return;
  const MatInfo M = P.mats[it.mat];
  constexpr int ES = Op<OP>::bytes;  // operand element size
  constexpr int KS = ROWB / ES;      // k elements per slab

  __shared__ __attribute__((aligned(16))) char sA[BM * ROWB];
  __shared__ __attribute__((aligned(16))) char sB[BM * ROWB];

  const int ti = it.a, tj = it.b;
  const char* opA;
  const char* opB;
  int64_t lda_b, ldb_b, K;
  if (KIND == GRAM) {  // rows of X (mp x np): A[i][j] = sum_k X[i][k] X[j][k]
    const char* X = P.ws + M.xo_off[P.cur];
    lda_b = ldb_b = int64_t(M.np) * ES;
    opA = X + int64_t(ti) * BM * lda_b;
    opB = X + int64_t(tj) * BM * ldb_b;
    K = M.np;
  } else if (KIND == POLY) {  // rows of A (mp x mp), symmetric: (A A)[i][j] = sum_k A[i][k] A[j][k]
    const char* Am = P.ws + M.a_off;
    lda_b = ldb_b = int64_t(M.mp) * ES;
    opA = Am + int64_t(ti) * BM * lda_b;
    opB = Am + int64_t(tj) * BM * ldb_b;
    K = M.mp;
  } else {  // rows of B (mp x mp) times columns tj of X (mp x np)
    const char* Bm = P.ws + M.b_off;
    lda_b = int64_t(M.mp) * ES;
    ldb_b = int64_t(M.np) * ES;
    opA = Bm + int64_t(ti) * BM * lda_b;
    opB = P.ws + M.xo_off[P.cur] + int64_t(tj) * BM * ES;
    K = M.mp;
  }

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 ra[4], rb[4];
  load_rows(ra, opA, lda_b, 0);
  if (KIND == UPDATE) load_cols<ES>(rb, opB, ldb_b, 0);
  else load_rows(rb, opB, ldb_b, 0);
  for (int64_t k0 = 0; k0 < K; k0 += KS) {
    __syncthreads();
    store_rows(sA, ra);
    if (KIND == UPDATE) store_cols<ES>(sB, rb);
    else store_rows(sB, rb);
    __syncthreads();
    if (k0 + KS < K) {
      load_rows(ra, opA, lda_b, (k0 + KS) * ES);
      if (KIND == UPDATE) load_cols<ES>(rb, opB, ldb_b, k0 + KS);
      else load_rows(rb, opB, ldb_b, (k0 + KS) * ES);
    }
    mma_slab<OP>(acc, sA, sB, wm, wn);
  }

  // ------------------------------------------------------------ epilogue
  // acc[i][j][r] is C[row][col] with row = wm*64 + i*16 + 4*(lane>>4) + r,
  // col = wn*64 + j*16 + (lane & 15) inside the tile.
  const int lr = lane & 15, lg = lane >> 4;
  if (KIND == GRAM || KIND == POLY) {
    char* C = P.ws + (KIND == GRAM ? M.a_off : M.b_off);
    const char* Am = P.ws + M.a_off;
    const int64_t ld = M.mp;
    const bool diag = ti == tj;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int gi0 = ti * BM + wm * 64 + i * 16 + 4 * lg;
        const int gj = tj * BM + wn * 64 + j * 16 + lr;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc[i][j][r];
        if (KIND == POLY) {
          // b A[gi][gj] read from the mirrored (contiguous) position A[gj][gi0..]
#pragma unroll
          for (int r = 0; r < 4; ++r)
            v[r] = __fmaf_rn(P.c, v[r], P.b * Op<OP>::load(Am, int64_t(gj) * ld + gi0 + r));
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int gi = gi0 + r;
          if (!diag || gi <= gj) Op<OP>::store(C, int64_t(gi) * ld + gj, v[r]);
          if (!diag || gi < gj) Op<OP>::store(C, int64_t(gj) * ld + gi, v[r]);
        }
      }
  } else {
    const int64_t ldx = M.np;
    if (!P.last) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int gi0 = ti * BM + wm * 64 + i * 16 + 4 * lg;
          const int gj = tj * BM + wn * 64 + j * 16 + lr;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int64_t off = int64_t(gi0 + r) * ldx + gj;
            if constexpr (OP != OP_F32) {
              float* xm = reinterpret_cast<float*>(P.ws + M.xm_off);
              const float v = __fmaf_rn(P.a, xm[off], acc[i][j][r]);
              xm[off] = v;
              Op<OP>::store(P.ws + M.xo_off[P.cur ^ 1], off, v);
            } else {
              const float* xc = reinterpret_cast<const float*>(P.ws + M.xo_off[P.cur]);
              const float v = __fmaf_rn(P.a, xc[off], acc[i][j][r]);
              reinterpret_cast<float*>(P.ws + M.xo_off[P.cur ^ 1])[off] = v;
            }
          }
        }
    } else {
      // last step: out in the caller's layout and dtype, valid region only
      const float* xsrc = reinterpret_cast<const float*>(
          P.ws + (OP != OP_F32 ? M.xm_off : M.xo_off[P.cur]));
      char* o = static_cast<char*>(M.out);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int gi0 = ti * BM + wm * 64 + i * 16 + 4 * lg;
          const int gj = tj * BM + wn * 64 + j * 16 + lr;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int gi = gi0 + r;
            if (gi < M.m && gj < M.n) {
              const float v = __fmaf_rn(P.a, xsrc[int64_t(gi) * ldx + gj], acc[i][j][r]);
              const int64_t co = M.tall ? int64_t(gj) * M.ld + gi : int64_t(gi) * M.ld + gj;
              Elem<T>::store(o, co, v);
            }
          }
        }
    }
  }
}

// --------------------------------------------------------------- launchers

template <typename T, int OP>
static hipError_t launch_t(int kind, const StepArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  dim3 g(grid), b(256);
  switch (kind) {
    case MUON_K_MOMENTUM: hipLaunchKernelGGL(momentum_kernel<T>, g, b, 0, s, a); break;
    case MUON_K_NORMALIZE: hipLaunchKernelGGL((normalize_kernel<T, OP>), g, b, 0, s, a); break;
    case MUON_K_GRAM: hipLaunchKernelGGL((gemm_kernel<T, OP, GRAM>), g, b, 0, s, a); break;
    case MUON_K_POLY: hipLaunchKernelGGL((gemm_kernel<T, OP, POLY>), g, b, 0, s, a); break;
    case MUON_K_UPDATE: hipLaunchKernelGGL((gemm_kernel<T, OP, UPDATE>), g, b, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_kernel(int kind, muon_dtype dt, int precision, const StepArgs& a, int grid,
                         hipStream_t s) {
  if (dt == MUON_F32) return launch_t<float, OP_F32>(kind, a, grid, s);
  if (precision == MUON_PRECISION_BF16_OPERANDS) return launch_t<uint16_t, OP_BF16>(kind, a, grid, s);
  return launch_t<uint16_t, OP_F16>(kind, a, grid, s);
}

}  // namespace muon
