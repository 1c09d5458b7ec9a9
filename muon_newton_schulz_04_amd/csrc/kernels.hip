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
#include <type_traits>

#include "launch.hpp"

namespace muon {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 bits

// float -> bfloat16 bits, round to nearest, ties to even (gfx950's
// v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
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
  // X = hi + lo * 2^-11: hi is the operand, lo the scaled residual (about
  // 22 significant bits together; the scaling keeps lo out of subnormals)
  static __device__ __forceinline__ void split(float x, uint32_t& hi, uint32_t& lo) {
    const _Float16 h = static_cast<_Float16>(x);
    hi = __builtin_bit_cast(uint16_t, h);
    lo = __builtin_bit_cast(uint16_t, static_cast<_Float16>((x - static_cast<float>(h)) * 2048.f));
  }
  static __device__ __forceinline__ float join(uint32_t hi, uint32_t lo) {
    return __fmaf_rn(load16(lo), 1.f / 2048.f, load16(hi));
  }
  static __device__ __forceinline__ float load16(uint32_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
  }
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
  // X = hi + lo (about 17 significant bits together)
  static __device__ __forceinline__ void split(float x, uint32_t& hi, uint32_t& lo) {
    hi = f2bf(x);
    lo = f2bf(x - bf2f(static_cast<uint16_t>(hi)));
  }
  static __device__ __forceinline__ float join(uint32_t hi, uint32_t lo) {
    return bf2f(static_cast<uint16_t>(hi)) + bf2f(static_cast<uint16_t>(lo));
  }
  static __device__ __forceinline__ float load16(uint32_t h) { return bf2f(static_cast<uint16_t>(h)); }
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

// Component e (compile-time after unrolling) of a 16-byte register vector.
__device__ __forceinline__ uint32_t comp(const uint4& v, int e) {
  return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

// Offset of operand buffer `which` (0/1) without indexing the record's
// array by a run-time value (which would move the record to scratch).
__device__ __forceinline__ int64_t xo_sel(const MatInfo& M, int which) {
  return which ? M.xo_off[1] : M.xo_off[0];
}

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
  const MatInfo& M = A.mats[it.mat];
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

// fp16 operand sets keep the low part of X in the update kernel's
// accumulator order: per 256 x 128 tile, per wave, per accumulator group
// (i, j, g) a contiguous 64-lane x 4-element block. Lane loads and stores of
// the update epilogue are then contiguous across the wave. Element index of
// X(m, n) in that layout (np = padded row length):
__device__ __forceinline__ int64_t lo_index(int m, int n, int np) {
  const int tile = (m >> 8) * (np >> 7) + (n >> 7);
  const int mm = m & 255, nn = n & 127;
  const int wave = (mm >> 7) * 2 + (nn >> 6);
  const int lane = (mm & 31) + 32 * ((nn >> 2) & 1);
  const int grp = (((mm >> 5) & 3) * 2 + ((nn >> 5) & 1)) * 4 + ((nn >> 3) & 3);
  return (((int64_t(tile) * 4 + wave) * 32 + grp) * 64 + lane) * 4 + (nn & 3);
}

template <typename T, int OP>
__global__ __launch_bounds__(256) void normalize_kernel(StepArgs A) {
  const WorkItem it = A.items[blockIdx.x];
  if (it.mat < 0) return;
  const MatInfo& M = A.mats[it.mat];
  __shared__ float red[4];
  __shared__ float tile[64][65];

  // 1. scale from this matrix's partial sums, in slot order
  float s = 0.f;
  for (int32_t p = threadIdx.x; p < M.part_cnt; p += 256) s += A.parts[M.part_off + p];
  s = block_sum_256(s, red);
  const float scale = 1.0f / (sqrtf(s) + A.eps);

  // 2. caller-side tile rows cr0.., cols cc0..; thread handles 2 runs of 8
  //    consecutive caller columns: run h covers row (tid + 256 h) / 8,
  //    columns 8 * (tid % 8)..+7
  const int32_t i0 = it.a * 64, j0 = it.b * 64;  // X0 (rows<=cols) coordinates
  const int32_t cr0 = M.tall ? j0 : i0, cc0 = M.tall ? i0 : j0;
  const T* g = static_cast<const T*>(M.grad);
  const T* mb = static_cast<const T*>(M.mom);
  float u[2][8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int v = threadIdx.x + 256 * h;
    const int32_t cr = cr0 + (v >> 3), cc = cc0 + (v & 7) * 8;
    const int64_t off = int64_t(cr) * M.ld + cc;
    if (cr < M.rows && M.vec_ok && cc + 8 <= M.cols) {
      float gv[8], bv[8];
      if constexpr (sizeof(T) == 2) {
        const u32x4_t gw = *reinterpret_cast<const u32x4_t*>(g + off);
        u32x4_t bw = {0u, 0u, 0u, 0u};
        if (A.use_mom) bw = *reinterpret_cast<const u32x4_t*>(mb + off);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          gv[e] = bf2f(static_cast<uint16_t>(gw[e >> 1] >> (16 * (e & 1))));
          bv[e] = bf2f(static_cast<uint16_t>(bw[e >> 1] >> (16 * (e & 1))));
        }
      } else {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const f32x4_t gw = *reinterpret_cast<const f32x4_t*>(g + off + 4 * q);
          f32x4_t bw = {0.f, 0.f, 0.f, 0.f};
          if (A.use_mom) bw = *reinterpret_cast<const f32x4_t*>(mb + off + 4 * q);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            gv[4 * q + e] = gw[e];
            bv[4 * q + e] = bw[e];
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) u[h][e] = form_u(gv[e], bv[e], A) * scale;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = 0.f;
        if (cr < M.rows && cc + e < M.cols) {
          const float gf = Elem<T>::load(g, off + e);
          const float nb = A.use_mom ? Elem<T>::load(mb, off + e) : 0.f;
          x = form_u(gf, nb, A) * scale;
        }
        u[h][e] = x;
      }
    }
  }

  if (A.direct) {  // zero steps: X0 is the result, in the caller's layout
    T* o = static_cast<T*>(M.out);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int v = threadIdx.x + 256 * h;
      const int32_t cr = cr0 + (v >> 3), cc = cc0 + (v & 7) * 8;
      if (cr >= M.rows) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (cc + e < M.cols) Elem<T>::store(o, int64_t(cr) * M.ld + cc + e, u[h][e]);
    }
    return;
  }

  // 3. X0 rows i0.., cols j0.. of the padded layout (row stride np), written
  //    as runs of 8 (fp32 master + operand copy); tall tiles go through LDS
  if (M.tall) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int v = threadIdx.x + 256 * h;
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[(v & 7) * 8 + e][v >> 3] = u[h][e];
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int v = threadIdx.x + 256 * h;
#pragma unroll
      for (int e = 0; e < 8; ++e) u[h][e] = tile[v >> 3][(v & 7) * 8 + e];
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int v = threadIdx.x + 256 * h;
    const int64_t off = int64_t(i0 + (v >> 3)) * M.np + j0 + (v & 7) * 8;
    if constexpr (OP != OP_F32) {
      u32x4_t whi, wlo;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t h0, l0, h1, l1;
        Op<OP>::split(u[h][2 * q], h0, l0);
        Op<OP>::split(u[h][2 * q + 1], h1, l1);
        whi[q] = h0 | (h1 << 16);
        wlo[q] = l0 | (l1 << 16);
      }
      *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(A.ws + M.xo_off[0]) + off) = whi;
      uint16_t* lo = reinterpret_cast<uint16_t*>(A.ws + M.xl_off);
      if constexpr (OP == OP_F16) {  // two runs of 4 in accumulator order
        const int m = i0 + (v >> 3), n = j0 + (v & 7) * 8;
        *reinterpret_cast<uint2*>(lo + lo_index(m, n, M.np)) = make_uint2(wlo[0], wlo[1]);
        *reinterpret_cast<uint2*>(lo + lo_index(m, n + 4, M.np)) = make_uint2(wlo[2], wlo[3]);
      } else {
        *reinterpret_cast<u32x4_t*>(lo + off) = wlo;
      }
    } else {
      float* x0 = reinterpret_cast<float*>(A.ws + M.xo_off[0]) + off;
      reinterpret_cast<f32x4_t*>(x0)[0] = f32x4_t{u[h][0], u[h][1], u[h][2], u[h][3]};
      reinterpret_cast<f32x4_t*>(x0)[1] = f32x4_t{u[h][4], u[h][5], u[h][6], u[h][7]};
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
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      // columns 2d (low halves) and 2d+1 (high halves)
      const uint32_t w0 = comp(r[0], d), w1 = comp(r[1], d), w2 = comp(r[2], d), w3 = comp(r[3], d);
      uint2 lo, hi;
      lo.x = (w0 & 0xffffu) | (w1 << 16);
      lo.y = (w2 & 0xffffu) | (w3 << 16);
      hi.x = (w0 >> 16) | (w1 & 0xffff0000u);
      hi.y = (w2 >> 16) | (w3 & 0xffff0000u);
      const int n0 = ng * 8 + 2 * d;
      *reinterpret_cast<uint2*>(lds + lds_off(n0, kq >> 1) + (kq & 1) * 8) = lo;
      *reinterpret_cast<uint2*>(lds + lds_off(n0 + 1, kq >> 1) + (kq & 1) * 8) = hi;
    }
  } else {
    // k-quad kq covers fp32 k = 4kq..4kq+3: exactly chunk kq
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint4 v = make_uint4(comp(r[0], e), comp(r[1], e), comp(r[2], e), comp(r[3], e));
      *reinterpret_cast<uint4*>(lds + lds_off(ng * 4 + e, kq)) = v;
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
                __uint_as_float(comp(af[i], e)), __uint_as_float(comp(bfr[j], e)), acc[i][j], 0,
                0, 0);
    }
  }
}

// fp32 sets. Item {mat, ti, tj} of 128 x 128 tiles. GRAM/POLY: C = Op Op^T
// on upper-triangle tiles (ti <= tj) mirrored into the lower triangle;
// UPDATE: X = a X + B X on all tiles.
template <typename T, int OP, int KIND>
__global__ __launch_bounds__(256, 1) void gemm32_kernel(StepArgs P) {
  static_assert(OP == OP_F32, "the 128 x 128 engine serves fp32 sets");
  const WorkItem it = P.items[blockIdx.x];
  if (it.mat < 0) return;
  const MatInfo& M = P.mats[it.mat];
  constexpr int ES = Op<OP>::bytes;  // operand element size
  constexpr int KS = ROWB / ES;      // k elements per slab

  __shared__ __attribute__((aligned(16))) char sA[BM * ROWB];
  __shared__ __attribute__((aligned(16))) char sB[BM * ROWB];

  const int ti = it.a, tj = it.b;
  const char* opA;
  const char* opB;
  int64_t lda_b, ldb_b, K;
  if (KIND == GRAM) {  // rows of X (mp x np): A[i][j] = sum_k X[i][k] X[j][k]
    const char* X = P.ws + xo_sel(M, P.cur);
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
    opB = P.ws + xo_sel(M, P.cur) + int64_t(tj) * BM * ES;
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
            const float* xc = reinterpret_cast<const float*>(P.ws + xo_sel(M, P.cur));
            const float v = __fmaf_rn(P.a, xc[off], acc[i][j][r]);
            reinterpret_cast<float*>(P.ws + xo_sel(M, P.cur ^ 1))[off] = v;
          }
        }
    } else {
      // last step: out in the caller's layout and dtype, valid region only
      const float* xsrc = reinterpret_cast<const float*>(P.ws + xo_sel(M, P.cur));
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


// ------------------------------------------- 16-bit operand engine (bf16 sets)
//
// Output tile 256 (rows) x 128 (cols), k-slab 64 elements (128 bytes). Four
// waves in 2 x 2, each owning 128 x 64 = 4 x 2 accumulators of
// v_mfma_f32_32x32x16_{f16,bf16}. The MFMA is fed (column operand, row
// operand), so lane l holds, for accumulator (i, j) and register e,
//   C[m][n], m = row0 + 32 i + l % 32, n = col0 + 32 j + 8 (e / 4) + 4 (l / 32) + e % 4,
// i.e. runs of 4 consecutive output columns: vector epilogue loads/stores.
//   Row operand (k contiguous in memory): LDS [row][k], 128-byte rows.
//   Column operand, k contiguous (Gram, A A):  LDS [col][k], 128-byte rows.
//   Column operand, k along memory rows (X in B X): LDS [k][col], 256-byte
//     rows, read with ds_read_b64_tr_b16: in each 16-lane group, lane s
//     addresses row k0 + s/4, columns c0 + 4(s%4)..+3, and lane i receives
//     column c0 + i of rows k0..k0+3.
// Two LDS stages and two register sets; the loop is unrolled by two so
// stage and register-set choices are constants: multiply stage 0, write the
// next slab (registers) to stage 1, barrier, load the slab three ahead,
// multiply stage 1, and so on.

#ifndef MUON_GEMM_PIPE
#define MUON_GEMM_PIPE 1
#endif

namespace e16 {

constexpr int TM = 256, TN = 128;
// PIPE 2: two LDS stages + two register sets, one workgroup per CU.
// PIPE 1: one LDS stage + one register set, two workgroups per CU.
// PIPE 3: ring of NST direct-to-LDS stages of 32-k slabs (NST <= 3: two
//         workgroups per CU; larger: one).
constexpr int PIPE = MUON_GEMM_PIPE;
#ifndef MUON_GEMM_NST
#define MUON_GEMM_NST 6
#endif
constexpr int NST = MUON_GEMM_NST;
constexpr int WG_PER_CU = (PIPE == 1 || (PIPE == 3 && NST <= 3)) ? 2 : 1;
// PIPE 4: PIPE 2's buffers with one barrier per slab: while slab t is
//         multiplied, slab t+1 goes from registers to the other LDS stage and
//         slab t+3 is loaded into the registers just freed.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int off_rows(int row, int chunk) {   // 128-byte rows
  return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}
// [k][col] tile, 256-byte rows; the XOR spreads the rows touched by one
// transposed read over distinct 32-byte bank groups (2 passes, the minimum)
__device__ __forceinline__ int off_kn(int k, int chunk) {
  return k * 256 + ((chunk ^ (((k ^ ((k >> 3) << 2)) & 7) << 1)) << 4);
}

// Operand slabs are read with buffer loads: a scalar resource descriptor
// per slab (so offsets stay small for any matrix size) and one 32-bit
// per-lane offset, instead of a 64-bit address per load.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const char* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, 0x7fffffff, 0x00020000);
}

template <int R>  // R rows x 128 bytes at base + row*ldb + k0b
__device__ __forceinline__ void load_rows(u32x4 (&r)[R / 32], const char* base, int64_t ldb,
                                          int64_t k0b) {
  const int t = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rs = slab_rsrc(base + k0b);
  const int32_t vo = (t >> 3) * int32_t(ldb) + (t & 7) * 16;
#pragma unroll
  for (int q = 0; q < R / 32; ++q)
    r[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, vo, 32 * q * int32_t(ldb), 0);
}
template <int R>
__device__ __forceinline__ void store_rows(char* lds, const u32x4 (&r)[R / 32]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int q = 0; q < R / 32; ++q)
    *reinterpret_cast<u32x4*>(lds + off_rows((t >> 3) + 32 * q, t & 7)) = r[q];
}
// 64 k-rows x 256 bytes at base + (k0 + k)*ldb
__device__ __forceinline__ void load_kn(u32x4 (&r)[4], const char* base, int64_t ldb, int64_t k0) {
  const int t = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rs = slab_rsrc(base + k0 * ldb);
  const int32_t vo = (t >> 4) * int32_t(ldb) + (t & 15) * 16;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    r[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, vo, 16 * q * int32_t(ldb), 0);
}
__device__ __forceinline__ void store_kn(char* lds, const u32x4 (&r)[4]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<u32x4*>(lds + off_kn((t >> 4) + 16 * q, t & 15)) = r[q];
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

template <int OP>
__device__ __forceinline__ f32x16_t mfma(const u32x4& colop, const u32x4& rowop, f32x16_t c) {
  if constexpr (OP == OP_F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, colop),
                                                  __builtin_bit_cast(f16x8_t, rowop), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, colop),
                                                   __builtin_bit_cast(bf16x8_t, rowop), c, 0, 0, 0);
}

// One 64-k slab of this wave's 128 x 64 block: 4 k-steps of 16.
template <int OP, bool KN>
__device__ __forceinline__ void mma_slab(f32x16_t (&acc)[4][2], const char* sA, const char* sB,
                                         int wm, int wn) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int ch = ks * 2 + lh;  // 16-byte k chunk of this lane half
    u32x4 bf[2], af[4];
    if constexpr (!KN) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bf[j] = *reinterpret_cast<const u32x4*>(sB + off_rows(wn * 64 + j * 32 + l32, ch));
    } else {
      const int s = lane & 15, h = lane >> 4;        // 16-lane group h
      const int krow = ks * 16 + (h >> 1) * 8 + (s >> 2);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = wn * 64 + j * 32 + (h & 1) * 16 + 4 * (s & 3);
        const int chunk = col >> 3, byte = (col & 7) * 2;
        i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(sB + off_kn(krow, chunk) + byte));
        i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(sB + off_kn(krow + 4, chunk) + byte));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        bf[j] = u32x4{l2.x, l2.y, h2.x, h2.y};
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[i] = *reinterpret_cast<const u32x4*>(sA + off_rows(wm * 128 + i * 32 + l32, ch));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma<OP>(bf[j], af[i], acc[i][j]);
  }
}

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d, bool f16) {
  uint2 r;
  if (f16) {
    r.x = uint32_t(Op<OP_F16>::bits(a)) | (uint32_t(Op<OP_F16>::bits(b)) << 16);
    r.y = uint32_t(Op<OP_F16>::bits(c)) | (uint32_t(Op<OP_F16>::bits(d)) << 16);
  } else {
    r.x = uint32_t(f2bf(a)) | (uint32_t(f2bf(b)) << 16);
    r.y = uint32_t(f2bf(c)) | (uint32_t(f2bf(d)) << 16);
  }
  return r;
}



// One 64-k slab like mma_slab, with `hook(ks)` called before each of the 4
// k-steps; used to spread the next slab's LDS stores and global loads over
// the multiplies (sched_barrier keeps each k-step's group together).
template <int OP, bool KN, class Hook>
__device__ __forceinline__ void mma_slab_hooked(f32x16_t (&acc)[4][2], const char* sA,
                                                const char* sB, int wm, int wn, Hook&& hook) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int ch = ks * 2 + lh;
    u32x4 bf[2], af[4];
    if constexpr (!KN) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bf[j] = *reinterpret_cast<const u32x4*>(sB + off_rows(wn * 64 + j * 32 + l32, ch));
    } else {
      const int s = lane & 15, h = lane >> 4;
      const int krow = ks * 16 + (h >> 1) * 8 + (s >> 2);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = wn * 64 + j * 32 + (h & 1) * 16 + 4 * (s & 3);
        const int chunk = col >> 3, byte = (col & 7) * 2;
        i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(sB + off_kn(krow, chunk) + byte));
        i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(sB + off_kn(krow + 4, chunk) + byte));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        bf[j] = u32x4{l2.x, l2.y, h2.x, h2.y};
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[i] = *reinterpret_cast<const u32x4*>(sA + off_rows(wm * 128 + i * 32 + l32, ch));
    hook(ks);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma<OP>(bf[j], af[i], acc[i][j]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---- PIPE 3: direct-to-LDS ring of 32-k slabs (64-byte rows for k-contiguous
// operands, 256-byte rows for the [k][col] operand). Each
// global_load_lds_dwordx4 fills 1 KB of LDS: lane i writes base + 16 i, so
// the XOR swizzle is applied by choosing which global chunk lane i fetches.
__device__ __forceinline__ int off_rows64(int row, int chunk) {
  return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4);
}
typedef __attribute__((address_space(3))) void lds_void_t;

// Issues the DMA of one 32-k slab: row operand R rows (k contiguous), column
// operand either TN rows (k contiguous) or 32 k-rows x TN columns.
template <bool KN>
__device__ __forceinline__ void dma_slab(char* sA, char* sB, const char* opA, int64_t lda,
                                         const char* opB, int64_t ldb, int64_t k0) {
  const int w = threadIdx.x >> 6, i = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < 4; ++q) {  // A: 16 instructions of 16 rows x 64 B
    const int I = w + 4 * q, row = 16 * I + (i >> 2), lch = (i & 3) ^ ((row >> 2) & 3);
    __builtin_amdgcn_global_load_lds(opA + row * lda + k0 * 2 + lch * 16,
                                     (lds_void_t*)(sA + I * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int I = w + 4 * q;
    if constexpr (!KN) {  // 8 instructions of 16 rows x 64 B
      const int row = 16 * I + (i >> 2), lch = (i & 3) ^ ((row >> 2) & 3);
      __builtin_amdgcn_global_load_lds(opB + row * ldb + k0 * 2 + lch * 16,
                                       (lds_void_t*)(sB + I * 1024), 16, 0, 0);
    } else {              // 8 instructions of 4 k-rows x 256 B
      const int kr = 4 * I + (i >> 4);
      const int lch = (i & 15) ^ ((((kr ^ ((kr >> 3) << 2)) & 7)) << 1);
      __builtin_amdgcn_global_load_lds(opB + (k0 + kr) * ldb + lch * 16,
                                       (lds_void_t*)(sB + I * 1024), 16, 0, 0);
    }
  }
}

// One 32-k slab of this wave's 128 x 64 block (2 k-steps of 16).
template <int OP, bool KN>
__device__ __forceinline__ void mma_slab32(f32x16_t (&acc)[4][2], const char* sA, const char* sB,
                                           int wm, int wn) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int ch = ks * 2 + lh;
    u32x4 bf[2], af[4];
    if constexpr (!KN) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bf[j] = *reinterpret_cast<const u32x4*>(sB + off_rows64(wn * 64 + j * 32 + l32, ch));
    } else {
      const int s = lane & 15, h = lane >> 4;
      const int krow = ks * 16 + (h >> 1) * 8 + (s >> 2);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = wn * 64 + j * 32 + (h & 1) * 16 + 4 * (s & 3);
        const int chunk = col >> 3, byte = (col & 7) * 2;
        i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(sB + off_kn(krow, chunk) + byte));
        i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_t*)(sB + off_kn(krow + 4, chunk) + byte));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        bf[j] = u32x4{l2.x, l2.y, h2.x, h2.y};
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[i] = *reinterpret_cast<const u32x4*>(sA + off_rows64(wm * 128 + i * 32 + l32, ch));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma<OP>(bf[j], af[i], acc[i][j]);
  }
}

// s_waitcnt with only the vector-memory counter limited to n (gfx9 encoding).
#define MUON_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0F70)

}  // namespace e16

// bf16 sets. Item {mat, TI, TJ} of 256 x 128 tiles. GRAM/POLY: tiles that
// reach the upper triangle (TJ >= 2 TI); each stored element (m <= n) is
// mirrored to (n, m). UPDATE: X = a X + B X on all tiles.
template <typename T, int OP, int KIND, bool LAST>
__global__ __launch_bounds__(256, e16::WG_PER_CU) void gemm16_kernel(StepArgs P) {
  using namespace e16;
  const WorkItem it = P.items[blockIdx.x];
  if (it.mat < 0) return;
  // Matrix record fields read once into registers: re-reading them after a
  // global store would force a reload (the compiler cannot rule out aliasing).
  struct {
    int32_t m, n, mp, np, tall, vec_ok;
    int64_t ld, a_off, b_off, xl_off, xo_cur, xo_nxt;
    void* out;
  } M;
  {
    const MatInfo& R = P.mats[it.mat];
    M.m = R.m; M.n = R.n; M.mp = R.mp; M.np = R.np; M.tall = R.tall; M.vec_ok = R.vec_ok;
    M.ld = R.ld; M.a_off = R.a_off; M.b_off = R.b_off; M.xl_off = R.xl_off;
    M.xo_cur = xo_sel(R, P.cur); M.xo_nxt = xo_sel(R, P.cur ^ 1); M.out = R.out;
  }
  constexpr bool KN = KIND == UPDATE;

  // LDS: operand stages (PIPE 1: one, PIPE 2: two); reused by the epilogue.
  constexpr int STAGE = (TM + TN) * 128;
  constexpr int STAGE32 = (TM + TN) * 64;  // PIPE 3: 32-k slab
  constexpr int LDS_BYTES = PIPE == 3 ? NST * STAGE32 : (PIPE == 1 ? 1 : 2) * STAGE;
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  char* const sA0 = lds;
  char* const sB0 = lds + TM * 128;
  char* const sA1 = lds + (PIPE == 1 ? 0 : STAGE);  // (PIPE 1/2/4)
  char* const sB1 = sA1 + TM * 128;

  const int TI = it.a, TJ = it.b;
  const char* opA;
  const char* opB;
  int64_t lda, ldb, K;
  if (KIND == GRAM) {
    const char* X = P.ws + M.xo_cur;
    lda = ldb = int64_t(M.np) * 2;
    opA = X + int64_t(TI) * TM * lda;
    opB = X + int64_t(TJ) * TN * ldb;
    K = M.np;
  } else if (KIND == POLY) {
    const char* Am = P.ws + M.a_off;
    lda = ldb = int64_t(M.mp) * 2;
    opA = Am + int64_t(TI) * TM * lda;
    opB = Am + int64_t(TJ) * TN * ldb;
    K = M.mp;
  } else {
    lda = int64_t(M.mp) * 2;
    ldb = int64_t(M.np) * 2;
    opA = P.ws + M.b_off + int64_t(TI) * TM * lda;
    opB = P.ws + M.xo_cur + int64_t(TJ) * TN * 2;
    K = M.mp;
  }

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // Two register sets hold the next two slabs, so each global load has two
  // slabs of multiplies to land before its data is written to LDS.
  u32x4 ra0[TM / 32], rb0[4], ra1[TM / 32], rb1[4];
  auto load = [&](u32x4 (&ra)[TM / 32], u32x4 (&rb)[4], int64_t slab) {
    const int64_t k0 = slab * 64;
    load_rows<TM>(ra, opA, lda, k0 * 2);
    if constexpr (KN) load_kn(rb, opB, ldb, k0);
    else load_rows<TN>(rb, opB, ldb, k0 * 2);
  };
  auto store = [&](const u32x4 (&ra)[TM / 32], const u32x4 (&rb)[4], char* a, char* b) {
    store_rows<TM>(a, ra);
    if constexpr (KN) store_kn(b, rb);
    else store_rows<TN>(b, rb);
  };
  // K is a multiple of 128: an even number (>= 2) of 64-element slabs.
  // Loads past the last slab are clamped to it (valid, unused).
  const int nslab = static_cast<int>(K >> 6);
  if constexpr (PIPE == 4) {
    // per-thread pieces of a slab: A rows in ra[0..7], B rows (or k-rows) in rb[0..3]
    auto st_piece = [&](const u32x4 (&ra)[TM / 32], const u32x4 (&rb)[4], char* a, char* b, int q) {
      const int t = threadIdx.x;
      if (q < 8) {
        *reinterpret_cast<u32x4*>(a + off_rows((t >> 3) + 32 * q, t & 7)) = ra[q];
      } else {
        const int r = q - 8;
        if constexpr (KN) *reinterpret_cast<u32x4*>(b + off_kn((t >> 4) + 16 * r, t & 15)) = rb[r];
        else *reinterpret_cast<u32x4*>(b + off_rows((t >> 3) + 32 * r, t & 7)) = rb[r];
      }
    };
    auto ld_piece = [&](u32x4 (&ra)[TM / 32], u32x4 (&rb)[4], int64_t slab, int q) {
      const int t = threadIdx.x;
      const int64_t k0 = slab * 64;
      if (q < 8) {
        ra[q] = *reinterpret_cast<const u32x4*>(opA + int64_t((t >> 3) + 32 * q) * lda + k0 * 2 + (t & 7) * 16);
      } else {
        const int r = q - 8;
        if constexpr (KN)
          rb[r] = *reinterpret_cast<const u32x4*>(opB + (k0 + (t >> 4) + 16 * r) * ldb + (t & 15) * 16);
        else
          rb[r] = *reinterpret_cast<const u32x4*>(opB + int64_t((t >> 3) + 32 * r) * ldb + k0 * 2 + (t & 7) * 16);
      }
    };
    load(ra0, rb0, 0);
    store(ra0, rb0, sA0, sB0);
    load(ra0, rb0, 1);
    load(ra1, rb1, min(2, nslab - 1));
    __syncthreads();
    for (int t = 0; t < nslab - 2; t += 2) {
      // slab t from stage 0; slab t+1 (ra0) -> stage 1; ra0 <- slab t+3
      mma_slab_hooked<OP, KN>(acc, sA0, sB0, wm, wn, [&](int ks) {
#pragma unroll
        for (int q = 3 * ks; q < 3 * ks + 3; ++q) {
          st_piece(ra0, rb0, sA1, sB1, q);
          ld_piece(ra0, rb0, t + 3, q);
        }
      });
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      // slab t+1 from stage 1; slab t+2 (ra1) -> stage 0; ra1 <- slab t+4
      const int64_t s4 = min(t + 4, nslab - 1);
      mma_slab_hooked<OP, KN>(acc, sA1, sB1, wm, wn, [&](int ks) {
#pragma unroll
        for (int q = 3 * ks; q < 3 * ks + 3; ++q) {
          st_piece(ra1, rb1, sA0, sB0, q);
          ld_piece(ra1, rb1, s4, q);
        }
      });
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    mma_slab_hooked<OP, KN>(acc, sA0, sB0, wm, wn, [&](int ks) {
#pragma unroll
      for (int q = 3 * ks; q < 3 * ks + 3; ++q) st_piece(ra0, rb0, sA1, sB1, q);
    });
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    mma_slab<OP, KN>(acc, sA1, sB1, wm, wn);
  } else if constexpr (PIPE == 3) {
    // ring of NST stages; slab t (32 k) lives in stage t % NST, NST-1 in flight
    const int n32 = static_cast<int>(K >> 5);
    auto stA = [&](int st) { return lds + st * STAGE32; };
    auto stB = [&](int st) { return lds + st * STAGE32 + TM * 64; };
#pragma unroll
    for (int p = 0; p < NST - 1; ++p)
      dma_slab<KN>(stA(p), stB(p), opA, lda, opB, ldb, int64_t(min(p, n32 - 1)) * 32);
    int st = 0;
    for (int t = 0; t < n32; ++t) {
      MUON_WAIT_VMCNT(6 * (NST - 2));  // this wave's loads of slab t are done
      // Everyone's are, and slab t-1 is consumed. A bare s_barrier: the
      // workgroup fence of __syncthreads would wait for all loads in flight;
      // the memory clobber keeps the compiler from moving LDS accesses across.
      asm volatile("s_barrier" ::: "memory");
      const int stn = st == 0 ? NST - 1 : st - 1;  // stage of slab t+NST-1 (= t-1's)
      dma_slab<KN>(stA(stn), stB(stn), opA, lda, opB, ldb,
                   int64_t(min(t + NST - 1, n32 - 1)) * 32);  // past the end: a valid, unused slab
      __builtin_amdgcn_sched_barrier(0);
      mma_slab32<OP, KN>(acc, stA(st), stB(st), wm, wn);
      st = st == NST - 1 ? 0 : st + 1;
    }
    MUON_WAIT_VMCNT(0);  // drain the trailing loads before the LDS is reused
  } else if constexpr (PIPE == 1) {
    load(ra0, rb0, 0);
    for (int t = 0; t < nslab; ++t) {
      __syncthreads();
      store(ra0, rb0, sA0, sB0);
      __syncthreads();
      load(ra0, rb0, min(t + 1, nslab - 1));
      __builtin_amdgcn_sched_barrier(0);
      mma_slab<OP, KN>(acc, sA0, sB0, wm, wn);
    }
  } else {
  load(ra0, rb0, 0);
  store(ra0, rb0, sA0, sB0);
  load(ra0, rb0, 1);
  load(ra1, rb1, min(2, nslab - 1));
  __syncthreads();
  // sched_barrier(0) keeps the compiler from moving the loads past the
  // multiplies that are meant to hide their latency.
  for (int t = 0; t < nslab - 2; t += 2) {
    mma_slab<OP, KN>(acc, sA0, sB0, wm, wn);
    store(ra0, rb0, sA1, sB1);
    __syncthreads();
    load(ra0, rb0, t + 3);
    __builtin_amdgcn_sched_barrier(0);
    mma_slab<OP, KN>(acc, sA1, sB1, wm, wn);
    store(ra1, rb1, sA0, sB0);
    __syncthreads();
    load(ra1, rb1, min(t + 4, nslab - 1));
    __builtin_amdgcn_sched_barrier(0);
  }
  mma_slab<OP, KN>(acc, sA0, sB0, wm, wn);
  store(ra0, rb0, sA1, sB1);
  __syncthreads();
  mma_slab<OP, KN>(acc, sA1, sB1, wm, wn);
  }

  // ---------------------------------------------------------------- epilogue
  // acc[i][j][4 g + r] = C[m][n], m = mb + 32 i + l32, n = nb + 32 j + 8 g + 4 lh + r
  // with mb = TI*256 + wm*128, nb = TJ*128 + wn*64. Each row group i (32 rows
  // x 64 columns per wave) is staged through LDS (fp32, 68-float pitch) so
  // global accesses are row-contiguous: "direct" reads 4 columns of a row,
  // "transposed" reads 8 consecutive rows of one column.
  const int l32 = lane & 31, lh = lane >> 5;
  constexpr bool F16 = OP == OP_F16;
  constexpr int PITCH = 68;
  const int mb = TI * TM + wm * 128, nb = TJ * TN + wn * 64;
  float* const stg = reinterpret_cast<float*>(lds) + wave * (32 * PITCH);
  __syncthreads();  // every wave is done reading the operand stages

  auto stage_acc = [&](auto ic) {
    constexpr int i = decltype(ic)::value;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4_t*>(stg + l32 * PITCH + 32 * j + 8 * g + 4 * lh) =
            f32x4_t{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
  };
  // staging of a run-time row group (one small copy of the stores per group)
  auto stage_acc_rt = [&](int i) {
    switch (i) {
      case 0: stage_acc(std::integral_constant<int, 0>{}); break;
      case 1: stage_acc(std::integral_constant<int, 1>{}); break;
      case 2: stage_acc(std::integral_constant<int, 2>{}); break;
      default: stage_acc(std::integral_constant<int, 3>{}); break;
    }
  };
  // direct access q (0..7): row 4 q + lane / 16 of the group, columns 4 (lane % 16)..+3
  auto drow = [&](int q) { return 4 * q + (lane >> 4); };
  const int dcol = 4 * (lane & 15);
  // transposed access q (0..3): column (lane + 64 q) / 4, rows 8 ((lane + 64 q) % 4)..+7
  auto tcol = [&](int q) { return (lane + 64 * q) >> 2; };
  auto trow = [&](int q) { return 8 * ((lane + 64 * q) & 3); };

  if (KIND == GRAM || KIND == POLY) {
    char* C = P.ws + (KIND == GRAM ? M.a_off : M.b_off);
    const char* Am = P.ws + M.a_off;
    const int64_t ld = M.mp;
    const bool strict = TJ * TN >= (TI + 1) * TM;  // every element above the diagonal
    auto round = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      stage_acc(ic);
      __syncthreads();
      const int m0 = mb + 32 * i;
      // direct rows (POLY: bias loads first, then b A + c acc back into LDS)
      u32x2 bias[8];
      if (KIND == POLY) {
#pragma unroll
        for (int q = 0; q < 8; ++q)
          bias[q] = *reinterpret_cast<const u32x2*>(Am + (int64_t(m0 + drow(q)) * ld + nb + dcol) * 2);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int m = m0 + drow(q), n = nb + dcol;
        f32x4_t v = *reinterpret_cast<const f32x4_t*>(stg + drow(q) * PITCH + dcol);
        if (KIND == POLY) {
          const u32x2 bq = bias[q];
          const float a4[4] = {Op<OP>::load16(bq.x & 0xffffu), Op<OP>::load16(bq.x >> 16),
                               Op<OP>::load16(bq.y & 0xffffu), Op<OP>::load16(bq.y >> 16)};
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = __fmaf_rn(P.c, v[r], P.b * a4[r]);
          if constexpr (OP == OP_F16) {
            // fp16 operands: B' = a I + b A + c A A, so the update is B' X
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (m == n + r && m < M.m) v[r] += P.a;  // padding stays zero
          }
          *reinterpret_cast<f32x4_t*>(stg + drow(q) * PITCH + dcol) = v;
        }
        if (strict || m <= n) {
          *reinterpret_cast<uint2*>(C + (int64_t(m) * ld + n) * 2) = pack4(v[0], v[1], v[2], v[3], F16);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (m <= n + r) Op<OP>::store(C, int64_t(m) * ld + n + r, v[r]);
        }
      }
      if (KIND == POLY) __syncthreads();
      // mirrored rows: C[n][m..m+7] = C[m..m+7][n]
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cc = tcol(q), rr = trow(q);
        const int n = nb + cc, m = m0 + rr;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = stg[(rr + e) * PITCH + cc];
        if (strict || m + 7 < n) {
          const uint2 lo = pack4(v[0], v[1], v[2], v[3], F16), hi = pack4(v[4], v[5], v[6], v[7], F16);
          *reinterpret_cast<uint4*>(C + (int64_t(n) * ld + m) * 2) = make_uint4(lo.x, lo.y, hi.x, hi.y);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (m + e < n) Op<OP>::store(C, int64_t(n) * ld + m + e, v[e]);
        }
      }
      __syncthreads();
    };
    round(std::integral_constant<int, 0>{});
    round(std::integral_constant<int, 1>{});
    round(std::integral_constant<int, 2>{});
    round(std::integral_constant<int, 3>{});
  } else if constexpr (OP == OP_F16) {
    // X' = B' hi + a 2^-11 lo  (B' = a I + B carries the a X term of the high
    // part). lo lives in accumulator order, so no staging is needed.
    const int64_t ldx = M.np;
    uint16_t* lo = reinterpret_cast<uint16_t*>(P.ws + M.xl_off) +
                   (((int64_t(TI) * (M.np >> 7) + TJ) * 4 + wave) * 32) * 256 + lane * 4;
    char* xn = P.ws + M.xo_nxt;
    const float a2 = P.a * (1.f / 2048.f);
    auto round = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      u32x2 lv[2][4];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          lv[j][g] = *reinterpret_cast<const u32x2*>(lo + ((i * 2 + j) * 4 + g) * 256);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t lw[4] = {lv[j][g].x & 0xffffu, lv[j][g].x >> 16, lv[j][g].y & 0xffffu,
                                  lv[j][g].y >> 16};
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[i][j][4 * g + r] = __fmaf_rn(a2, Op<OP>::load16(lw[r]), acc[i][j][4 * g + r]);
          if constexpr (!LAST) {
            const int m = mb + 32 * i + l32, n0 = nb + 32 * j + 8 * g + 4 * lh;
            uint32_t nh[4], nl[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) Op<OP>::split(acc[i][j][4 * g + r], nh[r], nl[r]);
            *reinterpret_cast<uint2*>(xn + (int64_t(m) * ldx + n0) * 2) =
                make_uint2(nh[0] | (nh[1] << 16), nh[2] | (nh[3] << 16));
            *reinterpret_cast<uint2*>(lo + ((i * 2 + j) * 4 + g) * 256) =
                make_uint2(nl[0] | (nl[1] << 16), nl[2] | (nl[3] << 16));
          }
        }
    };
    round(std::integral_constant<int, 0>{});
    round(std::integral_constant<int, 1>{});
    round(std::integral_constant<int, 2>{});
    round(std::integral_constant<int, 3>{});
    if constexpr (LAST) {
      // `out` in the caller's layout: stage X' through LDS
      T* o = static_cast<T*>(M.out);
      auto out_round = [&](auto ic) {
        constexpr int i = decltype(ic)::value;
        stage_acc(ic);
        __syncthreads();
        const int m0 = mb + 32 * i;
        if (!M.tall) {
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int m = m0 + drow(q), n = nb + dcol;
            if (m >= M.m) continue;
            const f32x4_t x = *reinterpret_cast<const f32x4_t*>(stg + drow(q) * PITCH + dcol);
            const int64_t co = int64_t(m) * M.ld + n;
            if (M.vec_ok && n + 3 < M.n) {
              if constexpr (sizeof(T) == 2)
                *reinterpret_cast<uint2*>(o + co) = pack4(x[0], x[1], x[2], x[3], false);
              else
                *reinterpret_cast<f32x4_t*>(o + co) = x;
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (n + r < M.n) Elem<T>::store(o, co + r, x[r]);
            }
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int cc = tcol(q), rr = trow(q);
            const int n = nb + cc, m = m0 + rr;
            if (n >= M.n) continue;
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = stg[(rr + e) * PITCH + cc];
            const int64_t co = int64_t(n) * M.ld + m;
            if (M.vec_ok && m + 7 < M.m) {
              if constexpr (sizeof(T) == 2) {
                const uint2 l4 = pack4(v[0], v[1], v[2], v[3], false), h4 = pack4(v[4], v[5], v[6], v[7], false);
                *reinterpret_cast<uint4*>(o + co) = make_uint4(l4.x, l4.y, h4.x, h4.y);
              } else {
                *reinterpret_cast<f32x4_t*>(o + co) = f32x4_t{v[0], v[1], v[2], v[3]};
                *reinterpret_cast<f32x4_t*>(o + co + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
              }
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (m + e < M.m) Elem<T>::store(o, co + e, v[e]);
            }
          }
        }
        __syncthreads();
      };
      out_round(std::integral_constant<int, 0>{});
      out_round(std::integral_constant<int, 1>{});
      out_round(std::integral_constant<int, 2>{});
      out_round(std::integral_constant<int, 3>{});
    }
  } else {
    const int64_t ldx = M.np;
    const char* xh = P.ws + M.xo_cur;      // hi part of X (operand)
    char* xl = P.ws + M.xl_off;                      // lo part, updated in place
    char* xn = P.ws + M.xo_nxt;        // next hi part
    T* o = static_cast<T*>(M.out);
auto round = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      __builtin_amdgcn_sched_barrier(0);  // keep each round's loads inside it
      stage_acc(ic);
      __syncthreads();
      const int m0 = mb + 32 * i;
#pragma unroll
      for (int qb = 0; qb < 8; qb += 4) {
      u32x2 hv[8], lv[8];
#pragma unroll
      for (int q = qb; q < qb + 4; ++q) {
        const int64_t off = int64_t(m0 + drow(q)) * ldx + nb + dcol;
        hv[q] = *reinterpret_cast<const u32x2*>(xh + off * 2);
        lv[q] = *reinterpret_cast<const u32x2*>(xl + off * 2);
      }
#pragma unroll
      for (int q = qb; q < qb + 4; ++q) {
        const int m = m0 + drow(q), n = nb + dcol;
        const int64_t off = int64_t(m) * ldx + n;
        f32x4_t x = *reinterpret_cast<const f32x4_t*>(stg + drow(q) * PITCH + dcol);
        const uint32_t hw[4] = {hv[q].x & 0xffffu, hv[q].x >> 16, hv[q].y & 0xffffu, hv[q].y >> 16};
        const uint32_t lw[4] = {lv[q].x & 0xffffu, lv[q].x >> 16, lv[q].y & 0xffffu, lv[q].y >> 16};
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = __fmaf_rn(P.a, Op<OP>::join(hw[r], lw[r]), x[r]);
        if constexpr (!LAST) {
          uint32_t nh[4], nl[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) Op<OP>::split(x[r], nh[r], nl[r]);
          *reinterpret_cast<uint2*>(xn + off * 2) = make_uint2(nh[0] | (nh[1] << 16), nh[2] | (nh[3] << 16));
          *reinterpret_cast<uint2*>(xl + off * 2) = make_uint2(nl[0] | (nl[1] << 16), nl[2] | (nl[3] << 16));
        } else if (!M.tall) {
          // last step, rows<=cols matrix: `out` rows m, columns n..n+3
          if (m < M.m) {
            const int64_t co = int64_t(m) * M.ld + n;
            if (M.vec_ok && n + 3 < M.n) {
              if constexpr (sizeof(T) == 2)
                *reinterpret_cast<uint2*>(o + co) = pack4(x[0], x[1], x[2], x[3], false);
              else
                *reinterpret_cast<f32x4_t*>(o + co) = x;
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (n + r < M.n) Elem<T>::store(o, co + r, x[r]);
            }
          }
        } else {
          *reinterpret_cast<f32x4_t*>(stg + drow(q) * PITCH + dcol) = x;  // for the transposed write
        }
      }
      }
      if (LAST && M.tall) {
        __syncthreads();
        // `out` is the transpose: out rows n, columns m..m+7
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int cc = tcol(q), rr = trow(q);
          const int n = nb + cc, m = m0 + rr;
          if (n >= M.n) continue;
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = stg[(rr + e) * PITCH + cc];
          const int64_t co = int64_t(n) * M.ld + m;
          if (M.vec_ok && m + 7 < M.m) {
            if constexpr (sizeof(T) == 2) {
              const uint2 lo = pack4(v[0], v[1], v[2], v[3], false), hi = pack4(v[4], v[5], v[6], v[7], false);
              *reinterpret_cast<uint4*>(o + co) = make_uint4(lo.x, lo.y, hi.x, hi.y);
            } else {
              *reinterpret_cast<f32x4_t*>(o + co) = f32x4_t{v[0], v[1], v[2], v[3]};
              *reinterpret_cast<f32x4_t*>(o + co + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (m + e < M.m) Elem<T>::store(o, co + e, v[e]);
          }
        }
      }
      __syncthreads();
    };
    round(std::integral_constant<int, 0>{});
    round(std::integral_constant<int, 1>{});
    round(std::integral_constant<int, 2>{});
    round(std::integral_constant<int, 3>{});
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
    case MUON_K_GRAM:
      if constexpr (OP == OP_F32) hipLaunchKernelGGL((gemm32_kernel<T, OP, GRAM>), g, b, 0, s, a);
      else hipLaunchKernelGGL((gemm16_kernel<T, OP, GRAM, false>), g, b, 0, s, a);
      break;
    case MUON_K_POLY:
      if constexpr (OP == OP_F32) hipLaunchKernelGGL((gemm32_kernel<T, OP, POLY>), g, b, 0, s, a);
      else hipLaunchKernelGGL((gemm16_kernel<T, OP, POLY, false>), g, b, 0, s, a);
      break;
    case MUON_K_UPDATE:
      if constexpr (OP == OP_F32) hipLaunchKernelGGL((gemm32_kernel<T, OP, UPDATE>), g, b, 0, s, a);
      else if (a.last) hipLaunchKernelGGL((gemm16_kernel<T, OP, UPDATE, true>), g, b, 0, s, a);
      else hipLaunchKernelGGL((gemm16_kernel<T, OP, UPDATE, false>), g, b, 0, s, a);
      break;
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
