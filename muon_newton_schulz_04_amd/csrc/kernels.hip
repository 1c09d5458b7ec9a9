// gfx950 (CDNA4) kernels of the Muon update.
//
//   momentum_kernel   buf' = mu buf + G, u = G + mu buf' | buf' | G, and one
//                     fixed-order sum of u^2 per work item        (HBM-bound)
//   normalize_kernel  X0 = u / (sqrt(sum u^2) + eps) in the rows<=cols
//                     orientation, zero-padded: fp32 sets an fp32 master,
//                     bf16 sets a 16-bit operand (hi, in 32-column panels)
//                     and a low part (lo)                          (HBM-bound)
//   gemm*_kernel<GRAM>   A = X X^T          upper-triangle tiles, mirrored
//                                           (small bf16 sets: long k loops
//                                           split into parts, summed in a
//                                           second pass)
//   gemm*_kernel<POLY>   B = b A + c A A    upper-triangle tiles, mirrored
//   gemm*_kernel<UPDATE> X = a X + B X      the last step writes `out`, or
//                                           applies X to the weights
//
// Two matrix-core engines:
//  - gemm32_kernel (fp32 sets): 128 x 128 output tiles, 4 waves each owning
//    64 x 64 as 4 x 4 v_mfma_f32_16x16x4_f32 accumulators, operands staged
//    through LDS from registers (the next k-slab prefetched while the
//    current one is multiplied).
//  - gemm16_kernel (bf16 sets; fp16 operands by default): 256 x 256 output
//    tiles, 8 waves, operands DMA'd straight into a 4-stage LDS ring (see
//    the section below); X kept as an fp16 high part plus an e4m3 low byte.
//
// Every launch takes a schedule of work items; block b runs item b. The
// schedules keep one matrix's tiles on one XCD (block b runs on XCD b % 8).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "launch.hpp"

namespace muon {

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
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const void* p, int64_t i) {
    return bf2f(static_cast<const uint16_t*>(p)[i]);
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = f2bf(v);
  }
};

// Operand formats of the matrix products (X, A, B in the workspace).
enum OpFmt { OP_F32 = 0, OP_F16 = 1 };
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
  static __device__ __forceinline__ float load16(uint32_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
  }
  // The X master of fp16-operand sets: X = hi + lo 2^-18 with hi = RN16(X)
  // and lo one byte, the OCP e4m3 rounding (to nearest even) of
  // (X - hi) 2^18: 4 significant bits below hi's last one. Validation keeps
  // every iterate's entries below 2 in magnitude (singular values of the
  // accepted polynomials stay in [-2, 2]), so |X - hi| <= ulp(hi) / 2 <=
  // 2^-10 and |lo| <= 2^8, inside the format's range (448).
  static constexpr float kLoScale = 262144.f;  // 2^18
  // the four lo bytes of residuals r0..r3 (x - hi, exact in fp32), byte q
  // holding r_q: gfx950's scaled conversion divides by its scale operand,
  // so a scale of 2^-18 gives e4m3(r 2^18) in one instruction per pair
  // (bitwise the separate multiply and conversion)
  static __device__ __forceinline__ uint32_t lo4(float r0, float r1, float r2, float r3) {
    typedef short s2_t __attribute__((ext_vector_type(2)));
    const s2_t z = {0, 0};
    const s2_t a = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, r0, r1, 1.f / kLoScale, false);
    const s2_t b = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(a, r2, r3, 1.f / kLoScale, true);
    return __builtin_bit_cast(uint32_t, b);
  }
  // the four lo bytes of w as floats (lo, not yet scaled by 2^-18), two per
  // conversion
  static __device__ __forceinline__ void lo_vals(uint32_t w, float (&v)[4]) {
    typedef float f2_t __attribute__((ext_vector_type(2)));
    const int x = static_cast<int>(w);
    const f2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(x, false);
    const f2_t b = __builtin_amdgcn_cvt_pk_f32_fp8(x, true);
    v[0] = a.x;
    v[1] = a.y;
    v[2] = b.x;
    v[3] = b.y;
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

// Sums of squares relative to a power of two: a partial sum s with exponent
// e stands for s 4^e, e being the exponent of the largest |u| it covers, so
// its terms stay below 4 and no finite u overflows fp32 (a plain fp32 sum of
// u^2 does once entries pass about 2^60). Scaling by powers of two is exact,
// so away from fp32's range limits every partial, and the norm, is bitwise
// that of the plain sum in the same order.
// The exponent e of x in [2^e, 2^(e+1)), clamped to [-126, 126]; 0 for
// zero, NaN and infinities.
__device__ __forceinline__ int exp_of(float x) {
  if (!(x > 0.f) || !(x <= 3.40282347e38f)) return 0;
  const int e = static_cast<int>((__float_as_uint(x) >> 23) & 255u) - 127;
  return min(max(e, -126), 126);
}
// 2^k for k in [-126, 127]
__device__ __forceinline__ float pow2i(int k) { return __uint_as_float(static_cast<uint32_t>(k + 127) << 23); }
// Running sum of squares of one thread, relative to 4^e (e the largest
// exponent seen so far, starting at -126).
struct ScaledSsq {
  float s = 0.f;
  int e = -126;
  __device__ __forceinline__ void add(float u) {
    const int eu = exp_of(fabsf(u));
    if (u != 0.f && eu > e) {  // rescale what was summed so far (exact unless it underflows)
      s = ldexpf(s, 2 * (e - eu));
      e = eu;
    }
    const float x = u * pow2i(-e);
    s = __fmaf_rn(x, x, s);
  }
};
// Block combination of the threads' scaled sums (fixed order): {s, e}.
__device__ __forceinline__ ScaledSsq block_ssq_256(ScaledSsq t, float* red, int* ered) {
  int e = t.e;
  for (int o = 32; o > 0; o >>= 1) e = max(e, __shfl_xor(e, o, 64));
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) ered[w] = e;
  __syncthreads();
  ScaledSsq r;
  r.e = max(max(ered[0], ered[1]), max(ered[2], ered[3]));
  r.s = block_sum_256(ldexpf(t.s, 2 * (t.e - r.e)), red);
  return r;
}

// StepArgs (kernel arguments) is declared in launch.hpp.

// Component e (compile-time after unrolling) of a 16-byte register vector.
__device__ __forceinline__ uint32_t comp(const uint4& v, int e) {
  return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

// The 16-bit matrix-core operands of bf16 sets (X's high part, A and B) are
// stored in 32-column panels: panel p holds columns 32 p .. 32 p + 31 of
// every row, 64 bytes per row, rows consecutive. Element (r, c) of a matrix
// with `rows` (padded) rows is at this element index. A 32-k stage of 256
// rows is then one contiguous 16 KB run, and 32 k-rows of a column block are
// whole 128-byte lines, so every LDS DMA request of the engine is a full
// cache line.
__device__ __forceinline__ int64_t pidx(int r, int c, int rows) {
  return (int64_t(c >> 5) * rows + r) * 32 + (c & 31);
}

// Offset of operand buffer `which` (0/1) without indexing the record's
// array by a run-time value (which would move the record to scratch).
__device__ __forceinline__ int64_t xo_sel(const MatInfo& M, int which) {
  return which ? M.xo_off[1] : M.xo_off[0];
}

// Weight application: W' = W (1 - lr' wd') - lr' x with lr' = lr lr_mul and
// wd' = wd wd_mul, in fp32.
struct WApply {
  float keep, step;  // 1 - lr' wd', lr'
  __device__ __forceinline__ WApply(const StepArgs& A, const MatInfo& M)
      : keep(1.f - (A.lr * M.lr_mul) * (A.wd * M.wd_mul)), step(A.lr * M.lr_mul) {}
  __device__ __forceinline__ float operator()(float w, float x) const {
    return __fmaf_rn(-step, x, w * keep);
  }
};

// buf' = mu buf + g rounded once to the buffer's type, returned as a float
// (the caller stores it; the store is exact). For fp32 state the fused
// multiply-add is that rounding. For bf16 state s = fma(mu, b, g) is the
// float32 nearest to the exact value, and rounding s to bf16 (ties to even)
// gives the bf16 nearest to the exact value unless s lies exactly halfway
// between two bf16 values while the exact value does not (double rounding).
// Then the sign of the residual (mu b + g) - s decides, evaluated exactly
// in float64: mu b is exact there (at most 32 significant bits), the sum
// with g splits into its rounded value S and exact error E (Knuth's
// TwoSum), and S - s is exact (the two are within a factor of two:
// Sterbenz's lemma), so (S - s) + E has the residual's sign. s then moves
// one float32 ulp toward the exact value, off the halfway point, before the
// bf16 rounding. The float64 path runs only on halfway points.
__device__ __forceinline__ float momentum_bf16(float mu, float b, float g) {
  const float s = __fmaf_rn(mu, b, g);
  const uint32_t bits = __float_as_uint(s);
  if ((bits & 0xffffu) == 0x8000u) {
    const double P = __dmul_rn(double(mu), double(b));
    const double S = __dadd_rn(P, double(g));
    const double bb = __dsub_rn(S, P);
    const double E = __dadd_rn(__dsub_rn(P, __dsub_rn(S, bb)), __dsub_rn(double(g), bb));
    const double d = __dadd_rn(__dsub_rn(S, double(s)), E);
    if (d != 0.0 && d == d) {
      const bool away = (d > 0.0) == (s > 0.0);  // toward the exact value
      return bf2f(f2bf(__uint_as_float(away ? bits + 1u : bits - 1u)));
    }
  }
  return bf2f(f2bf(s));
}
template <typename T>
__device__ __forceinline__ float momentum_new(float mu, float b, float g) {
  if constexpr (sizeof(T) == 2) return momentum_bf16(mu, b, g);
  else return __fmaf_rn(mu, b, g);
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
  ScaledSsq acc;
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
          const float nb = momentum_new<T>(A.mu, Elem<T>::load(be, e), gf);
          Elem<T>::store(oe, e, nb);
          acc.add(form_u(gf, nb, A));
        }
        *reinterpret_cast<uint4*>(mb + off) = ov;
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) acc.add(Elem<T>::load(ge, e));
      }
    }
  } else {
    const int32_t ne = nr * M.cols;
    for (int32_t e = threadIdx.x; e < ne; e += 256) {
      const int64_t off = int64_t(r0 + e / M.cols) * M.ld + (e % M.cols);
      const float gf = Elem<T>::load(g, off);
      float u = gf;
      if (A.use_mom) {
        const float nb = momentum_new<T>(A.mu, Elem<T>::load(mb, off), gf);
        Elem<T>::store(mb, off, nb);
        u = form_u(gf, nb, A);
      }
      acc.add(u);
    }
  }
  __shared__ float red[4];
  __shared__ int ered[4];
  const ScaledSsq b = block_ssq_256(acc, red, ered);
  if (threadIdx.x == 0) {
    A.parts[it.c] = b.s;
    A.part_exp[it.c] = static_cast<float>(b.e);
  }
}

// -------------------------------------------------------- normalize kernel
//
// Item {mat, ti, tj}: a 64 x 64 tile of X0 in the rows<=cols orientation
// (rows ti*64.., cols tj*64.. of the mp x np padded layout). The caller-side
// tile (transposed for tall matrices) is read into LDS, scaled, and written
// out row-major, zeros in the padding. With zero steps the scaled values go
// straight to `out` in the caller's layout.

// fp16 operand sets keep the low byte of X (Op<OP_F16>::lo4) in the update
// kernel's accumulator order: per 256 x TN tile (TM * TN bytes), per 32-row
// block u, per wave column wn and accumulator column block j, a 1 KB run
// holds 16 bytes per lane: lane l32 + 32 lh has row 32 u + l32, columns
// 64 wn + 32 j + 8 g + 4 lh + r at byte 4 g + r. One 16-byte load or store
// per lane and accumulator block, contiguous across the wave. Byte offset
// of X(m, n) (np = padded row length):
__device__ __forceinline__ int64_t lo8_index(int m, int n, int np) {
  constexpr int TN = kTileN16, WN = TN / 64;
  const int tile = (m >> 8) * (np / TN) + n / TN;
  const int mm = m & 255, nn = n % TN;
  const int lane = (mm & 31) + 32 * ((nn >> 2) & 1);
  return ((((int64_t(tile) * 8 + (mm >> 5)) * WN + (nn >> 6)) * 2 + ((nn >> 5) & 1)) * 64 + lane) * 16 +
         ((nn >> 3) & 3) * 4 + (nn & 3);
}

template <typename T, int OP>
__global__ __launch_bounds__(256) void normalize_kernel(StepArgs A) {
  const WorkItem it = A.items[blockIdx.x];
  if (it.mat < 0) return;
  const MatInfo& M = A.mats[it.mat];
  __shared__ float red[4];
  __shared__ float tile[64][65];

  // 1. scale from this matrix's partial sums (each relative to 4^e), in
  //    slot order, relative to 4^E for the largest e
  __shared__ int ered[4];
  int E = -126;
  for (int32_t p = threadIdx.x; p < M.part_cnt; p += 256) E = max(E, static_cast<int>(A.part_exp[M.part_off + p]));
  for (int o = 32; o > 0; o >>= 1) E = max(E, __shfl_xor(E, o, 64));
  if ((threadIdx.x & 63) == 0) ered[threadIdx.x >> 6] = E;
  __syncthreads();
  E = max(max(ered[0], ered[1]), max(ered[2], ered[3]));
  float s = 0.f;
  for (int32_t p = threadIdx.x; p < M.part_cnt; p += 256)
    s += ldexpf(A.parts[M.part_off + p], 2 * (static_cast<int>(A.part_exp[M.part_off + p]) - E));
  s = block_sum_256(s, red);
  const float scale = 1.0f / (ldexpf(sqrtf(s), E) + A.eps);

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
    const WApply wa(A, M);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int v = threadIdx.x + 256 * h;
      const int32_t cr = cr0 + (v >> 3), cc = cc0 + (v & 7) * 8;
      if (cr >= M.rows) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (cc + e >= M.cols) continue;
        if (A.apply) {
          const int64_t wi = int64_t(cr) * M.wld + cc + e;
          Elem<T>::store(M.w, wi, wa(Elem<T>::load(M.w, wi), u[h][e]));
        } else {
          Elem<T>::store(M.out, int64_t(cr) * M.ld + cc + e, u[h][e]);
        }
      }
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
      const int64_t poff = pidx(i0 + (v >> 3), j0 + (v & 7) * 8, M.mp);
      u32x4_t whi;  // the high parts; the low bytes go out below
#pragma unroll
      for (int q = 0; q < 4; ++q)
        whi[q] = uint32_t(Op<OP>::bits(u[h][2 * q])) | (uint32_t(Op<OP>::bits(u[h][2 * q + 1])) << 16);
      *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(A.ws + M.xo_off[0]) + poff) = whi;
    } else {
      float* x0 = reinterpret_cast<float*>(A.ws + M.xo_off[0]) + off;
      reinterpret_cast<f32x4_t*>(x0)[0] = f32x4_t{u[h][0], u[h][1], u[h][2], u[h][3]};
      reinterpret_cast<f32x4_t*>(x0)[1] = f32x4_t{u[h][4], u[h][5], u[h][6], u[h][7]};
    }
  }
  if constexpr (OP == OP_F16) {
    // Low bytes in accumulator order. Each 32-row half of this tile is one
    // contiguous 2 KB run of that layout (64 columns: one wave column, both
    // column blocks j); thread t writes the 16 bytes of lane t % 64 of block
    // j = t / 64 % 2 of half b = t / 128: row 32 b + t % 32, columns
    // 32 j + 8 g + 4 (t / 32 % 2) + r at byte 4 g + r.
    __syncthreads();  // the tall path above has finished reading the tile
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int v = threadIdx.x + 256 * h;
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[v >> 3][(v & 7) * 8 + e] = u[h][e];
    }
    __syncthreads();
    const int t = threadIdx.x, b = t >> 7, j = (t >> 6) & 1, ln = t & 63;
    const int row = 32 * b + (ln & 31), col = 32 * j + 4 * (ln >> 5);
    uint32_t w[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float r[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float x = tile[row][col + 8 * g + q];
        r[q] = x - Op<OP>::load16(Op<OP>::bits(x));
      }
      w[g] = Op<OP>::lo4(r[0], r[1], r[2], r[3]);
    }
    char* lo = A.ws + M.xl_off + lo8_index(i0 + 32 * b, j0, M.np);
    *reinterpret_cast<u32x4_t*>(lo + (j * 64 + ln) * 16) = u32x4_t{w[0], w[1], w[2], w[3]};
  }
}

// ------------------------------------------ X0's operand of bf16 sets
//
// With at least one Newton-Schulz step, bf16 sets do not store X0 = u /
// (||u|| + eps) itself (the norm is known only after a pass over u): the
// momentum pass stores U = u p, p a power of two, as its fp16 rounding hi
// (the matrix-core operand) and one e4m3 byte holding (U - hi) 2^5, and
// the first Gram and update scale their fp32 sums by sigma^2 and sigma,
// sigma = 1 / ((||u|| + eps) p). p puts the matrix's largest |u| in
// [2^12, 2^13): fp16's range holds it, entries down to 2^-26 of the largest
// stay normal fp16 numbers, and |U - hi| <= 2 keeps the byte below 64. The
// momentum pass takes p from the previous call's largest |u| (a hint the
// plan keeps); the scale pass compares it with the p of this call's largest
// |u| and the operand and bytes of the matrices where the two differ are
// written again, so they depend on this call's inputs only. The byte
// matters: the polynomial amplifies X0's rounding noise in the directions
// of small singular values by up to a^k, which an fp16 X0 alone leaves far
// above the bf16 tolerance for low-rank inputs.

// 2^k with mx 2^k in [2^12, 2^13) (k clamped to normal floats); 1 when mx
// is zero, NaN or infinite.
__device__ __forceinline__ float x0_pow2(float mx) {
  if (!(mx > 0.f) || !(mx <= 3.40282347e38f)) return 1.f;
  const int e = static_cast<int>((__float_as_uint(mx) >> 23) & 255u) - 127;
  const int k = min(max(12 - e, -126), 126);
  return __uint_as_float(static_cast<uint32_t>(k + 127) << 23);
}

// max that keeps a NaN once seen
__device__ __forceinline__ float nan_max(float m, float v) { return (v > m || v != v) ? v : m; }

__device__ __forceinline__ float block_max_256(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = nan_max(v, __shfl_xor(v, o, 64));
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  return nan_max(nan_max(red[0], red[1]), nan_max(red[2], red[3]));
}

// u of one 64 x 64 tile of X0's orientation, read from the caller's layout
// (caller rows cr0.., columns cc0..; transposed for tall matrices): thread t
// holds two runs of 8 consecutive caller columns, run h at caller row
// (t + 256 h) / 8 of the tile and columns 8 (t % 8) ... Zero outside the
// matrix. STEP: the momentum step happens here (buf' written back);
// otherwise u is formed from the stored buf'.
template <bool STEP>
__device__ __forceinline__ void tile_u_bf16(const StepArgs& A, const MatInfo& M, int32_t cr0, int32_t cc0,
                                            float (&u)[2][8]) {
  const uint16_t* g = static_cast<const uint16_t*>(M.grad);
  uint16_t* mb = static_cast<uint16_t*>(M.mom);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int v = threadIdx.x + 256 * h;
    const int32_t cr = cr0 + (v >> 3), cc = cc0 + (v & 7) * 8;
    const int64_t off = int64_t(cr) * M.ld + cc;
    if (cr < M.rows && M.vec_ok && cc + 8 <= M.cols) {
      const u32x4_t gw = *reinterpret_cast<const u32x4_t*>(g + off);
      u32x4_t bw = {0u, 0u, 0u, 0u};
      if (A.use_mom) bw = *reinterpret_cast<const u32x4_t*>(mb + off);
      u32x4_t nw = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gf = bf2f(static_cast<uint16_t>(gw[e >> 1] >> (16 * (e & 1))));
        float nb = bf2f(static_cast<uint16_t>(bw[e >> 1] >> (16 * (e & 1))));
        if (STEP && A.use_mom) {
          nb = momentum_new<uint16_t>(A.mu, nb, gf);
          nw[e >> 1] |= uint32_t(f2bf(nb)) << (16 * (e & 1));
        }
        u[h][e] = form_u(gf, nb, A);
      }
      if (STEP && A.use_mom) *reinterpret_cast<u32x4_t*>(mb + off) = nw;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = 0.f;
        if (cr < M.rows && cc + e < M.cols) {
          const float gf = bf2f(g[off + e]);
          float nb = A.use_mom ? bf2f(mb[off + e]) : 0.f;
          if (STEP && A.use_mom) {
            nb = momentum_new<uint16_t>(A.mu, nb, gf);
            mb[off + e] = f2bf(nb);
          }
          x = form_u(gf, nb, A);
        }
        u[h][e] = x;
      }
    }
  }
}

// U = u p of the tile at rows i0.., columns j0.. of X0's orientation: its
// fp16 rounding into the first operand buffer (panels; tall tiles are
// transposed through LDS) and the byte e4m3((U - hi) 2^5) into the low-byte
// layout (accumulator order, as the update reads it).
constexpr float kX0LoScale = 32.f;  // 2^5
__device__ __forceinline__ void tile_store_x0(const StepArgs& A, const MatInfo& M, int32_t i0, int32_t j0,
                                              float (&u)[2][8], float p, float (*tile)[65]) {
  if (M.tall) {
    __syncthreads();  // an earlier tile's reads of `tile` are done
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
  uint16_t* x = reinterpret_cast<uint16_t*>(A.ws + M.xo_off[0]);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int v = threadIdx.x + 256 * h;
    u32x4_t w;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u[h][2 * q] *= p;  // exact: a power of two
      u[h][2 * q + 1] *= p;
      w[q] = uint32_t(Op<OP_F16>::bits(u[h][2 * q])) | (uint32_t(Op<OP_F16>::bits(u[h][2 * q + 1])) << 16);
    }
    *reinterpret_cast<u32x4_t*>(x + pidx(i0 + (v >> 3), j0 + (v & 7) * 8, M.mp)) = w;
  }
  // Low bytes in accumulator order: each 32-row half of the tile is one
  // contiguous 2 KB run of that layout (64 columns: one wave column, both
  // column blocks j); thread t writes the 16 bytes of lane t % 64 of block
  // j = t / 64 % 2 of half b = t / 128: row 32 b + t % 32, columns
  // 32 j + 8 g + 4 (t / 32 % 2) + r at byte 4 g + r.
  __syncthreads();  // the tall path above has finished reading the tile
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int v = threadIdx.x + 256 * h;
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[v >> 3][(v & 7) * 8 + e] = u[h][e];
  }
  __syncthreads();
  const int t = threadIdx.x, b = t >> 7, j = (t >> 6) & 1, ln = t & 63;
  const int row = 32 * b + (ln & 31), col = 32 * j + 4 * (ln >> 5);
  uint32_t w[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float U = tile[row][col + 8 * g + q];
      // U - hi is exact; 2^5 / 2^18 puts it at lo4's fixed 2^18
      r[q] = (U - Op<OP_F16>::load16(Op<OP_F16>::bits(U))) * (kX0LoScale / Op<OP_F16>::kLoScale);
    }
    w[g] = Op<OP_F16>::lo4(r[0], r[1], r[2], r[3]);
  }
  char* lo = A.ws + M.xl_off + lo8_index(i0 + 32 * b, j0, M.np);
  *reinterpret_cast<u32x4_t*>(lo + (j * 64 + ln) * 16) = u32x4_t{w[0], w[1], w[2], w[3]};
}

// Momentum step and X0's operand in one pass. Item {mat, ti, tj}: one 64 x
// 64 tile of mp x np (X0's orientation; tiles in the padding store zeros).
// Per tile: the largest |u| and the sum of u^2 relative to 4^e for e its
// exponent (each thread's 16 terms in order, then the block's fixed tree).
__global__ __launch_bounds__(256) void momentum_x0_kernel(StepArgs A) {
  const WorkItem it = A.items[blockIdx.x];
  if (it.mat < 0) return;
  const MatInfo& M = A.mats[it.mat];
  __shared__ float red[4];
  __shared__ float tile[64][65];
  const int32_t i0 = it.a * 64, j0 = it.b * 64;
  float u[2][8];
  tile_u_bf16<true>(A, M, M.tall ? j0 : i0, M.tall ? i0 : j0, u);
  float mx = 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = nan_max(mx, fabsf(u[h][e]));
  mx = block_max_256(mx, red);
  // the tile's sum of squares relative to 4^e, e = exp_of(largest |u|)
  const float inv = pow2i(-exp_of(mx));
  float ss = 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = u[h][e] * inv;
      ss = __fmaf_rn(x, x, ss);
    }
  ss = block_sum_256(ss, red);
  const float p = x0_pow2(A.hint[it.mat]);
  if (threadIdx.x == 0) {
    const int32_t slot = M.tile_off + it.a * (M.np / 64) + it.b;
    reinterpret_cast<float*>(A.ws + A.tsum_off)[slot] = ss;
    reinterpret_cast<float*>(A.ws + A.tmax_off)[slot] = mx;
    if (it.a == 0 && it.b == 0) reinterpret_cast<float*>(A.ws + A.x0s_off)[4 * it.mat + 2] = p;
  }
  tile_store_x0(A, M, i0, j0, u, p, tile);
}

// Scale pass. Item {mat}: one workgroup per matrix takes the largest |u|
// and sums its tile sums (fixed order), then stores {sigma, p, p of the
// momentum pass, rewrite flag} and the new hint. The flag is set where the
// momentum pass's p differs from this one. With a chained schedule it also
// clears the matrix's completion counter (and block 0 the tickets).
__global__ __launch_bounds__(256) void x0_scale_kernel(StepArgs A) {
  const WorkItem it = A.items[blockIdx.x];
  if (A.chain_off >= 0 && threadIdx.x < kNumXcd + 1) {
    int32_t* ctr = reinterpret_cast<int32_t*>(A.ws + A.chain_off);
    if (threadIdx.x < kNumXcd) {
      if (blockIdx.x == 0) ctr[threadIdx.x] = 0;
    } else if (it.mat >= 0) {
      ctr[kNumXcd + it.mat] = 0;
    }
  }
  if (it.mat < 0) return;
  const MatInfo& M = A.mats[it.mat];
  __shared__ float red[4];
  const float* ts = reinterpret_cast<const float*>(A.ws + A.tsum_off) + M.tile_off;
  const float* tm = reinterpret_cast<const float*>(A.ws + A.tmax_off) + M.tile_off;
  float mx = 0.f;
  for (int32_t q = threadIdx.x; q < M.tile_cnt; q += 256) mx = nan_max(mx, tm[q]);
  mx = block_max_256(mx, red);
  // tile sums are relative to 4^exp_of(tile max); sum them relative to the
  // matrix's 4^E
  const int E = exp_of(mx);
  float s = 0.f;
  for (int32_t q = threadIdx.x; q < M.tile_cnt; q += 256) s += ldexpf(ts[q], 2 * (exp_of(tm[q]) - E));
  s = block_sum_256(s, red);
  if (threadIdx.x == 0) {
    const float scale = 1.0f / (ldexpf(sqrtf(s), E) + A.eps);
    const float p = x0_pow2(mx);
    float* xs = reinterpret_cast<float*>(A.ws + A.x0s_off) + 4 * it.mat;
    xs[0] = scale / p;  // exact (p is a power of two) unless it underflows
    xs[1] = p;
    xs[3] = xs[2] == p ? 0.f : 1.f;
    if (mx > 0.f && mx <= 3.40282347e38f) A.hint[it.mat] = mx;
  }
}

// Operand rewrite: the tiles of the matrices whose flag is set, u again
// from G and the stored buf'. Runs over the momentum pass's tile schedule
// with a smaller grid, block b taking items b, b + grid, ... (grid a
// multiple of 8, so each item stays on the XCD the schedule placed it on).
// Most calls have no flag set: every workgroup first reads the flags of all
// non-empty matrices at once and leaves when none is set, instead of
// walking its items (two dependent loads each, one item after another).
__global__ __launch_bounds__(256) void x0_rewrite_kernel(StepArgs A) {
  __shared__ float tile[64][65];
  const float* x0s = reinterpret_cast<const float*>(A.ws + A.x0s_off);
  int any = 0;
  for (int32_t i = threadIdx.x; i < A.n_mats; i += blockDim.x)
    any |= A.mats[i].m > 0 && x0s[4 * i + 3] != 0.f;
  if (!__syncthreads_or(any)) return;
  for (int32_t q = blockIdx.x; q < A.n_items; q += gridDim.x) {
    const WorkItem it = A.items[q];
    if (it.mat < 0 || x0s[4 * it.mat + 3] == 0.f) continue;
    const MatInfo& M = A.mats[it.mat];
    const int32_t i0 = it.a * 64, j0 = it.b * 64;
    if (i0 >= M.m || j0 >= M.n) continue;  // padding: zeros already
    float u[2][8];
    tile_u_bf16<false>(A, M, M.tall ? j0 : i0, M.tall ? i0 : j0, u);
    tile_store_x0(A, M, i0, j0, u, x0s[4 * it.mat + 1], tile);
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

// 16 bytes as a native vector: the staging arrays of the fp32 engine stay in
// registers (arrays of the uint4 struct were kept in scratch memory).
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t comp(const v4u32& v, int e) { return v[e]; }

// Loads a 128-row x 128-byte slab of a row-major operand whose k index is
// contiguous (rows r0.., bytes k0b..): 4 x 16 bytes per thread.
__device__ __forceinline__ void load_rows(v4u32 (&r)[4], const char* base, int64_t ld_bytes,
                                          int64_t k0b) {
  const int t = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = (t >> 3) + 32 * q, ch = t & 7;
    r[q] = *reinterpret_cast<const v4u32*>(base + row * ld_bytes + k0b + ch * 16);
  }
}
__device__ __forceinline__ void store_rows(char* lds, const v4u32 (&r)[4]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = (t >> 3) + 32 * q, ch = t & 7;
    *reinterpret_cast<v4u32*>(lds + lds_off(row, ch)) = r[q];
  }
}

// Operand with k along memory rows (X[k][n], n contiguous): the slab is
// KS k-rows x 128 n-columns (KS = 64 bf16 or 32 fp32). Thread t loads a
// block of 4 k-rows x V columns (V = 8 bf16 / 4 fp32, 16 bytes) and later
// writes it transposed into the [n][k] LDS tile.
template <int ES>
__device__ __forceinline__ void load_cols(v4u32 (&r)[4], const char* base, int64_t ld_bytes,
                                          int64_t k0) {
  constexpr int V = 16 / ES;
  constexpr int NG = 128 / V;  // column groups per slab (16 bf16, 32 fp32)
  const int t = threadIdx.x;
  const int kq = t / NG, ng = t % NG;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    r[q] = *reinterpret_cast<const v4u32*>(base + (k0 + 4 * kq + q) * ld_bytes + ng * 16);
}
template <int ES>
__device__ __forceinline__ void store_cols(char* lds, const v4u32 (&r)[4]) {
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
      const v4u32 v = {comp(r[0], e), comp(r[1], e), comp(r[2], e), comp(r[3], e)};
      *reinterpret_cast<v4u32*>(lds + lds_off(ng * 4 + e, kq)) = v;
    }
  }
}

// One k-slab (128 bytes of k per row) of fp32 MFMAs for this wave's 64 x 64.
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

  v4u32 ra[4], rb[4];
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
    mma_slab(acc, sA, sB, wm, wn);
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
      const WApply wa(P, M);
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
              if (P.apply) {
                const int64_t wi = M.tall ? int64_t(gj) * M.wld + gi : int64_t(gi) * M.wld + gj;
                Elem<T>::store(M.w, wi, wa(Elem<T>::load(M.w, wi), v));
              } else {
                const int64_t co = M.tall ? int64_t(gj) * M.ld + gi : int64_t(gi) * M.ld + gj;
                Elem<T>::store(o, co, v);
              }
            }
          }
        }
    }
  }
}


// ------------------------------------------- 16-bit operand engine (bf16 sets)
//
// Output tile 256 x 256, 512 threads: eight waves in 2 (rows) x 4 (cols),
// each owning 128 x 64 = 4 x 2 accumulators of v_mfma_f32_32x32x16_{f16,bf16}.
// The MFMA is fed (column operand, row operand), so lane l holds, for
// accumulator (i, j) and register e,
//   C[m][n], m = row0 + 32 i + l % 32, n = col0 + 32 j + 8 (e / 4) + 4 (l / 32) + e % 4,
// i.e. runs of 4 consecutive output columns: vector epilogue loads/stores.
//
// k advances in stages of 32. Operands (stored in 32-column panels, so a
// stage of one operand is whole 128-byte lines) go from global memory
// straight into a ring of NS LDS stages (global_load_lds_dwordx4: lane i of
// a 1 KB piece writes base + 16 i, so the bank swizzle is applied by choosing
// which global 16-byte chunk lane i fetches). While stage g is multiplied,
// stages g+1 .. g+NS-2 are in flight and the slot that stage g-1 freed is
// refilled, its DMA spread over the two k-steps; one barrier per stage.
//   Row operand (k contiguous in memory): [row][k], 64-byte rows.
//   Column operand, k contiguous (Gram, A A): [col][k], 64-byte rows.
//   Column operand, k along memory rows (X in B X): [k][col], 512-byte rows,
//     read with ds_read_b64_tr_b16: in each 16-lane group, lane s addresses
//     row k0 + s/4, columns c0 + 4(s%4)..+3, and lane i receives column
//     c0 + i of rows k0..k0+3.

namespace e16 {

constexpr int TM = 256;                // output tile rows
constexpr int TN = kTileN16;           // output tile columns
constexpr int WN = TN / 64;            // waves per tile row (2 rows of waves)
constexpr int NWAVE = 2 * WN;
constexpr int NTHR = 64 * NWAVE;
constexpr int KS = 32;                 // k per stage
// Ring depth: one workgroup per CU with four 32 KB stages.
constexpr int NS = 4;
constexpr int HALF_A = TM * KS * 2;    // row operand of one stage: 16 KB
constexpr int HALF_B = TN * KS * 2;    // column operand of one stage
constexpr int STAGE = HALF_A + HALF_B;
constexpr int LDS_BYTES = NS * STAGE;
constexpr int KROW = TN * 2;           // bytes of one k-row of the [k][col] layout
static_assert(TN == 256 && NS == 4, "the ring and its DMA split assume 256 x 256 tiles, 4 stages");

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// LDS of gfx950 serves 256 bytes (64 banks of 4 bytes) per clock; a
// ds_read_b128 is served 16 lanes at a time.
// [row][k] layout: 16-byte chunk c (8 k) of row r. A fragment read puts 16
// consecutive rows (64 bytes apart, same chunk) in one phase: rows r, r+4,
// r+8, r+12 share a 64-byte bank quarter, and the XOR gives them four
// distinct chunks (measured: conflict-free; XOR with (r >> 1) & 3 alone
// leaves 2-way conflicts).
__device__ __forceinline__ int off_r(int r, int c) {
  return r * 64 + ((c ^ (((r >> 1) ^ (r >> 2)) & 3)) << 4);
}
// [k][col] layout: chunk c (8 columns) of k-row k (KROW-byte rows, a
// multiple of the 256-byte bank row). The XOR moves the four k-rows of one
// transposed read to four different 64-byte quarters of the bank row
// (measured: as fast as a contiguous transposed read).
__device__ __forceinline__ int off_k(int k, int c) { return k * KROW + ((c ^ ((k & 3) << 2)) << 4); }

// One 1 KB piece of LDS DMA: lane i copies the 16 bytes at `src` to LDS
// address lds_base + 16 i (lds_base wave-uniform, taken through M0).
// Written as asm on purpose: the instruction has no register result, and
// hiding it from the compiler keeps it from guarding every later LDS read
// with a wait for all DMA in flight (it cannot tell the ring slots apart,
// and it cannot see the alias scopes of the transposing LDS reads). The
// ring's own waits (s_waitcnt vmcnt + s_barrier) order the accesses.
// M0 is a reserved register, so clang warns that it does not save it around
// the asm; the generated code of this file holds no live value in M0 (its
// only writes are these), so the warning is silenced here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// COH: a device-scope load (sc1), which never hits an L1 copy older than
// the XCD's L2 (the chained launch, whose tiles read what other CUs of the
// XCD wrote earlier in the same launch).
template <bool COH = false>
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  if constexpr (COH)
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off sc1"
        :
        : "s"(lds_base), "v"(src)
        : "memory", "m0");
  else
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off"
        :
        : "s"(lds_base), "v"(src)
        : "memory", "m0");
}
#pragma clang diagnostic pop

// DMA of one stage in pieces of 1 KB: 16 of the row operand, TN/16 of the
// column operand. Operands are in 32-column panels (pidx) and lda / ldb are
// panel strides in bytes: a row operand's stage (256 rows at opA, k0 ..
// k0+31) is panel k0/32, 16 KB contiguous; the column operand is either the
// same (opB) or k-rows k0 .. k0+31 of TN columns (TN/32 panels from opB,
// 64 bytes per k-row in each). Wave w issues pieces w, w + NWAVE, ...; its
// q-th piece is dma_piece(q).
// Waves 0 .. DMA_WAVES-1 issue the ring's DMA. With half of the waves (one
// per SIMD: waves w and w + 4 share a SIMD) the other wave of each SIMD
// never waits behind a DMA issue; measured against every wave issuing, on
// one device back to back: the update launch 2 % faster, Gram and poly the
// same.
constexpr int DMA_WAVES = NWAVE / 2;
static_assert(NWAVE % DMA_WAVES == 0 && (16 + TN / 16) % DMA_WAVES == 0 && 16 % DMA_WAVES == 0, "DMA waves");
constexpr int DMA_PER_STAGE = (16 + TN / 16) / DMA_WAVES;  // pieces per DMA wave per stage
template <bool KN, bool COH = false>
__device__ __forceinline__ void dma_piece(char* st, const char* opA, int64_t lda, const char* opB,
                                          int64_t ldb, int64_t k0, int q, uint32_t tid) {
  const int w = tid >> 6, i = tid & 63;
  constexpr int QA = 16 / DMA_WAVES;  // row-operand pieces per wave
  const int I = w + DMA_WAVES * (q < QA ? q : q - QA);
  const uint32_t dst = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(st)) + (q < QA ? 0 : HALF_A) + I * 1024);
  if (q < QA) {
    const int row = 16 * I + (i >> 2), g = (i & 3) ^ (((row >> 1) ^ (row >> 2)) & 3);
    dma16<COH>(opA + (k0 >> 5) * lda + row * 64 + g * 16, dst);
  } else if constexpr (!KN) {
    const int row = 16 * I + (i >> 2), g = (i & 3) ^ (((row >> 1) ^ (row >> 2)) & 3);
    dma16<COH>(opB + (k0 >> 5) * ldb + row * 64 + g * 16, dst);
  } else {
    constexpr int RPP = 1024 / KROW;  // k-rows per piece
    const int kr = RPP * I + i / (64 / RPP), g = (i % (64 / RPP)) ^ ((kr & 3) << 2);
    dma16<COH>(opB + (g >> 2) * ldb + (k0 + kr) * 64 + (g & 3) * 16, dst);
  }
}
// The same piece q of a stage-sized (32 KB) contiguous block at src: stage
// byte offset (q < 4 ? 0 : 16 KB) + 1 KB (w + 4 (q % 4)) for DMA wave w,
// the offset it also has at src (the update's low bytes of X, prefetched
// through the ring in the k loop's last passes).
template <bool COH = false>
__device__ __forceinline__ void dma_block_piece(char* st, const char* src, int q, uint32_t tid) {
  const int w = tid >> 6, i = tid & 63;
  constexpr int QA = 16 / DMA_WAVES;
  const int off = (q < QA ? 0 : HALF_A) + (w + DMA_WAVES * (q < QA ? q : q - QA)) * 1024;
  const uint32_t dst = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(st)) + off);
  dma16<COH>(src + off + i * 16, dst);
}
static_assert(HALF_A == 16384 && STAGE == 32768, "the low-byte prefetch fills whole stages");
template <bool KN, bool COH = false>
__device__ __forceinline__ void dma_stage(char* st, const char* opA, int64_t lda, const char* opB,
                                          int64_t ldb, int64_t k0, uint32_t tid) {
#pragma unroll
  for (int q = 0; q < DMA_PER_STAGE; ++q) dma_piece<KN, COH>(st, opA, lda, opB, ldb, k0, q, tid);
}

template <int OP>
__device__ __forceinline__ f32x16_t mfma(const u32x4& colop, const u32x4& rowop, f32x16_t c) {
  static_assert(OP == OP_F16, "the 16-bit engine takes fp16 operands");
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, colop),
                                                __builtin_bit_cast(f16x8_t, rowop), c, 0, 0, 0);
}

// Operand fragments of one k-step (16 k) of this wave's 128 x 64 block.
struct Frag {
  u32x4 a[4];  // row operand: rows wm*128 + 32 i + l%32, 8 k per lane half
  u32x4 b[2];  // column operand: columns wn*64 + 32 j + l%32
};

// Fragment reads of k-step ks (0/1) of the stage at `st`: row-operand block
// i, column-operand block j. The reads stay in flight until the MFMAs that
// use them.
__device__ __forceinline__ void frag_load_a(Frag& f, const char* st, int ks, int wm, int i, uint32_t tid) {
  const int lane = tid & 63;
  const int ch = ks * 2 + (lane >> 5);  // 16-byte k chunk of this lane half
  f.a[i] = *reinterpret_cast<const u32x4*>(st + off_r(wm * 128 + i * 32 + (lane & 31), ch));
}
template <bool KN>
__device__ __forceinline__ void frag_load_b(Frag& f, const char* st, int ks, int wn, int j, uint32_t tid) {
  const char* sB = st + HALF_A;
  const int lane = tid & 63;
  if constexpr (KN) {
    const int s = lane & 15, h = lane >> 4;  // 16-lane group h
    const int krow = ks * 16 + (h >> 1) * 8 + (s >> 2);
    const int col = wn * 64 + j * 32 + (h & 1) * 16 + 4 * (s & 3);
    const int chunk = col >> 3, byte = (col & 7) * 2;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4_t*)(sB + off_k(krow, chunk) + byte));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4_t*)(sB + off_k(krow + 4, chunk) + byte));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    f.b[j] = u32x4{l2.x, l2.y, h2.x, h2.y};
  } else {
    const int ch = ks * 2 + (lane >> 5);
    f.b[j] = *reinterpret_cast<const u32x4*>(sB + off_r(wn * 64 + j * 32 + (lane & 31), ch));
  }
}
template <bool KN>
__device__ __forceinline__ void frag_load(Frag& f, const char* st, int ks, int wm, int wn, uint32_t tid) {
#pragma unroll
  for (int j = 0; j < 2; ++j) frag_load_b<KN>(f, st, ks, wn, j, tid);
#pragma unroll
  for (int i = 0; i < 4; ++i) frag_load_a(f, st, ks, wm, i, tid);
}

// One k-step with DMA spread over it: the 8 MFMAs of fragment set fm, the
// LDS reads of fragment set fl (k-step ks of the stage at `st`) and NCH DMA
// pieces, dma(c) at the start of chunk c. Each chunk takes 4 / NCH row
// blocks of MFMAs with their share of the reads, so a wave never has more
// than one DMA in front of its next MFMAs and the address unit drains
// between the chunks.
template <int OP, bool KN, int NCH, typename D>
__device__ __forceinline__ void kstep_dma(f32x16_t (&acc)[4][2], const Frag& fm, Frag& fl,
                                          const char* st, int ks, int wm, int wn, uint32_t tid, D&& dma) {
  static_assert(4 % NCH == 0, "row blocks per chunk");
  constexpr int IPC = 4 / NCH;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    __builtin_amdgcn_sched_barrier(0);
    dma(c);
#pragma unroll
    for (int ii = 0; ii < IPC; ++ii)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[c * IPC + ii][j] = mfma<OP>(fm.b[j], fm.a[c * IPC + ii], acc[c * IPC + ii][j]);
    if (c == 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j) frag_load_b<KN>(fl, st, ks, wn, j, tid);
    }
#pragma unroll
    for (int ii = 0; ii < IPC; ++ii) frag_load_a(fl, st, ks, wm, c * IPC + ii, tid);
    constexpr int NM = 2 * IPC;
    const int nr = IPC + (c == 0 ? (KN ? 4 : 2) : 0);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      if (k < nr) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// RN16(x0) | RN16(x1) << 16: one v_cvt_pk_f16_f32 (round to nearest even)
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef float f2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk16(float x0, float x1) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{x0, x1}, h2_t));
}

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d, bool f16) {
  uint2 r;
  if (f16) {
    r.x = pk16(a, b);
    r.y = pk16(c, d);
  } else {
    r.x = uint32_t(f2bf(a)) | (uint32_t(f2bf(b)) << 16);
    r.y = uint32_t(f2bf(c)) | (uint32_t(f2bf(d)) << 16);
  }
  return r;
}

// Mixed-precision FMAs (v_fma_mix_f32) for the fp16 update epilogue: the
// residual x - f16(low / high half of h) in one rounding (exact here).
// VALU-only asm (no memory access).
__device__ __forceinline__ float sub_l(float x, uint32_t h) {
  float r;
  asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(x));
  return r;
}
__device__ __forceinline__ float sub_h(float x, uint32_t h) {
  float r;
  asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(x));
  return r;
}

// POLY: acc[i][J] += f A[m][n] at this lane's accumulator positions of
// column block J (row blocks i < NR, rows rbase + 32 i ..), read from the
// row-operand half of the stage at `st`, which holds A[m][k] for the 32 k
// that are these n (the caller picks the stage).
template <int OP, int J, int NR>
__device__ __forceinline__ void fold_rows(f32x16_t (&acc)[4][2], const char* st, int rbase, float f,
                                          uint32_t tid) {
  const int lane = tid & 63, l32 = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    u32x2 v[4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
      v[g] = *reinterpret_cast<const u32x2*>(st + off_r(rbase + 32 * i + l32, g) + lh * 8);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t w[4] = {v[g].x & 0xffffu, v[g].x >> 16, v[g].y & 0xffffu, v[g].y >> 16};
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[i][J][4 * g + r] = __fmaf_rn(f, Op<OP>::load16(w[r]), acc[i][J][4 * g + r]);
    }
  }
}

// Diagonal tiles (TI == TJ) of the symmetric products (Gram, poly). Of the
// 8 x 8 grid of 32 x 32 blocks only the 36 on or above the diagonal are
// needed, and the row and column operands are the same 256 rows, so a stage
// carries the row operand only (16 KB, four 1 KB pieces per DMA wave) and
// column fragments are read from it too. The 36 blocks are shared so that
// each SIMD runs 9 (its two waves w and w + 4), against 16 on other tiles:
//   waves 0..3   (strip)       block rows 0..3 of block column 4 + w (the
//                              upper-right quadrant, 4 blocks each);
//   waves 4, 6   (triangle A)  block columns 0 and 3 of the upper-left (4)
//                              or lower-right (6) quadrant: 1 and 4 blocks;
//   waves 5, 7   (triangle B)  its block columns 1 and 2: 2 and 3 blocks.
// acc[i][j] holds block row i (rows rbase + 32 i ..) of block column j
// (columns cb[j] ..), for i < nr[j].
template <int ROLE> struct DiagRole;
template <> struct DiagRole<0> { static constexpr int NJ = 1, NR0 = 4, NR1 = 0; };
template <> struct DiagRole<1> { static constexpr int NJ = 2, NR0 = 1, NR1 = 4; };
template <> struct DiagRole<2> { static constexpr int NJ = 2, NR0 = 2, NR1 = 3; };

struct DiagGeo {
  int rbase, cb0, cb1;  // first row, first column of block columns 0 and 1
};
__device__ __forceinline__ int diag_role(int wave) { return wave < 4 ? 0 : ((wave & 1) ? 2 : 1); }
__device__ __forceinline__ DiagGeo diag_geo(int wave) {
  if (wave < 4) return DiagGeo{0, 128 + 32 * wave, 128 + 32 * wave};
  const int q = 128 * ((wave >> 1) & 1);  // waves 4, 5: upper-left; 6, 7: lower-right
  return (wave & 1) ? DiagGeo{q, q + 32, q + 64} : DiagGeo{q, q, q + 96};
}

// A fragment of 32 rows (row0 ..) of k-step ks from the row-operand half.
__device__ __forceinline__ u32x4 frag_rows(const char* st, int ks, int row0, uint32_t tid) {
  const int lane = tid & 63;
  return *reinterpret_cast<const u32x4*>(st + off_r(row0 + (lane & 31), ks * 2 + (lane >> 5)));
}

// Half C (0/1) of a diagonal-tile k-step: its share of the role's MFMAs on
// fragment set fm and of the LDS reads of fragment set fl (k-step ks of the
// stage at `st`), interleaved.
template <int OP, int ROLE, int C>
__device__ __forceinline__ void kchunk_diag(f32x16_t (&acc)[4][2], const Frag& fm, Frag& fl,
                                            const char* st, int ks, const DiagGeo& geo, uint32_t tid) {
  using R = DiagRole<ROLE>;
  constexpr int NM = R::NR0 + R::NR1;
  constexpr int NA = R::NR0 > R::NR1 ? R::NR0 : R::NR1;
  constexpr int NRD = R::NJ + NA;
  constexpr int mb = C * NM / 2, me = (C + 1) * NM / 2;
  constexpr int rb = C * NRD / 2, re = (C + 1) * NRD / 2;
#pragma unroll
  for (int t = mb; t < me; ++t) {
    const int j = t < R::NR0 ? 0 : 1, i = t < R::NR0 ? t : t - R::NR0;
    acc[i][j] = mfma<OP>(fm.b[j], fm.a[i], acc[i][j]);
  }
#pragma unroll
  for (int t = rb; t < re; ++t) {
    if (t < R::NJ) fl.b[t] = frag_rows(st, ks, t == 0 ? geo.cb0 : geo.cb1, tid);
    else fl.a[t - R::NJ] = frag_rows(st, ks, geo.rbase + 32 * (t - R::NJ), tid);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k < me - mb) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    if (k < re - rb) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
  }
}
template <int OP, int ROLE, typename D>
__device__ __forceinline__ void kstep_diag(f32x16_t (&acc)[4][2], const Frag& fm, Frag& fl,
                                           const char* st, int ks, const DiagGeo& geo, uint32_t tid, D&& dma) {
  __builtin_amdgcn_sched_barrier(0);
  dma(0);
  kchunk_diag<OP, ROLE, 0>(acc, fm, fl, st, ks, geo, tid);
  __builtin_amdgcn_sched_barrier(0);
  dma(1);
  kchunk_diag<OP, ROLE, 1>(acc, fm, fl, st, ks, geo, tid);
  __builtin_amdgcn_sched_barrier(0);
}

// s_waitcnt with only the vector-memory counter limited to n (gfx9 encoding).
#define MUON_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0F70)
// s_waitcnt lgkmcnt(0) only (LDS and scalar memory; vector memory may stay
// in flight).
#define MUON_WAIT_LGKMCNT0() __builtin_amdgcn_s_waitcnt(0xC07F)

// The k loop of a diagonal tile for wave role ROLE: the ring of the other
// tiles (same slots, same one barrier per stage, the stage's DMA split over
// its two k-steps) carrying the row operand only (opA, panel stride lda).
// FOLD (poly): block column j also adds f A at its accumulator positions
// while stage fs[j] is resident (the stage holding its 32 columns as k).
template <int OP, int ROLE, bool FOLD, bool COH = false>
__device__ __forceinline__ void kloop_diag(f32x16_t (&acc)[4][2], char* lds, const char* opA, int64_t lda,
                                           int nst, bool dma_wave, const DiagGeo& geo, int fs0, int fs1,
                                           float f, uint32_t tid) {
  using R = DiagRole<ROLE>;
  constexpr int DPS = 16 / DMA_WAVES;  // row-operand pieces per DMA wave per stage
  constexpr int H = DPS / 2;           // pieces per k-step
  static_assert(H == 2, "two chunks per k-step");
#pragma unroll
  for (int p = 0; p < NS - 2; ++p)
#pragma unroll
    for (int q = 0; q < DPS; ++q)
      if (dma_wave) dma_piece<false, COH>(lds + p * STAGE, opA, lda, opA, lda, int64_t(p) * KS, q, tid);
#pragma unroll
  for (int q = 0; q < H; ++q)
    if (dma_wave) dma_piece<false, COH>(lds + (NS - 2) * STAGE, opA, lda, opA, lda, int64_t(NS - 2) * KS, q, tid);
  MUON_WAIT_VMCNT(DPS * (NS - 3) + H);  // stage 0 landed (this wave's pieces)
  asm volatile("s_barrier" ::: "memory");
  constexpr int NA = R::NR0 > R::NR1 ? R::NR0 : R::NR1;
  Frag f0, f1;
  f0.b[0] = frag_rows(lds, 0, geo.cb0, tid);
  if constexpr (R::NJ == 2) f0.b[1] = frag_rows(lds, 0, geo.cb1, tid);
#pragma unroll
  for (int i = 0; i < NA; ++i) f0.a[i] = frag_rows(lds, 0, geo.rbase + 32 * i, tid);
  int cur = 0;
  // one pass over stage g; J >= 0 also folds block column J (see the other
  // tiles' loop: the fold passes are loops of their own)
  // TAIL (Gram: the last three passes, 1 .. 3 for g = nst-3 .. nst-1)
  // issues no stage past the end and waits for every stage issued.
  auto pass = [&](int g, auto fold_j, auto tail) {
    constexpr int J = decltype(fold_j)::value;
    constexpr int TAIL = decltype(tail)::value;
    const int nxt = cur == NS - 1 ? 0 : cur + 1;
    const int old = cur == 0 ? NS - 1 : cur - 1;
    {
      const int s2 = cur + NS - 2 < NS ? cur + NS - 2 : cur - 2;
      const int64_t k2 = int64_t(min(g + NS - 2, nst - 1)) * KS;
      kstep_diag<OP, ROLE>(acc, f0, f1, lds + cur * STAGE, 1, geo, tid, [&](int c) {
        if constexpr (TAIL <= 1)
          if (dma_wave) dma_piece<false, COH>(lds + s2 * STAGE, opA, lda, opA, lda, k2, H + c, tid);
      });
    }
    if constexpr (TAIL >= 2)
      MUON_WAIT_VMCNT(0);
    else
      MUON_WAIT_VMCNT(DPS * (NS - 3));
    asm volatile("s_barrier" ::: "memory");
    {
      const int64_t k3 = int64_t(min(g + NS - 1, nst - 1)) * KS;
      kstep_diag<OP, ROLE>(acc, f1, f0, lds + nxt * STAGE, 0, geo, tid, [&](int c) {
        if constexpr (TAIL == 0)
          if (dma_wave) dma_piece<false, COH>(lds + old * STAGE, opA, lda, opA, lda, k3, c, tid);
      });
    }
    if constexpr (J >= 0) {
      __builtin_amdgcn_sched_barrier(0);
      fold_rows<OP, J, J == 0 ? R::NR0 : R::NR1>(acc, lds + cur * STAGE, geo.rbase, f, tid);
    }
    cur = nxt;
  };
  using NoFold = std::integral_constant<int, -1>;
  using T0 = std::integral_constant<int, 0>;
  int g = 0;
  if constexpr (FOLD) {
    // (poly: past the end the DMA repeats the last stage, valid addresses,
    // unused: the last diagonal tile's fold passes fall among the last
    // passes, and tail passes for each of them cost more registers than the
    // chained launch has)
    if (fs0 >= 0) {
      for (; g < fs0; ++g) pass(g, NoFold{}, T0{});
      pass(g++, std::integral_constant<int, 0>{}, T0{});
      if constexpr (R::NJ == 2) {
        for (; g < fs1; ++g) pass(g, NoFold{}, T0{});
        pass(g++, std::integral_constant<int, 1>{}, T0{});
      }
    }
    for (; g < nst; ++g) pass(g, NoFold{}, T0{});
  } else {
    for (; g < nst - 3; ++g) pass(g, NoFold{}, T0{});
    pass(g++, NoFold{}, std::integral_constant<int, 1>{});
    pass(g++, NoFold{}, std::integral_constant<int, 2>{});
    pass(g++, NoFold{}, std::integral_constant<int, 3>{});
  }
  MUON_WAIT_VMCNT(0);  // every stage issued lands before the LDS is reused or freed
}



}  // namespace e16

// bf16 sets. Item {mat, TI, TJ} of 256 x 256 tiles. GRAM/POLY: tiles on or
// above the diagonal (TJ >= TI); each stored element (m <= n) is mirrored to
// (n, m). UPDATE: X = a X + B X on all tiles.
// SK (Gram only): the variant that also runs split tiles and the reduce
// pass, launched for plans that split Gram tiles.
// One work item (tile) of the 16-bit engine on the workgroup's LDS ring
// `lds` (LDS_BYTES). The launches below run one item per workgroup; the
// chained launch (chain16_kernel) runs the items of every step in one
// launch.
// at_epilogue() runs once the k loop is done, before the epilogue (the
// chained launch fetches its next ticket there).
struct NoHook {
  __device__ void operator()() const {}
};
template <typename T, int OP, int KIND, bool LAST, bool SK = false, bool X0S = false, bool COH = false,
          typename Hook = NoHook>
__device__ __forceinline__ void tile16(const StepArgs& P, const WorkItem it, char* lds, uint32_t tid,
                                       Hook at_epilogue = Hook{}) {
  using namespace e16;
  if (it.mat < 0) return;
  // Matrix record fields read once into registers: re-reading them after a
  // global store would force a reload (the compiler cannot rule out aliasing).
  struct {
    int32_t m, n, mp, np, tall, vec_ok, w_vec_ok;
    int64_t ld, a_off, b_off, xl_off, xo_cur, xo_nxt, wld;
    void* out;
    void* w;
    float keep, step;  // weight application (see WApply)
  } M;
  {
    const MatInfo& R = P.mats[it.mat];
    M.m = R.m; M.n = R.n; M.mp = R.mp; M.np = R.np; M.tall = R.tall; M.vec_ok = R.vec_ok;
    M.ld = R.ld; M.a_off = R.a_off; M.b_off = R.b_off; M.xl_off = R.xl_off;
    M.xo_cur = xo_sel(R, P.cur); M.xo_nxt = xo_sel(R, P.cur ^ 1); M.out = R.out;
    M.w = R.w; M.wld = R.wld; M.w_vec_ok = R.w_vec_ok;
    const WApply wa(P, R);
    M.keep = wa.keep; M.step = wa.step;
  }
  constexpr bool KN = KIND == UPDATE;

  const int TI = it.a, TJ = it.b;
  const char* opA;
  const char* opB;
  int64_t lda, ldb, K;
  // Every operand has mp rows, so one panel stride serves both.
  lda = ldb = int64_t(M.mp) * 64;
  // Split Gram tiles: part sp of S covers k in [sp K / S, (sp + 1) K / S)
  // and stores an fp32 partial tile; the reduce pass sums the S partials.
  const int S = SK ? max(it.c & 255, 1) : 1;
  const int sp = SK ? (it.c >> 8) & 255 : 0;
  const int pbase = SK ? (it.c >> 16) : 0;
  const bool reducing = SK && P.reduce;
  const bool partial = SK && !reducing && S > 1;
  if (KIND == GRAM) {
    const char* X = P.ws + M.xo_cur;
    K = M.np / S;
    opA = X + int64_t(TI) * TM * 64 + (sp * K / 32) * lda;
    opB = X + int64_t(TJ) * TN * 64 + (sp * K / 32) * ldb;
  } else if (KIND == POLY) {
    const char* Am = P.ws + M.a_off;
    opA = Am + int64_t(TI) * TM * 64;
    opB = Am + int64_t(TJ) * TN * 64;
    K = M.mp;
  } else {
    opA = P.ws + M.b_off + int64_t(TI) * TM * 64;
    opB = P.ws + M.xo_cur + int64_t(TJ) * (TN / 32) * ldb;
    K = M.mp;
  }

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const bool dma_wave = wave < DMA_WAVES;  // (waves 0 .. 3 sit on the four SIMDs)
  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // K is a multiple of 256 (at least 8 stages). Each stage is two k-steps;
  // the fragments of the next k-step are read while the MFMAs of the current
  // one run, and the ring barrier sits between the two k-steps of a stage:
  //   mma(g, 0) | read (g, 1) | stage g+1 landed, barrier, DMA g+NS-1 into
  //   the slot of g-1 | mma(g, 1) | read (g+1, 0)
  // Every pass issues one stage, so the wait count is the same in every pass;
  // past the end the DMA of poly repeats the last stage (valid addresses,
  // unused), while the last passes of Gram and of the update are passes of
  // their own (TAIL below) that issue no stage past the end.
  const bool fold = KIND == POLY && P.c != 0.f;
  // This wave's blocks: acc[i][j] is rows rbase + 32 i .. of the tile and
  // columns cb0 .. (j = 0) or cb1 .. (j = 1), for i < nr0 / nr1. Diagonal
  // tiles of the symmetric products share their 36 needed blocks out by
  // role (kloop_diag); every other tile is wm, wn's 128 x 64.
  int rbase = wm * 128, cb0 = wn * 64, cb1 = wn * 64 + 32, nr0 = 4, nr1 = 4;
  bool diag = false;
  if constexpr ((KIND == GRAM || KIND == POLY) && !SK) {
    if (TI == TJ) {
      diag = true;
      const DiagGeo geo = diag_geo(wave);
      const int role = diag_role(wave);
      rbase = geo.rbase;
      cb0 = geo.cb0;
      cb1 = geo.cb1;
      const int nst = static_cast<int>(K / KS);
      // poly: block column j's 32 columns are the k of stage TJ * 8 + cb / 32
      const int fs0 = TJ * (TN / KS) + cb0 / KS, fs1 = TJ * (TN / KS) + cb1 / KS;
      // (without the fold, fs0 = fs1 = -1 never match a stage)
      const float fb = fold ? P.b / P.c : 0.f;
      const int f0s = fold ? fs0 : -1, f1s = fold ? fs1 : -1;
      constexpr bool FOLD = KIND == POLY;
      if (role == 0) {
        nr0 = DiagRole<0>::NR0, nr1 = DiagRole<0>::NR1;
        kloop_diag<OP, 0, FOLD, COH>(acc, lds, opA, lda, nst, dma_wave, geo, f0s, f1s, fb, tid);
      } else if (role == 1) {
        nr0 = DiagRole<1>::NR0, nr1 = DiagRole<1>::NR1;
        kloop_diag<OP, 1, FOLD, COH>(acc, lds, opA, lda, nst, dma_wave, geo, f0s, f1s, fb, tid);
      } else {
        nr0 = DiagRole<2>::NR0, nr1 = DiagRole<2>::NR1;
        kloop_diag<OP, 2, FOLD, COH>(acc, lds, opA, lda, nst, dma_wave, geo, f0s, f1s, fb, tid);
      }
    }
  }
  if (!reducing && !diag) {
  const int nst = static_cast<int>(K / KS);
  constexpr int H = DMA_PER_STAGE / 2;  // pieces per k-step (the DMA of a stage is split over two)
  static_assert(DMA_PER_STAGE % 2 == 0 && 4 % H == 0, "DMA split");
  // stages 0 .. NS-3 and the first half of stage NS-2 (its second half
  // goes out with the first k-step of stage 0)
#pragma unroll
  for (int p = 0; p < NS - 2; ++p)
    if (dma_wave) dma_stage<KN, COH>(lds + p * STAGE, opA, lda, opB, ldb, int64_t(p) * KS, tid);
#pragma unroll
  for (int q = 0; q < H; ++q)
    if (dma_wave) dma_piece<KN, COH>(lds + (NS - 2) * STAGE, opA, lda, opB, ldb, int64_t(NS - 2) * KS, q, tid);
  MUON_WAIT_VMCNT(DMA_PER_STAGE * (NS - 3) + H);  // stage 0 landed (this wave's pieces)
  asm volatile("s_barrier" ::: "memory");
  // POLY with c != 0 folds the b A term into the accumulators on the way:
  // acc = A A + (b / c) A, and the epilogue scales by c. Column n of this
  // wave's block j is k = n of the row operand, which is in stage
  // bias0 + j (the A tile of rows TI and columns TJ passes through LDS).
  const int bias0 = fold ? TJ * (TN / KS) + wn * (64 / KS) : -2;
  const float fb = fold ? P.b / P.c : 0.f;
  Frag f0, f1;
  frag_load<KN>(f0, lds, 0, wm, wn, tid);
  int cur = 0;  // ring slot of stage g
  // The update's low bytes of X (64 KB per tile, contiguous) take the place
  // of stages nst and nst+1 (slots nst % NS and (nst+1) % NS), which
  // otherwise repeat the last stage: the epilogue reads them from LDS.
  constexpr bool LO_DMA = KIND == UPDATE;
  const char* lo_src = LO_DMA ? P.ws + M.xl_off + (int64_t(TI) * (M.np / TN) + TJ) * (TM * TN) : nullptr;
  // One pass over stage g. Poly's b A term is folded into the accumulators
  // of block column J in the pass over the stage that holds those columns
  // as k; those two passes are loops of their own, so that no other pass
  // carries the fold's branch. TAIL (the last three passes, g = nst-3 ..
  // nst-1): the update's (1 .. 3) fetch the low bytes where stages nst and
  // nst+1 would go, and its last pass issues nothing (nothing waits for it);
  // Gram's (4 .. 6) issue no stage past the end and wait for every stage
  // issued.
  auto pass = [&](int g, auto fold_j, auto tail) {
    constexpr int J = decltype(fold_j)::value;
    constexpr int TAIL = decltype(tail)::value;
    const int nxt = cur == NS - 1 ? 0 : cur + 1;  // slot of stage g+1
    const int old = cur == 0 ? NS - 1 : cur - 1;  // slot of stage g-1 (unused for g = 0)
    {
      // second half of stage g+NS-2 (its slot was freed at the previous
      // barrier; the first half went out then)
      const int s2 = cur + NS - 2 < NS ? cur + NS - 2 : cur - 2;
      const int64_t k2 = int64_t(min(g + NS - 2, nst - 1)) * KS;
      kstep_dma<OP, KN, H>(acc, f0, f1, lds + cur * STAGE, 1, wm, wn, tid, [&](int c) {
        if constexpr (TAIL == 2 || TAIL == 3) {  // stage nst or nst+1: low bytes, second half
          if (dma_wave) dma_block_piece<COH>(lds + s2 * STAGE, lo_src + (TAIL - 2) * STAGE, H + c, tid);
        } else if constexpr (TAIL <= 1 || TAIL == 4) {
          if (dma_wave) dma_piece<KN, COH>(lds + s2 * STAGE, opA, lda, opB, ldb, k2, H + c, tid);
        }
      });
    }
    // This wave's pieces of stage g+1 have landed (stages up to g+NS-2 may
    // still be in flight). A bare s_barrier: the workgroup fence of
    // __syncthreads would also wait for those; the memory clobber keeps the
    // compiler from moving LDS accesses across it.
    if constexpr (TAIL >= 5)
      MUON_WAIT_VMCNT(0);
    else
      MUON_WAIT_VMCNT(DMA_PER_STAGE * (NS - 3));
    asm volatile("s_barrier" ::: "memory");
    // every wave has finished reading stage g-1: refill its slot, the first
    // half of stage g+NS-1 now and the second half with the next k-step
    // (after the last stage the fragment reads come from a stale slot; the
    // values are unused)
    {
      const int64_t k3 = int64_t(min(g + NS - 1, nst - 1)) * KS;
      kstep_dma<OP, KN, H>(acc, f1, f0, lds + nxt * STAGE, 0, wm, wn, tid, [&](int c) {
        if constexpr (TAIL == 1 || TAIL == 2) {  // stage nst or nst+1: low bytes, first half
          if (dma_wave) dma_block_piece<COH>(lds + old * STAGE, lo_src + (TAIL - 1) * STAGE, c, tid);
        } else if constexpr (TAIL == 0) {
          if (dma_wave) dma_piece<KN, COH>(lds + old * STAGE, opA, lda, opB, ldb, k3, c, tid);
        }
      });
    }
    if constexpr (J >= 0) {
      // (stage g stays in its slot until every wave has passed the next
      // barrier)
      __builtin_amdgcn_sched_barrier(0);
      fold_rows<OP, J, 4>(acc, lds + cur * STAGE, wm * 128, fb, tid);
    }
    cur = nxt;
  };
  using NoFold = std::integral_constant<int, -1>;
  using T0 = std::integral_constant<int, 0>;
  using Fold0 = std::integral_constant<int, 0>;
  using Fold1 = std::integral_constant<int, 1>;
  using T4 = std::integral_constant<int, 4>;
  using T5 = std::integral_constant<int, 5>;
  using T6 = std::integral_constant<int, 6>;
  if (fold) {
    // (poly: past the end the DMA repeats the last stage, valid addresses,
    // unused: a fold pass can be one of the last three passes, and tail
    // passes for those cases cost more registers than the chained launch
    // has)
    int g = 0;
    for (; g < bias0; ++g) pass(g, NoFold{}, T0{});
    pass(g++, Fold0{}, T0{});
    pass(g++, Fold1{}, T0{});
    for (; g < nst; ++g) pass(g, NoFold{}, T0{});
  } else if constexpr (LO_DMA) {
    int g = 0;
    for (; g < nst - 3; ++g) pass(g, NoFold{}, T0{});
    pass(g++, NoFold{}, std::integral_constant<int, 1>{});
    pass(g++, NoFold{}, std::integral_constant<int, 2>{});
    pass(g++, NoFold{}, std::integral_constant<int, 3>{});
  } else {
    // Gram (and poly with c = 0): the last three passes (TAIL 4 .. 6) issue
    // no stage past the end and wait for every stage issued
    int g = 0;
    for (; g < nst - 3; ++g) pass(g, NoFold{}, T0{});
    pass(g++, NoFold{}, T4{});
    pass(g++, NoFold{}, T5{});
    pass(g++, NoFold{}, T6{});
  }
  MUON_WAIT_VMCNT(0);  // every stage issued lands before the LDS is reused or freed
  }

  // ---------------------------------------------------------------- epilogue
  // acc[i][j][4 g + r] = C[m][n], m = mb + 32 i + l32, n = nb + 32 j + 8 g + 4 lh + r
  // with mb = TI*256 + wm*128, nb = TJ*TN + wn*64. Results are staged as a
  // 16-bit 256 x TN tile in LDS (the ring is free now) and written out from
  // there: rows with 16-byte reads (whole 128-byte lines per store), columns
  // (mirror, transposed output) with transposing reads, 8 rows per lane.
  const int l32 = lane & 31, lh = lane >> 5;
  constexpr int ROWB = TN * 2;   // bytes per staged row
  constexpr int CPR = TN / 8;    // 16-byte chunks per staged row
  const int m0 = TI * TM, n0 = TJ * TN;  // tile origin
  __builtin_amdgcn_sched_barrier(0);
  at_epilogue();
  __syncthreads();  // every wave is done reading the operand stages

  // Split Gram tiles: a part stores its fp32 accumulators in accumulator
  // order (per wave and block (i, j): 64 lanes x 64 bytes); the reduce pass
  // sums the parts in order straight into the staged tile (below) and goes
  // on as an ordinary tile.
  auto part_ptr = [&](int q, int i, int j) {
    return reinterpret_cast<const f32x4_t*>(P.ws + P.split_off + int64_t(pbase + q) * (TM * TN * 4) +
                                            ((((wave * 4 + i) * 2 + j) * 64) + lane) * 64);
  };
  if constexpr (SK) {
    if (partial) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            f32x4_t* d = const_cast<f32x4_t*>(part_ptr(sp, i, j));
#pragma unroll
            for (int v = 0; v < 4; ++v)
              d[v] = f32x4_t{acc[i][j][4 * v], acc[i][j][4 * v + 1], acc[i][j][4 * v + 2], acc[i][j][4 * v + 3]};
          }
      return;
    }
  }

  // Staged address of (row r, chunk c). The XOR gives 16 consecutive rows
  // distinct chunk positions (accumulator-order writes) and keeps the four
  // rows of a transposing read on distinct 32-byte pairs.
  auto soff = [](int r, int c) {
    const int x = ((r & 3) << 1) | ((r >> 2) & 1) | (((r >> 3) & 1) << 3);
    return r * ROWB + ((c ^ x) << 4);
  };
  // acc (or values derived from it) -> staged 16-bit tile
  auto stage16 = [&](bool f16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (i >= (j ? nr1 : nr0)) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r = rbase + 32 * i + l32, c = (j ? cb1 : cb0) / 8 + g;
          *reinterpret_cast<uint2*>(lds + soff(r, c) + lh * 8) =
              e16::pack4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                         acc[i][j][4 * g + 3], f16);
        }
      }
  };
  // Visits the staged tile by rows: fn(m, n, 16 bytes of n..n+7).
  auto rows_out = [&](auto&& fn) {
#pragma unroll 4
    for (int q = 0; q < TM * CPR / NTHR; ++q) {
      const int r = q * (NTHR / CPR) + tid / CPR, c = tid % CPR;
      fn(m0 + r, n0 + 8 * c, *reinterpret_cast<const uint4*>(lds + soff(r, c)));
    }
  };
  // Visits the staged tile by columns: fn(n, m, 16 bytes of rows m..m+7 of
  // column n). A wave covers 16 columns x 32 rows per pass; 16-lane group h
  // takes rows 8h..8h+7 of the block (two transposing reads of 4 rows).
  auto cols_out = [&](auto&& fn) {
    const int s = lane & 15, h = lane >> 4;
#pragma unroll 4
    for (int p = 0; p < (TM / 32) * (TN / 16) / NWAVE; ++p) {
      const int P = wave + NWAVE * p, cb = P % (TN / 16), rb = P / (TN / 16);
      const int r = rb * 32 + 8 * h + (s >> 2), col = cb * 16 + 4 * (s & 3);
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4_t*)(lds + soff(r, col >> 3) + (col & 7) * 2));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4_t*)(lds + soff(r + 4, col >> 3) + (col & 7) * 2));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      fn(n0 + cb * 16 + s, m0 + rb * 32 + 8 * h, make_uint4(l2.x, l2.y, h2.x, h2.y));
    }
  };
  auto half = [](const uint4& v, int e) {  // 16-bit element e of 16 bytes
    const uint32_t w = comp(v, e >> 1);
    return (e & 1) ? (w >> 16) : (w & 0xffffu);
  };

  if constexpr (KIND == GRAM || KIND == POLY) {
    char* C = P.ws + (KIND == GRAM ? M.a_off : M.b_off);
    const int mp = M.mp;
    const bool strict = TJ * TN >= (TI + 1) * TM;  // every element above the diagonal
    if constexpr (KIND == POLY) {
      // B = c (A A) + b A (+ a I for fp16 operands, so that the update is
      // B' X).
      if (fold) {
        // acc = A A + (b / c) A already. Only a 32 x 32 block that a diagonal
        // tile's diagonal crosses (its rows and columns start together; the
        // offsets are wave-uniform) holds elements of a I.
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            if (i >= (j ? nr1 : nr0)) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] *= P.c;
            if (TI == TJ && rbase + 32 * i == (j ? cb1 : cb0)) {
#pragma unroll
              for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  if (l32 == 8 * g + 4 * lh + r && m0 + rbase + 32 * i + l32 < M.m)  // padding stays zero
                    acc[i][j][4 * g + r] += P.a;
            }
          }
        stage16(true);
      } else {
      // c = 0: the A tile goes into the staging layout by DMA (whole rows,
      // coalesced); each lane then reads its accumulator positions, combines
      // and writes the result back to the same positions (no other lane
      // touches them, so no barrier is needed in between).
      const char* Am = P.ws + M.a_off;
      constexpr int RPP = 1024 / ROWB;  // staged rows per 1 KB piece
      constexpr int LPR = 64 / RPP;     // lanes per row
#pragma unroll
      for (int q = 0; q < TM * ROWB / 1024 / NWAVE; ++q) {
        const int I = wave + NWAVE * q;
        const int r = RPP * I + lane / LPR, sl = lane % LPR;
        const int x = ((r & 3) << 1) | ((r >> 2) & 1) | (((r >> 3) & 1) << 3);
        const uint32_t base = __builtin_amdgcn_readfirstlane(
            static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)) + I * 1024);
        e16::dma16<COH>(Am + pidx(m0 + r, n0 + 8 * (sl ^ x), mp) * 2, base);
      }
      MUON_WAIT_VMCNT(0);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (i >= (j ? nr1 : nr0)) continue;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int cb = j ? cb1 : cb0;
            char* sp = lds + soff(rbase + 32 * i + l32, cb / 8 + g) + lh * 8;
            const u32x2 bq = *reinterpret_cast<const u32x2*>(sp);
            const float a4[4] = {Op<OP>::load16(bq.x & 0xffffu), Op<OP>::load16(bq.x >> 16),
                                 Op<OP>::load16(bq.y & 0xffffu), Op<OP>::load16(bq.y >> 16)};
            const int m = m0 + rbase + 32 * i + l32, n = n0 + cb + 8 * g + 4 * lh;
            // (a I only in the blocks a diagonal tile's diagonal crosses)
            const bool dblk = TI == TJ && rbase + 32 * i == cb;
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              v[r] = __fmaf_rn(P.c, acc[i][j][4 * g + r], P.b * a4[r]);
              if (dblk && m == n + r && m < M.m) v[r] += P.a;  // padding stays zero
            }
            *reinterpret_cast<uint2*>(sp) = e16::pack4(v[0], v[1], v[2], v[3], true);
          }
        }
      }
    } else if (SK && reducing) {
      // one 128 x 128 quarter (qr, qc) of the tile: its 64 KB of each part's
      // accumulator-order partial (waves qr*4 + 2qc and the next) summed in
      // part order by all threads, 16 bytes (4 floats of one lane and block)
      // at a time, into the staged tile
      const int qr = sp >> 1, qc = sp & 1;
      // the first step's Gram: A0 = sigma^2 (sum of the operand's products)
      float gsc = 1.f;
      if (P.x0_scaled) {
        const float sg = reinterpret_cast<const float*>(P.ws + P.x0s_off)[4 * it.mat];
        gsc = sg * sg;
      }
      const char* qbase = P.ws + P.split_off + int64_t(pbase) * (TM * TN * 4) + (qr * 4 + 2 * qc) * 32768;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4_t sum[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) sum[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int q0 = 0; q0 < S; q0 += 4) {
          f32x4_t x[4][4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (q0 + q < S)
#pragma unroll
              for (int u = 0; u < 4; ++u)
                x[q][u] = *reinterpret_cast<const f32x4_t*>(qbase + int64_t(q0 + q) * (TM * TN * 4) +
                                                            ((h * 4 + u) * NTHR + tid) * 16);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (q0 + q < S)
#pragma unroll
              for (int u = 0; u < 4; ++u) sum[u] += x[q][u];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int o = ((h * 4 + u) * NTHR + tid) * 16;
          const int wl = o >> 15, blk = (o >> 12) & 7, ln = (o >> 6) & 63, v = (o >> 4) & 3;
          const int r = qr * 128 + 32 * (blk >> 1) + (ln & 31);
          const int c = (2 * qc + wl) * 8 + 4 * (blk & 1) + v;
          *reinterpret_cast<uint2*>(lds + soff(r, c) + (ln >> 5) * 8) =
              e16::pack4(sum[u][0] * gsc, sum[u][1] * gsc, sum[u][2] * gsc, sum[u][3] * gsc, true);
        }
      }
    } else {
      if (P.x0_scaled) {
        // the first step's Gram: A0 = sigma^2 (sum of the operand's products)
        const float sg = reinterpret_cast<const float*>(P.ws + P.x0s_off)[4 * it.mat];
        const float s2 = sg * sg;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] *= s2;
      }
      stage16(true);
    }
    __syncthreads();
    if (!strict && !(SK && reducing)) {
      // Diagonal tile: only its upper triangle is staged (and only it is
      // needed). The lower triangle is completed inside LDS from the upper
      // one (so C stays bitwise symmetric): the 16 bytes at row n, columns
      // m .. m+7 (m + 7 < n) are column n of rows m .. m+7, read transposed;
      // a chunk that the diagonal crosses (m <= n <= m+7) takes its columns
      // below n the same way and keeps the rest. Then every row goes out
      // with whole 16-byte stores and no mirror pass is needed.
      cols_out([&](int n, int m, const uint4& v) {
        const int rn = n - n0, cm = m - m0;
        if (cm >= rn) return;
        uint4* d = reinterpret_cast<uint4*>(lds + soff(rn, cm >> 3));
        if (cm + 7 < rn) {
          *d = v;
        } else {
          const uint4 t = *d;
          uint32_t w[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t lo = cm + 2 * q < rn ? half(v, 2 * q) : half(t, 2 * q);
            const uint32_t hi = cm + 2 * q + 1 < rn ? half(v, 2 * q + 1) : half(t, 2 * q + 1);
            w[q] = lo | (hi << 16);
          }
          *d = make_uint4(w[0], w[1], w[2], w[3]);
        }
      });
      __syncthreads();
      rows_out([&](int m, int n, const uint4& v) {
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(C) + pidx(m, n, mp)) = v;
      });
    } else {
      // (the reduce pass of a split tile stores its quarter only)
      auto in_quarter = [&](int m, int n) {
        if constexpr (!SK) return true;
        if (!reducing) return true;
        return ((m - m0) >> 7) == (sp >> 1) && ((n - n0) >> 7) == (sp & 1);
      };
      // C[m][n..n+7] where m <= n
      rows_out([&](int m, int n, const uint4& v) {
        if (!in_quarter(m, n)) return;
        uint16_t* d = reinterpret_cast<uint16_t*>(C) + pidx(m, n, mp);
        if (strict || m <= n) {
          *reinterpret_cast<uint4*>(d) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (m <= n + e) d[e] = static_cast<uint16_t>(half(v, e));
        }
      });
      // mirror: C[n][m..m+7] = C[m..m+7][n] where m < n
      cols_out([&](int n, int m, const uint4& v) {
        if (!in_quarter(m, n)) return;
        uint16_t* d = reinterpret_cast<uint16_t*>(C) + pidx(n, m, mp);
        if (strict || m + 7 < n) {
          *reinterpret_cast<uint4*>(d) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (m + e < n) d[e] = static_cast<uint16_t>(half(v, e));
        }
      });
    }
  } else {
    // UPDATE. The low bytes are read (and, unless this is the last step,
    // written back) in accumulator order, one 16-byte access per lane and
    // accumulator block, all loads first (one latency for the tile).
    {
      char* lo_t = P.ws + M.xl_off + (int64_t(TI) * (M.np / TN) + TJ) * (TM * TN) + lane * 16;
      auto lo_ptr = [&](int i, int j) { return lo_t + (((wm * 4 + i) * WN + wn) * 2 + j) * 1024; };
      u32x4 lq[4][2];
      {
        // the low bytes arrived with the k loop's last passes: block bi
        // (1 KB, 16 bytes per lane) is at offset (bi % 32) KB of ring slot
        // (nst + bi / 32) % NS; every wave reads its blocks before any wave
        // stages its result over the ring
        const int nst = static_cast<int>(K / KS);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int bi = ((wm * 4 + i) * WN + wn) * 2 + j;
            lq[i][j] = *reinterpret_cast<const u32x4*>(lds + ((nst + (bi >> 5)) % NS) * STAGE + (bi & 31) * 1024 +
                                                       lane * 16);
          }
        MUON_WAIT_LGKMCNT0();
        asm volatile("s_barrier" ::: "memory");
      }
      // X' = B' hi + a 2^-18 lo  (B' = a I + B carries a hi). The first step
      // (X0S, a kernel of its own so that the other steps' register
      // allocation is untouched) starts from X0 = sigma (U) with U = hi +
      // lo 2^-5: X1 = sigma (B' hi + a 2^-5 lo).
      const float as = P.a * (X0S ? 1.f / kX0LoScale : 1.f / Op<OP>::kLoScale);
      float sg = 1.f;
      if constexpr (X0S) sg = reinterpret_cast<const float*>(P.ws + P.x0s_off)[4 * it.mat];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          uint32_t qw[4];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            {
              float lv[4];
              Op<OP>::lo_vals(lq[i][j][g], lv);
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                acc[i][j][4 * g + r] = __fmaf_rn(as, lv[r], acc[i][j][4 * g + r]);
                if constexpr (X0S) acc[i][j][4 * g + r] *= sg;
              }
            }
            if constexpr (!LAST) {
              // split back into hi (staged straight into the LDS tile, the
              // ring is free) and the low bytes; x - hi is exact (sub_l/h)
              uint32_t hp[2];
              float rs[4];
#pragma unroll
              for (int q = 0; q < 2; ++q) {
                const float v0 = acc[i][j][4 * g + 2 * q], v1 = acc[i][j][4 * g + 2 * q + 1];
                hp[q] = e16::pk16(v0, v1);
                rs[2 * q] = e16::sub_l(v0, hp[q]);
                rs[2 * q + 1] = e16::sub_h(v1, hp[q]);
              }
              qw[g] = Op<OP>::lo4(rs[0], rs[1], rs[2], rs[3]);
              *reinterpret_cast<uint2*>(lds + soff(wm * 128 + 32 * i + l32, wn * 8 + 4 * j + g) + lh * 8) =
                  make_uint2(hp[0], hp[1]);
            }
          }
          if constexpr (!LAST) *reinterpret_cast<u32x4*>(lo_ptr(i, j)) = u32x4{qw[0], qw[1], qw[2], qw[3]};
        }
      if constexpr (!LAST) {
        // the staged hi tile is complete once every wave's LDS writes are;
        // a bare barrier, so the low-byte stores above stay in flight (the
        // workgroup fence of __syncthreads would wait for them)
        MUON_WAIT_LGKMCNT0();
        asm volatile("s_barrier" ::: "memory");
        uint16_t* xn = reinterpret_cast<uint16_t*>(P.ws + M.xo_nxt);
        rows_out([&](int m, int n, const uint4& v) {
          *reinterpret_cast<uint4*>(xn + pidx(m, n, M.mp)) = v;
        });
        return;
      }
    }
    // the last step: X is the result
    if (P.apply) {
      // weight application: W' = W keep - step X in the caller's layout
      // (transposed for tall matrices); X is staged as fp16, three more
      // significant bits than the set's bf16
      stage16(true);
      __syncthreads();
      uint16_t* wm16 = static_cast<uint16_t*>(M.w);
      const float keep = M.keep, step = M.step;
      auto putw = [&](int row, int col, int nrow, int ncol, const uint4& v) {
        if (row >= nrow) return;
        uint16_t* d = wm16 + int64_t(row) * M.wld + col;
        if (M.w_vec_ok && col + 7 < ncol) {
          const uint4 wv = *reinterpret_cast<const uint4*>(d);
          uint32_t r[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float x0 = Op<OP_F16>::load16(half(v, 2 * q)), x1 = Op<OP_F16>::load16(half(v, 2 * q + 1));
            const float w0 = bf2f(static_cast<uint16_t>(half(wv, 2 * q)));
            const float w1 = bf2f(static_cast<uint16_t>(half(wv, 2 * q + 1)));
            r[q] = uint32_t(f2bf(__fmaf_rn(-step, x0, w0 * keep))) |
                   (uint32_t(f2bf(__fmaf_rn(-step, x1, w1 * keep))) << 16);
          }
          *reinterpret_cast<uint4*>(d) = make_uint4(r[0], r[1], r[2], r[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (col + e < ncol)
              d[e] = f2bf(__fmaf_rn(-step, Op<OP_F16>::load16(half(v, e)), bf2f(d[e]) * keep));
        }
      };
      if (!M.tall)
        rows_out([&](int m, int n, const uint4& v) { putw(m, n, M.m, M.n, v); });
      else
        cols_out([&](int n, int m, const uint4& v) { putw(n, m, M.n, M.m, v); });
    } else {
      // `out` in the caller's layout (bf16), transposed for tall matrices
      stage16(false);
      __syncthreads();
      uint16_t* o = static_cast<uint16_t*>(M.out);
      auto put = [&](int row, int col, int nrow, int ncol, const uint4& v) {
        if (row >= nrow) return;
        uint16_t* d = o + int64_t(row) * M.ld + col;
        if (M.vec_ok && col + 7 < ncol) {
          *reinterpret_cast<uint4*>(d) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (col + e < ncol) d[e] = static_cast<uint16_t>(half(v, e));
        }
      };
      if (!M.tall)
        rows_out([&](int m, int n, const uint4& v) { put(m, n, M.m, M.n, v); });
      else
        cols_out([&](int n, int m, const uint4& v) { put(n, m, M.n, M.m, v); });
    }
  }
}

template <typename T, int OP, int KIND, bool LAST, bool SK = false, bool X0S = false>
__global__ __launch_bounds__(e16::NTHR, 1) void gemm16_kernel(StepArgs P) {
  __shared__ __attribute__((aligned(16))) char lds[e16::LDS_BYTES];
  tile16<T, OP, KIND, LAST, SK, X0S>(P, P.items[blockIdx.x], lds, threadIdx.x);
}

// ------------------------------------------------------- chained schedule
// One launch runs every Gram, poly and update tile of all steps (plan.hpp:
// per-XCD lists, tickets, per-matrix completion counters). All tiles of a
// matrix run on one XCD, so everything they pass to each other goes through
// that XCD's L2, which every CU of the XCD shares: a tile's stores have
// reached it once the wave's vector-memory count is zero, and a reader sees
// them if it does not take an older copy from its CU's L1. The chained
// tiles read their operands with device-scope loads (COH), which the L1
// does not serve from an older copy. (An L1 invalidate is not the tool: the
// workgroup-scope one need not touch the L1 of a workgroup that sits on one
// CU, and tiles then read stale lines; the device-scope one also drops the
// XCD's L2, which cost 10 % of the step.)

// The XCD (accelerator complex die) this workgroup runs on: hardware
// register XCC_ID, bits 3:0.
__device__ __forceinline__ int xcc_id() {
  return static_cast<int>(__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20));
}

// A wait is bounded (ChainArgs::wait_ticks of the 100 MHz real-time
// counter); one that runs out records the fact in the plan's error word and
// its workgroup skips its item, so a broken schedule ends the launch
// instead of hanging it.
__device__ __forceinline__ bool chain_wait(const int32_t* cnt, int32_t need, int32_t* err, uint64_t bound) {
  if (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= need) return true;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    __builtin_amdgcn_s_sleep(2);
    if (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= need) return true;
    if (__builtin_amdgcn_s_memrealtime() - t0 > bound) {
      __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
  }
}

// Persistent: one workgroup per CU; each takes tickets from its XCD's list
// until the list is drained. The ticket for the next pass is fetched when
// the current tile's k loop is done (its epilogue hides the atomic's
// latency; fetched earlier, a long tile would hold a ticket that others
// wait for), by a lane of wave 4 (waves 0 .. 3 issue the ring's DMA and
// count it with their vector-memory counters, which must not hold anything
// else). A workgroup holding a ticket is always running, and it finishes
// its current tile before it waits for the next one, so the lowest
// unfinished ticket is always some workgroup's current tile and its inputs
// are done.
constexpr int kChainOwner = 4 * 64;  // the thread that takes tickets and waits
__global__ __launch_bounds__(e16::NTHR, 1) void chain16_kernel(StepArgs P, ChainArgs C) {
  __shared__ __attribute__((aligned(16))) char lds[e16::LDS_BYTES];
  __shared__ int32_t slot[2];
  const int x = xcc_id();
  if (x >= kNumXcd) {
    if (threadIdx.x == 0) __hip_atomic_store(C.err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  int32_t* tick = reinterpret_cast<int32_t*>(P.ws + P.chain_off);
  int32_t* done = tick + kNumXcd;
  const int32_t beg = C.beg[x], len = C.beg[x + 1] - beg, total = len * C.steps;
  int32_t next = 0, prev = -1;  // (owner) the tickets of the next and the last pass
  int32_t seen = -1;             // (owner) an early reading of the next tile's counter
  if (threadIdx.x == kChainOwner)
    next = __hip_atomic_fetch_add(tick + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (;;) {
    if (threadIdx.x == kChainOwner) {
      const int32_t t = next;
      bool ok = true;
      if (t <= prev) {  // tickets only grow: a pass without a fetch ends the loop
        __hip_atomic_store(C.err, 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = false;
      } else if (t < total) {
        const int32_t step = t / len;
        const ChainItem ci = C.items[beg + t - step * len];
        // (counters only grow: an earlier reading that already meets the
        // need proves it)
        const int32_t need = step * (ci.kind_n >> 8) + ci.need;
        if (seen < need) ok = chain_wait(done + ci.mat, need, C.err, C.wait_ticks);
      }
      prev = t;
      slot[0] = t;
      slot[1] = ok ? 1 : 0;
    }
    __syncthreads();
    const int32_t t = __builtin_amdgcn_readfirstlane(slot[0]);
    if (t >= total || __builtin_amdgcn_readfirstlane(slot[1]) == 0) break;
    // The lane index through an empty move: a value the compiler cannot
    // carry from one pass to the next, so the tile's lane arithmetic is
    // recomputed per tile instead of being held in registers across passes.
    uint32_t tid;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"(static_cast<uint32_t>(threadIdx.x)));
    const int32_t step = t / len;
    const ChainItem ci = C.items[beg + t - step * len];
    StepArgs Q = P;
    Q.cur = step & 1;
    Q.last = step == C.steps - 1 ? 1 : 0;
    Q.x0_scaled = step == 0 ? 1 : 0;
    const WorkItem it{ci.mat, ci.ti, ci.tj, 0};
    const int kind = ci.kind_n & 255;
    auto fetch = [&]() {
      if (threadIdx.x == kChainOwner)
        next = __hip_atomic_fetch_add(tick + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    if (kind == MUON_K_GRAM) {
      tile16<uint16_t, OP_F16, GRAM, false, false, false, true>(Q, it, lds, tid, fetch);
    } else if (kind == MUON_K_POLY) {
      tile16<uint16_t, OP_F16, POLY, false, false, false, true>(Q, it, lds, tid, fetch);
    } else if (step == 0) {
      if (Q.last) tile16<uint16_t, OP_F16, UPDATE, true, false, true, true>(Q, it, lds, tid, fetch);
      else tile16<uint16_t, OP_F16, UPDATE, false, false, true, true>(Q, it, lds, tid, fetch);
    } else {
      if (Q.last) tile16<uint16_t, OP_F16, UPDATE, true, false, false, true>(Q, it, lds, tid, fetch);
      else tile16<uint16_t, OP_F16, UPDATE, false, false, false, true>(Q, it, lds, tid, fetch);
    }
    // the next tile's record and an early reading of its counter, while
    // the stores drain (the pass's wait then usually has nothing to wait for)
    seen = -1;
    if (threadIdx.x == kChainOwner && next < total) {
      const int32_t ns = next / len;
      const ChainItem nci = C.items[beg + next - ns * len];
      seen = __hip_atomic_load(done + nci.mat, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // release: every wave's stores have reached L2, then the count goes up
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == kChainOwner)
      __hip_atomic_fetch_add(done + ci.mat, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// --------------------------------------------------------------- launchers

template <typename T, int OP>
static hipError_t launch_t(int kind, const StepArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  const bool engine16 = OP != OP_F32 && (kind == MUON_K_GRAM || kind == MUON_K_POLY || kind == MUON_K_UPDATE);
  dim3 g(grid), b(engine16 ? e16::NTHR : 256);
  switch (kind) {
    case MUON_K_MOMENTUM: hipLaunchKernelGGL(momentum_kernel<T>, g, b, 0, s, a); break;
    case MUON_K_NORMALIZE: hipLaunchKernelGGL((normalize_kernel<T, OP>), g, b, 0, s, a); break;
    case kKernelMomentumX0:
      if constexpr (OP == OP_F32) return hipErrorInvalidValue;
      else hipLaunchKernelGGL(momentum_x0_kernel, g, b, 0, s, a);
      break;
    case kKernelX0Scale:
      if constexpr (OP == OP_F32) return hipErrorInvalidValue;
      else hipLaunchKernelGGL(x0_scale_kernel, g, b, 0, s, a);
      break;
    case kKernelX0Rewrite:
      if constexpr (OP == OP_F32) return hipErrorInvalidValue;
      else hipLaunchKernelGGL(x0_rewrite_kernel, dim3(grid < kX0RewriteGrid ? grid : kX0RewriteGrid), b, 0, s, a);
      break;
    case MUON_K_GRAM:
      if constexpr (OP == OP_F32) hipLaunchKernelGGL((gemm32_kernel<T, OP, GRAM>), g, b, 0, s, a);
      else if (a.split_off >= 0) hipLaunchKernelGGL((gemm16_kernel<T, OP, GRAM, false, true>), g, b, 0, s, a);
      else hipLaunchKernelGGL((gemm16_kernel<T, OP, GRAM, false>), g, b, 0, s, a);
      break;
    case MUON_K_POLY:
      if constexpr (OP == OP_F32) hipLaunchKernelGGL((gemm32_kernel<T, OP, POLY>), g, b, 0, s, a);
      else hipLaunchKernelGGL((gemm16_kernel<T, OP, POLY, false>), g, b, 0, s, a);
      break;
    case MUON_K_UPDATE:
      if constexpr (OP == OP_F32) hipLaunchKernelGGL((gemm32_kernel<T, OP, UPDATE>), g, b, 0, s, a);
      else if (a.x0_scaled && a.last) hipLaunchKernelGGL((gemm16_kernel<T, OP, UPDATE, true, false, true>), g, b, 0, s, a);
      else if (a.x0_scaled) hipLaunchKernelGGL((gemm16_kernel<T, OP, UPDATE, false, false, true>), g, b, 0, s, a);
      else if (a.last) hipLaunchKernelGGL((gemm16_kernel<T, OP, UPDATE, true>), g, b, 0, s, a);
      else hipLaunchKernelGGL((gemm16_kernel<T, OP, UPDATE, false>), g, b, 0, s, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_chain(const StepArgs& a, const ChainArgs& c, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(chain16_kernel, dim3(grid), dim3(e16::NTHR), 0, s, a, c);
  return hipGetLastError();
}

hipError_t launch_kernel(int kind, muon_dtype dt, const StepArgs& a, int grid, hipStream_t s) {
  if (dt == MUON_F32) return launch_t<float, OP_F32>(kind, a, grid, s);
  return launch_t<uint16_t, OP_F16>(kind, a, grid, s);
}

}  // namespace muon
