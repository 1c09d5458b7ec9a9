// Adam branch of the optimizer step (include/muon_adam.h): one fused
// elementwise kernel over a whole list of parameter tensors, its plan
// (validated tensor table and work items in device memory) and the C ABI.
//
// The update (mhpq.cn, modded-nanogpt track_1_short technical guide, section
// 6.2: Adam with betas (0.9, 0.99) and per-group lr_mul / wd_mul for the
// parameters off the Muon path), per element, in fp32:
//   m = beta1 m + (1 - beta1) g;  v = beta2 v + (1 - beta2) g^2
//   p = p (1 - lr' wd') - (lr' / bc1) m / (sqrt(v) / sqrt(bc2) + eps)
// with lr' = lr lr_mul, wd' = wd wd_mul, bc_i = 1 - beta_i^t (the bias-
// corrected form m/bc1 / (sqrt(v/bc2) + eps), rearranged so that the per-call
// factors 1/bc1 and 1/sqrt(bc2) are computed once on the host).
//
// HBM-bound: per element it reads p, g, m, v and writes p, m, v (22 bytes
// for bf16 parameters, 28 for fp32). Each block streams one work item of at
// most 16384 consecutive elements of one tensor, 8 per thread per pass with
// 16-byte accesses when the tensor's buffers allow it.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/muon_adam.h"

namespace muon_adam {

constexpr int kChunk = 16384;  // elements per work item
constexpr int kThreads = 256;
constexpr int kVec = 8;        // elements per thread per pass

struct Tensor {
  void* p;
  const void* g;
  float* m;
  float* v;
  int64_t numel;
  float lr_mul, wd_mul;
  int32_t vec;  // 16-byte vector access legal for all four buffers
  int32_t pad_;
};

struct Item {
  int32_t t;      // tensor index
  int32_t chunk;  // elements chunk * kChunk .. + kChunk - 1 of the tensor
};

struct Args {
  const Tensor* ts;
  const Item* items;
  float lr, b1, b2, eps, wd;
  float inv_bc1, inv_sqrt_bc2;  // 1 / (1 - beta1^t), 1 / sqrt(1 - beta2^t)
};

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) {  // round to nearest even
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);  // NaN
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

template <typename T> struct PElem;
template <> struct PElem<float> {
  static __device__ __forceinline__ float load(const void* p, int64_t i) { return static_cast<const float*>(p)[i]; }
  static __device__ __forceinline__ void store(void* p, int64_t i, float v) { static_cast<float*>(p)[i] = v; }
};
template <> struct PElem<uint16_t> {
  static __device__ __forceinline__ float load(const void* p, int64_t i) {
    return bf2f(static_cast<const uint16_t*>(p)[i]);
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = f2bf(v);
  }
};

struct Consts {
  float b1, c1, b2, c2, eps, keep, step, isb2;
};

// One element: updates m, v in place and returns the new parameter value.
__device__ __forceinline__ float adam_elem(float p, float g, float& m, float& v, const Consts& k) {
  m = __fmaf_rn(k.b1, m, k.c1 * g);
  v = __fmaf_rn(k.b2, v, k.c2 * (g * g));
  const float denom = __fsqrt_rn(v) * k.isb2 + k.eps;
  return __fmaf_rn(-k.step, __fdiv_rn(m, denom), p * k.keep);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Eight consecutive elements of one tensor in registers.
struct Vec8 {
  float p[kVec], g[kVec], m[kVec], v[kVec];
};

template <typename T>
__device__ __forceinline__ void load8(const Tensor& t, int64_t e0, Vec8& x) {
  if constexpr (sizeof(T) == 2) {
    const u32x4 pw = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(t.p) + e0);
    const u32x4 gw = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(t.g) + e0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x.p[2 * q] = __uint_as_float(pw[q] << 16);
      x.p[2 * q + 1] = __uint_as_float(pw[q] & 0xffff0000u);
      x.g[2 * q] = __uint_as_float(gw[q] << 16);
      x.g[2 * q + 1] = __uint_as_float(gw[q] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 pv = *reinterpret_cast<const f32x4*>(static_cast<const float*>(t.p) + e0 + 4 * h);
      const f32x4 gv = *reinterpret_cast<const f32x4*>(static_cast<const float*>(t.g) + e0 + 4 * h);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        x.p[4 * h + q] = pv[q];
        x.g[4 * h + q] = gv[q];
      }
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const f32x4 mv = *reinterpret_cast<const f32x4*>(t.m + e0 + 4 * h);
    const f32x4 vv = *reinterpret_cast<const f32x4*>(t.v + e0 + 4 * h);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x.m[4 * h + q] = mv[q];
      x.v[4 * h + q] = vv[q];
    }
  }
}

template <typename T>
__device__ __forceinline__ void store8(const Tensor& t, int64_t e0, const Vec8& x) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    *reinterpret_cast<f32x4*>(t.m + e0 + 4 * h) =
        f32x4{x.m[4 * h], x.m[4 * h + 1], x.m[4 * h + 2], x.m[4 * h + 3]};
    *reinterpret_cast<f32x4*>(t.v + e0 + 4 * h) =
        f32x4{x.v[4 * h], x.v[4 * h + 1], x.v[4 * h + 2], x.v[4 * h + 3]};
  }
  if constexpr (sizeof(T) == 2) {
    u32x4 pw;
#pragma unroll
    for (int q = 0; q < 4; ++q) pw[q] = uint32_t(f2bf(x.p[2 * q])) | (uint32_t(f2bf(x.p[2 * q + 1])) << 16);
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(t.p) + e0) = pw;
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      *reinterpret_cast<f32x4*>(static_cast<float*>(t.p) + e0 + 4 * h) =
          f32x4{x.p[4 * h], x.p[4 * h + 1], x.p[4 * h + 2], x.p[4 * h + 3]};
  }
}

__device__ __forceinline__ void update8(Vec8& x, const Consts& k) {
#pragma unroll
  for (int e = 0; e < kVec; ++e) x.p[e] = adam_elem(x.p[e], x.g[e], x.m[e], x.v[e], k);
}

// Elements e0 .. min(e0 + 8, end) - 1, vector or scalar.
template <typename T>
__device__ __forceinline__ void run8(const Tensor& t, int64_t e0, int64_t end, const Consts& k) {
  if (t.vec && e0 + kVec <= end) {
    Vec8 x;
    load8<T>(t, e0, x);
    update8(x, k);
    store8<T>(t, e0, x);
  } else {
    const int64_t e1 = e0 + kVec < end ? e0 + kVec : end;
    for (int64_t e = e0; e < e1; ++e) {
      float m = t.m[e], v = t.v[e];
      const float p = adam_elem(PElem<T>::load(t.p, e), PElem<T>::load(t.g, e), m, v, k);
      t.m[e] = m;
      t.v[e] = v;
      PElem<T>::store(t.p, e, p);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void adam_kernel(Args A) {
  const Item it = A.items[blockIdx.x];
  const Tensor t = A.ts[it.t];
  const float lr_e = A.lr * t.lr_mul;
  Consts k;
  k.b1 = A.b1;
  k.c1 = 1.f - A.b1;
  k.b2 = A.b2;
  k.c2 = 1.f - A.b2;
  k.eps = A.eps;
  k.keep = 1.f - lr_e * (A.wd * t.wd_mul);
  k.step = lr_e * A.inv_bc1;
  k.isb2 = A.inv_sqrt_bc2;
  const int64_t base = int64_t(it.chunk) * kChunk;
  const int64_t end = base + kChunk < t.numel ? base + kChunk : t.numel;
  // two vectors per thread per pass, both loaded before either is updated
  constexpr int64_t kPass = int64_t(kThreads) * kVec;
  for (int64_t e0 = base + int64_t(threadIdx.x) * kVec; e0 < end; e0 += 2 * kPass) {
    const int64_t e1 = e0 + kPass;
    if (t.vec && e1 + kVec <= end) {
      Vec8 x, y;
      load8<T>(t, e0, x);
      load8<T>(t, e1, y);
      update8(x, k);
      update8(y, k);
      store8<T>(t, e0, x);
      store8<T>(t, e1, y);
    } else {
      run8<T>(t, e0, end, k);
      if (e1 < end) run8<T>(t, e1, end, k);
    }
  }
}

// ------------------------------------------------------------------ host

struct Interval {
  uintptr_t lo, hi;
  bool write;
};

muon_status build(const muon_adam_tensor* ts, int32_t n, muon_dtype dtype, std::vector<Tensor>* out,
                  std::vector<Item>* items) {
  if (dtype != MUON_F32 && dtype != MUON_BF16) return MUON_E_DTYPE;
  if (n < 0 || n > MUON_ADAM_MAX_TENSORS) return MUON_E_SHAPE;
  if (n > 0 && ts == nullptr) return MUON_E_INVALID;
  const size_t es = dtype == MUON_F32 ? 4 : 2;
  std::vector<Interval> iv;
  out->assign(static_cast<size_t>(n), Tensor{});
  items->clear();
  for (int32_t i = 0; i < n; ++i) {
    const muon_adam_tensor& T = ts[i];
    if (T.numel < 0 || T.numel > MUON_ADAM_MAX_NUMEL) return MUON_E_SHAPE;
    if (T.numel == 0) continue;
    if (!T.param || !T.grad || !T.exp_avg || !T.exp_avg_sq) return MUON_E_INVALID;
    if (!std::isfinite(T.lr_mul) || !std::isfinite(T.wd_mul)) return MUON_E_INVALID;
    auto addr = [](const void* p) { return reinterpret_cast<uintptr_t>(p); };
    if (addr(T.param) % es || addr(T.grad) % es || addr(T.exp_avg) % 4 || addr(T.exp_avg_sq) % 4)
      return MUON_E_ALIGN;
    const uintptr_t pb = static_cast<uintptr_t>(T.numel) * es, sb = static_cast<uintptr_t>(T.numel) * 4;
    iv.push_back({addr(T.param), addr(T.param) + pb, true});
    iv.push_back({addr(T.grad), addr(T.grad) + pb, false});
    iv.push_back({addr(T.exp_avg), addr(T.exp_avg) + sb, true});
    iv.push_back({addr(T.exp_avg_sq), addr(T.exp_avg_sq) + sb, true});
    Tensor& D = (*out)[i];
    D.p = T.param;
    D.g = T.grad;
    D.m = T.exp_avg;
    D.v = T.exp_avg_sq;
    D.numel = T.numel;
    D.lr_mul = T.lr_mul;
    D.wd_mul = T.wd_mul;
    D.vec = (addr(T.param) | addr(T.grad) | addr(T.exp_avg) | addr(T.exp_avg_sq)) % 16 == 0;
    const int64_t chunks = (T.numel + kChunk - 1) / kChunk;
    for (int64_t c = 0; c < chunks; ++c) items->push_back({i, static_cast<int32_t>(c)});
  }
  std::sort(iv.begin(), iv.end(), [](const Interval& x, const Interval& y) { return x.lo < y.lo; });
  uintptr_t max_hi_any = 0, max_hi_w = 0;
  for (const Interval& x : iv) {
    if (x.lo < max_hi_w || (x.write && x.lo < max_hi_any)) return MUON_E_INVALID;
    max_hi_any = std::max(max_hi_any, x.hi);
    if (x.write) max_hi_w = std::max(max_hi_w, x.hi);
  }
  return MUON_OK;
}

}  // namespace muon_adam

struct muon_adam_plan_s {
  int device = -1;
  muon_dtype dtype = MUON_BF16;
  void* dmem = nullptr;
  const muon_adam::Tensor* d_ts = nullptr;
  const muon_adam::Item* d_items = nullptr;
  int64_t nitems = 0;
};

extern "C" {

muon_status muon_adam_work_items(const muon_adam_tensor* ts, int32_t n, muon_dtype dtype,
                                 int64_t* items) {
  if (items == nullptr) return MUON_E_INVALID;
  std::vector<muon_adam::Tensor> t;
  std::vector<muon_adam::Item> it;
  const muon_status st = muon_adam::build(ts, n, dtype, &t, &it);
  if (st != MUON_OK) return st;
  *items = static_cast<int64_t>(it.size());
  return MUON_OK;
}

muon_status muon_adam_plan_create(const muon_adam_tensor* ts, int32_t n, muon_dtype dtype,
                                  muon_adam_plan** plan) {
  if (plan == nullptr) return MUON_E_INVALID;
  *plan = nullptr;
  std::vector<muon_adam::Tensor> t;
  std::vector<muon_adam::Item> it;
  muon_status st = muon_adam::build(ts, n, dtype, &t, &it);
  if (st != MUON_OK) return st;
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess ||
      std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return MUON_E_DEVICE;
  muon_adam_plan_s* p = new (std::nothrow) muon_adam_plan_s();
  if (!p) return MUON_E_ALLOC;
  p->device = dev;
  p->dtype = dtype;
  p->nitems = static_cast<int64_t>(it.size());
  const size_t tb = (sizeof(muon_adam::Tensor) * std::max<size_t>(1, t.size()) + 255) / 256 * 256;
  const size_t bytes = tb + sizeof(muon_adam::Item) * std::max<size_t>(1, it.size());
  std::vector<char> h(bytes, 0);
  if (!t.empty()) std::memcpy(h.data(), t.data(), sizeof(muon_adam::Tensor) * t.size());
  if (!it.empty()) std::memcpy(h.data() + tb, it.data(), sizeof(muon_adam::Item) * it.size());
  if (hipMalloc(&p->dmem, bytes) != hipSuccess) {
    (void)hipGetLastError();
    delete p;
    return MUON_E_ALLOC;
  }
  if (hipMemcpy(p->dmem, h.data(), bytes, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(p->dmem);
    delete p;
    return MUON_E_DEVICE;
  }
  p->d_ts = static_cast<const muon_adam::Tensor*>(p->dmem);
  p->d_items = reinterpret_cast<const muon_adam::Item*>(static_cast<char*>(p->dmem) + tb);
  *plan = p;
  return MUON_OK;
}

muon_status muon_adam_plan_step(muon_adam_plan* plan, const muon_adam_config* cfg, void* stream) {
  if (plan == nullptr || cfg == nullptr) return MUON_E_INVALID;
  if (!std::isfinite(cfg->lr) || !std::isfinite(cfg->beta1) || !std::isfinite(cfg->beta2) ||
      !std::isfinite(cfg->eps) || !std::isfinite(cfg->wd))
    return MUON_E_INVALID;
  if (cfg->beta1 < 0.f || cfg->beta1 >= 1.f || cfg->beta2 < 0.f || cfg->beta2 >= 1.f ||
      cfg->eps < 0.f || cfg->step < 1)
    return MUON_E_INVALID;
  if (plan->nitems == 0) return MUON_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != plan->device) return MUON_E_DEVICE;
  muon_adam::Args a{};
  a.ts = plan->d_ts;
  a.items = plan->d_items;
  a.lr = cfg->lr;
  a.b1 = cfg->beta1;
  a.b2 = cfg->beta2;
  a.eps = cfg->eps;
  a.wd = cfg->wd;
  a.inv_bc1 = static_cast<float>(1.0 / (1.0 - std::pow(double(cfg->beta1), double(cfg->step))));
  a.inv_sqrt_bc2 =
      static_cast<float>(1.0 / std::sqrt(1.0 - std::pow(double(cfg->beta2), double(cfg->step))));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(plan->nitems)), block(muon_adam::kThreads);
  if (plan->dtype == MUON_F32)
    hipLaunchKernelGGL(muon_adam::adam_kernel<float>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(muon_adam::adam_kernel<uint16_t>, grid, block, 0, s, a);
  return hipGetLastError() == hipSuccess ? MUON_OK : MUON_E_LAUNCH;
}

void muon_adam_plan_destroy(muon_adam_plan* plan) {
  if (!plan) return;
  (void)hipDeviceSynchronize();
  if (plan->dmem) (void)hipFree(plan->dmem);
  delete plan;
}

}  // extern "C"
