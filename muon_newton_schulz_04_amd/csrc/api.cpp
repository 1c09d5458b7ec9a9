// C ABI of the Muon update library: validation, plans (device tables),
// launches, per-kernel timing and the plan cache behind muon_step.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstring>
#include <list>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "launch.hpp"
#include "plan.hpp"

using muon::HostPlan;
using muon::MatInfo;
using muon::WorkItem;

struct TimedLaunch {
  int kind;
  hipEvent_t start, stop;
};

struct muon_plan_s {
  HostPlan host;
  int device = -1;
  void* dmem = nullptr;                       // MatInfo table + schedules
  const MatInfo* d_mats = nullptr;
  const WorkItem* d_items[muon::kKinds] = {};
  const WorkItem* d_whole[muon::kKinds] = {};  // one-group schedules (timing)
  float* d_hint = nullptr;                    // per matrix: largest |u| of the last call (0: none)
  const muon::ChainItem* d_chain = nullptr;   // chained schedule: the per-XCD lists
  int32_t* d_err = nullptr;                   // chained launches: a wait past its bound (sticky)
  bool chain_on = true;                       // muon_plan_set_chained
  bool chain_ok = false;                      // the device has the 8 x 32 CUs the lists assume
  int64_t chain_wait_us = 2000000;            // muon_plan_set_chain_timeout
  // groups > 1: one stream per group (default priority) and the events that
  // fork them from, and join them back to, the caller's stream
  hipStream_t gstream[muon::kMaxGroups] = {};
  hipEvent_t fork_ev = nullptr;
  hipEvent_t join_ev[muon::kMaxGroups] = {};
  // 0: off; 1: each kernel over the whole set in its own launch, timed;
  // 2: the step's own launches timed as they run (the chained launch as one)
  int timing = 0;
  std::vector<TimedLaunch> pending;           // recorded, not yet read
  std::vector<hipEvent_t> free_events;
  // per muon_kernel_kind, then the chained launch (index MUON_K_COUNT)
  double acc_ms[MUON_K_COUNT + 1] = {};
  int64_t acc_n[MUON_K_COUNT + 1] = {};
  bool has_weights = false;                   // muon_plan_set_weights succeeded
  void* scratch = nullptr;                    // this device's fixed scratch array
};

namespace {

muon_status upload(muon_plan_s* p) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MUON_E_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MUON_E_DEVICE;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MUON_E_DEVICE;
  p->device = dev;
  // the chained lists are per XCD of a whole MI355X (8 XCDs of 32 CUs); on a
  // partitioned device the plan uses the separate launches
  p->chain_ok = prop.multiProcessorCount == muon::kNumCu;
  // set-up time: the device address of this GPU's scratch array (once per
  // device) for muon_plan_step_noalloc
  if (muon::scratch_address(&p->scratch) != hipSuccess) {
    (void)hipGetLastError();
    p->scratch = nullptr;
  }
  size_t bytes = sizeof(MatInfo) * std::max<size_t>(1, p->host.info.size());
  size_t offs[muon::kKinds], woffs[muon::kKinds];
  for (int k = 0; k < muon::kKinds; ++k) {
    bytes = (bytes + 255) / 256 * 256;
    offs[k] = bytes;
    bytes += sizeof(WorkItem) * std::max<size_t>(1, p->host.sched[k].items.size());
    bytes = (bytes + 255) / 256 * 256;
    woffs[k] = bytes;
    bytes += sizeof(WorkItem) * std::max<size_t>(1, p->host.whole[k].items.size());
  }
  bytes = (bytes + 255) / 256 * 256;
  const size_t hint_off = bytes;
  bytes += sizeof(float) * std::max<size_t>(1, p->host.info.size());
  bytes = (bytes + 255) / 256 * 256;
  const size_t err_off = bytes;
  bytes += 256;
  const size_t chain_off = bytes;
  bytes += sizeof(muon::ChainItem) * std::max<size_t>(1, p->host.chain.size());
  std::vector<char> h(bytes, 0);
  if (!p->host.chain.empty())
    std::memcpy(h.data() + chain_off, p->host.chain.data(), sizeof(muon::ChainItem) * p->host.chain.size());
  if (!p->host.info.empty())
    std::memcpy(h.data(), p->host.info.data(), sizeof(MatInfo) * p->host.info.size());
  for (int k = 0; k < muon::kKinds; ++k) {
    const auto& it = p->host.sched[k].items;
    if (!it.empty()) std::memcpy(h.data() + offs[k], it.data(), sizeof(WorkItem) * it.size());
    const auto& wt = p->host.whole[k].items;
    if (!wt.empty()) std::memcpy(h.data() + woffs[k], wt.data(), sizeof(WorkItem) * wt.size());
  }
  if (p->host.ngroups > 1) {
    auto fail = [&]() {
      (void)hipGetLastError();
      return MUON_E_ALLOC;
    };
    if (hipEventCreateWithFlags(&p->fork_ev, hipEventDisableTiming) != hipSuccess) return fail();
    for (int g = 0; g < p->host.ngroups; ++g) {
      if (hipStreamCreateWithFlags(&p->gstream[g], hipStreamNonBlocking) != hipSuccess) return fail();
      if (hipEventCreateWithFlags(&p->join_ev[g], hipEventDisableTiming) != hipSuccess) return fail();
    }
  }
  if (hipMalloc(&p->dmem, bytes) != hipSuccess) {
    p->dmem = nullptr;
    (void)hipGetLastError();
    return MUON_E_ALLOC;
  }
  if (hipMemcpy(p->dmem, h.data(), bytes, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(p->dmem);
    p->dmem = nullptr;
    (void)hipGetLastError();
    return MUON_E_DEVICE;
  }
  char* base = static_cast<char*>(p->dmem);
  p->d_mats = reinterpret_cast<const MatInfo*>(base);
  for (int k = 0; k < muon::kKinds; ++k) {
    p->d_items[k] = reinterpret_cast<const WorkItem*>(base + offs[k]);
    p->d_whole[k] = reinterpret_cast<const WorkItem*>(base + woffs[k]);
  }
  p->d_hint = reinterpret_cast<float*>(base + hint_off);
  p->d_err = reinterpret_cast<int32_t*>(base + err_off);
  p->d_chain = reinterpret_cast<const muon::ChainItem*>(base + chain_off);
  return MUON_OK;
}

void release(muon_plan_s* p) {
  if (!p) return;
  (void)hipDeviceSynchronize();
  for (auto& t : p->pending) {
    (void)hipEventDestroy(t.start);
    (void)hipEventDestroy(t.stop);
  }
  for (auto e : p->free_events) (void)hipEventDestroy(e);
  for (int g = 0; g < muon::kMaxGroups; ++g) {
    if (p->gstream[g]) (void)hipStreamDestroy(p->gstream[g]);
    if (p->join_ev[g]) (void)hipEventDestroy(p->join_ev[g]);
  }
  if (p->fork_ev) (void)hipEventDestroy(p->fork_ev);
  if (p->dmem) (void)hipFree(p->dmem);
  delete p;
}

hipEvent_t get_event(muon_plan_s* p) {
  if (!p->free_events.empty()) {
    hipEvent_t e = p->free_events.back();
    p->free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

muon_status step_impl(muon_plan_s* p, const muon_config* cfg, void* ws, size_t ws_bytes,
                      void* stream, bool orthogonalize_only, const muon_apply* ap = nullptr,
                      bool allow_timing = true) {
  if (p == nullptr) return MUON_E_INVALID;
  const HostPlan& H = p->host;
  muon_status st = muon::validate_config(cfg, H.dtype);
  if (st != MUON_OK) return st;
  if (H.ws_bytes == 0) return MUON_OK;  // nothing to do (all matrices empty)
  if (ws == nullptr || ws_bytes < H.ws_bytes || reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return MUON_E_WORKSPACE;
  const bool use_mom = !orthogonalize_only && cfg->momentum != 0.f;
  if (use_mom)
    for (const MatInfo& I : H.info)
      if (I.m > 0 && I.mom == nullptr) return MUON_E_INVALID;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != p->device) return MUON_E_DEVICE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  muon::StepArgs a{};
  a.mats = p->d_mats;
  a.n_mats = static_cast<int32_t>(H.info.size());
  a.ws = static_cast<char*>(ws);
  a.parts = static_cast<float*>(ws);
  a.part_exp = a.parts + H.total_partials;
  a.a = cfg->a;
  a.b = cfg->b;
  a.c = cfg->c;
  a.mu = use_mom ? cfg->momentum : 0.f;
  a.eps = cfg->eps;
  a.nesterov = cfg->nesterov;
  a.use_mom = use_mom ? 1 : 0;
  a.direct = cfg->steps == 0 ? 1 : 0;
  a.split_off = H.split_off;
  // bf16 sets with at least one step: the momentum pass also stores X0's
  // operand (scaled by a power of two), the normalise slot runs the scale
  // pass, and the first Gram and update apply the scale
  const bool fused = H.dtype == MUON_BF16 && cfg->steps > 0 && H.x0s_off >= 0;
  a.tsum_off = H.tsum_off;
  a.tmax_off = H.tmax_off;
  a.x0s_off = H.x0s_off;
  a.hint = p->d_hint;
  // the chained schedule (not under per-kernel timing, which times each
  // kernel's own launch)
  const bool chain = fused && H.chained && p->chain_ok && p->chain_on && !(p->timing == 1 && allow_timing);
  // per-kernel timing: asked for (1), or the step's own launches (2) of a
  // step that has no chained launch
  const bool per_kernel = allow_timing && (p->timing == 1 || (p->timing == 2 && !chain));
  const bool as_run = allow_timing && p->timing == 2 && chain;
  a.chain_off = chain ? H.chain_off : -1;
  if (ap) {
    a.apply = 1;
    a.lr = ap->lr;
    a.wd = ap->wd;
  }

  // Step slot `kind` (a muon_kernel_kind, or the sums of split Gram tiles,
  // which run as a second pass of the Gram kernel) -> its kernels (one, or
  // two in a row), the schedule each runs, and the kind its time is
  // reported under.
  struct Slot {
    int report, n;
    int kernel[2], sched[2];
  };
  auto slot_of = [fused](int kind) -> Slot {
    if (kind == muon::kGramReduce) return {MUON_K_GRAM, 1, {MUON_K_GRAM, 0}, {kind, 0}};
    if (fused && kind == MUON_K_MOMENTUM)
      return {MUON_K_MOMENTUM, 1, {muon::kKernelMomentumX0, 0}, {MUON_K_NORMALIZE, 0}};
    if (fused && kind == MUON_K_NORMALIZE)
      return {MUON_K_NORMALIZE, 2, {muon::kKernelX0Scale, muon::kKernelX0Rewrite},
              {muon::kX0Scale, MUON_K_NORMALIZE}};
    return {kind, 1, {kind, 0}, {kind, 0}};
  };
  // Kernel `kernel` over `count` items from `items` on stream `q`.
  auto run = [&](int kind, int kernel, const WorkItem* items, int32_t count, hipStream_t q) -> hipError_t {
    a.items = items;
    a.n_items = count;
    a.reduce = kind == muon::kGramReduce ? 1 : 0;
    const hipError_t r = muon::launch_kernel(kernel, H.dtype, a, count, q);
    a.reduce = 0;
    return r;
  };
  // The launches of step slot `kind` for group g on stream `q`.
  auto launch = [&](int kind, int g, hipStream_t q) -> muon_status {
    const Slot o = slot_of(kind);
    for (int k = 0; k < o.n; ++k) {
      const int32_t b = H.gbeg[g][o.sched[k]], e = H.gbeg[g + 1][o.sched[k]];
      if (e == b) continue;
      if (run(kind, o.kernel[k], p->d_items[o.sched[k]] + b, e - b, q) != hipSuccess) return MUON_E_LAUNCH;
    }
    return MUON_OK;
  };
  // fn() (launches on the caller's stream), bracketed by HIP events whose
  // interval is reported under `report` when `on`.
  auto bracket = [&](bool on, int report, auto&& fn) -> muon_status {
    if (!on) return fn() == hipSuccess ? MUON_OK : MUON_E_LAUNCH;
    TimedLaunch t{report, get_event(p), get_event(p)};
    auto give_back = [&]() {
      if (t.start) p->free_events.push_back(t.start);
      if (t.stop) p->free_events.push_back(t.stop);
      return MUON_E_LAUNCH;
    };
    if (!t.start || !t.stop || hipEventRecord(t.start, s) != hipSuccess) return give_back();
    if (fn() != hipSuccess || hipEventRecord(t.stop, s) != hipSuccess) return give_back();
    p->pending.push_back(t);
    return MUON_OK;
  };
  // Step slot `kind` over the whole set (the one-group schedules) on the
  // caller's stream.
  auto whole_slot = [&](int kind) -> hipError_t {
    const Slot o = slot_of(kind);
    hipError_t r = hipSuccess;
    for (int k = 0; k < o.n && r == hipSuccess; ++k) {
      const auto& w = H.whole[o.sched[k]].items;
      if (!w.empty()) r = run(kind, o.kernel[k], p->d_whole[o.sched[k]], static_cast<int32_t>(w.size()), s);
    }
    return r;
  };
  // Per-kernel timing: step slot `kind` over the whole set, bracketed by
  // HIP events.
  auto timed = [&](int kind) -> muon_status {
    const Slot o = slot_of(kind);
    if (H.whole[o.sched[0]].items.empty()) return MUON_OK;
    return bracket(true, o.report, [&]() { return whole_slot(kind); });
  };
  // The whole sequence of one group on stream q: momentum, normalise (or
  // the scale pass), k x (gram, poly, update).
  auto sequence = [&](int g, hipStream_t q) -> muon_status {
    muon_status r;
    if ((r = launch(MUON_K_MOMENTUM, g, q)) != MUON_OK) return r;
    if ((r = launch(MUON_K_NORMALIZE, g, q)) != MUON_OK) return r;
    for (int t = 0; t < cfg->steps; ++t) {
      a.cur = t & 1;
      a.last = t == cfg->steps - 1 ? 1 : 0;
      a.x0_scaled = fused && t == 0 ? 1 : 0;
      for (int kind : {int(MUON_K_GRAM), muon::kGramReduce, int(MUON_K_POLY), int(MUON_K_UPDATE)})
        if ((r = launch(kind, g, q)) != MUON_OK) return r;
    }
    return MUON_OK;
  };

  if (per_kernel) {
    muon_status r;
    if ((r = timed(MUON_K_MOMENTUM)) != MUON_OK) return r;
    if ((r = timed(MUON_K_NORMALIZE)) != MUON_OK) return r;
    for (int t = 0; t < cfg->steps; ++t) {
      a.cur = t & 1;
      a.last = t == cfg->steps - 1 ? 1 : 0;
      a.x0_scaled = fused && t == 0 ? 1 : 0;
      for (int kind : {int(MUON_K_GRAM), muon::kGramReduce, int(MUON_K_POLY), int(MUON_K_UPDATE)})
        if ((r = timed(kind)) != MUON_OK) return r;
    }
    return MUON_OK;
  }
  if (chain) {
    // momentum, the scale pass (which clears the chain's counters) and the
    // rewrite over the whole set (the one-group schedules), then every Gram,
    // poly and update tile of all steps in one persistent launch of one
    // workgroup per CU (timing 2: each of the three slots bracketed)
    muon_status r;
    for (int kind : {int(MUON_K_MOMENTUM), int(MUON_K_NORMALIZE)})
      if ((r = bracket(as_run, kind, [&]() { return whole_slot(kind); })) != MUON_OK) return r;
    muon::ChainArgs c{};
    c.items = p->d_chain;
    c.steps = cfg->steps;
    c.err = p->d_err;
    c.wait_ticks = static_cast<uint64_t>(p->chain_wait_us) * 100u;
    for (int x = 0; x <= muon::kNumXcd; ++x) c.beg[x] = H.chain_beg[x];
    a.cur = 0;
    a.last = 0;
    a.x0_scaled = 1;
    return bracket(as_run, MUON_K_COUNT, [&]() { return muon::launch_chain(a, c, muon::kNumCu, s); });
  }
  if (H.ngroups == 1) return sequence(0, s);
  // several groups, no timing: each group runs its whole sequence on its
  // own stream, forked once and joined once. Every group that was forked is
  // joined back to the caller's stream, also when a launch fails part way,
  // so no work of this call outlives the stream order the caller sees (if a
  // join itself cannot be enqueued, the host waits for that group).
  if (hipEventRecord(p->fork_ev, s) != hipSuccess) return MUON_E_LAUNCH;
  muon_status res = MUON_OK;
  int forked = 0;
  for (int g = 0; g < H.ngroups && res == MUON_OK; ++g) {
    if (hipStreamWaitEvent(p->gstream[g], p->fork_ev, 0) != hipSuccess) {
      res = MUON_E_LAUNCH;
      break;
    }
    forked = g + 1;
    res = sequence(g, p->gstream[g]);
  }
  for (int g = 0; g < forked; ++g) {
    if (hipEventRecord(p->join_ev[g], p->gstream[g]) != hipSuccess ||
        hipStreamWaitEvent(s, p->join_ev[g], 0) != hipSuccess) {
      (void)hipStreamSynchronize(p->gstream[g]);
      if (res == MUON_OK) res = MUON_E_LAUNCH;
    }
  }
  return res;
}

// ---- plan cache for muon_step / muon_orthogonalize

struct CacheEntry {
  std::string key;
  muon_plan_s* plan;
};
std::mutex g_cache_mu;
std::list<CacheEntry> g_cache;  // front = most recently used
constexpr size_t kCacheMax = 16;

std::string make_key(const muon_matrix* mats, int32_t n, muon_dtype dt) {
  std::string k(reinterpret_cast<const char*>(&dt), sizeof(dt));
  int dev = -1;
  (void)hipGetDevice(&dev);
  k.append(reinterpret_cast<const char*>(&dev), sizeof(dev));
  if (n > 0) k.append(reinterpret_cast<const char*>(mats), sizeof(muon_matrix) * size_t(n));
  return k;
}

muon_status cached_step(const muon_matrix* mats, int32_t n, muon_dtype dt, const muon_config* cfg,
                        void* ws, size_t ws_bytes, void* stream, bool ortho) {
  muon_status st = muon::validate_config(cfg, dt);
  if (st != MUON_OK) return st;
  st = muon::validate_matrices(mats, n, dt, !ortho && cfg->momentum != 0.f);
  if (st != MUON_OK) return st;
  std::lock_guard<std::mutex> lock(g_cache_mu);
  const std::string key = make_key(mats, n, dt);
  for (auto it = g_cache.begin(); it != g_cache.end(); ++it) {
    if (it->key == key) {
      g_cache.splice(g_cache.begin(), g_cache, it);
      return step_impl(it->plan, cfg, ws, ws_bytes, stream, ortho);
    }
  }
  muon_plan_s* p = new (std::nothrow) muon_plan_s();
  if (!p) return MUON_E_ALLOC;
  st = muon::build_plan(mats, n, dt, &p->host);
  if (st != MUON_OK) {
    delete p;
    return st;
  }
  // check the workspace before allocating anything
  if (p->host.ws_bytes > 0 &&
      (ws == nullptr || ws_bytes < p->host.ws_bytes || reinterpret_cast<uintptr_t>(ws) % 256 != 0)) {
    delete p;
    return MUON_E_WORKSPACE;
  }
  if ((st = upload(p)) != MUON_OK) {
    release(p);  // also frees the streams and events of a partial upload
    return st;
  }
  g_cache.push_front({key, p});
  if (g_cache.size() > kCacheMax) {
    release(g_cache.back().plan);
    g_cache.pop_back();
  }
  return step_impl(p, cfg, ws, ws_bytes, stream, ortho);
}

}  // namespace

extern "C" {

int32_t muon_abi_version(void) { return MUON_ABI_VERSION; }

const char* muon_status_str(int32_t s) {
  switch (s) {
    case MUON_OK: return "ok";
    case MUON_E_INVALID: return "invalid argument";
    case MUON_E_DTYPE: return "unsupported dtype";
    case MUON_E_SHAPE: return "invalid shape";
    case MUON_E_ALIGN: return "misaligned pointer";
    case MUON_E_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case MUON_E_DEVICE: return "no usable gfx950 device or HIP runtime error";
    case MUON_E_LAUNCH: return "kernel launch failed";
    case MUON_E_ALLOC: return "allocation failed";
    case MUON_E_SCRATCH: return "set needs more workspace than the fixed scratch array holds";
    default: return "unknown status";
  }
}

muon_status muon_workspace_bytes(const muon_matrix* mats, int32_t n, muon_dtype dtype,
                                 size_t* bytes) {
  if (bytes == nullptr) return MUON_E_INVALID;
  HostPlan P;
  muon_status st = muon::build_plan(mats, n, dtype, &P);
  if (st != MUON_OK) return st;
  *bytes = P.ws_bytes;
  return MUON_OK;
}

muon_status muon_plan_create(const muon_matrix* mats, int32_t n, muon_dtype dtype,
                             muon_plan** plan) {
  if (plan == nullptr) return MUON_E_INVALID;
  *plan = nullptr;
  muon_plan_s* p = new (std::nothrow) muon_plan_s();
  if (!p) return MUON_E_ALLOC;
  muon_status st = muon::build_plan(mats, n, dtype, &p->host);
  if (st != MUON_OK) {
    delete p;
    return st;
  }
  if ((st = upload(p)) != MUON_OK) {
    release(p);  // also frees the streams and events of a partial upload
    return st;
  }
  *plan = p;
  return MUON_OK;
}

muon_status muon_plan_step(muon_plan* plan, const muon_config* cfg, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return step_impl(plan, cfg, workspace, workspace_bytes, stream, false);
}

muon_status muon_plan_step_noalloc(muon_plan* plan, const muon_config* cfg, void* stream) {
  if (plan == nullptr) return MUON_E_INVALID;
  if (plan->host.ws_bytes > muon::kScratchBytes) return MUON_E_SCRATCH;
  if (plan->host.ws_bytes > 0 && plan->scratch == nullptr) return MUON_E_DEVICE;
  return step_impl(plan, cfg, plan->scratch, muon::kScratchBytes, stream, false, nullptr, false);
}

muon_status muon_plan_set_weights(muon_plan* plan, const muon_weight* w, int32_t n) {
  if (plan == nullptr) return MUON_E_INVALID;
  muon_status st = muon::validate_weights(plan->host, w, n);
  if (st != MUON_OK) return st;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != plan->device) return MUON_E_DEVICE;
  std::vector<MatInfo> info = plan->host.info;
  const size_t es = muon::elem_size(plan->host.dtype);
  for (int32_t i = 0; i < n; ++i) {
    MatInfo& I = info[i];
    if (I.m == 0) continue;
    I.w = w[i].weight;
    I.wld = w[i].ld;
    I.lr_mul = w[i].lr_mul;
    I.wd_mul = w[i].wd_mul;
    I.w_vec_ok = reinterpret_cast<uintptr_t>(w[i].weight) % 16 == 0 && (w[i].ld * es) % 16 == 0 &&
                 (static_cast<size_t>(plan->host.mats[i].cols) * es) % 16 == 0;
  }
  // the table is read by the plan's kernels: let earlier work finish first
  if (hipDeviceSynchronize() != hipSuccess) return MUON_E_DEVICE;
  if (!info.empty() && hipMemcpy(plan->dmem, info.data(), sizeof(MatInfo) * info.size(),
                                 hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipGetLastError();
    return MUON_E_DEVICE;
  }
  plan->host.info = info;
  plan->has_weights = true;
  return MUON_OK;
}

muon_status muon_plan_step_apply(muon_plan* plan, const muon_config* cfg, const muon_apply* ap,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (plan == nullptr) return MUON_E_INVALID;
  muon_status st = muon::validate_apply(ap);
  if (st != MUON_OK) return st;
  if (!plan->has_weights) return MUON_E_INVALID;
  return step_impl(plan, cfg, workspace, workspace_bytes, stream, false, ap);
}

void muon_plan_destroy(muon_plan* plan) { release(plan); }

muon_status muon_step(const muon_matrix* mats, int32_t n, muon_dtype dtype, const muon_config* cfg,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return cached_step(mats, n, dtype, cfg, workspace, workspace_bytes, stream, false);
}

muon_status muon_orthogonalize(const muon_matrix* mats, int32_t n, muon_dtype dtype,
                               const muon_config* cfg, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return cached_step(mats, n, dtype, cfg, workspace, workspace_bytes, stream, true);
}

muon_status muon_schedule_query(const muon_matrix* mats, int32_t n, muon_dtype dtype, int32_t kind,
                                int32_t* items, int64_t cap, int64_t* count) {
  if (count == nullptr || kind < 0 || kind > MUON_K_COUNT + 2 || cap < 0 ||
      (cap > 0 && items == nullptr))
    return MUON_E_INVALID;
  HostPlan P;
  muon_status st = muon::build_plan(mats, n, dtype, &P);
  if (st != MUON_OK) return st;
  if (kind == MUON_K_COUNT + 2) {  // the chained schedule's lists, XCD by XCD
    *count = static_cast<int64_t>(P.chain.size());
    const int64_t w = std::min<int64_t>(cap, *count);
    int x = 0;
    for (int64_t i = 0; i < w; ++i) {
      while (i >= P.chain_beg[x + 1]) ++x;
      const muon::ChainItem& c = P.chain[i];
      items[4 * i + 0] = c.mat;
      items[4 * i + 1] = (int32_t(c.ti) << 16) | int32_t(c.tj);
      items[4 * i + 2] = (x << 8) | (c.kind_n & 255);
      items[4 * i + 3] = c.need;
    }
    return MUON_OK;
  }
  const auto& v = P.sched[kind].items;
  *count = static_cast<int64_t>(v.size());
  const int64_t w = std::min<int64_t>(cap, *count);
  for (int64_t i = 0; i < w; ++i) {
    items[4 * i + 0] = v[i].mat;
    items[4 * i + 1] = v[i].a;
    items[4 * i + 2] = v[i].b;
    items[4 * i + 3] = v[i].c;
  }
  return MUON_OK;
}

muon_status muon_plan_set_timing(muon_plan* plan, int32_t enable) {
  if (plan == nullptr || enable < 0 || enable > 2) return MUON_E_INVALID;
  plan->timing = enable;
  return MUON_OK;
}

namespace {
// Waits for the recorded events and adds their intervals to the plan's sums.
muon_status drain_events(muon_plan* plan) {
  for (auto& t : plan->pending) {
    if (hipEventSynchronize(t.stop) != hipSuccess) return MUON_E_DEVICE;
    float e = 0.f;
    if (hipEventElapsedTime(&e, t.start, t.stop) != hipSuccess) return MUON_E_DEVICE;
    plan->acc_ms[t.kind] += e;
    plan->acc_n[t.kind] += 1;
    plan->free_events.push_back(t.start);
    plan->free_events.push_back(t.stop);
  }
  plan->pending.clear();
  return MUON_OK;
}
}  // namespace

muon_status muon_plan_chain_times(muon_plan* plan, double* ms, int64_t* launches) {
  if (plan == nullptr || ms == nullptr || launches == nullptr) return MUON_E_INVALID;
  muon_status st = drain_events(plan);
  if (st != MUON_OK) return st;
  *ms = plan->acc_ms[MUON_K_COUNT];
  *launches = plan->acc_n[MUON_K_COUNT];
  plan->acc_ms[MUON_K_COUNT] = 0.0;
  plan->acc_n[MUON_K_COUNT] = 0;
  return MUON_OK;
}

muon_status muon_plan_kernel_times(muon_plan* plan, double* ms, int64_t* launches) {
  if (plan == nullptr || ms == nullptr || launches == nullptr) return MUON_E_INVALID;
  muon_status st = drain_events(plan);
  if (st != MUON_OK) return st;
  for (int k = 0; k < MUON_K_COUNT; ++k) {
    ms[k] = plan->acc_ms[k];
    launches[k] = plan->acc_n[k];
    plan->acc_ms[k] = 0.0;
    plan->acc_n[k] = 0;
  }
  return MUON_OK;
}

muon_status muon_plan_set_chained(muon_plan* plan, int32_t enable) {
  if (plan == nullptr) return MUON_E_INVALID;
  plan->chain_on = enable != 0;
  return MUON_OK;
}

muon_status muon_plan_set_chain_timeout(muon_plan* plan, int64_t microseconds) {
  if (plan == nullptr || microseconds < 0 || microseconds > int64_t(3600) * 1000000) return MUON_E_INVALID;
  plan->chain_wait_us = microseconds;
  return MUON_OK;
}

muon_status muon_plan_chain_state(muon_plan* plan, int32_t* chained, int32_t* error) {
  if (plan == nullptr || chained == nullptr || error == nullptr) return MUON_E_INVALID;
  *chained = plan->host.chained && plan->chain_ok && plan->chain_on ? 1 : 0;
  *error = 0;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != plan->device) return MUON_E_DEVICE;
  if (hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(error, plan->d_err, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemset(plan->d_err, 0, sizeof(int32_t)) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess) {
    (void)hipGetLastError();
    return MUON_E_DEVICE;
  }
  return MUON_OK;
}

muon_status muon_plan_buffer_info(const muon_plan* plan, int32_t idx, muon_buffer_info* info) {
  if (plan == nullptr || info == nullptr) return MUON_E_INVALID;
  if (idx < 0 || idx >= static_cast<int32_t>(plan->host.info.size())) return MUON_E_INVALID;
  const MatInfo& I = plan->host.info[idx];
  info->m = I.m;
  info->n = I.n;
  info->mp = I.mp;
  info->np = I.np;
  info->x_lo = I.xl_off;
  info->x_op0 = I.xo_off[0];
  info->x_op1 = I.xo_off[1];
  info->gram = I.a_off;
  info->poly = I.b_off;
  info->x0_scale = I.m > 0 && plan->host.x0s_off >= 0 ? plan->host.x0s_off + 16 * int64_t(idx) : -1;
  return MUON_OK;
}

}  // extern "C"
