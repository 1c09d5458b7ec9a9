/*
 * muon_adam.h -- C ABI of the Adam branch of the same optimizer step, for the
 * parameters that do not take the Muon path (embeddings, biases, norm scales,
 * gates), as one fused elementwise kernel over a whole parameter list.
 *
 * Source: mhpq.cn, modded-nanogpt track_1_short technical guide, section 6.2
 * (training hyper-parameters): parameter groups that are not projection
 * matrices run Adam with betas (0.9, 0.99), each group with its own lr_mul,
 * and wd_mul = 0 for biases and scales, while the projection matrices take
 * the Muon path. The pages do not write the Adam update out; the reading
 * taken is textbook Adam with bias correction and decoupled weight decay, the
 * multipliers scaling the rate and the decay wherever they appear:
 *
 *   lr' = lr * lr_mul,  wd' = wd * wd_mul,  t = step (1, 2, ...)
 *   m  = beta1 * m + (1 - beta1) * g
 *   v  = beta2 * v + (1 - beta2) * g^2
 *   p  = p * (1 - lr' * wd') - lr' * (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
 *
 * Arithmetic is fp32; m and v are stored fp32; p is stored at the set's
 * dtype (round to nearest even). Conventions are those of muon.h: pointers
 * are device memory owned by the caller, arguments are validated before any
 * work is enqueued, work is asynchronous on `stream`, results are
 * deterministic, NaN/Inf propagate.
 */
#ifndef MUON_ADAM_H
#define MUON_ADAM_H

#include <stddef.h>
#include <stdint.h>

#include "muon.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Largest tensor (elements) and list length accepted. */
#define MUON_ADAM_MAX_NUMEL 2147483648LL /* 2^31 */
#define MUON_ADAM_MAX_TENSORS 1048576

/* One parameter tensor, flattened: numel contiguous elements. numel == 0 is
 * skipped (its pointers are ignored). param and grad are of the set's dtype
 * and aligned to its size; exp_avg / exp_avg_sq are fp32, 4-byte aligned.
 * 16-byte alignment of all four selects the vector path. param, exp_avg and
 * exp_avg_sq are read and written; grad is read; no buffer may overlap
 * another one of the list (grad with grad excepted). */
typedef struct {
  int64_t numel;
  void* param;
  const void* grad;
  float* exp_avg;
  float* exp_avg_sq;
  float lr_mul;
  float wd_mul;
} muon_adam_tensor;

/* Per-call scalars: all finite; 0 <= beta1, beta2 < 1; eps >= 0; step >= 1
 * (the 1-based count of updates including this one, for the bias
 * corrections). */
typedef struct {
  float lr;
  float beta1;
  float beta2;
  float eps;
  float wd;
  int32_t step;
} muon_adam_config;

typedef struct muon_adam_plan_s muon_adam_plan;

/* Validates the list, splits it into work items of at most 16384 elements
 * and uploads the tensor table and the schedule to the current device (a few
 * KB to MB owned by the plan; *plan receives NULL on error). */
muon_status muon_adam_plan_create(const muon_adam_tensor* ts, int32_t n, muon_dtype dtype,
                                  muon_adam_plan** plan);

/* Enqueues one Adam update of every tensor of the plan on `stream` (one
 * kernel launch). */
muon_status muon_adam_plan_step(muon_adam_plan* plan, const muon_adam_config* cfg, void* stream);

/* Frees a plan after waiting for the device (NULL is a no-op). */
void muon_adam_plan_destroy(muon_adam_plan* plan);

/* Host-only: the number of work items (kernel blocks) a list needs. */
muon_status muon_adam_work_items(const muon_adam_tensor* ts, int32_t n, muon_dtype dtype,
                                 int64_t* items);

#ifdef __cplusplus
}
#endif

#endif /* MUON_ADAM_H */
