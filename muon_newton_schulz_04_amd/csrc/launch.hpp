// Kernel arguments and the launcher shared by the C-ABI layer and kernels.
#pragma once

#include <hip/hip_runtime_api.h>

#include "plan.hpp"

namespace muon {

// Everything a kernel of one step needs (passed by value as kernel args).
struct StepArgs {
  const MatInfo* mats;     // device table, one record per matrix
  const WorkItem* items;   // device schedule of this launch
  char* ws;                // workspace base
  float* parts;            // sum-of-squares partials (workspace head)
  float* part_exp;         // their exponents: a partial s with exponent e stands for s 4^e
  float a, b, c, mu, eps;
  int32_t nesterov;
  int32_t use_mom;  // momentum state present and mu != 0
  int32_t cur;      // which operand buffer holds the current X
  int32_t last;     // last Newton-Schulz step: write `out`
  int32_t direct;   // zero steps: the normalise kernel writes `out`
  int32_t apply;    // write W <- W (1 - lr' wd') - lr' X instead of `out` (lr' = lr lr_mul, wd' = wd wd_mul)
  float lr, wd;
  int32_t reduce;   // Gram: sum split partial tiles and store A (second pass)
  int64_t split_off;  // workspace offset of the split Gram partials (-1: none)
  // bf16 sets with at least one step: X0 = sigma * (its fp16 operand),
  // which holds u scaled by a power of two p; the first Gram scales its sums
  // by sigma^2 and the first update by sigma (x0_scaled).
  int32_t x0_scaled;
  int64_t tsum_off, tmax_off, x0s_off;  // workspace offsets (see HostPlan)
  float* hint;  // plan memory, per matrix: the largest |u| of the last call (0: none)
  int32_t n_items;  // items of the schedule (kernels whose grid is smaller)
  int32_t n_mats;   // matrices of the set (the rewrite checks every matrix's flag first)
  // chained schedule: workspace offset of its counters (the scale pass
  // clears them), -1 without one
  int64_t chain_off;
};

// The chained launch (plan.hpp): the lists, their bounds per XCD, the
// number of steps, the plan word that records a wait past its bound, and
// that bound.
struct ChainArgs {
  const ChainItem* items;
  int32_t beg[kNumXcd + 1];
  int32_t steps;
  int32_t* err;
  uint64_t wait_ticks;  // bound of one wait, in 100 MHz real-time counter ticks
};

hipError_t launch_kernel(int kind, muon_dtype dt, const StepArgs& a, int grid, hipStream_t s);
// All Gram, poly and update tiles of every step in one launch of `grid`
// workgroups (bf16 sets).
hipError_t launch_chain(const StepArgs& a, const ChainArgs& c, int grid, hipStream_t s);

// Device address of the current device's fixed scratch array (kScratchBytes,
// 256-byte aligned), looked up on the first call per device and kept.
hipError_t scratch_address(void** out);

}  // namespace muon
