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
};

// precision: muon_precision (operand format of bf16 sets).
hipError_t launch_kernel(int kind, muon_dtype dt, int precision, const StepArgs& a, int grid,
                         hipStream_t s);

}  // namespace muon
