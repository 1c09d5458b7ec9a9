// Host-side planning for the Muon update: argument validation, per-matrix
// workspace layout and the XCD-aware work schedules of every kernel.
// Plain C++ (no HIP headers) so the same code runs in CPU-only tests.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "../../include/muon.h"

namespace muon {

// Tile sizes shared by the planner and the kernels.
constexpr int kGemmTile = 128;         // output tile of the matrix-core kernels (fp32 sets)
constexpr int kTileM16 = 256;          // 16-bit-operand engine (bf16 sets): 256 x 256 tiles
constexpr int kTileN16 = 256;
constexpr int kNormTile = 64;          // tile of the normalise / layout kernel
constexpr int kMomentumElems = 16384;  // target elements per momentum work item
constexpr int kNumXcd = 8;             // accelerator complex dies of an MI355X
constexpr int kNumCu = 256;            // compute units of an MI355X
constexpr size_t kWsAlign = 256;
// Size of the fixed device scratch array of muon_plan_step_noalloc.
constexpr size_t kScratchBytes = size_t(MUON_SCRATCH_BYTES);
// Internal schedules after the public kernel kinds: the sums of split Gram
// tiles (bf16 sets), launched as a second Gram pass, and the scale pass of
// X0 (bf16 sets with at least one step: one item per matrix).
constexpr int kGramReduce = MUON_K_COUNT;
constexpr int kX0Scale = MUON_K_COUNT + 1;
constexpr int kKinds = MUON_K_COUNT + 2;
// Kernels beyond the public kinds (launch_kernel): bf16 sets with at least
// one step run the momentum step and X0's operand in one pass over the
// normalise tiles, then the scale pass (normalisation scale and power of
// two per matrix) and the operand rewrite of the matrices whose power of
// two the momentum pass guessed wrong (over the normalise tiles with a grid
// of at most kX0RewriteGrid).
constexpr int kKernelMomentumX0 = 16;
constexpr int kKernelX0Scale = 17;
constexpr int kKernelX0Rewrite = 18;
constexpr int kX0RewriteGrid = 2048;
// Split Gram tiles: k ranges of at least 8 stages of 32; each partial is a
// 256 x TN fp32 tile in the workspace.
constexpr int32_t kSplitMaxParts = 32767;
constexpr int32_t kSplitMinStages = 24;

// Per-matrix record read by the kernels (device table; plain data).
struct MatInfo {
  const void* grad;
  void* mom;
  void* out;
  int64_t ld;        // caller row stride (elements)
  int32_t rows, cols;
  int32_t m, n;      // m = min(rows, cols), n = max(rows, cols)
  int32_t mp, np;    // m, n padded to the engine's tile multiples
  int32_t tall;      // rows > cols: the iteration runs on the transpose
  int32_t vec_ok;    // 16-byte vector access legal for grad/mom/out
  int64_t xl_off;    // bf16 sets: low part of X, one OCP e4m3 byte per
                     // element holding (X - hi) 2^18, -1 otherwise
  int64_t xo_off[2]; // bf16 sets: ping-pong high parts (the matrix-core
                     // operand); fp32 sets: ping-pong fp32 X
  int64_t a_off;     // A = X X^T
  int64_t b_off;     // B = b A + c A A
  int32_t part_off;  // first slot of this matrix's sum-of-squares partials
  int32_t part_cnt;
  int32_t tile_off;  // bf16 sets: first slot of this matrix's per-tile sums
  int32_t tile_cnt;  // and maxima (64 x 64 tiles of mp x np, row-major)
  // Weight application (muon_plan_step_apply): W in the caller's dtype and
  // orientation, row-major with leading dimension wld; lr and wd multipliers.
  void* w;
  int64_t wld;
  float lr_mul, wd_mul;
  int32_t w_vec_ok;  // 16-byte vector access legal for W
  int32_t pad_;
};

// Gram items of bf16 sets: c = 0, or for a tile whose k range is split into
// S parts, c = pbase << 16 | s << 8 | S (part s of S, stored in partial
// slot pbase + s); reduce items: c = pbase << 16 | q << 8 | S for quarter q
// (rows 128 (q >> 1), columns 128 (q & 1) of the tile).
struct WorkItem {
  int32_t mat, a, b, c;
};

struct Schedule {
  std::vector<WorkItem> items;  // launch order; block i runs items[i]; mat < 0 = empty
};

// Sets whose update launch is a few waves of tiles deep are split into
// groups of matrices that run concurrently on streams of their own, so one
// group's kernels fill the CUs that another group's tail (the last, partial
// wave of tiles) and launch gaps leave idle: three groups below 8 waves of
// 256 tiles, two below 24, one beyond (build_plan).
constexpr int kMaxGroups = 3;
constexpr int kGroupMinTiles = 512;  // matrix-core tiles per update launch to split

struct HostPlan {
  muon_dtype dtype = MUON_BF16;
  std::vector<muon_matrix> mats;
  std::vector<MatInfo> info;
  // Schedules of all groups, concatenated: group g's items of kernel k are
  // sched[k].items[gbeg[g][k] .. gbeg[g + 1][k]) (each a multiple of 8).
  Schedule sched[kKinds];
  int32_t ngroups = 1;
  int32_t gbeg[kMaxGroups + 1][kKinds] = {};
  // The same work as one group (per-kernel timing runs each kernel over the
  // whole set in one launch).
  Schedule whole[kKinds];
  int32_t total_partials = 0;
  // bf16 sets: per normalise tile, the sum of u^2 and the largest |u|
  // (momentum pass), and per matrix four floats {sigma, p, p of the
  // momentum pass, 0} (scale pass): X0 = sigma * (fp16 operand).
  int32_t total_tiles = 0;
  int64_t tsum_off = -1, tmax_off = -1, x0s_off = -1;
  // Split Gram tiles (small bf16 sets whose longest Gram tiles would set
  // the launch time): partial tiles in the workspace at split_off.
  int32_t split_parts = 0;
  int64_t split_off = -1;
  size_t ws_bytes = 0;
};

// Validates the matrix set (shapes, dtype, alignment, overlaps).
muon_status validate_matrices(const muon_matrix* mats, int32_t n, muon_dtype dtype,
                              bool need_momentum);
// Validates per-call scalars for a set of `dtype`.
muon_status validate_config(const muon_config* cfg, muon_dtype dtype);
// Validates the weights of a plan's matrices (one record per matrix; empty
// matrices' records are ignored) against the set's buffers.
muon_status validate_weights(const HostPlan& plan, const muon_weight* w, int32_t n);
// Validates the scalars of a weight application.
muon_status validate_apply(const muon_apply* ap);
// Builds the full host plan (no device calls). need_momentum: momentum
// pointers are part of the set (false for orthogonalisation-only plans).
muon_status build_plan(const muon_matrix* mats, int32_t n, muon_dtype dtype, HostPlan* out);

size_t elem_size(muon_dtype dt);

}  // namespace muon
