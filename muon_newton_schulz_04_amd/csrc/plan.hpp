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
  int32_t chain_n;   // chained schedule: Gram + poly + update items per step
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

// Chained schedule (bf16 sets with at least one step): one launch runs the
// Gram, poly and update tiles of every Newton-Schulz step. All items of a
// matrix go to one XCD, whose L2 then holds everything the matrix's tiles
// pass to each other. Each XCD has a list, ordered by a list-scheduling
// simulation of its CUs (every item after the items it depends on); the
// workgroups running on an XCD take tickets from its list in order, ticket
// t meaning item t % len of step t / len. An item waits until its matrix has
// completed step * chain_n + need items: the Gram tiles of step s wait for
// the updates of step s - 1, poly for Gram, the update for poly. Waits only
// reach back to lower tickets, taken by running workgroups, so the launch
// always progresses.
struct ChainItem {
  int32_t mat;
  int16_t ti, tj;  // tile row and column
  int32_t need;    // items of the matrix's own step to wait for
  int32_t kind_n;  // MUON_K_GRAM, MUON_K_POLY or MUON_K_UPDATE | the matrix's chain_n << 8
};
constexpr int kChainCus = kNumCu / kNumXcd;  // CUs per XCD
// Chained only when the matrices spread over the XCDs with the heaviest
// XCD at most this much above the mean, and when the update launch is less
// than kChainMaxWaves waves of tiles deep: there the separate launches lose
// their tails and launch gaps (measured: GPT-2-124M, 5 waves, 3.5 % faster
// chained; GPT-2-350M, 18 waves, 2 %), while deeper launches have little
// tail and run faster separately (2048 x 8192 set, 64 waves: 5 % slower
// chained, the tiles of an XCD then share less of its L2).
constexpr double kChainMaxImbalance = 1.10;
constexpr int kChainMaxWaves = 24;

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
  // Chained schedule: per-XCD lists, chain[chain_beg[x] .. chain_beg[x + 1]);
  // workspace at chain_off: one ticket counter per XCD, then one completion
  // counter per matrix (int32 each, cleared by the scale pass of each call).
  bool chained = false;
  std::vector<ChainItem> chain;
  int32_t chain_beg[kNumXcd + 1] = {};
  int64_t chain_off = -1;
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
