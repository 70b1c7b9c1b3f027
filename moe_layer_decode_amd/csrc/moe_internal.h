// Internal interface between the C ABI (host orchestration) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_decode.h"

namespace moe {

constexpr int kWaves = 4;            // waves per block of every kernel
constexpr int kThreads = 64 * kWaves;
constexpr int kRouteChunk = 512;     // d elements one router wave covers (64 lanes x 8)
constexpr int kTokInline = 4;        // tokens carried inline in a work descriptor
constexpr int kWideRows = 64;        // rows / columns of a bf16 large-group tile (unless split K)
constexpr int kSplitKMaxT = 32;      // K-split gate/up tiles: T at most (two 16-row token tiles)
constexpr int kSplitKDownMaxT = 16;  // K-split down tiles: T at most (one token tile)
constexpr int kDownRowCols = 128;    // down row tiles (T > kSplitKDownMaxT): output columns per block
constexpr int kSplitKCols = 32;      // K-split down tiles: output columns per block,
constexpr int kSplitKDownMinD = 2048;  //   d above it
constexpr int kSplitKMinK = 256;     //   and intermediate width at least (a full K tile per wave)
constexpr int kSplitKMaxGroups = 16; // d > 2048, T > 8: K-split only if a launch holds at most this
                                     //   many large groups
constexpr int kPlanThreads = 1024;   // threads of the single-block top-k / plan kernel
// Top-k + plan in one block (a wave per token, at most 256 experts), or the
// per-token selections across the chip followed by a one-block plan launch.
inline bool topk_in_one_block(int T, int E) {
  return T <= kPlanThreads / 64 && (E + 63) / 64 <= 4;
}
constexpr int kMaxRouteSplit = 8;   // partial-logit planes of the bf16 router at most
constexpr int kMaxParts = 6;         // 3 matrix families x (small groups, large groups)
// Plan header entries beyond the public ones: lengths of the compacted work
// lists of small (<= kTokInline rows) and large groups.
constexpr int kHdrSmall = 8, kHdrLarge = 9, kHdrDeptSmall = 10, kHdrDeptLarge = 11;

// One active matrix of a family and its row group, written by the dispatch
// phase so an expert block starts from a single 32-byte read.
struct WorkDesc {
  int mat;                 // expert or department index
  int r0;                  // first row of its group in the plan's row order
  int n;                   // rows (tokens) in the group
  int tok[kTokInline];     // the first tokens of the group
  int pad;
};

// Everything the routing + dispatch phase reads and writes.
struct PlanArgs {
  int T, E, k, m;
  int factorised;          // 1: also write plan.row_pair and pair-indexed inline rows
  moe_plan plan;
  WorkDesc* work;          // [2E] active experts: small groups from 0, large groups from E
  WorkDesc* dwork;         // [2m] the same for departments
  moe_step_stats* stats;   // device stats of the step, or nullptr
  // weight bytes one step streams: fixed (router, shared expert) plus per
  // active expert and per active department (the host's byte count)
  unsigned long long bytes_fixed, bytes_expert, bytes_dept;
};

struct RouteArgs {
  const void* x;           // [T][d]
  const void* wr;          // [E][d]
  const float* bias;       // [E] or nullptr
  int T, d, E, k;
  int score_fn, renorm;
  float scale;
  int m, k_dept;           // department-limited top-k when 0 < k_dept < m (or strict)
  int strict;              // 1: exactly k_dept departments per token
  int n_chunks;            // ceil(d / kRouteChunk)
  int ksplit;              // partial-logit planes: logits holds [ksplit][T][E], summed in order
  float* logits;           // [ksplit][T][E]
  int32_t* ids_out;        // [T][k] or nullptr
  float* w_out;            // [T][k] or nullptr
  float* sel_out;          // [T][E] or nullptr
};

// One part of a family of same-shape matrices (routed experts -- private
// slices in the department form --, department slices, or the shared
// expert): the slots whose group has at most kTokInline rows (small part,
// register GEMV) or more (large part, matrix-core tiles).
struct Family {
  const void* gate;        // [n_mats][rows][d]
  const void* up;          // [n_mats][rows][d]
  const void* down;        // [n_mats][d][rows]
  int rows;
  const WorkDesc* work;    // per active slot; nullptr: the shared expert (all T tokens)
  const int* n_active;     // device count of active slots (nullptr: 1)
  const int* grp_token;    // token of each row (nullptr: row r is token r)
  void* h;                 // [rows_total][rows] gate/up output in the layer's dtype (see epi)
  void* h2;                // [rows_total][rows] second gate/up output (epi 1), else nullptr
  float* out;              // [rows_total][d]    unweighted down output
  const void* x_gate;      // gate/up inputs [in_rows][d]; nullptr: the launch's x for both
  const void* x_up;        //   (the factorised form's private transforms read two matrices)
  int in_rows;             // rows the gate/up inputs hold (row indices are clamped to it)
  int epi;                 // gate/up: 0 h = SiLU(g)*u, 1 h = SiLU(g) and h2 = SiLU(u);
                           // down: 0 out = W h, 1 out = SiLU(W h)
  int max_slots;           // host bound on the slots this part can serve
  int tiles;               // blocks per slot in the current launch
  int n_mats;              // matrices in the family (bounds check of work descriptors)
  int max_rows;            // rows h / out hold (bounds check of work descriptors)
  int large;               // 0: groups of <= kTokInline rows; 1: larger groups
  int routed;              // 1: the routed experts (many groups of a few rows each)
  int splitk;              // large part of bf16 weights: 1 K-split tiles at decode batches
                           // (gate/up: 16 rows, down: kSplitKCols columns per block); 2 (down
                           // past kSplitKDownMaxT, routed experts) kDownRowCols columns per
                           // block, row tiles for groups of at most 16 rows; 0 64-row /
                           // 64-column tiles
  const float* gate_scale; // FP8 weights: per-row scales [n_mats][rows] (gate, up)
  const float* up_scale;   //   and [n_mats][d] (down); unused otherwise
  const float* down_scale;
};

struct FamilySet {
  Family f[kMaxParts];
  int n;
  int blk_start[kMaxParts + 1];   // prefix sums of max_slots * tiles
};

struct CombineArgs {
  const int32_t* inv_perm;
  const float* row_weight;
  const float* row_out;    // nullptr: no per-row term (factorised form)
  const int32_t* dept_inv;
  const float* dept_scale; // nullptr: department outputs are added unscaled
  const float* dept_out;   // nullptr when no department term
  const float* shared_out; // nullptr when no shared expert
  int T, k, m, d;
  int max_rows;            // rows of row_out (plan entries at or past it are skipped)
  int max_dept_rows;       // rows of dept_out
};

// Down projection with the combine as its epilogue, for decode batches of at
// most kTokInline tokens (every group is then a small one): each wave owns one
// output column and streams that column's weight row of every active matrix
// of every family, so y is written once, with no per-row outputs, atomics or
// second launch.
constexpr int kDcWaves = 8;          // waves (output columns) per block
constexpr int kDcFamilies = 3;       // routed experts, department slices, shared expert
constexpr int kDcMaxRows = 2048;     // longest intermediate row it streams (4 steps of 512)
struct DcFamily {
  const void* down;        // [n_mats][d][rows] (bf16, or FP8 codes)
  const float* down_scale; // FP8: per-column scales [n_mats][d]; else nullptr
  const WorkDesc* work;    // small-group descriptors; nullptr: the shared expert (one group, all T tokens)
  const int* n_items;      // device count of descriptors (unused when work is nullptr)
  const float* wrow;       // weight of h row r (routing weight or c_{t,J}); nullptr: 1
  const void* h;           // gate/up outputs, row r at h + r * rows (layer dtype)
  const int* n_hrows;      // device count of rows of h in use; nullptr: T
  int rows;                // row length (intermediate size)
  int max_items;           // host bound on descriptors
  int max_hrows;           // host bound on the rows of h staged
  int lds_off;             // element offset of the family's rows of h in LDS
  int n_mats;              // matrices in the family (bounds check of descriptors)
};
struct DownCombineArgs {
  DcFamily f[kDcFamilies];
  int nf;                  // families in use (the first nf)
  int T, d;
  int h_elems;             // staged elements of h over all families (multiple of 8)
  int max_items;           // sum of the families' max_items
  int fp8;                 // 1: FP8 weights (E4M3 codes + per-column scales)
};
size_t down_combine_lds_bytes(const DownCombineArgs& a);

// Factorised form: weighted sum of a (token, department) pair's private
// outputs, the input of the department down projection.
struct PairCombineArgs {
  const int32_t* n_pairs;    // device count of pairs (plan header)
  const int32_t* pair_token; // [pairs]
  const int32_t* pair_dept;  // [pairs]
  const int32_t* inv_perm;   // [T*k]
  const int32_t* row_expert; // [rows]
  const float* row_weight;   // [rows]
  const float* z;            // [rows][cols] private outputs
  int T, k, group, cols;     // group = experts per department
  int max_rows;
};

struct GemvConfig {
  int rows_per_wave;   // gate/up: rows of each matrix per wave (1)
  int rows_per_pass;   // gate/up: rows a wave streams at once (1)
  int lpr;             // down: lanes per weight row (16, 32, 64)
  int col_groups;      // down: column groups per wave, 1 or 2 (columns per wave = col_groups * 64 / lpr)
};

// Optional timing of one kernel: the runtime writes `start` when the kernel
// begins and `stop` when it ends (hipExtLaunchKernel), so the interval is the
// kernel alone, with no event packets of its own in the stream.
struct KernelEvents {
  hipEvent_t start, stop;
};

// Launchers: each returns hipGetLastError() after its launch.  `ev` may be
// null; launch_route takes two (router kernel, top-k/plan kernel).
hipError_t launch_route(int w_dtype, const RouteArgs& ra, const PlanArgs* pa, hipStream_t st,
                        const KernelEvents* ev);
hipError_t launch_dispatch(const int32_t* ids, const float* w, const PlanArgs& pa, hipStream_t st);
hipError_t launch_gateup(int w_dtype, const FamilySet& set, const void* x, int T, int d,
                         int rows_per_wave, int rows_per_pass, hipStream_t st,
                         const KernelEvents* ev);
hipError_t launch_down(int w_dtype, const FamilySet& set, int T, int d, int lpr, int col_groups,
                       hipStream_t st, const KernelEvents* ev);
hipError_t launch_combine(int act_dtype, const CombineArgs& a, void* y, hipStream_t st,
                          const KernelEvents* ev);
// bf16 activations (bf16 or FP8 weights); the caller checks T <= kTokInline,
// the LDS size and kDcMaxRows.
hipError_t launch_down_combine(const DownCombineArgs& a, void* y, hipStream_t st,
                               const KernelEvents* ev);
// FP8 expert weights (E4M3 codes + per-row scales, bf16 activations): every
// part of the set is tiled like a small part (one gate/up row per wave; down:
// 64 / lpr columns per wave), groups of any size taken kTokInline tokens at a
// time.  d and every row length are multiples of 16 and at most
// MOE_FP8_MAX_WIDTH.
constexpr int kFp8RowsPerWave = 2;   // gate/up rows per wave (tiles of 4 * 2 rows)
constexpr int kFp8DownColGroups = 2; // down: columns per wave = 2 * 64 / lpr
constexpr int kFp8DnAhead = 2;       // down: 16-code steps requested ahead per column
hipError_t launch_gateup_fp8(const FamilySet& set, const void* x, int T, int d, hipStream_t st,
                             const KernelEvents* ev);
hipError_t launch_down_fp8(const FamilySet& set, int T, int d, int lpr, hipStream_t st,
                           const KernelEvents* ev);
// FP8 experts at larger batches: every group on matrix-core tiles (gate/up:
// 64 rows per block, tiles = ceil(rows / kWideRows); down: 64 columns per
// block, tiles = ceil(d / kWideRows)), the codes widened to bf16.
hipError_t launch_fp8_wide(bool gateup, const FamilySet& set, const void* x, int T, int d,
                           hipStream_t st, const KernelEvents* ev);
hipError_t launch_zero(unsigned int* p, size_t n, hipStream_t st);
hipError_t launch_stream_read(const void* src, size_t blocks, float* sink, hipStream_t st);
hipError_t launch_pair_combine(int act_dtype, const PairCombineArgs& a, void* zc, int max_pairs,
                               hipStream_t st);

}  // namespace moe
