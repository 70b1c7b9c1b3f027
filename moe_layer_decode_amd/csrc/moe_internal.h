// Internal interface between the C ABI (host orchestration) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_decode.h"

namespace moe {

// Gate/up GEMV tiling: a block is 4 waves, each wave owns kRowsPerWave rows of
// gate and up, so a block covers kGuTile intermediate rows.
constexpr int kGuWaves = 4;
constexpr int kRowsPerWave = 4;
constexpr int kGuTile = kGuWaves * kRowsPerWave;
// Down GEMV tiling: each wave owns kColsPerWave output columns of d.
constexpr int kDnWaves = 4;
constexpr int kColsPerWave = 4;
constexpr int kDnTile = kDnWaves * kColsPerWave;
// Threads of the single-block top-k / dispatch kernel.
constexpr int kPlanThreads = 1024;

// One family of same-shape matrices (routed experts, department slices, or
// the shared expert) and the row groups that use them.
struct MatSeg {
  const void* gate;      // [n_mats][rows][d]
  const void* up;        // [n_mats][rows][d]
  const void* down;      // [n_mats][d][rows]
  int rows;              // intermediate width of this family
  const int* active;     // active matrix ids (nullptr: the single matrix 0)
  const int* n_active;   // device count of `active` (nullptr: 1)
  const int* grp_off;    // [n_mats+1] row ranges (nullptr: rows 0..T-1)
  const int* grp_token;  // token of each row (nullptr: row r is token r)
  float* h;              // [rows_total][rows] fp32 SiLU(g)*u
  float* out;            // [rows_total][d] fp32 unweighted down output
  int max_slots;         // host upper bound on *n_active
  int tiles_gu;          // ceil(rows / kGuTile)
  int tiles_dn;          // ceil(d / kDnTile)
};

struct SegSet {
  MatSeg s[3];
  int n;
  int blk_start[4];      // prefix sums of blocks per family
};

struct TopkArgs {
  const float* logits;   // [T][E]
  const float* bias;     // [E] or nullptr
  int T, E, k;
  int score_fn, renorm;
  float scale;
  int32_t* ids_out;      // [T][k] or nullptr
  float* w_out;          // [T][k] or nullptr
  float* sel_out;        // [T][E] or nullptr
};

struct DispatchArgs {
  const int32_t* ids_in;  // used when the kernel does not run top-k itself
  const float* w_in;
  int T, E, k, m;
  moe_plan plan;
};

struct CombineArgs {
  const int32_t* inv_perm;
  const float* row_weight;
  const float* row_out;
  const int32_t* dept_inv;
  const float* dept_scale;
  const float* dept_out;   // nullptr when no department term
  const float* shared_out; // nullptr when no shared expert
  int T, k, m, d;
};

// Launchers (each returns the hipGetLastError() of its launch).
hipError_t launch_router_logits(int w_dtype, const void* x, const void* w_router, int T, int d,
                                int E, float* logits, hipStream_t st);
hipError_t launch_topk_dispatch(const TopkArgs* topk, const DispatchArgs* disp, hipStream_t st);
hipError_t launch_gateup(int w_dtype, const SegSet& set, const void* x, int T, int d,
                         hipStream_t st);
hipError_t launch_down(int w_dtype, const SegSet& set, int T, int d, hipStream_t st);
hipError_t launch_combine(int act_dtype, const CombineArgs& a, void* y, hipStream_t st);

}  // namespace moe
