// gfx950 kernels of the MoE decode step.
//
//   router_logits_kernel  l[t][e] = x_t . W_r[e]   (DeaMoE section 2.1, Eq. (2))
//   topk_dispatch_kernel  top-k + routing weights (Eq. (2)-(3); the DeepSeekMoE
//                         guide's bias routing), then the dispatch plan: counting
//                         sort by expert, inverse map, active lists, department
//                         pairs ("How a batch becomes expert-specific matrices")
//   gateup_kernel         h = SiLU(W_gate x) * (W_up x) per dispatched row (Eq. (1))
//   down_kernel           o = W_down h per dispatched row (Eq. (1))
//   combine_kernel        y_t = sum_j p_j o_{t,j} + department + shared terms (Eq. (3))
//
// Decode streams every active expert's weights once per step at one to a few
// rows per expert, so the expert kernels are weight-streaming GEMVs: every lane
// reads 16 contiguous bytes per row per step (a wave covers 1 KiB of a row per
// load instruction), accumulates in fp32 in registers, and the 64 lanes are
// reduced once per row block with a reduce-scatter butterfly.
#include "moe_device.h"
#include "moe_internal.h"

#include <climits>

namespace moe {

// ---------------------------------------------------------------------------
// Router logits: one wave per expert, lanes split d, tokens in chunks of 8.
// The per-expert reduction order does not depend on the expert index, so
// equal router rows give bitwise-equal logits.
// ---------------------------------------------------------------------------
template <typename T_>
__global__ __launch_bounds__(256) void router_logits_kernel(const T_* __restrict__ x,
                                                            const T_* __restrict__ wr, int T,
                                                            int d, int E,
                                                            float* __restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const T_* wrow = wr + (size_t)e * d;
  for (int t0 = 0; t0 < T; t0 += 8) {
    const int nv = min(8, T - t0);
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.f;
    for (int c = lane * 8; c < d; c += 8 * kWave) {
      float w[8];
      load8(wrow + c, w);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < nv) {
          float xv[8];
          load8(x + (size_t)(t0 + j) * d + c, xv);
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[j] = fmaf(w[q], xv[q], acc[j]);
        }
      }
    }
    const float r = wave_reduce_scatter<8>(acc, lane);
    const int j = (lane >> 3) & 7;
    if ((lane & 7) == 0 && j < nv) logits[(size_t)(t0 + j) * E + e] = r;
  }
}

// ---------------------------------------------------------------------------
// Top-k of one token by one wave.  Lane l holds experts l, l+64, ...; k rounds
// of a wave-wide argmax under the order (score desc, index asc).  Lane j keeps
// slot j, so slots come out in that order.
// ---------------------------------------------------------------------------
template <int NPL>
__device__ void topk_one(const TopkArgs& p, int t, int lane, int* s_ids, float* s_w) {
  const float* lrow = p.logits + (size_t)t * p.E;
  float sel[NPL], aux[NPL], lg[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + kWave * i;
    float l = 0.f, s = 0.f, a = 0.f;
    if (e < p.E) {
      l = lrow[e];
      const float b = p.bias ? p.bias[e] : 0.f;
      if (p.score_fn == MOE_SCORE_SIGMOID) {
        a = 1.0f / (1.0f + expf(-l));
        s = a + b;
      } else if (p.score_fn == MOE_SCORE_SOFTMAX_BIAS) {
        a = l;
        s = l + b;
      } else {
        a = l;
        s = l;
      }
      if (p.sel_out) p.sel_out[(size_t)t * p.E + e] = s;
    }
    sel[i] = s;
    aux[i] = a;
    lg[i] = l;
  }
  uint32_t taken = 0;
  int my_id = -1;
  float my_aux = 0.f;
  for (int j = 0; j < p.k; ++j) {
    float bv = 0.f, ba = 0.f;
    int be = INT_MAX;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + kWave * i;
      // indices grow with i, so a strict '>' keeps the lower index on ties
      if (e < p.E && !((taken >> i) & 1u) && (be == INT_MAX || sel[i] > bv)) {
        bv = sel[i];
        be = e;
        ba = aux[i];
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oe = __shfl_xor(be, o, kWave);
      const float oa = __shfl_xor(ba, o, kWave);
      const bool better = oe != INT_MAX && (be == INT_MAX || ov > bv || (ov == bv && oe < be));
      if (better) {
        bv = ov;
        be = oe;
        ba = oa;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) {
      my_id = be;
      my_aux = ba;
    }
  }
  const bool mine = lane < p.k;
  float w;
  if (p.score_fn == MOE_SCORE_SIGMOID) {
    const float tot = wave_sum(mine ? my_aux : 0.f);
    w = p.renorm ? my_aux / tot : my_aux;
  } else if (p.renorm) {
    const float mx = wave_max(mine ? my_aux : -INFINITY);
    const float ex = mine ? expf(my_aux - mx) : 0.f;
    const float tot = wave_sum(ex);
    w = ex / tot;
  } else {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (lane + kWave * i < p.E) mx = fmaxf(mx, lg[i]);
    mx = wave_max(mx);
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (lane + kWave * i < p.E) z += expf(lg[i] - mx);
    z = wave_sum(z);
    w = expf(my_aux - mx) / z;
  }
  w *= p.scale;
  if (mine) {
    const int a = t * p.k + lane;
    if (p.ids_out) p.ids_out[a] = my_id;
    if (p.w_out) p.w_out[a] = w;
    s_ids[a] = my_id;
    s_w[a] = w;
  }
}

// Exclusive scan of in[0, n) into out[0, n], out[n] = total; LDS arrays, whole block.
__device__ void block_exclusive_scan(const int* in, int* out, int n, int (*s_scan)[16]) {
  const int tid = threadIdx.x, nth = blockDim.x;
  const int lane = tid & 63, wid = tid >> 6, nw = nth >> 6;
  const int per = (n + nth - 1) / nth;
  const int beg = min(n, tid * per), end = min(n, beg + per);
  int local = 0;
  for (int i = beg; i < end; ++i) local += in[i];
  int v = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  if (lane == 63) s_scan[0][wid] = v;
  __syncthreads();
  if (wid == 0) {
    const int tot = lane < nw ? s_scan[0][lane] : 0;
    int w = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(w, o, kWave);
      if (lane >= o) w += u;
    }
    if (lane < nw) s_scan[1][lane] = w - tot;
  }
  __syncthreads();
  int run = s_scan[1][wid] + v - local;
  for (int i = beg; i < end; ++i) {
    out[i] = run;
    run += in[i];
  }
  if (tid == nth - 1) out[n] = run;
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Top-k for all tokens, then the dispatch plan, in one block.
// ---------------------------------------------------------------------------
template <int NPL>
__global__ __launch_bounds__(kPlanThreads) void topk_dispatch_kernel(TopkArgs tk, DispatchArgs dp,
                                                                     int do_topk, int do_dispatch) {
  __shared__ int s_ids[MOE_MAX_ASSIGNMENTS];
  __shared__ float s_w[MOE_MAX_ASSIGNMENTS];
  __shared__ int s_a[MOE_MAX_EXPERTS];
  __shared__ int s_b[MOE_MAX_EXPERTS + 1];
  __shared__ unsigned char s_flag[MOE_MAX_DEPT_PAIRS];
  __shared__ int s_scan[2][16];
  __shared__ int s_invalid;

  const int tid = threadIdx.x, nth = blockDim.x;
  const int lane = tid & 63, wid = tid >> 6, nw = nth >> 6;
  const int T = dp.T, k = dp.k, A = T * k;

  if (do_topk) {
    for (int t = wid; t < tk.T; t += nw) topk_one<NPL>(tk, t, lane, s_ids, s_w);
  } else {
    for (int a = tid; a < A; a += nth) {
      s_ids[a] = dp.ids_in[a];
      s_w[a] = dp.w_in[a];
    }
  }
  if (!do_dispatch) return;
  const int E = dp.E;
  const moe_plan& P = dp.plan;
  for (int e = tid; e < E; e += nth) s_a[e] = 0;
  if (tid == 0) s_invalid = 0;
  __syncthreads();

  // rows per expert
  for (int a = tid; a < A; a += nth) {
    const int e = s_ids[a];
    if (e >= 0 && e < E)
      atomicAdd(&s_a[e], 1);
    else
      atomicAdd(&s_invalid, 1);
  }
  __syncthreads();
  block_exclusive_scan(s_a, s_b, E, s_scan);

  // row of assignment a = offset of its expert + earlier assignments to it
  for (int a = tid; a < A; a += nth) {
    const int e = s_ids[a];
    if (e >= 0 && e < E) {
      int rank = 0;
      for (int b = 0; b < a; ++b) rank += (s_ids[b] == e);
      const int row = s_b[e] + rank;
      P.row_token[row] = a / k;
      P.row_slot[row] = a % k;
      P.row_expert[row] = e;
      P.row_weight[row] = s_w[a];
      P.inv_perm[a] = row;
    } else {
      P.inv_perm[a] = -1;
    }
  }
  for (int e = tid; e < E; e += nth) {
    P.counts[e] = s_a[e];
    P.offsets[e] = s_b[e];
  }
  if (tid == 0) P.offsets[E] = s_b[E];
  __syncthreads();
  for (int e = tid; e < E; e += nth) s_a[e] = s_a[e] > 0 ? 1 : 0;
  __syncthreads();
  block_exclusive_scan(s_a, s_b, E, s_scan);
  for (int e = tid; e < E; e += nth)
    if (s_a[e]) P.active[s_b[e]] = e;
  if (tid == 0) {
    P.header[MOE_PLAN_N_ROWS] = A - s_invalid;
    P.header[MOE_PLAN_N_ACTIVE] = s_b[E];
    P.header[MOE_PLAN_N_INVALID] = s_invalid;
  }
  __syncthreads();

  if (dp.m > 0) {
    // (token, department) pairs: department j is active for token t when t
    // selected at least one of its experts; c_{t,j} sums those weights.
    const int m = dp.m, G = E / m, TM = T * m;
    for (int p = tid; p < TM; p += nth) {
      const int t = p / m, J = p - t * m;
      int has = 0;
      for (int j = 0; j < k; ++j) {
        const int e = s_ids[t * k + j];
        if (e >= 0 && e < E && e / G == J) has = 1;
      }
      s_flag[p] = (unsigned char)has;
    }
    __syncthreads();
    for (int J = tid; J < m; J += nth) {
      int c = 0;
      for (int t = 0; t < T; ++t) c += s_flag[t * m + J];
      s_a[J] = c;
    }
    __syncthreads();
    block_exclusive_scan(s_a, s_b, m, s_scan);
    for (int p = tid; p < TM; p += nth) {
      const int t = p / m, J = p - t * m;
      if (s_flag[p]) {
        int rank = 0;
        for (int u = 0; u < t; ++u) rank += s_flag[u * m + J];
        const int q = s_b[J] + rank;
        float sc = 0.f;
        for (int j = 0; j < k; ++j) {
          const int e = s_ids[t * k + j];
          if (e >= 0 && e < E && e / G == J) sc += s_w[t * k + j];
        }
        P.dept_row_token[q] = t;
        P.dept_row_dept[q] = J;
        P.dept_row_scale[q] = sc;
        P.dept_inv[p] = q;
      } else {
        P.dept_inv[p] = -1;
      }
    }
    for (int J = tid; J < m; J += nth) {
      P.dept_counts[J] = s_a[J];
      P.dept_offsets[J] = s_b[J];
    }
    if (tid == 0) {
      P.dept_offsets[m] = s_b[m];
      P.header[MOE_PLAN_N_DEPT_ROWS] = s_b[m];
    }
    __syncthreads();
    for (int J = tid; J < m; J += nth) s_a[J] = s_a[J] > 0 ? 1 : 0;
    __syncthreads();
    block_exclusive_scan(s_a, s_b, m, s_scan);
    for (int J = tid; J < m; J += nth)
      if (s_a[J]) P.active_depts[s_b[J]] = J;
    if (tid == 0) P.header[MOE_PLAN_N_ACTIVE_DEPTS] = s_b[m];
  } else if (tid == 0) {
    P.header[MOE_PLAN_N_DEPT_ROWS] = 0;
    P.header[MOE_PLAN_N_ACTIVE_DEPTS] = 0;
  }
}

// ---------------------------------------------------------------------------
// Grouped expert GEMVs.  A block maps to (family, active slot, tile); slots
// beyond the device-side active count exit at once, so the grid can be sized
// on the host from T alone.
// ---------------------------------------------------------------------------
struct BlockTask {
  const void* gate;
  const void* up;
  const void* down;
  const int* grp_token;
  float* h;
  float* out;
  int rows, mat, r0, n, tile;
};

// Copies the fields of this block's family into registers (a pointer into the
// kernel-argument struct would force it into scratch memory).
__device__ __forceinline__ bool map_block(const SegSet& set, int T, bool gateup, BlockTask& bt) {
  const int b = blockIdx.x;
  int si = 0;
  while (si + 1 < set.n && b >= set.blk_start[si + 1]) ++si;
  const MatSeg S = set.s[si];
  const int tiles = gateup ? S.tiles_gu : S.tiles_dn;
  const int lb = b - set.blk_start[si];
  const int slot = lb / tiles;
  const int na = S.n_active ? *S.n_active : 1;
  if (slot >= na) return false;
  bt.gate = S.gate;
  bt.up = S.up;
  bt.down = S.down;
  bt.grp_token = S.grp_token;
  bt.h = S.h;
  bt.out = S.out;
  bt.rows = S.rows;
  bt.tile = lb - slot * tiles;
  bt.mat = S.active ? S.active[slot] : 0;
  bt.r0 = S.grp_off ? S.grp_off[bt.mat] : 0;
  bt.n = S.grp_off ? S.grp_off[bt.mat + 1] - bt.r0 : T;
  return bt.n > 0;
}

// RW rows of gate and up starting at i0, against the n tokens of rows
// r0..r0+n-1 in chunks of NT.  h[row][i] = SiLU(g) * u.
template <typename T_, int RW, int NT>
__device__ __forceinline__ void gateup_pass(const T_* __restrict__ Wg, const T_* __restrict__ Wu,
                                            int d, int rows, int i0, const T_* __restrict__ x,
                                            const int* __restrict__ grp_token, int r0, int n,
                                            float* __restrict__ h, int lane) {
  const T_* gp[RW];
  const T_* up[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int i = min(i0 + r, rows - 1);
    gp[r] = Wg + (size_t)i * d;
    up[r] = Wu + (size_t)i * d;
  }
  for (int tc = 0; tc < n; tc += NT) {
    const int nv = min(NT, n - tc);
    const T_* xp[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int rr = r0 + tc + min(t, nv - 1);
      const int tok = grp_token ? grp_token[rr] : rr;
      xp[t] = x + (size_t)tok * d;
    }
    float ag[RW][NT], au[RW][NT];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int t = 0; t < NT; ++t) ag[r][t] = au[r][t] = 0.f;
    for (int c = lane * 8; c < d; c += 8 * kWave) {
      float wg[RW][8], wu[RW][8];
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        load8_stream(gp[r] + c, wg[r]);
        load8_stream(up[r] + c, wu[r]);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t < nv) {
          float xv[8];
          load8(xp[t] + c, xv);
#pragma unroll
          for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              ag[r][t] = fmaf(wg[r][q], xv[q], ag[r][t]);
              au[r][t] = fmaf(wu[r][q], xv[q], au[r][t]);
            }
        }
      }
    }
    constexpr int N = 2 * RW * NT;
    constexpr int SH = 6 - Log2<N>::value;
    float v[N];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        v[r * NT + t] = ag[r][t];
        v[RW * NT + r * NT + t] = au[r][t];
      }
    const float red = wave_reduce_scatter<N>(v, lane);
    const float upv = __shfl_xor(red, 32, kWave);  // index + N/2 lives in lane ^ 32
    const int idx = (lane >> SH) & (N - 1);
    if (idx < N / 2 && (lane & ((1 << SH) - 1)) == 0) {
      const int r = idx / NT, t = idx - (idx / NT) * NT;
      if (t < nv && i0 + r < rows) h[(size_t)(r0 + tc + t) * rows + i0 + r] = silu(red) * upv;
    }
  }
}

template <typename T_>
__global__ __launch_bounds__(256) void gateup_kernel(SegSet set, const T_* __restrict__ x, int T,
                                                     int d) {
  BlockTask bt;
  if (!map_block(set, T, true, bt)) return;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int rows = bt.rows;
  const int i0 = bt.tile * kGuTile + wid * kRowsPerWave;
  if (i0 >= rows) return;
  const size_t mstride = (size_t)rows * d;
  const T_* Wg = static_cast<const T_*>(bt.gate) + (size_t)bt.mat * mstride;
  const T_* Wu = static_cast<const T_*>(bt.up) + (size_t)bt.mat * mstride;
  if (bt.n <= 4) {
    gateup_pass<T_, 4, 4>(Wg, Wu, d, rows, i0, x, bt.grp_token, bt.r0, bt.n, bt.h, lane);
  } else if (bt.n <= 8) {
    gateup_pass<T_, 2, 8>(Wg, Wu, d, rows, i0, x, bt.grp_token, bt.r0, bt.n, bt.h, lane);
    gateup_pass<T_, 2, 8>(Wg, Wu, d, rows, i0 + 2, x, bt.grp_token, bt.r0, bt.n, bt.h, lane);
  } else {
#pragma unroll 1
    for (int r = 0; r < kRowsPerWave; ++r)
      gateup_pass<T_, 1, 16>(Wg, Wu, d, rows, i0 + r, x, bt.grp_token, bt.r0, bt.n, bt.h, lane);
  }
}

// CW output columns from c0 (rows of W_down [d][rows]) against the n rows of
// h from r0, in chunks of NT.  out[row][c] = W_down[c] . h[row].
template <typename T_, int CW, int NT>
__device__ __forceinline__ void down_pass(const T_* __restrict__ Wd, int d, int rows, int c0,
                                          const float* __restrict__ h, int r0, int n,
                                          float* __restrict__ out, int lane) {
  const T_* wp[CW];
#pragma unroll
  for (int cc = 0; cc < CW; ++cc) wp[cc] = Wd + (size_t)min(c0 + cc, d - 1) * rows;
  for (int tc = 0; tc < n; tc += NT) {
    const int nv = min(NT, n - tc);
    const float* hp[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) hp[t] = h + (size_t)(r0 + tc + min(t, nv - 1)) * rows;
    float acc[CW][NT];
#pragma unroll
    for (int cc = 0; cc < CW; ++cc)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[cc][t] = 0.f;
    for (int i = lane * 8; i < rows; i += 8 * kWave) {
      float wv[CW][8];
#pragma unroll
      for (int cc = 0; cc < CW; ++cc) load8_stream(wp[cc] + i, wv[cc]);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t < nv) {
          float hv[8];
          load8(hp[t] + i, hv);
#pragma unroll
          for (int cc = 0; cc < CW; ++cc)
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[cc][t] = fmaf(wv[cc][q], hv[q], acc[cc][t]);
        }
      }
    }
    constexpr int N = CW * NT;
    constexpr int SH = 6 - Log2<N>::value;
    float v[N];
#pragma unroll
    for (int cc = 0; cc < CW; ++cc)
#pragma unroll
      for (int t = 0; t < NT; ++t) v[cc * NT + t] = acc[cc][t];
    const float red = wave_reduce_scatter<N>(v, lane);
    const int idx = (lane >> SH) & (N - 1);
    if ((lane & ((1 << SH) - 1)) == 0) {
      const int cc = idx / NT, t = idx - (idx / NT) * NT;
      if (t < nv && c0 + cc < d) out[(size_t)(r0 + tc + t) * d + c0 + cc] = red;
    }
  }
}

template <typename T_>
__global__ __launch_bounds__(256) void down_kernel(SegSet set, int T, int d) {
  BlockTask bt;
  if (!map_block(set, T, false, bt)) return;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int rows = bt.rows;
  const int c0 = bt.tile * kDnTile + wid * kColsPerWave;
  if (c0 >= d) return;
  const T_* Wd = static_cast<const T_*>(bt.down) + (size_t)bt.mat * rows * d;
  if (bt.n <= 4) {
    down_pass<T_, 4, 4>(Wd, d, rows, c0, bt.h, bt.r0, bt.n, bt.out, lane);
  } else if (bt.n <= 8) {
    down_pass<T_, 2, 8>(Wd, d, rows, c0, bt.h, bt.r0, bt.n, bt.out, lane);
    down_pass<T_, 2, 8>(Wd, d, rows, c0 + 2, bt.h, bt.r0, bt.n, bt.out, lane);
  } else {
#pragma unroll 1
    for (int cc = 0; cc < kColsPerWave; ++cc)
      down_pass<T_, 1, 16>(Wd, d, rows, c0 + cc, bt.h, bt.r0, bt.n, bt.out, lane);
  }
}

// ---------------------------------------------------------------------------
// Combine: one thread per (token, column); slot order, then departments
// ascending, then the shared expert.
// ---------------------------------------------------------------------------
template <typename AT>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a, AT* __restrict__ y) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const int t = blockIdx.y;
  if (c >= a.d) return;
  float acc = 0.f;
  for (int j = 0; j < a.k; ++j) {
    const int r = a.inv_perm[t * a.k + j];
    if (r >= 0) acc = fmaf(a.row_weight[r], a.row_out[(size_t)r * a.d + c], acc);
  }
  if (a.dept_out) {
    for (int J = 0; J < a.m; ++J) {
      const int q = a.dept_inv[t * a.m + J];
      if (q >= 0) acc = fmaf(a.dept_scale[q], a.dept_out[(size_t)q * a.d + c], acc);
    }
  }
  if (a.shared_out) acc += a.shared_out[(size_t)t * a.d + c];
  store_act(y + (size_t)t * a.d + c, acc);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_router_logits(int w_dtype, const void* x, const void* w_router, int T, int d,
                                int E, float* logits, hipStream_t st) {
  const dim3 grid((E + 3) / 4), block(256);
  if (w_dtype == MOE_BF16)
    hipLaunchKernelGGL(router_logits_kernel<bf16_t>, grid, block, 0, st,
                       static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(w_router), T, d,
                       E, logits);
  else
    hipLaunchKernelGGL(router_logits_kernel<float>, grid, block, 0, st,
                       static_cast<const float*>(x), static_cast<const float*>(w_router), T, d, E,
                       logits);
  return hipGetLastError();
}

hipError_t launch_topk_dispatch(const TopkArgs* topk, const DispatchArgs* disp, hipStream_t st) {
  TopkArgs tk{};
  if (topk) tk = *topk;
  DispatchArgs dp{};
  if (disp) dp = *disp;
  const int do_topk = topk != nullptr, do_dispatch = disp != nullptr;
  if (do_topk && !do_dispatch) {  // the kernel reads T and k from the dispatch arguments
    dp.T = tk.T;
    dp.k = tk.k;
  }
  const int E = do_topk ? tk.E : dp.E;
  const dim3 grid(1), block(kPlanThreads);
#define MOE_TOPK_LAUNCH(NPL)                                                                   \
  hipLaunchKernelGGL(topk_dispatch_kernel<NPL>, grid, block, 0, st, tk, dp, do_topk, do_dispatch)
  if (!do_topk || E <= 64)
    MOE_TOPK_LAUNCH(1);
  else if (E <= 128)
    MOE_TOPK_LAUNCH(2);
  else if (E <= 256)
    MOE_TOPK_LAUNCH(4);
  else if (E <= 512)
    MOE_TOPK_LAUNCH(8);
  else if (E <= 1024)
    MOE_TOPK_LAUNCH(16);
  else
    MOE_TOPK_LAUNCH(32);
#undef MOE_TOPK_LAUNCH
  return hipGetLastError();
}

hipError_t launch_gateup(int w_dtype, const SegSet& set, const void* x, int T, int d,
                         hipStream_t st) {
  const int blocks = set.blk_start[set.n];
  if (blocks <= 0) return hipSuccess;
  if (w_dtype == MOE_BF16)
    hipLaunchKernelGGL(gateup_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st, set,
                       static_cast<const bf16_t*>(x), T, d);
  else
    hipLaunchKernelGGL(gateup_kernel<float>, dim3(blocks), dim3(256), 0, st, set,
                       static_cast<const float*>(x), T, d);
  return hipGetLastError();
}

hipError_t launch_down(int w_dtype, const SegSet& set, int T, int d, hipStream_t st) {
  const int blocks = set.blk_start[set.n];
  if (blocks <= 0) return hipSuccess;
  if (w_dtype == MOE_BF16)
    hipLaunchKernelGGL(down_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st, set, T, d);
  else
    hipLaunchKernelGGL(down_kernel<float>, dim3(blocks), dim3(256), 0, st, set, T, d);
  return hipGetLastError();
}

hipError_t launch_combine(int act_dtype, const CombineArgs& a, void* y, hipStream_t st) {
  const dim3 grid((a.d + 255) / 256, a.T), block(256);
  if (act_dtype == MOE_BF16)
    hipLaunchKernelGGL(combine_kernel<bf16_t>, grid, block, 0, st, a, static_cast<bf16_t*>(y));
  else
    hipLaunchKernelGGL(combine_kernel<float>, grid, block, 0, st, a, static_cast<float*>(y));
  return hipGetLastError();
}

}  // namespace moe
