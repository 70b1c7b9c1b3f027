// gfx950 kernels of the MoE decode step.
//
//   route_kernel      partial router logits (DeaMoE section 2.1, Eq. (2)),
//                     split over d-chunks across the whole chip
//   topk_plan_kernel  one block: sums the partials, takes the top-k with its
//                     weights (Eq. (3); the DeepSeekMoE guide's sigmoid/bias
//                     routing) and builds the dispatch plan ("How a batch
//                     becomes expert-specific matrices": group by expert, keep
//                     token ids and the inverse map), plus one work descriptor
//                     per active expert and department
//   topk_token_kernel the top-k of larger batches (or of more than 256
//                     experts), one wave per token across many blocks
//   dispatch_kernel   the plan alone, from caller-given ids or from the ids
//                     topk_token_kernel wrote
//   gateup_kernel     h = SiLU(W_gate x) * (W_up x) per dispatched row (Eq. (1))
//   down_kernel       o = W_down h per dispatched row (Eq. (1))
//   combine_kernel    y_t = sum_j p_j o_{t,j} + department + shared terms (Eq. (3))
//
// Decode reads every active expert's weights once per step at one to a few
// rows per expert, so the expert kernels are weight-streaming GEMVs: each lane
// reads 16 contiguous bytes of a weight row per step, the next step's weights
// are already in flight while the current ones are used, sums are fp32 in
// registers, and the lanes of a row are reduced once with a reduce-scatter
// butterfly.  Blocks whose slot is beyond the device-side active count exit at
// once, so every grid is sized on the host from T alone.
//
#include "moe_device.h"
#include "moe_internal.h"

#include <hip/hip_ext.h>

#include <climits>
#include <type_traits>

namespace moe {

// ---------------------------------------------------------------------------
// 16-byte weight vectors kept raw (bf16 stays packed) until they are used.
// ---------------------------------------------------------------------------
template <typename T_> struct Raw8;
template <> struct Raw8<bf16_t> {
  u32x4_t u;
  __device__ __forceinline__ void load(const bf16_t* p) {
    u = __builtin_nontemporal_load(as_global<u32x4_t>(p));
  }
  __device__ __forceinline__ void zero() { u = u32x4_t{0, 0, 0, 0}; }
  __device__ __forceinline__ void to_f32(float (&v)[8]) const {
    v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
    v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z); v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
  }
};
template <> struct Raw8<float> {
  f32x4_t a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = __builtin_nontemporal_load(as_global<f32x4_t>(p));
    b = __builtin_nontemporal_load(as_global<f32x4_t>(p + 4));
  }
  __device__ __forceinline__ void zero() { a = b = f32x4_t{0.f, 0.f, 0.f, 0.f}; }
  __device__ __forceinline__ void to_f32(float (&v)[8]) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

// Activation vectors of 8 elements and the 8-term dot product with a weight
// vector.  bf16 x bf16 uses the packed dot instruction (products are exact in
// fp32, two per instruction); fp32 uses plain fused multiply-adds.
template <typename T_> struct X8;
template <> struct X8<bf16_t> {
  u32x4_t u;
  __device__ __forceinline__ void load(const bf16_t* p) {
    u = *as_global<u32x4_t>(p);
  }
  __device__ __forceinline__ void zero() { u = u32x4_t{0, 0, 0, 0}; }
};
template <> struct X8<float> {
  f32x4_t a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *as_global<f32x4_t>(p);
    b = *as_global<f32x4_t>(p + 4);
  }
  __device__ __forceinline__ void zero() { a = b = f32x4_t{0.f, 0.f, 0.f, 0.f}; }
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}
__device__ __forceinline__ float dot8(const Raw8<bf16_t>& w, const X8<bf16_t>& x, float acc) {
  acc = dot2_bf16(w.u.x, x.u.x, acc);
  acc = dot2_bf16(w.u.y, x.u.y, acc);
  acc = dot2_bf16(w.u.z, x.u.z, acc);
  return dot2_bf16(w.u.w, x.u.w, acc);
}
__device__ __forceinline__ float dot8(const Raw8<float>& w, const X8<float>& x, float acc) {
  acc = fmaf(w.a.x, x.a.x, acc);
  acc = fmaf(w.a.y, x.a.y, acc);
  acc = fmaf(w.a.z, x.a.z, acc);
  acc = fmaf(w.a.w, x.a.w, acc);
  acc = fmaf(w.b.x, x.b.x, acc);
  acc = fmaf(w.b.y, x.b.y, acc);
  acc = fmaf(w.b.z, x.b.z, acc);
  return fmaf(w.b.w, x.b.w, acc);
}

// 16-byte loads with the default cache policy.  Weights read in the
// matrix-core operand layout (64-byte pieces of each row: the router's and the
// 64-row tiles') take it too: the two halves of a 128-byte line arrive from
// separate loads, and a non-temporal first half did not keep the line for the
// second (DeaMoE on the DeepSeek-V3 geometry, batch 128: 1168 -> 1085 us;
// the DeepSeek-V3-shaped router at batch 128: 18.7 -> 14.7 us).  Whole-line
// streams (the GEMVs, the LDS weight tiles) stay non-temporal.
__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4_t& u) {
  return __builtin_bit_cast(bf16x8_t, u);
}
__device__ __forceinline__ u32x4_t ld16(const bf16_t* p) { return *as_global<u32x4_t>(p); }


// Wave-uniform copies (one lane's value in a scalar register), for values
// that are uniform by construction but reach a function in vector registers.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float uni(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}
template <typename P>
__device__ __forceinline__ P* uni(P* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  return reinterpret_cast<P*>(lo | (hi << 32));
}

// Raw buffer loads.  A resource spans 2 GiB from a wave-uniform base; a load
// at an offset at or past its end returns zeros without touching memory, so a
// bounds test becomes a select on the load's offset (kDcOob) and the load
// itself stays unconditional.  (Loads under a branch make the compiler wait
// for every load in flight at the branch's end, which empties any prefetch.)
constexpr int kGfx9BufferDword3 = 0x00020000;  // raw (untyped) 32-bit buffer access
constexpr int kCpolNt = 2;                     // non-temporal: weights are read once
constexpr uint32_t kDcOob = 0x80000000u;       // buffer offset past every resource: reads 0
constexpr int kSpanBytes = 0x7fffffff;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(uni(const_cast<void*>(base)), (short)0, kSpanBytes,
                                           kGfx9BufferDword3);
}
__device__ __forceinline__ u32x4_t ld16_span(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
}

// ---------------------------------------------------------------------------
// Routing + plan
// ---------------------------------------------------------------------------
// Top-k staging: a chunk of tokens' router logits and selection keys in LDS
// (entry j = (t - t0) * E + e), filled by the whole block, then read by the
// token's wave.
constexpr int kTopkBuf = 10240;   // staged (token, expert) entries per chunk
constexpr int kCand = 128;        // compacted candidates per token
constexpr int kPlanWaves = kPlanThreads / kWave;
constexpr int kRankMaskWords = 1024;
constexpr int kDeptMaskMax = 64;
constexpr int kDeptMaskWords = 4;  // department token bits: up to 256 tokens
__device__ __forceinline__ bool dept_masks(int T, int m) {
  return m > 0 && m <= kDeptMaskMax && T <= 64 * kDeptMaskWords;
}
// Words of token bits per expert when E of them fit in `cap` words, else 0.
__device__ __forceinline__ int rank_mask_words(int T, int E, int cap = kRankMaskWords) {
  const int nwt = (T + 63) >> 6;
  return nwt * E <= cap ? nwt : 0;
}
struct TopkStage {
  float lg[kTopkBuf];
  uint32_t key[kTopkBuf];
  uint32_t cand_key[kPlanWaves][kCand];
  int cand_e[kPlanWaves][kCand];
  unsigned dmax[kPlanWaves][MOE_MAX_DEPTS_GROUPED];  // per wave: department keys / counts
};
// Plan-only arrays (used once every token is routed).
struct PlanWork {
  int off[MOE_MAX_EXPERTS + 1];           // experts: first row
  int slot[MOE_MAX_EXPERTS];              //          index in the small / large work list
  int doff[MOE_MAX_EXPERTS + 1];          // departments (m <= E): first pair
  int dslot[MOE_MAX_EXPERTS];
  int dcnt[MOE_MAX_EXPERTS];
  int tot[kPlanWaves][4];                 // per wave: rows, active, small
};
struct PlanShared {
  int ids[MOE_MAX_ASSIGNMENTS];           // chosen experts, t*k + slot
  float w[MOE_MAX_ASSIGNMENTS];           // their weights
  int cnt[MOE_MAX_EXPERTS];               // assignments per expert
  unsigned char flag[MOE_MAX_DEPT_PAIRS]; // (t, J): token t chose an expert of department J
  // Tokens of each expert as bits (word e * ceil(T / 64) + t / 64, bit t % 64)
  // when E * ceil(T / 64) words fit: an assignment's rank among its expert's
  // rows is then a popcount of the lower tokens instead of a scan of the
  // earlier assignments.
  unsigned long long tmask[kRankMaskWords];
  // Tokens of each department as bits (word t / 64 of department J, bit
  // t % 64) when T <= 64 kDeptMaskWords and m <= kDeptMaskMax: a pair's rank
  // among its department's pairs is then a popcount of the lower tokens
  // instead of a scan of the pair flags.
  unsigned long long dtok[kDeptMaskMax][kDeptMaskWords];
  union {
    TopkStage tk;
    // the plan-only launch stages no top-k: its expert token bits take the
    // staging area beside the plan's arrays (E * ceil(T / 64) up to
    // kRankMaskWordsBig words)
    struct {
      PlanWork pw;
      unsigned long long tbig[(sizeof(TopkStage) - sizeof(PlanWork)) / 8];
    };
  };
  int invalid;
};
constexpr int kRankMaskWordsBig = (int)((sizeof(TopkStage) - sizeof(PlanWork)) / 8);
static_assert(kRankMaskWordsBig >= 4096, "token bits of 864 experts at 256 tokens");

// Rank of token t among the tokens whose bits `w` holds (its lower ones).
__device__ __forceinline__ int bits_below(const unsigned long long* w, int t) {
  int r = 0;
  for (int q = 0; q < (t >> 6); ++q) r += __popcll(w[q]);
  return r + __popcll(w[t >> 6] & ((1ull << (t & 63)) - 1ull));
}

// Order-preserving 32-bit key of a score: a larger float gives a larger key,
// and +0 / -0 share one key (they compare equal as floats).  Key 0 lies below
// every float, so it marks lanes past the last expert.
__device__ __forceinline__ uint32_t score_key(float f) {
  const uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int wave_count(bool b) { return __popcll(__ballot(b)); }

// Value the routing weights start from: the sigmoid affinity in sigmoid mode,
// else the logit.
__device__ __forceinline__ float route_aux(const RouteArgs& p, float l) {
  return p.score_fn == MOE_SCORE_SIGMOID ? 1.0f / (1.0f + expf(-l)) : l;
}

// The ksplit partial logits of expert e for token t (planes past ksplit read
// 0), and its selection bias (0 without one).  Every load is unconditional --
// a plane past ksplit re-reads plane 0, the bias of a layer without one reads
// a logit -- and the values are selected afterwards: a load under a branch
// would end in a wait for every load in flight at the branch's join.
__device__ __forceinline__ void logit_parts(const RouteArgs& p, int t, int e,
                                            float (&v)[kMaxRouteSplit], float& b) {
  const float* bp = p.bias ? p.bias : p.logits;
  const float bv = bp[e];
#pragma unroll
  for (int q = 0; q < kMaxRouteSplit; ++q)
    v[q] = p.logits[((size_t)(q < p.ksplit ? q : 0) * p.T + t) * p.E + e];
#pragma unroll
  for (int q = 0; q < kMaxRouteSplit; ++q) v[q] = q < p.ksplit ? v[q] : 0.f;
  b = p.bias ? bv : 0.f;
}

// One token's row by its own wave (lane l: experts l, l+64, ...), for
// layers with few experts per lane: the planes of all NPL entries are
// requested before the first add waits, and no block barrier is needed.  The
// keys stay in registers; the row in LDS gets the logits, and the keys too
// when departments are ranked (their maxima are read department-major).
template <int NPL, bool GROUPED>
__device__ void stage_token(const RouteArgs& p, int t, int row, int lane, PlanShared& s,
                            uint32_t (&key)[NPL]) {
  const int E = p.E;
  // planes of experts in chunks of CH, each chunk's partial-logit loads all
  // requested before its first add waits (a layer with few experts is one chunk)
  constexpr int CH = NPL < 4 ? NPL : 4;
#pragma unroll
  for (int i0 = 0; i0 < NPL; i0 += CH) {
    float v[CH][kMaxRouteSplit], b[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) logit_parts(p, t, min(lane + kWave * (i0 + i), E - 1), v[i], b[i]);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int e = lane + kWave * (i0 + i);
      key[i0 + i] = 0u;
      if (e < E) {
        float l = 0.f;
#pragma unroll
        for (int q = 0; q < kMaxRouteSplit; ++q) l += v[i][q];
        const float sc = p.score_fn == MOE_SCORE_SOFTMAX ? l : route_aux(p, l) + b[i];
        if (p.sel_out) p.sel_out[(size_t)t * E + e] = sc;
        s.tk.lg[row + e] = l;
        key[i0 + i] = score_key(sc);
        if (GROUPED) s.tk.key[row + e] = key[i0 + i];
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// The k-th largest key of the wave (NP keys per lane; key 0 lies below every
// real key; k >= 1 and at most the number of keys): the largest value whose
// count of keys at or above it is at least k, built one bit at a time from
// the top.
template <int NP>
__device__ __forceinline__ uint32_t kth_largest_key(const uint32_t (&key)[NP], int k) {
  uint32_t thr = 0u;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = thr | (1u << b);
    int n = 0;
#pragma unroll
    for (int i = 0; i < NP; ++i) n += wave_count(key[i] >= c);
    if (n >= k) thr = c;
  }
  return thr;
}

// Radix select of the k largest of NP planes of keys (entry i of lane l has
// key key[i] and expert eid(i, l); planes and lanes in ascending expert
// order): a radix select finds the k-th largest key, and among entries tied
// at it the lowest experts are taken.  The k chosen are compacted in expert
// order into the wave's list (ck, ce); lane j < k then ranks entry j by
// (key desc, expert asc) against the other k - 1 and sets slot_id[rank].
template <int NP, typename EidOf>
__device__ __forceinline__ void select_rank(const uint32_t (&key)[NP], EidOf eid, int k, int lane,
                                            uint32_t* ck, int* ce, int* slot_id) {
  const uint32_t thr = kth_largest_key<NP>(key, k);
  int above = 0;
#pragma unroll
  for (int i = 0; i < NP; ++i) above += wave_count(key[i] > thr);
  const uint64_t below_me = (1ull << lane) - 1ull;
  int eq_before = 0, base = 0;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const uint64_t eq = __ballot(key[i] == thr);
    const int r = eq_before + __popcll(eq & below_me);
    const bool take = key[i] > thr || (key[i] == thr && r < k - above);
    eq_before += __popcll(eq);
    const uint64_t tm = __ballot(take);
    if (take) {
      const int pos = base + __popcll(tm & below_me);
      ck[pos] = key[i];
      ce[pos] = eid(i, lane);
    }
    base += __popcll(tm);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const uint32_t kj = lane < k ? ck[lane] : 0u;
  const int ej = lane < k ? ce[lane] : 0;
  int rank = 0;
  for (int i = 0; i < k; ++i) {
    const uint32_t k2 = (uint32_t)__builtin_amdgcn_readlane((int)kj, i);
    const int e2 = __builtin_amdgcn_readlane(ej, i);
    rank += (k2 > kj || (k2 == kj && e2 < ej)) ? 1 : 0;
  }
  if (lane < k) slot_id[rank] = ej;
}

// The k largest of NP planes of keys (entry i of lane l is expert l + 64 i),
// taken one at a time in rank order: round r finds the wave's largest
// remaining key (lowest expert among equal keys) and sets slot_id[r].  Every
// round is a wave maximum by row moves plus one ballot per plane: k rounds of
// mostly vector work, against the 32 scalar-bound rounds of a bitwise radix
// select plus a ranking pass (the scalar unit is the CU's, shared by the
// block's waves when every wave selects a token at once).  Taken entries drop
// to key 0 and stay out of later ties through the per-plane taken masks.
constexpr int kExtractMaxK = 16;
constexpr int kDeptRankMax = 32;  // departments ranked by a per-lane count at most
template <int NP>
__device__ __forceinline__ int extract_positions(uint32_t (&key)[NP], int k, int lane) {
  uint64_t taken[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) taken[i] = 0ull;
  int my_id = 0;
  for (int r = 0; r < k; ++r) {
    uint32_t lb = key[0];
#pragma unroll
    for (int i = 1; i < NP; ++i) lb = key[i] > lb ? key[i] : lb;
    const uint32_t M = wave_max_u32(lb);
    int pi = -1, pl = 0;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const uint64_t eq = __ballot(key[i] == M) & ~taken[i];
      if (pi < 0 && eq != 0ull) {
        pi = i;
        pl = __builtin_ctzll(eq);
      }
    }
    pi = __builtin_amdgcn_readfirstlane(pi);
    pl = __builtin_amdgcn_readfirstlane(pl);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (i == pi) {
        taken[i] |= 1ull << pl;
        key[i] = lane == pl ? 0u : key[i];
      }
    }
    my_id = lane == r ? pl + kWave * pi : my_id;
  }
  return my_id;
}
template <int NP>
__device__ __forceinline__ void select_extract(uint32_t (&key)[NP], int k, int lane,
                                               int* slot_id) {
  const int my_id = extract_positions<NP>(key, k, lane);
  if (lane < k) slot_id[lane] = my_id;
}

// The k-th largest of the wave's 64 keys (one per lane; k <= 64), by k
// rounds of a wave maximum that each retire one lane holding it.
__device__ __forceinline__ uint32_t kth_largest_extract(uint32_t v, int k, int lane) {
  uint32_t M = 0u;
  for (int r = 0; r < k; ++r) {
    M = wave_max_u32(v);
    const int l0 = __builtin_ctzll(__ballot(v == M));
    v = lane == l0 ? 0u : v;
  }
  return M;
}

// Top-k of token t by one wave from the staged row `row` (lane l holds experts
// l, l+64, ...).  With 8 or more planes: every key among the k largest, ties
// at the k-th included, is at least the k-th largest of the 64 lane maxima;
// those candidates (few for real scores) are compacted in expert order and
// selected on two planes.  With fewer planes, more candidates than fit, or
// fewer than k, the select runs on all planes.  The chosen experts are handed to lanes 0..k-1 through LDS, then the
// weights.
// `key` holds the row's keys on entry (lane l, plane i: expert l + 64 i; 0
// past the last expert); the logits are read from the staged row.
template <int NPL, bool GROUPED, bool TALLY = true>
__device__ void topk_token(const RouteArgs& p, int t, int row, int lane, PlanShared& s,
                           uint32_t (&key)[NPL]) {
  const int k = p.k, E = p.E, wid = threadIdx.x >> 6;
  const float* lgr = s.tk.lg + row;
  // department of expert e = floor((e + 0.5) / G) in fp32: exact, since
  // e < 2048 and the quotient is below m <= 64, so the rounding error
  // (under 64 * 2^-23) stays inside the 0.5 / G margin to each integer
  const float inv_g = GROUPED ? 1.0f / (float)(E / p.m) : 0.f;
  auto dept_of = [&](int e) { return (unsigned)(((float)e + 0.5f) * inv_g); };
  unsigned* dm = s.tk.dmax[wid];
  uint32_t dkey = 0u;           // lane J: department J's key
  uint64_t chosen_depts = 0ull; // bit J: department J chosen
  if (GROUPED) {
    // Department-limited top-k: a department's key is its best expert's key
    // (LDS max, one area per wave); the k_dept best departments are chosen
    // like experts (lane J holds department J; ties to the lower index) and
    // the experts of every other department drop to key 0, below every real
    // score.
    const int kd = p.k_dept;
    {
      // department-major read of the staged keys: L = 64/m lanes (rounded
      // down to a power of two) stride through each department's G keys,
      // then a max over the L lanes; lane J takes department J's result
      const int G = E / p.m, L = 1 << (31 - __builtin_clz(kWave / p.m));
      const int J = lane / L, sub = lane - J * L;
      uint32_t v = 0u;
      if (J < p.m)
        for (int e = J * G + sub; e < (J + 1) * G; e += L) {
          const uint32_t u = s.tk.key[row + e];
          v = u > v ? u : v;
        }
      for (int o = 1; o < L; o <<= 1) {
        const uint32_t u = (uint32_t)__shfl_xor((int)v, o, kWave);
        v = u > v ? u : v;
      }
      dkey = (uint32_t)__shfl((int)v, min(lane, p.m - 1) * L, kWave);
      dkey = lane < p.m ? dkey : 0u;
    }
    bool dtake;
    if (p.m <= kDeptRankMax) {
      // few departments: each lane counts the departments ranked above its
      // own (key desc, index asc) -- m vector steps instead of 32 rounds of
      // a bitwise select
      int above = 0;
      for (int j = 0; j < p.m; ++j) {
        const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)dkey, j);
        above += (kj > dkey || (kj == dkey && j < lane)) ? 1 : 0;
      }
      dtake = lane < p.m && above < kd;
    } else {
      const uint32_t dkeys[1] = {dkey};
      const uint32_t dthr = kth_largest_key<1>(dkeys, kd);
      const int dabove = wave_count(dkey > dthr);
      const uint64_t deq = __ballot(lane < p.m && dkey == dthr);
      dtake = lane < p.m && (dkey > dthr ||
                             (dkey == dthr && __popcll(deq & ((1ull << lane) - 1ull)) <
                                                  kd - dabove));
    }
    chosen_depts = __ballot(dtake);
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + kWave * i;
      if (e < E && !((chosen_depts >> dept_of(e)) & 1ull)) key[i] = 0u;
    }
  }
  // candidate cut (8 or more planes; with fewer a direct select is
  // cheaper): the k-th largest lane maximum, at least 1 so that key-0
  // entries never qualify; k rounds of a wave maximum for k <= kExtractMaxK,
  // else a bitwise select
  int n_cand = 0;
  uint32_t cut = 1u;
  if constexpr (NPL >= 8) {
    uint32_t lmax[1] = {0u};
#pragma unroll
    for (int i = 0; i < NPL; ++i) lmax[0] = key[i] > lmax[0] ? key[i] : lmax[0];
    const uint32_t c0 =
        k <= kExtractMaxK ? kth_largest_extract(lmax[0], k, lane) : kth_largest_key<1>(lmax, k);
    cut = c0 > 1u ? c0 : 1u;
#pragma unroll
    for (int i = 0; i < NPL; ++i) n_cand += wave_count(key[i] >= cut);
  }
  const uint64_t below_me = (1ull << lane) - 1ull;
  int* slot_id = s.ids + t * k;
  float* slot_aux = s.w + t * k;
  if (NPL >= 8 && n_cand >= k && n_cand <= kCand) {
    uint32_t* ck = s.tk.cand_key[wid];
    int* ce = s.tk.cand_e[wid];
    int base = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const bool c = key[i] >= cut;
      const uint64_t bm = __ballot(c);
      if (c) {
        const int pos = base + __popcll(bm & below_me);
        ck[pos] = key[i];
        ce[pos] = lane + kWave * i;
      }
      base += __popcll(bm);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    constexpr int NC = kCand / kWave;
    uint32_t ckey[NC];
    int cexp[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int pos = lane + kWave * i;
      ckey[i] = pos < n_cand ? ck[pos] : 0u;
      cexp[i] = pos < n_cand ? ce[pos] : 0;
    }
    // the list is rewritten with the chosen only after every lane has read it
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (k <= kExtractMaxK) {
      // candidates are in expert order, so the lowest position among equal
      // keys is the lowest expert
      const int pos = extract_positions<NC>(ckey, k, lane);
      if (lane < k) slot_id[lane] = ce[pos];
    } else {
      select_rank<NC>(ckey, [&](int i, int) { return cexp[i]; }, k, lane, ck, ce, slot_id);
    }
  } else if (NPL <= 4 && k <= kExtractMaxK) {
    select_extract<NPL>(key, k, lane, slot_id);
  } else {
    select_rank<NPL>(key, [](int i, int l) { return l + kWave * i; }, k, lane,
                     s.tk.cand_key[wid], s.tk.cand_e[wid], slot_id);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  int my_id = -1;
  float my_aux = 0.f;
  if (lane < k) {
    my_id = slot_id[lane];
    my_aux = route_aux(p, lgr[my_id]);
  }
  if (GROUPED && p.strict) {
    // Strict department coverage: while the k chosen experts (lane j holds
    // rank j) span fewer than k_dept departments, the lowest-ranked one
    // whose department keeps another chosen expert leaves and the best
    // expert of the best uncovered department enters.  Uncovered departments
    // are all among the chosen ones, and an entering expert ranks below
    // every kept one and below those entering before it, so the new order
    // is the kept experts in rank order followed by the entering ones.
    const unsigned my_dept = lane < k ? dept_of(my_id) : 0u;
    if (lane < p.m) dm[lane] = 0u;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (lane < k) atomicAdd(&dm[my_dept], 1u);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    int cnt = lane < k ? (int)dm[my_dept] : 0;  // chosen experts in my department
    uint64_t uncov = chosen_depts & ~__ballot(lane < p.m && dm[lane] > 0u);
    const int n_in = __popcll(uncov);
    if (n_in > 0) {
      bool removed = false;
      int in_id = -1;
      float in_aux = 0.f;
      for (int it = 0; it < n_in; ++it) {
        // best uncovered department: largest key, then lowest index
        const bool cand = (uncov >> lane) & 1ull;
        const uint32_t best = wave_max_u32(cand ? dkey : 0u);
        const int u = __builtin_ctzll(__ballot(cand && dkey == best));
        // its best expert: the lowest index holding the department's key
        int e_in = -1;
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
          const int e = lane + kWave * i;
          const uint64_t b = __ballot(e < E && dept_of(e) == (unsigned)u && key[i] == best);
          if (e_in < 0 && b) e_in = __builtin_ctzll(b) + kWave * i;
        }
        const uint64_t elig = __ballot(lane < k && !removed && cnt >= 2);
        if (e_in < 0 || !elig) break;  // neither happens when k >= k_dept
        const int r = 63 - __builtin_clzll(elig);
        const unsigned dr = (unsigned)__builtin_amdgcn_readlane((int)my_dept, r);
        if (lane < k && !removed && my_dept == dr) --cnt;
        if (lane == r) removed = true;
        if (lane == it) {
          in_id = e_in;
          in_aux = route_aux(p, lgr[e_in]);
        }
        uncov &= ~(1ull << u);
      }
      const uint64_t rem = __ballot(lane < k && removed);
      const int n_rem = __popcll(rem);
      if (lane < k && !removed) {
        const int j = lane - __popcll(rem & below_me);
        slot_id[j] = my_id;
        slot_aux[j] = my_aux;
      }
      if (lane < n_rem) {
        slot_id[k - n_rem + lane] = in_id;
        slot_aux[k - n_rem + lane] = in_aux;
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      if (lane < k) {
        my_id = slot_id[lane];
        my_aux = slot_aux[lane];
      }
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
    w = ex / wave_sum(ex);
  } else {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (lane + kWave * i < E) mx = fmaxf(mx, lgr[lane + kWave * i]);
    mx = wave_max(mx);
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (lane + kWave * i < E) z += expf(lgr[lane + kWave * i] - mx);
    w = expf(my_aux - mx) / wave_sum(z);
  }
  w *= p.scale;
  if (mine) {
    const int a = t * p.k + lane;
    if (p.ids_out) p.ids_out[a] = my_id;
    if (p.w_out) p.w_out[a] = w;
    if constexpr (TALLY) {
      s.ids[a] = my_id;
      s.w[a] = w;
      // the plan's tallies (the k experts of a token are distinct)
      atomicAdd(&s.cnt[my_id], 1);
      const int nwt = rank_mask_words(p.T, E);
      if (nwt > 0) atomicOr(&s.tmask[my_id * nwt + (t >> 6)], 1ull << (t & 63));
      if (p.m > 0) {
        const int J = my_id / (E / p.m);
        s.flag[t * p.m + J] = 1;
        if (dept_masks(p.T, p.m)) atomicOr(&s.dtok[J][t >> 6], 1ull << (t & 63));
      }
    }
  }
}

// Work descriptor of occupied entry e: compacted small list at work[slot],
// large list at work[cap + slot].
__device__ __forceinline__ WorkDesc* work_of(WorkDesc* work, int cap, int c, int slot) {
  return work + (c <= kTokInline ? slot : cap + slot);
}

// Departments, by one wave: pairs per department (from the pair flags),
// offsets, the ascending list of active departments, each one's index in the
// compacted list of small (<= kTokInline pairs) or of large groups, work
// descriptors and header totals.
__device__ void dept_scan(PlanShared& s, const PlanArgs& pa, int lane) {
  const int m = pa.m, T = pa.T;
  const moe_plan& P = pa.plan;
  const int per = (m + kWave - 1) / kWave;
  const int b = min(m, lane * per), en = min(m, b + per);
  int sc = 0, sa = 0, ss = 0;
  for (int J = b; J < en; ++J) {
    int c = 0;
    if (dept_masks(T, m))
      for (int q = 0; q < ((T + 63) >> 6); ++q) c += __popcll(s.dtok[J][q]);
    else
      for (int t = 0; t < T; ++t) c += s.flag[t * m + J];
    s.pw.dcnt[J] = c;
    sc += c;
    sa += c > 0 ? 1 : 0;
    ss += (c > 0 && c <= kTokInline) ? 1 : 0;
  }
  const int ic = wave_incl_scan(sc, lane), ia = wave_incl_scan(sa, lane),
            is = wave_incl_scan(ss, lane);
  int rc = ic - sc, ra = ia - sa, rs = is - ss, rl = (ia - sa) - (is - ss);
  for (int J = b; J < en; ++J) {
    const int c = s.pw.dcnt[J];
    s.pw.doff[J] = rc;
    P.dept_offsets[J] = rc;
    P.dept_counts[J] = c;
    if (c > 0) {
      P.active_depts[ra++] = J;
      const int sl = c <= kTokInline ? rs++ : rl++;
      s.pw.dslot[J] = sl;
      WorkDesc* wd = work_of(pa.dwork, m, c, sl);
      wd->mat = J;
      wd->r0 = rc;
      wd->n = c;
    }
    rc += c;
  }
  if (lane == kWave - 1) {
    P.dept_offsets[m] = ic;
    P.header[MOE_PLAN_N_DEPT_ROWS] = ic;
    P.header[MOE_PLAN_N_ACTIVE_DEPTS] = ia;
    P.header[kHdrDeptSmall] = is;
    P.header[kHdrDeptLarge] = ia - is;
  }
}

// Rank of token t's pair among department J's pairs (its lower tokens that
// chose one of J's experts).
__device__ __forceinline__ int pair_rank(const PlanShared& s, int T, int m, int t, int J) {
  if (dept_masks(T, m)) return bits_below(s.dtok[J], t);
  int r = 0;
  for (int u = 0; u < t; ++u) r += s.flag[u * m + J];
  return r;
}

// (token, department) pairs p = i0, i0 + stride, ...: department J is active
// for token t when t selected at least one of its experts; c_{t,J} sums those
// weights.  Needs the department offsets and slots of dept_scan.
__device__ void write_pairs(const PlanShared& s, const PlanArgs& pa, int i0, int stride) {
  const int T = pa.T, k = pa.k, E = pa.E, m = pa.m, G = E / m;
  const moe_plan& P = pa.plan;
  for (int p = i0; p < T * m; p += stride) {
    const int t = p / m, J = p - t * m;
    if (s.flag[p]) {
      const int rank = pair_rank(s, T, m, t, J);
      const int q = s.pw.doff[J] + rank;
      // the token's slots eight at a time: their ids and weights are read
      // together, then added in slot order (department J holds experts
      // [J G, J G + G))
      const int e0 = J * G;
      float sc2 = 0.f;
      for (int j0 = 0; j0 < k; j0 += 8) {
        int ev[8];
        float wv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int a = t * k + min(j0 + j, k - 1);
          ev[j] = s.ids[a];
          wv[j] = s.w[a];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j0 + j < k && ev[j] >= e0 && ev[j] < e0 + G && ev[j] < E) sc2 += wv[j];
      }
      P.dept_row_token[q] = t;
      P.dept_row_dept[q] = J;
      P.dept_row_scale[q] = sc2;
      P.dept_inv[p] = q;
      if (s.pw.dcnt[J] <= kTokInline) pa.dwork[s.pw.dslot[J]].tok[rank] = t;
    } else {
      P.dept_inv[p] = -1;
    }
  }
}

// The dispatch plan from s.ids / s.w (T*k assignments), s.cnt (rows per
// expert) and s.flag (pairs present).  Whole block, two barriers: a scan of
// the expert counts by at most kScanWaves waves (contiguous entries per lane,
// wave scans, wave totals through LDS) while the last wave scans the
// departments; then every assignment and every pair writes its row.  Waves
// with no entries stay out of the scan: cross-lane steps of idle waves would
// only queue on the LDS crossbar.  nwt > 0: tm holds the token bits of every
// expert, nwt words each (the tallies filled them; a token's k experts are
// distinct).
constexpr int kScanWaves = 4;
__device__ void plan_phase(PlanShared& s, const PlanArgs& pa, const unsigned long long* tm,
                           int nwt) {
  const int tid = threadIdx.x, nth = blockDim.x, lane = tid & 63, wid = tid >> 6;
  const int nw = nth >> 6;
  const int T = pa.T, k = pa.k, E = pa.E, A = T * k, m = pa.m;
  const moe_plan& P = pa.plan;
  const int per = max(1, (E + kScanWaves * kWave - 1) / (kScanWaves * kWave));
  const int nsw = (E + kWave * per - 1) / (kWave * per);  // scanning waves, <= kScanWaves
  const int b = min(E, tid * per), en = min(E, b + per);
  int sc = 0, sa = 0, ss = 0, ic = 0, ia = 0, is = 0;
  if (wid < nsw) {
    for (int e = b; e < en; ++e) {
      const int c = s.cnt[e];
      sc += c;
      sa += c > 0 ? 1 : 0;
      ss += (c > 0 && c <= kTokInline) ? 1 : 0;
    }
    ic = wave_incl_scan(sc, lane);
    ia = wave_incl_scan(sa, lane);
    is = wave_incl_scan(ss, lane);
    if (lane == kWave - 1) {
      s.pw.tot[wid][0] = ic;
      s.pw.tot[wid][1] = ia;
      s.pw.tot[wid][2] = is;
    }
  }
  if (m > 0 && wid == nw - 1) dept_scan(s, pa, lane);  // nw - 1 >= kScanWaves
  __syncthreads();
  if (tid == 0) {
    int gc = 0, gac = 0, gsc = 0;
    for (int w2 = 0; w2 < nsw; ++w2) {
      gc += s.pw.tot[w2][0];
      gac += s.pw.tot[w2][1];
      gsc += s.pw.tot[w2][2];
    }
    P.offsets[E] = gc;
    P.header[MOE_PLAN_N_ROWS] = gc;
    P.header[MOE_PLAN_N_ACTIVE] = gac;
    P.header[kHdrSmall] = gsc;
    P.header[kHdrLarge] = gac - gsc;
    P.header[MOE_PLAN_N_INVALID] = s.invalid;
    if (m <= 0) {
      P.header[MOE_PLAN_N_DEPT_ROWS] = 0;
      P.header[MOE_PLAN_N_ACTIVE_DEPTS] = 0;
      P.header[kHdrDeptSmall] = 0;
      P.header[kHdrDeptLarge] = 0;
    }
  }
  int pc = 0, pac = 0, psc = 0;  // totals of the scanning waves before mine
  for (int w2 = 0; w2 < wid && w2 < nsw; ++w2) {
    pc += s.pw.tot[w2][0];
    pac += s.pw.tot[w2][1];
    psc += s.pw.tot[w2][2];
  }
  int rc = pc + ic - sc, ra = pac + ia - sa, rs = psc + is - ss;
  int rl = ra - rs;  // large groups before mine: active minus small
  for (int e = b; e < en && wid < nsw; ++e) {
    const int c = s.cnt[e];
    s.pw.off[e] = rc;
    P.offsets[e] = rc;
    P.counts[e] = c;
    if (c > 0) {
      P.active[ra++] = e;
      const int sl = c <= kTokInline ? rs++ : rl++;
      s.pw.slot[e] = sl;
      WorkDesc* wd = work_of(pa.work, E, c, sl);
      wd->mat = e;
      wd->r0 = rc;
      wd->n = c;
    }
    rc += c;
  }
  __syncthreads();
  const int G = m > 0 ? E / m : 1;
  // row of assignment a = offset of its expert + earlier assignments to it;
  // in the factorised form a row's inputs are its (token, department) pair's
  // backbone outputs, so the pair index goes to row_pair and to the inline
  // entries of small groups
  for (int a = tid; a < A; a += nth) {
    const int e = s.ids[a];
    if (e >= 0 && e < E) {
      const int t = a / k;
      int rank = 0;
      if (nwt > 0) {
        // the earlier assignments to e are those of the lower tokens that chose it
        rank = bits_below(tm + e * nwt, t);
      } else {
        for (int b2 = 0; b2 < a; ++b2) rank += (s.ids[b2] == e) ? 1 : 0;
      }
      const int row = s.pw.off[e] + rank;
      P.row_token[row] = t;
      P.row_slot[row] = a - t * k;
      P.row_expert[row] = e;
      P.row_weight[row] = s.w[a];
      P.inv_perm[a] = row;
      int in = t;
      if (pa.factorised) {
        const int J = e / G;
        in = s.pw.doff[J] + pair_rank(s, T, m, t, J);
        P.row_pair[row] = in;
      }
      if (s.cnt[e] <= kTokInline) pa.work[s.pw.slot[e]].tok[rank] = in;
    } else {
      P.inv_perm[a] = -1;
    }
  }
  if (m > 0) write_pairs(s, pa, tid, nth);
}

// The plan by one wave, for at most 4 * 64 experts with the token bits of
// every expert in tm (nwt words each) and, in the department form, the token bits of
// every department in s.dtok: lane l takes the experts [l * per, (l + 1) *
// per), one wave scan of the counts gives their first rows and list slots
// (dept_scan does the same for the departments), and the same wave then
// writes every assignment's row and every pair's.  The lanes exchange
// offsets and slots through LDS inside the wave: no block barrier anywhere.
constexpr int kWavePlanPer = 4;  // experts per lane at most
constexpr int kWavePlanMaxA = 512;  // assignments the one-wave plan writes at most
// With departments only a lane's worth of assignments and of pairs: past it
// the block-wide plan measured faster (DeaMoE-7B-shaped top-k + plan at one
// token 7.9 -> 7.2 us with the wave, at 16 tokens 8.0 -> 9.4 us)
constexpr int kWavePlanMaxDeptA = kWave;
__device__ __forceinline__ bool wave_plan_fits(int T, int E, int k, int m, int nwt) {
  return E <= kWavePlanPer * kWave && nwt > 0 &&
         (m <= 0 ? T * k <= kWavePlanMaxA
                 : dept_masks(T, m) && T * k <= kWavePlanMaxDeptA && T * m <= kWavePlanMaxDeptA);
}
__device__ void plan_phase_wave(PlanShared& s, const PlanArgs& pa, int lane,
                                const unsigned long long* tm, int nwt) {
  const int T = pa.T, k = pa.k, E = pa.E, A = T * k, m = pa.m;
  const moe_plan& P = pa.plan;
  const int per = (E + kWave - 1) / kWave;
  const int b = min(E, lane * per), en = min(E, b + per);
  int c[kWavePlanPer];
  int sc = 0, sa = 0, ss = 0;
#pragma unroll
  for (int j = 0; j < kWavePlanPer; ++j) {
    c[j] = b + j < en ? s.cnt[b + j] : 0;
    sc += c[j];
    sa += c[j] > 0 ? 1 : 0;
    ss += (c[j] > 0 && c[j] <= kTokInline) ? 1 : 0;
  }
  const int ic = wave_incl_scan(sc, lane), ia = wave_incl_scan(sa, lane),
            is = wave_incl_scan(ss, lane);
  int rc = ic - sc, ra = ia - sa, rs = is - ss;
  int rl = ra - rs;  // large groups before mine: active minus small
#pragma unroll
  for (int j = 0; j < kWavePlanPer; ++j) {
    const int e = b + j;
    if (e < en) {
      s.pw.off[e] = rc;
      P.offsets[e] = rc;
      P.counts[e] = c[j];
      if (c[j] > 0) {
        P.active[ra++] = e;
        const int sl = c[j] <= kTokInline ? rs++ : rl++;
        s.pw.slot[e] = sl;
        WorkDesc* wd = work_of(pa.work, E, c[j], sl);
        wd->mat = e;
        wd->r0 = rc;
        wd->n = c[j];
      }
      rc += c[j];
    }
  }
  if (lane == kWave - 1) {
    P.offsets[E] = ic;
    P.header[MOE_PLAN_N_ROWS] = ic;
    P.header[MOE_PLAN_N_ACTIVE] = ia;
    P.header[kHdrSmall] = is;
    P.header[kHdrLarge] = ia - is;
    P.header[MOE_PLAN_N_INVALID] = s.invalid;
    if (m <= 0) {
      P.header[MOE_PLAN_N_DEPT_ROWS] = 0;
      P.header[MOE_PLAN_N_ACTIVE_DEPTS] = 0;
      P.header[kHdrDeptSmall] = 0;
      P.header[kHdrDeptLarge] = 0;
    }
  }
  if (m > 0) dept_scan(s, pa, lane);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const int G = m > 0 ? E / m : 1;
  for (int a = lane; a < A; a += kWave) {
    const int e = s.ids[a];
    if (e >= 0 && e < E) {
      const int t = a / k;
      // the earlier assignments to e are those of the lower tokens that chose it
      const int rank = bits_below(tm + e * nwt, t);
      const int row = s.pw.off[e] + rank;
      P.row_token[row] = t;
      P.row_slot[row] = a - t * k;
      P.row_expert[row] = e;
      P.row_weight[row] = s.w[a];
      P.inv_perm[a] = row;
      int in = t;
      if (pa.factorised) {
        const int J = e / G;
        in = s.pw.doff[J] + pair_rank(s, T, m, t, J);
        P.row_pair[row] = in;
      }
      if (s.cnt[e] <= kTokInline) pa.work[s.pw.slot[e]].tok[rank] = in;
    } else {
      P.inv_perm[a] = -1;
    }
  }
  if (m > 0) write_pairs(s, pa, lane, kWave);
}

// Routing statistics of the step (DeepSeekMoE Guide, "Sequence-Level and
// Batch-Level Expert Routing Balance Metrics": the load balance factor is
// the largest expert's token count over the mean count of the E routed
// experts), by one wave from the plan's LDS tallies: rows per expert, and in
// the department form the pair counts per department.  Both are final once
// the plan phase has passed its barriers, and neither is written after them.
__device__ void write_stats(const PlanShared& s, const PlanArgs& pa, int lane) {
  moe_step_stats* st = pa.stats;
  const int E = pa.E;
  int rows = 0, act = 0, mx = 0, adep = 0;
  for (int e = lane; e < E; e += kWave) {
    const int c = s.cnt[e];
    st->expert_rows[e] = c;
    rows += c;
    act += c > 0 ? 1 : 0;
    mx = c > mx ? c : mx;
  }
  for (int J = lane; J < pa.m; J += kWave) adep += s.pw.dcnt[J] > 0 ? 1 : 0;
  auto add = [](int a, int b) { return a + b; };
  rows = wave_reduce_i(rows, add);
  act = wave_reduce_i(act, add);
  adep = wave_reduce_i(adep, add);
  mx = wave_reduce_i(mx, [](int a, int b) { return a > b ? a : b; });
  if (lane == 0) {
    const float mean = (float)rows / (float)E;
    st->n_tokens = pa.T;
    st->n_assignments = rows;
    st->n_active_experts = act;
    st->n_active_depts = adep;
    st->max_expert_rows = mx;
    st->n_invalid = s.invalid;
    st->mean_expert_rows = mean;
    st->imbalance_ratio = rows > 0 ? (float)mx / mean : 0.f;
    st->loaded_weight_bytes =
        pa.bytes_fixed + (unsigned long long)act * pa.bytes_expert +
        (unsigned long long)adep * pa.bytes_dept;
  }
}

// Per-launch clearing of the plan's LDS tallies (before any top-k or count).
__device__ __forceinline__ void plan_clear(PlanShared& s, int T, int E, int m,
                                           unsigned long long* tm, int nwt) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) s.cnt[e] = 0;
  for (int i = threadIdx.x; i < nwt * E; i += blockDim.x) tm[i] = 0ull;
  for (int p = threadIdx.x; p < T * (m > 0 ? m : 0); p += blockDim.x) s.flag[p] = 0;
  if (dept_masks(T, m))
    for (int i = threadIdx.x; i < m * kDeptMaskWords; i += blockDim.x)
      s.dtok[i / kDeptMaskWords][i % kDeptMaskWords] = 0ull;
  if (threadIdx.x == 0) s.invalid = 0;
}

// Router logits l[t][e] = x_t . W_r[e].  A block owns EB experts; its four
// waves split d (wave w takes the 512-wide chunks w, w+4, ...), each wave
// reduces over its lanes, and the four wave sums are added in wave order.  The
// summation order depends only on the token's position in its group of 8,
// never on the expert, so equal router rows give bitwise-equal logits.
template <typename T_, int EB>
__global__ __launch_bounds__(kThreads) void route_kernel(RouteArgs ra) {
  __shared__ float part[kWaves][EB * 8];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int e0 = blockIdx.x * EB;
  const T_* x = static_cast<const T_*>(ra.x);
  const T_* wr = static_cast<const T_*>(ra.wr);
  constexpr int N = EB * 8;
  constexpr int SH = 6 - Log2<N>::value;
  for (int t0 = 0; t0 < ra.T; t0 += 8) {
    const int nv = min(8, ra.T - t0);
    float acc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.f;
    for (int c = wid; c < ra.n_chunks; c += kWaves) {
      const int col = c * kRouteChunk + lane * 8;
      if (col < ra.d) {
        Raw8<T_> w[EB];
#pragma unroll
        for (int eb = 0; eb < EB; ++eb) {
          if (e0 + eb < ra.E)
            w[eb].load(wr + (size_t)(e0 + eb) * ra.d + col);
          else
            w[eb].zero();
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (j < nv) {
            X8<T_> xv;
            xv.load(x + (size_t)(t0 + j) * ra.d + col);
#pragma unroll
            for (int eb = 0; eb < EB; ++eb) acc[eb * 8 + j] = dot8(w[eb], xv, acc[eb * 8 + j]);
          }
        }
      }
    }
    group_reduce_scatter<N, 64>(acc, lane);
    if ((lane & ((1 << SH) - 1)) == 0) part[wid][lane >> SH] = acc[0];
    __syncthreads();
    if (wid == 0 && lane < N) {
      const int eb = lane >> 3, j = lane & 7;
      if (e0 + eb < ra.E && j < nv)
        ra.logits[(size_t)(t0 + j) * ra.E + e0 + eb] =
            ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
    }
    __syncthreads();
  }
}

// Router logits on the matrix cores (bf16): block (x, y) owns experts
// 16x .. 16x+15 and K piece y of ksplit; its four waves split that piece
// again, each accumulating 16 experts x 16 tokens per 16x16x32 step for up to
// NCT token tiles, two K-steps of loads ahead.  The four wave tiles are added
// in wave order through LDS and written as partial plane y; the top-k adds the
// planes in order.  Every expert sees the same summation order, so equal
// router rows give bitwise-equal logits.
template <int NCT>
__global__ __launch_bounds__(kThreads) void route_mfma_kernel(RouteArgs ra) {
  constexpr int kAhead = 2;
  __shared__ f32x4_t part[kWaves][NCT][kWave];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int e0 = blockIdx.x * 16, d = ra.d, T = ra.T, E = ra.E;
  const int pieces = ra.ksplit * kWaves;
  const int kq = ((d + pieces * 32 - 1) / (pieces * 32)) * 32;
  const int kb = min(d, (blockIdx.y * kWaves + wid) * kq), ke = min(d, kb + kq);
  const bf16_t* xw = static_cast<const bf16_t*>(ra.x);
  const bf16_t* ap = static_cast<const bf16_t*>(ra.wr) + (size_t)min(e0 + r16, E - 1) * d + g * 8;
  float* out = ra.logits + (size_t)blockIdx.y * T * E;
  const u32x4_t z = {0, 0, 0, 0};
  for (int t0 = 0; t0 < T; t0 += 16 * NCT) {
    const bf16_t* bp[NCT];
    bool bv[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const int t = t0 + c * 16 + r16;
      bv[c] = t < T;
      bp[c] = xw + (size_t)(bv[c] ? t : 0) * d + g * 8;
    }
    f32x4_t acc[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    u32x4_t ra_[kAhead + 1], rb[kAhead + 1][NCT];
#pragma unroll
    for (int q = 0; q < kAhead; ++q) {
      const int k = kb + q * 32;
      const bool in = k + g * 8 < ke;
      ra_[q] = in ? ld16(ap + k) : z;
#pragma unroll
      for (int c = 0; c < NCT; ++c) rb[q][c] = (bv[c] && in) ? ld16(bp[c] + k) : z;
    }
    for (int k = kb; k < ke; k += 32 * (kAhead + 1)) {
#pragma unroll
      for (int q = 0; q <= kAhead; ++q) {
        const int kn = k + (q + kAhead) * 32;
        const int qn = (q + kAhead) % (kAhead + 1);
        const bool nin = kn + g * 8 < ke;
        ra_[qn] = nin ? ld16(ap + kn) : z;
#pragma unroll
        for (int c = 0; c < NCT; ++c) rb[qn][c] = (bv[c] && nin) ? ld16(bp[c] + kn) : z;
        if (k + q * 32 < ke) {
#pragma unroll
          for (int c = 0; c < NCT; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ra_[q]), as_bf16x8(rb[q][c]),
                                                             acc[c], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < NCT; ++c) part[wid][c][lane] = acc[c];
    __syncthreads();
    if (wid == 0) {
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        f32x4_t sum = part[0][c][lane];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) sum += part[w][c][lane];
        const int t = t0 + c * 16 + r16;
        if (t < T) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = e0 + 4 * g + i;
            if (e < E) out[(size_t)t * E + e] = sum[i];
          }
        }
      }
    }
    __syncthreads();
  }
}

// One block for batches of at most one token per wave and at most 256
// experts: each wave selects its token's top-k, then (do_plan) the block
// builds the dispatch plan from the LDS tallies.
template <int NPL, bool GROUPED>
__global__ __launch_bounds__(kPlanThreads) void topk_plan_kernel(RouteArgs ra, PlanArgs pa,
                                                                 int do_plan) {
  __shared__ PlanShared s;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nwt = rank_mask_words(ra.T, ra.E);
  plan_clear(s, ra.T, ra.E, ra.m, s.tmask, nwt);
  // up to 256 experts and one token per wave: each wave stages its own token
  // in its own row, its logits requested before the barrier that completes
  // the clearing (the staged row is not a tally)
  static_assert(NPL <= 4 && kPlanWaves * 4 * kWave <= kTopkBuf, "a row per wave");
  uint32_t key[NPL];
  if (wid < ra.T) stage_token<NPL, GROUPED>(ra, wid, wid * ra.E, lane, s, key);
  __syncthreads();  // the tallies are clear
  if (wid < ra.T) topk_token<NPL, GROUPED>(ra, wid, wid * ra.E, lane, s, key);
  if (!do_plan) return;
  __syncthreads();
  if (wave_plan_fits(pa.T, pa.E, pa.k, pa.m, nwt)) {
    if (wid == 0) plan_phase_wave(s, pa, lane, s.tmask, nwt);
  } else {
    plan_phase(s, pa, s.tmask, nwt);
  }
  // the tallies the statistics read were final before the plan phase (rows
  // per expert) or inside it, before its last barrier (pairs per department)
  if (pa.stats && wid == 0) write_stats(s, pa, lane);
}

// Top-k of many tokens at once, the ids and weights written to ra.ids_out /
// ra.w_out (and the ranked scores to ra.sel_out).  Serves batches past one
// token per wave of the single plan block, and layers with more than 256
// experts: the tokens then run side by side across the chip and a separate
// plan launch follows.  Up to 256 experts: four tokens per block, each wave
// stages and selects its own.  More experts: one token per block, whose four
// waves stage its row together (each thread a few experts, every partial
// plane requested at once), then one wave selects.
template <int NPL, bool GROUPED>
__global__ __launch_bounds__(kThreads) void topk_token_kernel(RouteArgs ra) {
  __shared__ PlanShared s;  // only the staging rows and the per-wave lists are used
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t key[NPL];
  if constexpr (NPL <= 4) {
    const int t = blockIdx.x * kWaves + wid;
    if (t >= ra.T) return;
    stage_token<NPL, GROUPED>(ra, t, wid * ra.E, lane, s, key);
    topk_token<NPL, GROUPED, false>(ra, t, wid * ra.E, lane, s, key);
  } else {
    const int t = blockIdx.x, E = ra.E;
    constexpr int PER = (NPL * kWave + kThreads - 1) / kThreads;  // experts per thread
    float v[PER][kMaxRouteSplit], b[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u)
      logit_parts(ra, t, min((int)threadIdx.x + u * kThreads, E - 1), v[u], b[u]);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = threadIdx.x + u * kThreads;
      if (e < E) {
        float l = 0.f;
#pragma unroll
        for (int q = 0; q < kMaxRouteSplit; ++q) l += v[u][q];
        const float sc = ra.score_fn == MOE_SCORE_SOFTMAX ? l : route_aux(ra, l) + b[u];
        if (ra.sel_out) ra.sel_out[(size_t)t * E + e] = sc;
        s.tk.lg[e] = l;
        s.tk.key[e] = score_key(sc);
      }
    }
    __syncthreads();
    if (wid != 0) return;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + kWave * i;
      key[i] = e < E ? s.tk.key[e] : 0u;
    }
    topk_token<NPL, GROUPED, false>(ra, t, 0, lane, s, key);
  }
}

// The dispatch plan from caller- or router-given ids and weights.  DISTINCT:
// every id is a valid expert and a token's ids are distinct (the router's
// top-k), so each expert's tokens are kept as bits and an assignment's row
// is a popcount; otherwise ids may repeat within a token or fall outside
// [0, E) (dropped and counted), and ranks come from a scan.
template <bool DISTINCT>
__global__ __launch_bounds__(kPlanThreads) void dispatch_kernel(const int32_t* ids, const float* w,
                                                                PlanArgs pa) {
  __shared__ PlanShared s;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  // no top-k staging here: the expert token bits take its area
  const int nwt = DISTINCT ? rank_mask_words(pa.T, pa.E, kRankMaskWordsBig) : 0;
  plan_clear(s, pa.T, pa.E, pa.m, s.tbig, nwt);
  __syncthreads();
  const int G = pa.m > 0 ? pa.E / pa.m : 1;
  for (int a = threadIdx.x; a < pa.T * pa.k; a += blockDim.x) {
    const int e = ids[a];
    s.ids[a] = e;
    s.w[a] = w[a];
    if (e >= 0 && e < pa.E) {
      const int t = a / pa.k;
      atomicAdd(&s.cnt[e], 1);
      if (nwt > 0) atomicOr(&s.tbig[e * nwt + (t >> 6)], 1ull << (t & 63));
      if (pa.m > 0) {
        s.flag[t * pa.m + e / G] = 1;
        if (dept_masks(pa.T, pa.m)) atomicOr(&s.dtok[e / G][t >> 6], 1ull << (t & 63));
      }
    } else {
      atomicAdd(&s.invalid, 1);
    }
  }
  __syncthreads();
  // (one wave writes every row: past kWavePlanMaxA assignments the block does)
  if (DISTINCT && wave_plan_fits(pa.T, pa.E, pa.k, pa.m, nwt)) {
    if (wid == 0) plan_phase_wave(s, pa, lane, s.tbig, nwt);
  } else {
    plan_phase(s, pa, s.tbig, nwt);
  }
  if (pa.stats && wid == 0) write_stats(s, pa, lane);
}

// ---------------------------------------------------------------------------
// Grouped expert GEMVs.  Every family of matrices is scheduled as two parts
// of one launch: the "small" part serves groups of at most four tokens with a
// register GEMV (most routed experts at decode batch sizes), the "large" part
// serves bigger groups (the shared expert, department backbones, hot experts)
// with 16x16x32 bf16 matrix-core tiles.  A block skips slots of the other part.
// ---------------------------------------------------------------------------
struct Slot {
  int mat, r0, n;
  int t0, t1, t2, t3;      // the first tokens of the group (inline_tok)
  bool inline_tok;
};

// Part of this block (a reference into the kernel-argument block, read with
// scalar loads; copying the part out would force a private stack copy).
__device__ __forceinline__ const Family& block_part(const FamilySet& set, int& tile) {
  const int b = blockIdx.x;
  int fi = 0;
#pragma unroll
  for (int i = 1; i < kMaxParts; ++i)
    if (i < set.n && b >= set.blk_start[i]) fi = i;
  tile = b - set.blk_start[fi];
  return set.f[fi];
}

// Slot and tile of this block in part F; false when the slot is not active,
// does not belong to this part, or its descriptor is out of range (so even a
// plan that was never written cannot send a block outside the weights or the
// row buffers).
__device__ __forceinline__ bool map_slot(const Family& F, int T, Slot& sl, int& tile) {
  const int slot = tile / F.tiles;
  tile -= slot * F.tiles;
  if (F.work) {
    // slot < max_slots keeps the descriptor read inside the work list, so it
    // is read together with the active count (one condition, no short
    // circuit) instead of after it
    static_assert(sizeof(WorkDesc) == 32, "a work descriptor is two 16-byte vectors");
    const int* na_ptr = F.n_active;
    const u32x4_t* wd_ptr = reinterpret_cast<const u32x4_t*>(F.work + slot);
    __asm__ volatile("" ::"s"(na_ptr), "s"(wd_ptr));  // both addresses first
    const int n_active = *na_ptr;
    const u32x4_t w0 = wd_ptr[0], w1 = wd_ptr[1];
    __asm__ volatile("" ::"s"(n_active), "s"(w0), "s"(w1));  // all three loads in flight at once
    WorkDesc wd;
    wd.mat = (int)w0.x;
    wd.r0 = (int)w0.y;
    wd.n = (int)w0.z;
    wd.tok[0] = (int)w0.w;
    wd.tok[1] = (int)w1.x;
    wd.tok[2] = (int)w1.y;
    wd.tok[3] = (int)w1.z;
    const bool ok = (slot < n_active) & (wd.mat >= 0) & (wd.mat < F.n_mats) & (wd.r0 >= 0) &
                    (wd.n <= F.max_rows - wd.r0);
    if (!ok) return false;
    sl.mat = wd.mat;
    sl.r0 = wd.r0;
    sl.n = wd.n;
    sl.t0 = wd.tok[0];
    sl.t1 = wd.tok[1];
    sl.t2 = wd.tok[2];
    sl.t3 = wd.tok[3];
    sl.inline_tok = sl.n <= kTokInline;
  } else {  // shared expert: every token, in order (row r is token r)
    sl.mat = 0;
    sl.r0 = 0;
    sl.n = T;
    sl.t0 = 0;
    sl.t1 = 1;
    sl.t2 = 2;
    sl.t3 = 3;
    sl.inline_tok = false;
  }
  if (sl.n <= 0) return false;
  return F.large ? sl.n > kTokInline : sl.n <= kTokInline;
}

// Where a part's gate/up results go.  epi 0: h = SiLU(g) * u (the SwiGLU
// intermediate).  epi 1: h = sigma(g), h2 = sigma(u) with sigma = SiLU (the
// department backbone outputs of the factorised form, DeaMoE section 3.2).
template <typename T_>
struct GuOut {
  T_* h;
  T_* h2;
  int epi;
};
template <typename T_>
__device__ __forceinline__ void gu_store(const GuOut<T_>& o, size_t idx, float g, float u) {
  if (o.epi) {
    store_act(o.h + idx, silu(g));
    store_act(o.h2 + idx, silu(u));
  } else {
    store_act(o.h + idx, silu(g) * u);
  }
}
// Down results: epi 0 stores the product, epi 1 its SiLU (the private down
// transform sigma((A_d)^T v) of the factorised form).
__device__ __forceinline__ void dn_store(float* out, size_t idx, float v, int epi) {
  out[idx] = epi ? silu(v) : v;
}

// Input row of row tc + t of the group (a token, or in the factorised form a
// (token, department) pair); t is a compile-time constant at every call site,
// so the inline case folds to one register.  Rows at or past the end of the
// group are never dereferenced and map to row 0; every index is clamped to
// the in_rows rows the input holds.
__device__ __forceinline__ int slot_token(const Slot& sl, const int* grp_token, int tc, int t,
                                          int nv, int in_rows) {
  int tok;
  if (sl.inline_tok)
    tok = t == 0 ? sl.t0 : t == 1 ? sl.t1 : t == 2 ? sl.t2 : sl.t3;
  else if (t >= nv)
    tok = 0;
  else
    tok = grp_token ? grp_token[sl.r0 + tc + t] : tc + t;
  return min(max(tok, 0), in_rows - 1);
}

// Input row of row t of a large group (per lane; t < n).
__device__ __forceinline__ int lane_token(const Slot& sl, const int* grp_token, int t,
                                          int in_rows) {
  const int tok = grp_token ? *as_global<int>(grp_token + sl.r0 + t) : t;
  return min(max(tok, 0), in_rows - 1);
}

// ---- small groups: register GEMV -------------------------------------------

// RW rows of gate and up from row i0 against the (at most four) input rows of
// the group (gate reads x, up reads xu: the same rows except in the two-input
// form).  Every load of step c+1 (weights and activations) is issued before
// step c is used: the vector-memory counter completes loads in order, so
// nothing requested after the next step's loads may be needed first.
template <typename T_, int RW, bool DUAL>
__device__ __forceinline__ void gu_small(const T_* __restrict__ Wg, const T_* __restrict__ Wu,
                                         int d, int rows, int i0, const T_* __restrict__ x,
                                         const T_* __restrict__ xu, int in_rows, const Slot& sl,
                                         const int* grp_token, const GuOut<T_>& o, int lane) {
  constexpr int NT = kTokInline, NX = DUAL ? 2 : 1;
  const int nv = sl.n;
  const T_* gp[RW];
  const T_* up[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const size_t i = (size_t)min(i0 + r, rows - 1);
    gp[r] = Wg + i * d;
    up[r] = Wu + i * d;
  }
  const T_* xp[NX][NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const size_t row = (size_t)slot_token(sl, grp_token, 0, t, nv, in_rows) * d;
    xp[0][t] = x + row;
    if constexpr (DUAL) xp[NX - 1][t] = xu + row;
  }
  float ag[RW][NT], au[RW][NT];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) ag[r][t] = au[r][t] = 0.f;

  int c = lane * 8;
  Raw8<T_> cg[RW], cu[RW];
  X8<T_> cx[NX][NT];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    if (c < d) {
      cg[r].load(gp[r] + c);
      cu[r].load(up[r] + c);
    } else {
      cg[r].zero();
      cu[r].zero();
    }
  }
#pragma unroll
  for (int v = 0; v < NX; ++v)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < nv && c < d)
        cx[v][t].load(xp[v][t] + c);
      else
        cx[v][t].zero();
    }
  for (; c < d; c += 8 * kWave) {
    const int cn = c + 8 * kWave;
    Raw8<T_> ng[RW], nu[RW];
    X8<T_> nx[NX][NT];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      if (cn < d) {
        ng[r].load(gp[r] + cn);
        nu[r].load(up[r] + cn);
      } else {
        ng[r].zero();
        nu[r].zero();
      }
    }
#pragma unroll
    for (int v = 0; v < NX; ++v)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t < nv && cn < d)
          nx[v][t].load(xp[v][t] + cn);
        else
          nx[v][t].zero();
      }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < nv) {
#pragma unroll
        for (int r = 0; r < RW; ++r) {
          ag[r][t] = dot8(cg[r], cx[0][t], ag[r][t]);
          au[r][t] = dot8(cu[r], cx[NX - 1][t], au[r][t]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      cg[r] = ng[r];
      cu[r] = nu[r];
    }
#pragma unroll
    for (int v = 0; v < NX; ++v)
#pragma unroll
      for (int t = 0; t < NT; ++t) cx[v][t] = nx[v][t];
  }
  constexpr int N = 2 * RW * NT;
  float v[N];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      v[r * NT + t] = ag[r][t];
      v[RW * NT + r * NT + t] = au[r][t];
    }
  group_reduce_scatter<N, 64>(v, lane);
  // gate index idx and up index idx + N/2 sit in lanes l and l ^ 32
  const float upv = xor32(v[0], lane);
  constexpr int SH = 6 - Log2<N>::value;
  const int idx = lane >> SH;
  if (idx < N / 2 && (lane & ((1 << SH) - 1)) == 0) {
    const int r = idx / NT, t = idx - (idx / NT) * NT;
    if (t < nv && i0 + r < rows) gu_store(o, (size_t)(sl.r0 + t) * rows + i0 + r, v[0], upv);
  }
}

// CG column groups of G = 64/LPR columns each (lane group g of LPR lanes takes
// column cb + q*G + g) against the (at most four) rows of h of the group.
// out[row][c] = W_down[c] . h[row].  Same load order as gu_small.
template <typename T_, int LPR, int CG>
__device__ __forceinline__ void dn_small(const T_* __restrict__ Wd, int d, int rows, int cb,
                                         const T_* __restrict__ h, const Slot& sl,
                                         float* __restrict__ out, int epi, int lane) {
  constexpr int NT = kTokInline;
  constexpr int G = 64 / LPR;
  const int g = lane / LPR, j = lane - g * LPR;
  const int nv = sl.n;
  const T_* wp[CG];
#pragma unroll
  for (int q = 0; q < CG; ++q) wp[q] = Wd + (size_t)min(cb + q * G + g, d - 1) * rows;
  const T_* hp[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) hp[t] = h + (size_t)(sl.r0 + min(t, nv - 1)) * rows;
  float acc[CG][NT];
#pragma unroll
  for (int q = 0; q < CG; ++q)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[q][t] = 0.f;
  int i = j * 8;
  Raw8<T_> cw[CG];
  X8<T_> ch[NT];
#pragma unroll
  for (int q = 0; q < CG; ++q) {
    if (i < rows)
      cw[q].load(wp[q] + i);
    else
      cw[q].zero();
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t < nv && i < rows)
      ch[t].load(hp[t] + i);
    else
      ch[t].zero();
  }
  for (; i < rows; i += 8 * LPR) {
    const int in = i + 8 * LPR;
    Raw8<T_> nw[CG];
    X8<T_> nh[NT];
#pragma unroll
    for (int q = 0; q < CG; ++q) {
      if (in < rows)
        nw[q].load(wp[q] + in);
      else
        nw[q].zero();
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < nv && in < rows)
        nh[t].load(hp[t] + in);
      else
        nh[t].zero();
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
      if (t < nv)
#pragma unroll
        for (int q = 0; q < CG; ++q) acc[q][t] = dot8(cw[q], ch[t], acc[q][t]);
#pragma unroll
    for (int q = 0; q < CG; ++q) cw[q] = nw[q];
#pragma unroll
    for (int t = 0; t < NT; ++t) ch[t] = nh[t];
  }
  constexpr int N = CG * NT;
  float v[N];
#pragma unroll
  for (int q = 0; q < CG; ++q)
#pragma unroll
    for (int t = 0; t < NT; ++t) v[q * NT + t] = acc[q][t];
  group_reduce_scatter<N, LPR>(v, lane);
  if constexpr (N >= LPR) {
    constexpr int PER = N / LPR;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int idx = j * PER + p;
      const int q = idx / NT, t = idx - (idx / NT) * NT;
      const int c = cb + q * G + g;
      if (t < nv && c < d) dn_store(out, (size_t)(sl.r0 + t) * d + c, v[p], epi);
    }
  } else {
    constexpr int SPAN = LPR / N;
    if (j % SPAN == 0) {
      const int idx = j / SPAN;
      const int q = idx / NT, t = idx - (idx / NT) * NT;
      const int c = cb + q * G + g;
      if (t < nv && c < d) dn_store(out, (size_t)(sl.r0 + t) * d + c, v[0], epi);
    }
  }
}

// ---- small groups, activations staged in LDS ------------------------------
//
// Every wave of a block works on the same group, so the block copies the
// group's (at most four) activation rows into LDS once and the waves read them
// with ds_read.  Only the weights then travel the vector-memory path: reading
// the activations per wave costs up to four extra 16-byte loads per weight load
// and, at four rows, makes that path (not HBM) the limit.  The copy is issued
// after the first weight loads, so both latencies overlap.

constexpr int kXLds = 2048;  // longest activation row staged (elements)

template <typename T_, int ROWS = kTokInline>
struct SmallLds {
  T_ x[ROWS][kXLds];
};

typedef __attribute__((address_space(3))) void lds_void_t;

// Block-wide: rows t < nv of `cols` elements, row t read from src(t), into
// lds.x[row0 + t], by direct global-to-LDS loads (each wave instruction moves
// 1 KB: lane l's 16 bytes land 16*l bytes past the wave-uniform destination),
// so the copy takes no registers.  cols is a multiple of 16 bytes' worth of
// elements and at most kXLds.  Only issues the loads: stage_wait() completes
// them for the whole block.
template <typename T_, int ROWS, typename Src>
__device__ __forceinline__ void stage_rows(SmallLds<T_, ROWS>& lds, int row0, int nv, int cols,
                                           Src src, int wid, int lane) {
  constexpr int EPL = 16 / sizeof(T_);     // elements per lane
  constexpr int EPI = EPL * kWave;         // elements per wave instruction
  const int per_row = (cols + EPI - 1) / EPI, total = nv * per_row;
  for (int q = wid; q < total; q += kWaves) {
    const int t = q / per_row, c0 = (q - t * per_row) * EPI;
    const int c = c0 + lane * EPL;
    if (c < cols)
      __builtin_amdgcn_global_load_lds(src(t) + c, (lds_void_t*)&lds.x[row0 + t][c0], 16, 0, 0);
  }
}

// Waits for every load this wave has issued (the weight prefetch included),
// then for the whole block, so every staged row is in LDS.
__device__ __forceinline__ void stage_wait() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

constexpr int kStageRing = 4;  // weight steps requested before the staging barrier

// Gate and up row i0 (one per wave) against the group's staged activations.
// Up to kStageRing steps of the row are requested before the staging, so they
// are all in flight through the barrier; after it, each consumed step's slot
// is refilled kStageRing steps ahead.  Same per-lane column order and
// reduction as gu_small.  NT: rows a group can have in this launch (1 at a
// batch of one token: a quarter of the accumulators and a shorter reduction).
template <typename T_, bool DUAL, int NT = kTokInline>
__device__ __forceinline__ void gu_small_lds(const T_* __restrict__ Wg, const T_* __restrict__ Wu,
                                             int d, int rows, int i0, const T_* __restrict__ x,
                                             const T_* __restrict__ xu, int in_rows,
                                             const Slot& sl, const int* grp_token,
                                             const GuOut<T_>& o, int lane, int wid,
                                             SmallLds<T_, DUAL ? 2 * kTokInline : kTokInline>& lds) {
  static_assert(NT >= 1 && NT <= kTokInline && (NT & (NT - 1)) == 0, "NT: 1, 2 or 4");
  constexpr int R = kStageRing, STEP = 8 * kWave;
  constexpr int UROW = DUAL ? NT : 0;  // LDS row of the up input of row t: UROW + t
  const int nv = sl.n;
  const size_t i = (size_t)min(i0, rows - 1);
  const T_* gp = Wg + i * d + lane * 8;
  const T_* up = Wu + i * d + lane * 8;
  const int dl = d - lane * 8;  // this lane's columns: lane*8 + k*STEP for k*STEP < dl
  Raw8<T_> rg[R], ru[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r * STEP < dl) {
      rg[r].load(gp + r * STEP);
      ru[r].load(up + r * STEP);
    } else {
      rg[r].zero();
      ru[r].zero();
    }
  }
  stage_rows(lds, 0, nv, d, [&](int t) {
    return x + (size_t)slot_token(sl, grp_token, 0, t, nv, in_rows) * d;
  }, wid, lane);
  if constexpr (DUAL)
    stage_rows(lds, UROW, nv, d, [&](int t) {
      return xu + (size_t)slot_token(sl, grp_token, 0, t, nv, in_rows) * d;
    }, wid, lane);
  stage_wait();
  float ag[NT], au[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) ag[t] = au[t] = 0.f;
  for (int c0 = 0; c0 < d; c0 += R * STEP) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int c = c0 + r * STEP;
      if (c < dl) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (t < nv) {
            const X8<T_> xv = *reinterpret_cast<const X8<T_>*>(&lds.x[t][lane * 8 + c]);
            ag[t] = dot8(rg[r], xv, ag[t]);
            if constexpr (DUAL) {
              const X8<T_> xw = *reinterpret_cast<const X8<T_>*>(&lds.x[UROW + t][lane * 8 + c]);
              au[t] = dot8(ru[r], xw, au[t]);
            } else {
              au[t] = dot8(ru[r], xv, au[t]);
            }
          }
        }
        if (c + R * STEP < dl) {
          rg[r].load(gp + c + R * STEP);
          ru[r].load(up + c + R * STEP);
        }
      }
    }
  }
  constexpr int N = 2 * NT;
  float v[N];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    v[t] = ag[t];
    v[NT + t] = au[t];
  }
  group_reduce_scatter<N, 64>(v, lane);
  // gate index t and up index t + NT sit in lanes l and l ^ 32
  const float upv = xor32(v[0], lane);
  constexpr int SH = 6 - Log2<N>::value;
  const int t = lane >> SH;
  if (t < NT && (lane & ((1 << SH) - 1)) == 0 && t < nv && i0 < rows)
    gu_store(o, (size_t)(sl.r0 + t) * rows + i0, v[0], upv);
}

// Down columns as dn_small, the group's rows of h staged in LDS; weights
// requested kStageRing steps ahead as in gu_small_lds.
template <typename T_, int LPR, int CG>
__device__ __forceinline__ void dn_small_lds(const T_* __restrict__ Wd, int d, int rows, int cb,
                                             const T_* __restrict__ h, const Slot& sl,
                                             float* __restrict__ out, int epi, int lane, int wid,
                                             SmallLds<T_>& lds) {
  // (wider column groups take a shallower ring: the same loads in flight)
  constexpr int NT = kTokInline, R = CG > 2 ? 2 * kStageRing / CG : kStageRing, STEP = 8 * LPR;
  constexpr int G = 64 / LPR;
  const int g = lane / LPR, j = lane - g * LPR;
  const int nv = sl.n;
  const int rl = rows - j * 8;  // this lane's elements: j*8 + k*STEP for k*STEP < rl
  const T_* wp[CG];
#pragma unroll
  for (int q = 0; q < CG; ++q) wp[q] = Wd + (size_t)min(cb + q * G + g, d - 1) * rows + j * 8;
  Raw8<T_> rw[R][CG];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int q = 0; q < CG; ++q) {
      if (r * STEP < rl)
        rw[r][q].load(wp[q] + r * STEP);
      else
        rw[r][q].zero();
    }
  stage_rows(lds, 0, nv, rows, [&](int t) { return h + (size_t)(sl.r0 + t) * rows; }, wid, lane);
  stage_wait();
  float acc[CG][NT];
#pragma unroll
  for (int q = 0; q < CG; ++q)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[q][t] = 0.f;
  for (int c0 = 0; c0 < rows; c0 += R * STEP) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int c = c0 + r * STEP;
      if (c < rl) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
          if (t < nv) {
            const X8<T_> hv = *reinterpret_cast<const X8<T_>*>(&lds.x[t][j * 8 + c]);
#pragma unroll
            for (int q = 0; q < CG; ++q) acc[q][t] = dot8(rw[r][q], hv, acc[q][t]);
          }
        if (c + R * STEP < rl) {
#pragma unroll
          for (int q = 0; q < CG; ++q) rw[r][q].load(wp[q] + c + R * STEP);
        }
      }
    }
  }
  constexpr int N = CG * NT;
  float v[N];
#pragma unroll
  for (int q = 0; q < CG; ++q)
#pragma unroll
    for (int t = 0; t < NT; ++t) v[q * NT + t] = acc[q][t];
  group_reduce_scatter<N, LPR>(v, lane);
  if constexpr (N >= LPR) {
    constexpr int PER = N / LPR;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int idx = j * PER + p;
      const int q = idx / NT, t = idx - (idx / NT) * NT;
      const int c = cb + q * G + g;
      if (t < nv && c < d) dn_store(out, (size_t)(sl.r0 + t) * d + c, v[p], epi);
    }
  } else {
    constexpr int SPAN = LPR / N;
    if (j % SPAN == 0) {
      const int idx = j / SPAN;
      const int q = idx / NT, t = idx - (idx / NT) * NT;
      const int c = cb + q * G + g;
      if (t < nv && c < d) dn_store(out, (size_t)(sl.r0 + t) * d + c, v[0], epi);
    }
  }
}

// ---- large groups, bf16: 16x16x32 matrix-core tiles ------------------------
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (lane l, g = l / 16): A row l%16
// with k = 8g..8g+7; B column l%16 with the same k; D rows 4g..4g+3 of column
// l%16.  A dot product is indifferent to the order of k, so each lane simply
// takes the 16-byte chunk at 8g of every 32-element step.

// K-split tiles (decode batches, T <= kSplitKMaxT): the four waves of a
// block share one 16-row tile (gate/up; two 16-column tiles for down) and
// each streams a quarter of K through a ring of LDS weight tiles (below), its
// token inputs read directly (L2); the four partial tiles are then added in
// wave order through LDS, so results do not depend on timing.


// Per-wave K range [kb, ke) of a K-split tile: quarters rounded up to 32.
__device__ __forceinline__ void k_quarter(int K, int wid, int& kb, int& ke) {
  const int kq = ((K + 4 * 32 - 1) / (4 * 32)) * 32;
  kb = min(K, wid * kq);
  ke = min(K, kb + kq);
}

// Weight tiles of the K-split gate/up go HBM -> LDS with buffer loads that
// write LDS directly (no registers): a tile is 16 rows x 64 elements of K,
// two loads of 8 rows x 128 contiguous bytes.  The matrix-core operand layout
// read straight from memory (lane l: row l % 16, 16 bytes at 8 (l / 16) of
// each 32-element step) visits 16 rows per load in 64-byte pieces, which
// measured 25% slower in HBM rate at the DeaMoE-7B-shaped batch 16; runs of
// 128 bytes or longer stream at the full rate.  In LDS, lane s of row a of a
// load holds chunk (s - rot) mod 8 of the row's 128 bytes, rot = a / 2 + 4 j
// for load j, so that the operand reads (16 rows at one chunk) fall in 16
// different 16-byte bank columns.
constexpr int kTileK = 64;                 // K elements of a tile
constexpr int kTileBytes = 16 * kTileK * 2;  // 2 KiB: 16 rows
constexpr int kTileSlots = 3;              // per wave: gate and up tiles in turn
struct MfmaLds {
  union {
    f32x4_t part[kWaves][2][2][kWave];                   // [wave][token chunk][gate / up][lane]
    unsigned char tile[kWaves][kTileSlots][kTileBytes];  // per wave: a ring of tiles
  };
};
__device__ __forceinline__ int tile_rot(int j, int a) { return ((a >> 1) + 4 * j) & 7; }

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Request one tile (rows i0.., K elements k0 .. k0 + 63) of the matrix behind
// `rs` into LDS tile `t` (wave-uniform): load j, lane l -> row 8 j + l / 8,
// chunk ((l % 8) - rot) mod 8; elements at or past ke, and rows at or past
// `rows`, read zeros.  Two vector-memory operations.
__device__ __forceinline__ void tile_request(unsigned char* t, __amdgpu_buffer_rsrc_t rs, int i0,
                                             int rows, int d, int k0, int ke, int lane) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int a = lane >> 3, r = 8 * j + a;
    const int chunk = ((lane & 7) - tile_rot(j, a)) & 7;
    const int k = k0 + 8 * chunk;
    const uint32_t off =
        (k < ke && i0 + r < rows) ? (uint32_t)(((size_t)(i0 + r) * d + k) * 2) : kDcOob;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(t + 1024 * j), 16, off, 0, 0,
                                             kCpolNt);
  }
}
// The operand of 32-element step m (0 or 1) of a tile in LDS.
__device__ __forceinline__ u32x4_t tile_operand(const unsigned char* t, int m, int lane) {
  const int r = lane & 15, j = r >> 3, a = r & 7;
  const int chunk = 4 * m + (lane >> 4);
  return *reinterpret_cast<const u32x4_t*>(t + 1024 * j +
                                           16 * (8 * a + ((chunk + tile_rot(j, a)) & 7)));
}

// K-split matrix-core tile: two 16-row tiles, A0 = rows a0.. of the matrix
// behind rs0 and A1 = rows a1.. of the matrix behind rs1 (nrows rows of kdim
// elements each), against up to 16 NT input rows (input row t at xrow(t) of
// x, and of xu for A1 when DUAL; rows t >= n read zeros), as NT 16-row token
// tiles.  Each wave takes a quarter of K in tiles of 64: tile q of A0 and
// tile q of A1 take turns in a ring of three LDS slots, so while one is used
// the next two are in flight; the inputs of tile q (two 32-element steps per
// token tile) come through registers, two sets in turn.  Loads past the
// wave's K range, and rows at or past nrows, read zeros, so every load is
// unconditional.  The waits are counted by hand (the compiler does not see
// the LDS data of these loads): per tile the vector-memory operations are,
// in order, A0 (2), inputs (2 NX NT), A1 (2).  The four waves' partial tiles
// are added in wave order through LDS, two token tiles at a time, and wave 0
// calls epi(t, i, s0, s1) with the sums of rows 4 (l / 16) + i of both
// tiles for input row t = 16 c + l % 16 < n of token tile c.
// KSPLIT false: the same pipeline without the split -- wave w owns rows
// 16 w.. of each matrix over the whole K and calls epi(t, 16 w + 4 (l / 16)
// + i, ...) itself, so a block covers 64 rows.
template <bool DUAL, int NT, bool KSPLIT = true, typename XRow, typename Epi>
__device__ void ksplit_mfma(__amdgpu_buffer_rsrc_t rs0, int a0, __amdgpu_buffer_rsrc_t rs1,
                            int a1, int nrows, int kdim, const bf16_t* __restrict__ x,
                            const bf16_t* __restrict__ xu, XRow xrow, int n, Epi epi, int lane,
                            int wid, MfmaLds& lds) {
  constexpr int NX = DUAL ? 2 : 1;   // activation inputs: A0's, and A1's when they differ
  constexpr int NXO = 2 * NX * NT;   // input loads of one tile
  static_assert(NT == 1 || NT == 2 || NT == 4, "token tiles per pass");
  const int t = lane & 15, g = lane >> 4;
  int kb = 0, ke = kdim;
  if constexpr (KSPLIT) {
    k_quarter(kdim, wid, kb, ke);
  } else {
    a0 += 16 * wid;
    a1 += 16 * wid;
  }
  kb = uni(kb);
  ke = uni(ke);
  __amdgpu_buffer_rsrc_t rx[NX];
  rx[0] = span_rsrc(x);
  if constexpr (DUAL) rx[NX - 1] = span_rsrc(xu);
  bool xv[NT];
  uint32_t xoff[NT];
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    xv[c] = 16 * c + t < n;
    xoff[c] = (uint32_t)(((size_t)(xv[c] ? xrow(16 * c + t) : 0) * kdim + g * 8) * 2);
  }
  // token tiles holding rows of the group (uniform): the matrix-core steps of
  // the others are skipped, their input loads read zeros
  const int ntl = min(NT, (n + 15) >> 4);
  f32x4_t acc0[NT], acc1[NT];
#pragma unroll
  for (int c = 0; c < NT; ++c) acc0[c] = acc1[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  unsigned char* slots = lds.tile[wid][0];
  u32x4_t xa[2][NX][NT], xb[2][NX][NT];
  auto request_x = [&](u32x4_t (&xr)[2][NX][NT], int k0) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int k = k0 + 32 * m;
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        const bool in = xv[c] && k + g * 8 < ke;
#pragma unroll
        for (int v = 0; v < NX; ++v)
          xr[m][v][c] = ld16_span(rx[v], in ? xoff[c] + (uint32_t)k * 2 : kDcOob);
      }
    }
  };
  // unit u = 2q (A0 tile q) or 2q + 1 (A1 tile q) lives in slot u % 3
  auto slot = [&](int u) { return slots + (u % kTileSlots) * kTileBytes; };
  auto mfma2 = [&](f32x4_t (&acc)[NT], const unsigned char* tl, const u32x4_t (&xr)[2][NX][NT],
                   int v) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const u32x4_t av = tile_operand(tl, m, lane);
#pragma unroll
      for (int c = 0; c < NT; ++c)
        if (c < ntl)
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(xr[m][v][c]),
                                                           acc[c], 0, 0, 0);
    }
  };
  // one tile, whose A0 and A1 units were requested before; requests the next
  // tile's units and inputs (into xn) as the slots free up
  auto step = [&](int q, u32x4_t (&xc)[2][NX][NT], u32x4_t (&xn)[2][NX][NT]) {
    const int k0 = kb + kTileK * q;
    __builtin_amdgcn_sched_barrier(0);
    tile_request(slot(2 * q + 2), rs0, a0, nrows, kdim, k0 + kTileK, ke, lane);
    request_x(xn, k0 + kTileK);
    // A0 tile q and inputs q: newer are A1 q, A0 q + 1, inputs q + 1
    wait_vmcnt<2 + 2 + NXO>();
    __builtin_amdgcn_sched_barrier(0);
    mfma2(acc0, slot(2 * q), xc, 0);
    __builtin_amdgcn_sched_barrier(0);
    // the slot of A0 tile q takes A1 tile q + 1: its reads have returned,
    // since the matrix-core steps issued above consumed them
    tile_request(slot(2 * q + 3), rs1, a1, nrows, kdim, k0 + kTileK, ke, lane);
    // A1 tile q: newer are A0 q + 1, inputs q + 1, A1 q + 1
    wait_vmcnt<2 + NXO + 2>();
    __builtin_amdgcn_sched_barrier(0);
    mfma2(acc1, slot(2 * q + 1), xc, NX - 1);
    __builtin_amdgcn_sched_barrier(0);
  };
  tile_request(slot(0), rs0, a0, nrows, kdim, kb, ke, lane);
  request_x(xa, kb);
  tile_request(slot(1), rs1, a1, nrows, kdim, kb, ke, lane);
  const int nq = (ke - kb + kTileK - 1) / kTileK;
  for (int q = 0; q < nq; q += 2) {
    step(q, xa, xb);
    if (q + 1 < nq) step(q + 1, xb, xa);
  }
  // no load may still write a slot when the area is reused below
  wait_vmcnt<0>();
  if constexpr (!KSPLIT) {
#pragma unroll
    for (int c = 0; c < NT; ++c)
      if (c < ntl && 16 * c + t < n) {
#pragma unroll
        for (int i = 0; i < 4; ++i) epi(16 * c + t, 16 * wid + 4 * g + i, acc0[c][i], acc1[c][i]);
      }
    return;
  }
#pragma unroll
  for (int c0 = 0; c0 < NT; c0 += 2) {
    if (c0 >= ntl) break;
    __syncthreads();
#pragma unroll
    for (int c = c0; c < c0 + 2 && c < NT; ++c) {
      lds.part[wid][c - c0][0][lane] = acc0[c];
      lds.part[wid][c - c0][1][lane] = acc1[c];
    }
    __syncthreads();
    if (wid == 0) {
#pragma unroll
      for (int c = c0; c < c0 + 2 && c < NT; ++c) {
        f32x4_t s0 = lds.part[0][c - c0][0][lane], s1 = lds.part[0][c - c0][1][lane];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) {
          s0 += lds.part[w][c - c0][0][lane];
          s1 += lds.part[w][c - c0][1][lane];
        }
        if (16 * c + t < n) {
#pragma unroll
          for (int i = 0; i < 4; ++i) epi(16 * c + t, 4 * g + i, s0[i], s1[i]);
        }
      }
    }
  }
  __syncthreads();
}

// 16 rows (i0..) of gate and up against the group's (at most 16 NT) rows.
template <bool DUAL, int NT>
__device__ void gu_mfma(const bf16_t* __restrict__ Wg, const bf16_t* __restrict__ Wu, int d,
                        int rows, int i0, const bf16_t* __restrict__ x,
                        const bf16_t* __restrict__ xu, int in_rows, const Slot& sl,
                        const int* grp_token, const GuOut<bf16_t>& o, int lane, int wid,
                        MfmaLds& lds) {
  ksplit_mfma<DUAL, NT>(
      span_rsrc(Wg), i0, span_rsrc(Wu), i0, rows, d, x, xu,
      [&](int t) { return lane_token(sl, grp_token, t, in_rows); }, sl.n,
      [&](int t, int i, float g, float u) {
        if (i0 + i < rows) gu_store(o, (size_t)(sl.r0 + t) * rows + i0 + i, g, u);
      },
      lane, wid, lds);
}

// Out-of-line entry of the K-split gate/up tile for NT 16-token tiles
// (groups of at most 16 NT rows), with plain-value arguments like
// gu_wide_call.
template <bool DUAL, int NT>
__device__ __attribute__((noinline)) void gu_mfma_call(
    const bf16_t* __restrict__ Wg, const bf16_t* __restrict__ Wu, int d, int rows, int i0,
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ xu, int in_rows, int r0, int n,
    const int* grp_token, GuOut<bf16_t> o, int lane, int wid, MfmaLds& lds) {
  Slot sl{};
  sl.r0 = r0;
  sl.n = n;
  gu_mfma<DUAL, NT>(Wg, Wu, d, rows, i0, x, xu, in_rows, sl, grp_token, o, lane, wid, lds);
}

// 64 rows (i0.., 16 per wave over the whole K) of gate and up against a
// group of at most 16 NT rows, through the LDS weight tiles of ksplit_mfma
// (one input set).  Out of line, like gu_mfma_call.
template <int NT>
__device__ __attribute__((noinline)) void gu_rows_call(
    const bf16_t* __restrict__ Wg, const bf16_t* __restrict__ Wu, int d, int rows, int i0,
    const bf16_t* __restrict__ x, int in_rows, int r0, int n, const int* grp_token,
    GuOut<bf16_t> o, int lane, int wid, MfmaLds& lds) {
  Slot sl{};
  sl.r0 = r0;
  sl.n = n;
  ksplit_mfma<false, NT, false>(
      span_rsrc(Wg), i0, span_rsrc(Wu), i0, rows, d, x, x,
      [&](int t) { return lane_token(sl, grp_token, t, in_rows); }, n,
      [&](int t, int i, float g, float u) {
        if (i0 + i < rows) gu_store(o, (size_t)(r0 + t) * rows + i0 + i, g, u);
      },
      lane, wid, lds);
}

// Down projection of a group of at most 16 NT rows of h as K-split tiles: 32
// output columns (c0..) per block, two 16-column tiles sharing each input
// step, K = the intermediate width split over the four waves.  out[r0 + t][c]
// (SiLU of it when epi) for every row t < n of the group.  Out of line, like
// gu_mfma_call.
template <int NT>
__device__ __attribute__((noinline)) void dn_mfma_call(const bf16_t* __restrict__ Wd, int d,
                                                       int rows, int c0,
                                                       const bf16_t* __restrict__ h, int r0,
                                                       int n, float* __restrict__ out, int epi,
                                                       int lane, int wid, MfmaLds& lds) {
  const __amdgpu_buffer_rsrc_t rw = span_rsrc(Wd);
  ksplit_mfma<false, NT>(
      rw, c0, rw, c0 + 16, d, rows, h + (size_t)r0 * rows, h, [](int t) { return t; }, n,
      [&](int t, int i, float a, float b) {
        float* o = out + (size_t)(r0 + t) * d;
        if (c0 + i < d) dn_store(o, c0 + i, a, epi);
        if (c0 + 16 + i < d) dn_store(o, c0 + 16 + i, b, epi);
      },
      lane, wid, lds);
}
// Down projection of a group of at most 16 NT rows of h over kDownRowCols
// output columns (c0..): wave w takes columns c0 + 16 w.. and c0 + 64 +
// 16 w.. over the whole K through the LDS weight tiles of ksplit_mfma.  Out
// of line, like gu_mfma_call.
template <int NT>
__device__ __attribute__((noinline)) void dn_rows_call(const bf16_t* __restrict__ Wd, int d,
                                                       int rows, int c0,
                                                       const bf16_t* __restrict__ h, int r0,
                                                       int n, float* __restrict__ out, int epi,
                                                       int lane, int wid, MfmaLds& lds) {
  const __amdgpu_buffer_rsrc_t rw = span_rsrc(Wd);
  ksplit_mfma<false, NT, false>(
      rw, c0, rw, c0 + kWideRows, d, rows, h + (size_t)r0 * rows, h, [](int t) { return t; }, n,
      [&](int t, int i, float a, float b) {
        float* o = out + (size_t)(r0 + t) * d;
        if (c0 + i < d) dn_store(o, c0 + i, a, epi);
        if (c0 + kWideRows + i < d) dn_store(o, c0 + kWideRows + i, b, epi);
      },
      lane, wid, lds);
}
// ---- large groups, bf16: 64-row tiles with LDS-shared inputs ---------------
//
// Four waves, each 16 rows (gate/up) or 16 output columns (down) over the whole
// K.  Every 64-wide K step of the group's inputs is loaded once per block by
// all 256 threads, written to LDS already in B-operand order, and read by each
// wave as one contiguous 1 KiB per 16-token tile: the inputs cross the memory
// path once per 64 rows, so at N tokens they add N/128 (gate/up, two 64-row
// matrices) or N/64 (down) of the weight bytes.  The inputs and weights of
// step i+1 are requested together before step i is used, so waiting for the
// inputs (loads complete in order) never waits for a later weight request.
// Groups of more than 16*NCMAX tokens take several passes over the weights.

constexpr int kDownNC = 4;     // 16-token tiles of a down pass (one accumulator set: room for 4)
using Slot0 = std::integral_constant<int, 0>;  // ring slots of the two-step pipeline
using Slot1 = std::integral_constant<int, 1>;
constexpr int kWideK = 64;     // K per step: two 32-wide matrix-core steps

// Two buffers of one step's inputs: [buffer][input][token tile][half][lane],
// lane l of (c, half) holding token 16c + l%16, k = 32 half + 8 (l/16) .. +7.
// H: 8-element k pieces per lane group and step (2: the 64-element step of
// bf16 weights; 4: the 128-element step of FP8 weights).
template <int NC, int NX, int H = 2>
struct WideLds {
  u32x4_t x[2][NX * NC * H * kWave];
};

// Per-thread share of one step's input chunks: chunk q = tid + kThreads * r
// of Q = NX*NC*64H, with l = q % 64, half = (q/64) % H, c = (q/(64H)) % NC,
// input v = q / (64 H NC).
template <int NC, int NX, int H = 2>
struct WideIn {
  static constexpr int Q = NX * NC * H * kWave;
  static constexpr int R = (Q + kThreads - 1) / kThreads;
  const bf16_t* p[R];  // input row + k offset of the chunk (nullptr: token past the group)
  int koff[R];
};

// The k of a chunk within the step: H = 2 (bf16 weights) k = 32 half +
// 8 (l/16); H = 4 (FP8 weights, whose lane group l/16 reads 32 consecutive
// codes) k = 32 (l/16) + 8 half.
template <int NC, int NX, int H = 2, typename RowOf>
__device__ __forceinline__ void wide_inputs(WideIn<NC, NX, H>& in, const bf16_t* const* src,
                                            int d, int tc, int n, RowOf row_of) {
#pragma unroll
  for (int r = 0; r < WideIn<NC, NX, H>::R; ++r) {
    const int q = threadIdx.x + kThreads * r;
    const int l = q & 63, half = (q >> 6) % H, rest = (q >> 6) / H;
    const int c = rest % NC, v = rest / NC;
    const int t = tc + 16 * c + (l & 15);
    in.koff[r] = H == 2 ? 32 * half + 8 * (l >> 4) : 32 * (l >> 4) + 8 * half;
    in.p[r] = (q < WideIn<NC, NX, H>::Q && t < n) ? src[v < NX ? v : 0] + (size_t)row_of(t) * d
                                                  : nullptr;
  }
}

template <int NC, int NX, int H = 2>
__device__ __forceinline__ void wide_load(u32x4_t* dst, const WideIn<NC, NX, H>& in, int k0,
                                          int K) {
  const u32x4_t z = {0, 0, 0, 0};
#pragma unroll
  for (int r = 0; r < WideIn<NC, NX, H>::R; ++r) {
    const int k = k0 + in.koff[r];
    dst[r] = (in.p[r] && k < K) ? ld16(in.p[r] + k) : z;
  }
}

template <int NC, int NX, int H = 2>
__device__ __forceinline__ void wide_stage(WideLds<NC, NX, H>& lds, int buf, const u32x4_t* v) {
#pragma unroll
  for (int r = 0; r < WideIn<NC, NX, H>::R; ++r) {
    const int q = threadIdx.x + kThreads * r;
    if (q < WideIn<NC, NX, H>::Q) lds.x[buf][q] = v[r];
  }
}

// 64 rows (i0..) of gate and up against 16*NC tokens (rows tc.. of the group
// [r0, r0 + n) of the plan).
template <int NC, bool DUAL>
__device__ __forceinline__ void gu_wide(const bf16_t* __restrict__ Wg,
                                                  const bf16_t* __restrict__ Wu, int d, int rows,
                                                  int i0, const bf16_t* __restrict__ x,
                                                  const bf16_t* __restrict__ xu, int in_rows,
                                                  int r0, int n, const int* grp_token, int tc,
                                                  GuOut<bf16_t> o, int lane, int wid,
                                                  WideLds<NC, DUAL ? 2 : 1>& lds) {
  constexpr int NX = DUAL ? 2 : 1;
  constexpr int R = WideIn<NC, NX>::R;
  const int r16 = lane & 15, g = lane >> 4;
  const size_t wrow = (size_t)min(i0 + 16 * wid + r16, rows - 1) * d + 8 * g;
  const bf16_t* ap = Wg + wrow;
  const bf16_t* bp = Wu + wrow;
  WideIn<NC, NX> in;
  const bf16_t* src[NX];
  src[0] = x;
  if constexpr (DUAL) src[NX - 1] = xu;
  wide_inputs<NC, NX>(in, src, d, tc, n, [&](int t) {
    const int tok = grp_token ? *as_global<int>(grp_token + r0 + t) : t;
    return min(max(tok, 0), in_rows - 1);
  });
  f32x4_t accg[NC], accu[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) accg[c] = accu[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const u32x4_t z = {0, 0, 0, 0};
  u32x4_t rx[2][R], ra[2][2], rb[2][2];
  auto request = [&](auto S, int k0) {
    constexpr int s = decltype(S)::value;
    wide_load<NC, NX>(rx[s], in, k0, d);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = k0 + 32 * h;
      ra[s][h] = k + 8 * g < d ? ld16(ap + k) : z;
      rb[s][h] = k + 8 * g < d ? ld16(bp + k) : z;
    }
  };
  auto use = [&](auto S) {
    constexpr int s = decltype(S)::value;
    wide_stage<NC, NX>(lds, s, rx[s]);
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u32x4_t bg = lds.x[s][(c * 2 + h) * kWave + lane];
        const u32x4_t bu = lds.x[s][((NX - 1) * NC * 2 + c * 2 + h) * kWave + lane];
        accg[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ra[s][h]), as_bf16x8(bg), accg[c], 0, 0, 0);
        accu[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(rb[s][h]), as_bf16x8(bu), accu[c], 0, 0, 0);
      }
  };
  const int nk = (d + kWideK - 1) / kWideK;
  const Slot0 s0;
  const Slot1 s1;
  request(s0, 0);
  for (int it = 0; it < nk; it += 2) {
    if (it + 1 < nk) request(s1, (it + 1) * kWideK);
    use(s0);
    if (it + 1 < nk) {
      if (it + 2 < nk) request(s0, (it + 2) * kWideK);
      use(s1);
    }
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int t = tc + c * 16 + r16;
    if (t < n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = i0 + 16 * wid + 4 * g + i;
        if (rr < rows) gu_store(o, (size_t)(r0 + t) * rows + rr, accg[c][i], accu[c][i]);
      }
    }
  }
  __syncthreads();  // the buffers are free for the next pass
}

// The same, out of line, for launches where large groups are rare (T <= 16):
// its registers then never raise the pressure, or cause spills, in the
// small-group path that shares the kernel.  Plain-value arguments, so the
// call makes the caller materialise nothing.
template <int NC, bool DUAL>
__device__ __attribute__((noinline)) void gu_wide_call(
    const bf16_t* __restrict__ Wg, const bf16_t* __restrict__ Wu, int d, int rows, int i0,
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ xu, int in_rows, int r0, int n,
    const int* grp_token, int tc, GuOut<bf16_t> o, int lane, int wid,
    WideLds<NC, DUAL ? 2 : 1>& lds) {
  gu_wide<NC, DUAL>(Wg, Wu, d, rows, i0, x, xu, in_rows, r0, n, grp_token, tc, o, lane, wid, lds);
}

// 64 output columns (c0..) against 16*NC rows of h (rows tc.. of the group).
// Out of line, like gu_wide.
template <int NC>
__device__ __attribute__((noinline)) void dn_wide(const bf16_t* __restrict__ Wd, int d, int rows,
                                                  int c0, const bf16_t* __restrict__ h, int r0,
                                                  int n, int tc, float* __restrict__ out, int epi,
                                                  int lane, int wid, WideLds<NC, 1>& lds) {
  constexpr int R = WideIn<NC, 1>::R;
  const int r16 = lane & 15, g = lane >> 4;
  const bf16_t* ap = Wd + (size_t)min(c0 + 16 * wid + r16, d - 1) * rows + 8 * g;
  WideIn<NC, 1> in;
  const bf16_t* const src[1] = {h};
  wide_inputs<NC, 1>(in, src, rows, tc, n, [&](int t) { return r0 + t; });
  f32x4_t acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const u32x4_t z = {0, 0, 0, 0};
  u32x4_t rx[2][R], ra[2][2];
  auto request = [&](auto S, int k0) {
    constexpr int s = decltype(S)::value;
    wide_load<NC, 1>(rx[s], in, k0, rows);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int k = k0 + 32 * hh;
      ra[s][hh] = k + 8 * g < rows ? ld16(ap + k) : z;
    }
  };
  auto use = [&](auto S) {
    constexpr int s = decltype(S)::value;
    wide_stage<NC, 1>(lds, s, rx[s]);
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u32x4_t b = lds.x[s][(c * 2 + hh) * kWave + lane];
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ra[s][hh]), as_bf16x8(b), acc[c], 0, 0, 0);
      }
  };
  const int nk = (rows + kWideK - 1) / kWideK;
  const Slot0 s0;
  const Slot1 s1;
  request(s0, 0);
  for (int it = 0; it < nk; it += 2) {
    if (it + 1 < nk) request(s1, (it + 1) * kWideK);
    use(s0);
    if (it + 1 < nk) {
      if (it + 2 < nk) request(s0, (it + 2) * kWideK);
      use(s1);
    }
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int t = tc + c * 16 + r16;
    if (t < n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = c0 + 16 * wid + 4 * g + i;
        if (col < d) dn_store(out, (size_t)(r0 + t) * d + col, acc[c][i], epi);
      }
    }
  }
  __syncthreads();
}

// ---- large groups, fp32 layers: plain GEMV ---------------------------------

// RW rows of gate and up against NT tokens from row tc of the group, no
// prefetch (fp32 layers are small).
template <int RW, int NT>
__device__ void gu_plain(const float* __restrict__ Wg, const float* __restrict__ Wu, int d,
                         int rows, int i0, const float* __restrict__ x,
                         const float* __restrict__ xu, int in_rows, const Slot& sl,
                         const int* grp_token, int tc, const GuOut<float>& o, int lane) {
  const int nv = min(NT, sl.n - tc);
  float ag[RW][NT], au[RW][NT];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) ag[r][t] = au[r][t] = 0.f;
  for (int c = lane * 8; c < d; c += 8 * kWave) {
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      Raw8<float> wg, wu;
      const size_t i = (size_t)min(i0 + r, rows - 1);
      wg.load(Wg + i * d + c);
      wu.load(Wu + i * d + c);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t < nv) {
          const size_t row = (size_t)lane_token(sl, grp_token, tc + t, in_rows) * d + c;
          X8<float> xv, xw;
          xv.load(x + row);
          xw.load(xu + row);
          ag[r][t] = dot8(wg, xv, ag[r][t]);
          au[r][t] = dot8(wu, xw, au[r][t]);
        }
      }
    }
  }
  constexpr int N = 2 * RW * NT;
  float v[N];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      v[r * NT + t] = ag[r][t];
      v[RW * NT + r * NT + t] = au[r][t];
    }
  group_reduce_scatter<N, 64>(v, lane);
  const float upv = xor32(v[0], lane);
  constexpr int SH = 6 - Log2<N>::value;
  const int idx = lane >> SH;
  if (idx < N / 2 && (lane & ((1 << SH) - 1)) == 0) {
    const int r = idx / NT, t = idx - (idx / NT) * NT;
    if (t < nv && i0 + r < rows) gu_store(o, (size_t)(sl.r0 + tc + t) * rows + i0 + r, v[0], upv);
  }
}

// CW columns from c0 against NT rows of h from row tc of the group.
template <int CW, int NT>
__device__ void dn_plain(const float* __restrict__ Wd, int d, int rows, int c0,
                         const float* __restrict__ h, const Slot& sl, int tc,
                         float* __restrict__ out, int epi, int lane) {
  const int nv = min(NT, sl.n - tc);
  float acc[CW][NT];
#pragma unroll
  for (int q = 0; q < CW; ++q)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[q][t] = 0.f;
  for (int i = lane * 8; i < rows; i += 8 * kWave) {
#pragma unroll
    for (int q = 0; q < CW; ++q) {
      Raw8<float> w;
      w.load(Wd + (size_t)min(c0 + q, d - 1) * rows + i);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t < nv) {
          X8<float> hv;
          hv.load(h + (size_t)(sl.r0 + tc + t) * rows + i);
          acc[q][t] = dot8(w, hv, acc[q][t]);
        }
      }
    }
  }
  constexpr int N = CW * NT;
  float v[N];
#pragma unroll
  for (int q = 0; q < CW; ++q)
#pragma unroll
    for (int t = 0; t < NT; ++t) v[q * NT + t] = acc[q][t];
  group_reduce_scatter<N, 64>(v, lane);
  constexpr int SH = 6 - Log2<N>::value;
  const int idx = lane >> SH;
  if ((lane & ((1 << SH) - 1)) == 0) {
    const int q = idx / NT, t = idx - (idx / NT) * NT;
    if (t < nv && c0 + q < d) dn_store(out, (size_t)(sl.r0 + tc + t) * d + c0 + q, v[0], epi);
  }
}

// ---- kernels -----------------------------------------------------------------

// Small groups: each wave owns RPW rows, taken RW at a time.
// Minimum waves per SIMD the expert kernels are built for.  The bf16 small-
// group GEMVs are latency-bound streams that want many waves in flight, so
// the register budget is capped where the matrix-core part still fits without
// spilling; fp32 layers keep the compiler's choice.
template <typename T_, int NCMAX, bool DUAL>
constexpr int gateup_min_waves() {
  // two-input launches carry twice the activations, and 64-token tiles four
  // accumulator pairs: a register budget of 4 waves
  return sizeof(T_) == 2 ? (DUAL || NCMAX >= 4 ? 4 : NCMAX > 1 ? 5 : 6) : 1;
}
template <typename T_>
constexpr int down_min_waves() { return sizeof(T_) == 2 ? 7 : 1; }

// LDS of an expert-kernel block: the matrix-core partial tiles of a large
// group or the staged activations of a small one (a block is only ever one).
template <typename T_, bool XL, bool DUAL = false, int NC = kDownNC>
constexpr size_t expert_lds_bytes() {
  const size_t w = sizeof(WideLds<NC, DUAL ? 2 : 1>);
  const size_t a = sizeof(T_) == 2 ? (w > sizeof(MfmaLds) ? w : sizeof(MfmaLds)) : 0;
  const size_t b = XL ? sizeof(SmallLds<T_, DUAL ? 2 * kTokInline : kTokInline>) : 0;
  return a > b ? a : (b > 0 ? b : 16);
}

// One pass of a 64-row large-group tile over 16*NC tokens from tc, with the
// LDS staging area of that width; out of line (CALL) or inlined.
template <int NC, bool DUAL, bool CALL, typename T_>
__device__ __forceinline__ void gu_wide_pass(const T_* __restrict__ Wg, const T_* __restrict__ Wu,
                                             int d, int rows, int i0, const T_* xg, const T_* xu,
                                             int in_rows, const Slot& sl, const int* grp_token,
                                             int tc, const GuOut<T_>& o, int lane, int wid,
                                             unsigned char* lds_raw) {
  if constexpr (sizeof(T_) == 2) {
    auto& lw = *reinterpret_cast<WideLds<NC, DUAL ? 2 : 1>*>(lds_raw);
    if constexpr (CALL)
      gu_wide_call<NC, DUAL>(Wg, Wu, d, rows, i0, xg, xu, in_rows, sl.r0, sl.n, grp_token, tc, o,
                             lane, wid, lw);
    else
      gu_wide<NC, DUAL>(Wg, Wu, d, rows, i0, xg, xu, in_rows, sl.r0, sl.n, grp_token, tc, o, lane,
                        wid, lw);
  }
}

// NCMAX: 16-token chunks a large-group tile takes at once (2 only when a
// group can exceed 16 rows, since the wider chunk costs registers).
// XL: small groups read their activations from LDS (rows of at most kXLds).
// DUAL: every part of the launch reads gate and up inputs from two different
// matrices (the private transforms of the factorised form).
// NTI: rows a small group can have in the launch (kTokInline, or 1 at T = 1).
template <typename T_, int RPW, int RW, int NCMAX, bool XL, bool DUAL, int NTI = kTokInline>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(
    gateup_min_waves<T_, NCMAX, DUAL>(), 8))) void gateup_kernel(FamilySet set,
                                                           const T_* __restrict__ x, int T,
                                                           int d) {
  int tile;
  const Family& F = block_part(set, tile);
  Slot sl;
  if (!map_slot(F, T, sl, tile)) return;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const size_t ms = (size_t)F.rows * d;
  const T_* Wg = static_cast<const T_*>(F.gate) + (size_t)sl.mat * ms;
  const T_* Wu = static_cast<const T_*>(F.up) + (size_t)sl.mat * ms;
  const T_* xg = F.x_gate ? static_cast<const T_*>(F.x_gate) : x;
  const T_* xu = DUAL ? static_cast<const T_*>(F.x_up) : xg;
  const GuOut<T_> o{static_cast<T_*>(F.h), static_cast<T_*>(F.h2), F.epi};
  __shared__ __align__(16) unsigned char lds_raw[expert_lds_bytes<T_, XL, DUAL, NCMAX>()];
  if (!F.large) {
    if constexpr (XL) {
      static_assert(RPW == 1 && RW == 1, "staged activations take one row per wave");
      gu_small_lds<T_, DUAL, NTI>(
          Wg, Wu, d, F.rows, tile * kWaves + wid, xg, xu, F.in_rows, sl, F.grp_token, o, lane, wid,
          *reinterpret_cast<SmallLds<T_, DUAL ? 2 * kTokInline : kTokInline>*>(lds_raw));
      return;
    }
    const int i0 = tile * (kWaves * RPW) + wid * RPW;
#pragma unroll 1
    for (int r = 0; r < RPW && i0 + r < F.rows; r += RW)
      gu_small<T_, RW, DUAL>(Wg, Wu, d, F.rows, i0 + r, xg, xu, F.in_rows, sl, F.grp_token, o,
                             lane);
    return;
  }
  if constexpr (sizeof(T_) == 2) {
    if (F.splitk) {
      // at most 16 NCMAX rows per group: one 16-row K-split tile per block
      const int i0 = tile * 16;
      if (i0 < F.rows)
        gu_mfma_call<DUAL, (NCMAX < 2 ? NCMAX : 2)>(Wg, Wu, d, F.rows, i0, xg, xu, F.in_rows,
                                                     sl.r0, sl.n, F.grp_token, o,
                           lane, wid, *reinterpret_cast<MfmaLds*>(lds_raw));
      return;
    }
    // large groups: the whole block on one 64-row tile, 16*NC tokens a pass
    const int i0 = tile * kWideRows;
    if (i0 >= F.rows) return;
    if constexpr (!DUAL) {
      // groups of at most 32 rows: each wave its 16 rows through the LDS
      // weight tiles, in one pass
      if (sl.n <= 32) {
        gu_rows_call<2>(Wg, Wu, d, F.rows, i0, xg, F.in_rows, sl.r0, sl.n, F.grp_token, o, lane,
                        wid, *reinterpret_cast<MfmaLds*>(lds_raw));
        return;
      }
    }
    // out of line where large groups are rare (T <= 16, or the two-input
    // private transforms, whose groups seldom pass four rows)
    constexpr bool kCall = NCMAX == 1 || DUAL;
#pragma unroll 1
    for (int tc = 0; tc < sl.n; tc += 16 * NCMAX) {
      const int rem = sl.n - tc;
      if (NCMAX >= 4 && rem > 32)
        gu_wide_pass<(NCMAX >= 4 ? 4 : 1), DUAL, kCall>(Wg, Wu, d, F.rows, i0, xg, xu, F.in_rows,
                                                        sl, F.grp_token, tc, o, lane, wid, lds_raw);
      else if (NCMAX >= 2 && rem > 16)
        gu_wide_pass<(NCMAX >= 2 ? 2 : 1), DUAL, kCall>(Wg, Wu, d, F.rows, i0, xg, xu, F.in_rows,
                                                        sl, F.grp_token, tc, o, lane, wid, lds_raw);
      else
        gu_wide_pass<1, DUAL, kCall>(Wg, Wu, d, F.rows, i0, xg, xu, F.in_rows, sl, F.grp_token,
                                     tc, o, lane, wid, lds_raw);
    }
  } else {
    // large groups, fp32 layers: the whole block on one 16-row tile
    const int i0 = tile * 16;
    if (i0 >= F.rows) return;
#pragma unroll 1
    for (int r = wid * 4; r < wid * 4 + 4; r += 2)
#pragma unroll 1
      for (int tc = 0; tc < sl.n; tc += 8)
        gu_plain<2, 8>(Wg, Wu, d, F.rows, i0 + r, xg, xu, F.in_rows, sl, F.grp_token, tc, o,
                       lane);
  }
}

template <typename T_, int LPR, int CG, bool XL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(
    down_min_waves<T_>(), 8))) void down_kernel(FamilySet set, int T, int d) {
  int tile;
  const Family& F = block_part(set, tile);
  Slot sl;
  if (!map_slot(F, T, sl, tile)) return;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const T_* Wd = static_cast<const T_*>(F.down) + (size_t)sl.mat * F.rows * d;
  const T_* h = static_cast<const T_*>(F.h);
  __shared__ __align__(16) unsigned char lds_raw[expert_lds_bytes<T_, XL>()];
  if (!F.large) {
    constexpr int CPW = CG * (64 / LPR);
    const int cb = tile * (kWaves * CPW) + wid * CPW;
    if constexpr (XL)  // every wave takes part in the staging
      dn_small_lds<T_, LPR, CG>(Wd, d, F.rows, cb, h, sl, F.out, F.epi, lane, wid,
                                *reinterpret_cast<SmallLds<T_>*>(lds_raw));
    else if (cb < d)
      dn_small<T_, LPR, CG>(Wd, d, F.rows, cb, h, sl, F.out, F.epi, lane);
    return;
  }
  if constexpr (sizeof(T_) == 2) {
    if (F.splitk == 1) {
      // at most 16 rows per group: 32 columns per block, K split over the waves
      const int c0 = tile * kSplitKCols;
      if (c0 < d)
        dn_mfma_call<1>(Wd, d, F.rows, c0, h, sl.r0, sl.n, F.out, F.epi, lane, wid,
                        *reinterpret_cast<MfmaLds*>(lds_raw));
      return;
    }
    // large groups: 64-column tiles, 16*NC rows of h a pass -- one per block,
    // or two (kDownRowCols columns) where groups of at most 16 rows take the
    // LDS weight tiles instead, each wave 16 + 16 columns over the whole K
    const int cols = F.splitk == 2 ? kDownRowCols : kWideRows;
    const int cb = tile * cols;
    if (cb >= d) return;
    if (F.splitk == 2 && sl.n <= 16) {
      dn_rows_call<1>(Wd, d, F.rows, cb, h, sl.r0, sl.n, F.out, F.epi, lane, wid,
                      *reinterpret_cast<MfmaLds*>(lds_raw));
      return;
    }
#pragma unroll 1
    for (int c0 = cb; c0 < cb + cols && c0 < d; c0 += kWideRows) {
#pragma unroll 1
      for (int tc = 0; tc < sl.n; tc += 16 * kDownNC) {
        const int rem = sl.n - tc;
        if (rem > 32)
          dn_wide<kDownNC>(Wd, d, F.rows, c0, h, sl.r0, sl.n, tc, F.out, F.epi, lane, wid,
                           *reinterpret_cast<WideLds<kDownNC, 1>*>(lds_raw));
        else if (rem > 16)
          dn_wide<2>(Wd, d, F.rows, c0, h, sl.r0, sl.n, tc, F.out, F.epi, lane, wid,
                     *reinterpret_cast<WideLds<2, 1>*>(lds_raw));
        else
          dn_wide<1>(Wd, d, F.rows, c0, h, sl.r0, sl.n, tc, F.out, F.epi, lane, wid,
                     *reinterpret_cast<WideLds<1, 1>*>(lds_raw));
      }
    }
  } else {
    // large groups, fp32 layers: the whole block on one 16-column tile
    const int c0 = tile * 16;
    if (c0 >= d) return;
#pragma unroll 1
    for (int q = wid * 4; q < wid * 4 + 4; q += 2)
#pragma unroll 1
      for (int tc = 0; tc < sl.n; tc += 8)
        dn_plain<2, 8>(Wd, d, F.rows, c0 + q, h, sl, tc, F.out, F.epi, lane);
  }
}

// Factorised form, between the private and the department down projections
// (DeaMoE section 3.2 collects every Z^{j,i} of department j for one W_d^j
// product; by linearity the Eq. (3) weights are applied before it):
//   zc[q][c] = sum over the slots s of token t (slot order) whose expert lies
//              in department J of row_weight[r] * z[r][c],  r = inv_perm[t*k+s]
// for pair q = (t, J).  One block per (256 columns, pair); pairs past the
// plan's count exit at once.
template <typename AT>
__global__ __launch_bounds__(kThreads) void pair_combine_kernel(PairCombineArgs a,
                                                                AT* __restrict__ zc) {
  const int c = blockIdx.x * kThreads + threadIdx.x;
  const int q = blockIdx.y;
  if (q >= *a.n_pairs || c >= a.cols) return;
  const int t = a.pair_token[q], J = a.pair_dept[q];
  if (t < 0 || t >= a.T) return;
  float acc = 0.f;
  for (int s = 0; s < a.k; ++s) {
    const int r = a.inv_perm[t * a.k + s];
    if (r >= 0 && r < a.max_rows && a.row_expert[r] / a.group == J)
      acc = fmaf(a.row_weight[r], a.z[(size_t)r * a.cols + c], acc);
  }
  store_act(zc + (size_t)q * a.cols + c, acc);
}

// One block per (256 columns, token): every thread one output element.
constexpr int kCombineBatch = 8;
constexpr int kCombineDeptList = kWave;  // departments listed per token at most
template <typename AT>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a, AT* __restrict__ y) {
  const int t = blockIdx.y;
  // past one batch of departments, the token's active ones, compacted by the
  // first wave (most of a token's department entries are empty), so the
  // column loop reads only them (DeaMoE on the DeepSeek-V3 geometry, 32
  // departments: combine 32.8 -> 14.1 us at 128 tokens, 8.6 -> 5.8 us at 16)
  __shared__ int dlist[kCombineDeptList];
  __shared__ float dscale[kCombineDeptList];
  __shared__ int dcount;
  const bool listed = a.dept_out && a.m > kCombineBatch && a.m <= kCombineDeptList;
  if (listed) {
    if (threadIdx.x < kWave) {
      const int J = threadIdx.x;
      const int r = J < a.m ? a.dept_inv[(size_t)t * a.m + J] : -1;
      const bool on = r >= 0 && r < a.max_dept_rows;
      const unsigned long long b = __ballot(on);
      if (on) {
        const int i = __popcll(b & ((1ull << J) - 1ull));
        dlist[i] = r;
        // no scales: the weights are already inside (factorised)
        dscale[i] = a.dept_scale ? a.dept_scale[r] : 1.f;
      }
      if (J == 0) dcount = __popcll(b);
    }
    __syncthreads();
  }
  const int c = blockIdx.x * kThreads + threadIdx.x;
  if (c >= a.d) return;
  // Slots (then departments) in order, kCombineBatch at a time: the batch's
  // row indices are read together, then its weights and rows (a missing row
  // reads row 0, and a select drops it), so a batch costs two round trips
  // instead of two per slot.
  constexpr int B = kCombineBatch;
  float acc = 0.f;
  if (a.row_out) {
    const int* ip = a.inv_perm + (size_t)t * a.k;
    for (int j0 = 0; j0 < a.k; j0 += B) {
      int r[B];
#pragma unroll
      for (int q = 0; q < B; ++q) r[q] = ip[min(j0 + q, a.k - 1)];
      float wv[B], ov[B];
      bool ok[B];
#pragma unroll
      for (int q = 0; q < B; ++q) {
        ok[q] = j0 + q < a.k && r[q] >= 0 && r[q] < a.max_rows;
        const int rr = ok[q] ? r[q] : 0;
        wv[q] = a.row_weight[rr];
        ov[q] = a.row_out[(size_t)rr * a.d + c];
      }
#pragma unroll
      for (int q = 0; q < B; ++q) acc = ok[q] ? fmaf(wv[q], ov[q], acc) : acc;
    }
  }
  if (listed) {
    const int n = dcount;
    for (int i0 = 0; i0 < n; i0 += B) {
      float ov[B];
#pragma unroll
      for (int q = 0; q < B; ++q) ov[q] = a.dept_out[(size_t)dlist[min(i0 + q, n - 1)] * a.d + c];
#pragma unroll
      for (int q = 0; q < B; ++q) acc = i0 + q < n ? fmaf(dscale[i0 + q], ov[q], acc) : acc;
    }
  } else if (a.dept_out) {
    const int* dp = a.dept_inv + (size_t)t * a.m;
    for (int J0 = 0; J0 < a.m; J0 += B) {
      int r[B];
#pragma unroll
      for (int q = 0; q < B; ++q) r[q] = dp[min(J0 + q, a.m - 1)];
      float wv[B], ov[B];
      bool ok[B];
#pragma unroll
      for (int q = 0; q < B; ++q) {
        ok[q] = J0 + q < a.m && r[q] >= 0 && r[q] < a.max_dept_rows;
        const int rr = ok[q] ? r[q] : 0;
        // no scales: the weights are already inside (factorised)
        wv[q] = a.dept_scale ? a.dept_scale[rr] : 1.f;
        ov[q] = a.dept_out[(size_t)rr * a.d + c];
      }
#pragma unroll
      for (int q = 0; q < B; ++q) acc = ok[q] ? fmaf(wv[q], ov[q], acc) : acc;
    }
  }
  if (a.shared_out) acc += a.shared_out[(size_t)t * a.d + c];
  store_act(y + (size_t)t * a.d + c, acc);
}

// FP8 (OCP E4M3) weight codes, used by the fused down + combine and the FP8
// expert kernels below.  Every E4M3 value is exactly a bf16 value, so
// v_cvt_scalef32_pk_bf16_fp8 with scale 1 widens two codes to a bf16 pair.
// Codes 4q .. 4q+3 of dword q as two bf16 pairs (byte 0 in the low half).
__device__ __forceinline__ void fp8x16_to_bf16(const u32x4_t& w, uint32_t (&o)[8]) {
  const uint32_t d4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    o[2 * q] = __builtin_bit_cast(uint32_t,
                                  __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d4[q], 1.0f, false));
    o[2 * q + 1] = __builtin_bit_cast(uint32_t,
                                      __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d4[q], 1.0f, true));
  }
}

// sum over 16 consecutive k of weight (widened codes) * activation, where
// the activations are 16 bf16 at p (16-byte aligned, LDS)
__device__ __forceinline__ float dot16(const uint32_t (&wb)[8], const bf16_t* p, float acc) {
  const u32x4_t a = *reinterpret_cast<const u32x4_t*>(p);
  const u32x4_t b = *reinterpret_cast<const u32x4_t*>(p + 8);
  acc = dot2_bf16(wb[0], a.x, acc);
  acc = dot2_bf16(wb[1], a.y, acc);
  acc = dot2_bf16(wb[2], a.z, acc);
  acc = dot2_bf16(wb[3], a.w, acc);
  acc = dot2_bf16(wb[4], b.x, acc);
  acc = dot2_bf16(wb[5], b.y, acc);
  acc = dot2_bf16(wb[6], b.z, acc);
  return dot2_bf16(wb[7], b.w, acc);
}

// ---------------------------------------------------------------------------
// Down projection with the combine as its epilogue, for batches of at most
// kTokInline tokens.  DeaMoE Eq. (3) sums each token's routing-weighted expert
// outputs, and W_down is linear, so output column c of token t is
//   y[t][c] = sum over groups g and rows j of g with token t of
//             w_{g,j} * (W_down[mat(g)][c] . h[row r_g + j])
// over the routed experts (w = routing weight), the department slices
// (w = c_{t,J}) and the shared expert (w = 1).  Wave c streams the weight rows
// W[mat][c] of every group of every family once, 16 bytes a lane per step,
// kDcRing steps ahead; each lane keeps one partial dot product per row of the
// current group and, when the group ends, adds it with the row's weight into
// its token's accumulator.  The accumulators are reduced over the wave once,
// at the end, and y is written in the layer dtype.  The groups' rows of h are
// staged in LDS for the whole block.  Summation order is fixed by the group
// order of the plan, so results do not depend on timing.
// ---------------------------------------------------------------------------
struct DcItem {
  const void* w;            // the group's matrix [d][rows] (bf16, or FP8 codes)
  uint32_t woff;            // byte offset of that matrix in the family's weights
  const float* scale;       // FP8: the matrix's per-column scales [d]; else nullptr
  int rows;                 // row length (elements)
  int nsteps;               // steps of 64 lanes x 8 elements per weight row
  int n;                    // rows of the group (0: invalid descriptor, streamed and unused)
  int hoff[kTokInline];     // LDS element offset of the group's row j of h
  int tok[kTokInline];      // token of row j
  float wt[kTokInline];     // weight of row j (0 past n)
  int thoff[kTokInline];    // per token t: LDS offset of the group's row of t (any row if none)
  float twt[kTokInline];    //   and its weight (0 if the group has no row of t)
};

size_t down_combine_lds_bytes(const DownCombineArgs& a) {
  return (((size_t)a.h_elems * 2 + 15) & ~(size_t)15) + (size_t)a.max_items * sizeof(DcItem);
}

constexpr int kDcLoads = 4;   // 16-byte weight loads in flight per lane
constexpr int kDcPrefetchMinD = 2048;  // first groups requested ahead of the table above this d
constexpr int kDcMaxSteps = kDcMaxRows / (8 * kWave);  // steps of the longest row

// Elements a lane takes per 16-byte step: 8 bf16 weights or 16 FP8 codes.
template <bool FP8> constexpr int dc_epl() { return FP8 ? 16 : 8; }

// Weight row of column c of group i < ie: NS steps of 64 lanes x 8 elements,
// through a buffer resource that spans exactly that row, so lanes past the
// row's end read zeros without a memory access; for i >= ie the resource is
// empty and every lane reads zeros.  The loads are thereby unconditional:
// a branch around them would make the compiler wait for all loads in flight
// before each use instead of only the oldest.

// FP8: also the column's scale (a scalar load, issued as far ahead).
template <int NS, bool FP8>
__device__ __forceinline__ void dc_load(const DcItem* items, int i, int ie, int c, int lane,
                                        u32x4_t (&dst)[NS], float& scl) {
  constexpr int EPL = dc_epl<FP8>(), ESZ = FP8 ? 1 : 2;
  const DcItem& it = items[min(i, ie - 1)];
  const int rows = uni(it.rows);
  const char* w = static_cast<const char*>(uni(it.w)) + (size_t)c * rows * ESZ;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(w), (short)0, i < ie ? rows * ESZ : 0, kGfx9BufferDword3);
#pragma unroll
  for (int s = 0; s < NS; ++s)
    dst[s] = __builtin_bit_cast(
        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                     rs, (lane * EPL + s * EPL * kWave) * ESZ, 0, kCpolNt));
  if constexpr (FP8) scl = *as_global<float>(uni(it.scale) + c);
}

// Group i's weight row of column c (matrix `mat` of the family, read from
// its work descriptor before the group table exists and clamped into the
// family, so a slot past the count -- whose data is never consumed -- still
// reads inside the weights), bf16.  Slots below 4 of a work list are 128
// bytes: inside its region, which is padded to 256 bytes like every
// workspace region.
template <int NS>
__device__ __forceinline__ void dc_prefetch(const DcFamily& F, int i, int mat, int d, int c,
                                            int lane, u32x4_t (&dst)[NS]) {
  const int rows = F.rows;
  const char* w = static_cast<const char*>(F.down) + ((size_t)mat * d + c) * rows * 2;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(w), (short)0, i < F.max_items ? rows * 2 : 0, kGfx9BufferDword3);
#pragma unroll
  for (int j = 0; j < NS; ++j)
    dst[j] = __builtin_bit_cast(
        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, (lane * 8 + j * 8 * kWave) * 2, 0,
                                                       kCpolNt));
}

// Dot products of group i's weight row with its rows of h (LDS), folded into
// the token accumulators with the rows' weights; nothing outside [ib, ie).
template <int NS, bool FP8>
__device__ __forceinline__ void dc_consume(const DcItem* items, int i, int ib, int ie,
                                           const bf16_t* hl,
                                           int lane, const u32x4_t (&wv)[NS], float scl,
                                           float (&acc)[kTokInline]) {
  constexpr int EPL = dc_epl<FP8>();
  const DcItem& it = items[min(max(i, ib), ie - 1)];
  const int rows = uni(it.rows), n = (i >= ib && i < ie) ? uni(it.n) : 0;
#pragma unroll
  for (int j = 0; j < kTokInline; ++j) {
    if (j < n) {
      const int ho = uni(it.hoff[j]);
      float part = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        // past the row's end the weights are zero and h is read at the row's
        // last EPL elements (finite values)
        const int e = min(lane * EPL + s * EPL * kWave, rows - EPL);
        if constexpr (FP8) {
          uint32_t wb[8];
          fp8x16_to_bf16(wv[s], wb);
          part = dot16(wb, hl + ho + e, part);
        } else {
          Raw8<bf16_t> w8;
          w8.u = wv[s];
          part = dot8(w8, *reinterpret_cast<const X8<bf16_t>*>(hl + ho + e), part);
        }
      }
      // a weight of 0 for the other tokens rather than a branch per token
      // keeps acc in registers; FP8 rows carry their column's scale
      const int tk = uni(it.tok[j]);
      const float wt = FP8 ? uni(it.wt[j]) * scl : uni(it.wt[j]);
#pragma unroll
      for (int t = 0; t < kTokInline; ++t) acc[t] = fmaf(tk == t ? wt : 0.f, part, acc[t]);
    }
  }
}

// Groups [ib, ie) of one family (rows of at most NS steps), D groups of loads
// ahead of the one being used.
template <int NS> constexpr int dc_ahead() { return kDcLoads / NS > 0 ? kDcLoads / NS : 1; }
template <int NS, bool FP8, bool PRE = false>
__device__ __forceinline__ void dc_family(const DcItem* items, int ib, int ie, int c,
                                          const bf16_t* hl, int lane, float (&acc)[kTokInline],
                                          const u32x4_t (*pre)[NS] = nullptr) {
  constexpr int D = dc_ahead<NS>();
  // The first pass only loads (groups before ib are not consumed): with no
  // loads ahead of the loop, the buffers need no copies on entry, and each
  // use waits only for its own group's loads.  PRE: groups ib .. ib + D - 1
  // were requested before the loop (into pre), so that pass is skipped.
  u32x4_t buf[D][NS];
  float scl[D];
#pragma unroll
  for (int q = 0; q < D; ++q) scl[q] = 1.f;
  if constexpr (PRE) {
#pragma unroll
    for (int q = 0; q < D; ++q)
#pragma unroll
      for (int j = 0; j < NS; ++j) buf[q][j] = pre[q][j];
  }
  for (int i0 = PRE ? ib : ib - D; i0 < ie; i0 += D) {
#pragma unroll
    for (int q = 0; q < D; ++q) {
      dc_consume<NS, FP8>(items, i0 + q, ib, ie, hl, lane, buf[q], scl[q], acc);
      dc_load<NS, FP8>(items, i0 + q + D, ie, c, lane, buf[q], scl[q]);
    }
  }
}

// Groups [ib, ie) of a bf16 family whose rows are LPI * 8 elements (LPI = 16
// or 32 lanes): one wave load takes column c's row of 64 / LPI groups at
// once, lane l serving group i + l / LPI.  The loads go through a buffer
// resource spanning the family's weights (`wbase`, `wbytes`), so a lane past
// the last group reads zeros without a memory access; every lane folds its
// own group's rows of h into the token accumulators (the weight of a lane
// outside [ib, ie) is 0), and the wave reduction at the end adds the lanes.
template <int LPI>
__device__ __forceinline__ void dcp_load(const DcItem* items, int i, int ie, int c, int lane,
                                         __amdgpu_buffer_rsrc_t rs, int rows, u32x4_t& dst) {
  const int gi = i + lane / LPI;
  const uint32_t off = gi < ie ? items[min(gi, ie - 1)].woff + (uint32_t)(c * rows * 2) +
                                     (uint32_t)((lane % LPI) * 16)
                               : kDcOob;
  dst = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kCpolNt));
}
template <int LPI>
__device__ __forceinline__ void dcp_consume(const DcItem* items, int i, int ib, int ie,
                                            const bf16_t* hl, int lane, const u32x4_t& wv,
                                            float (&acc)[kTokInline]) {
  const int gi = i + lane / LPI;
  const bool ok = gi >= ib && gi < ie;
  const DcItem& it = items[min(max(gi, ib), ie - 1)];
  const int e = (lane % LPI) * 8;
  Raw8<bf16_t> w8;
  w8.u = wv;
#pragma unroll
  for (int t = 0; t < kTokInline; ++t) {
    // (a lane outside [ib, ie) may hold a not-yet-loaded buffer: its dot
    // product is dropped by the select, never multiplied)
    const float dp = dot8(w8, *reinterpret_cast<const X8<bf16_t>*>(hl + it.thoff[t] + e), 0.f);
    acc[t] = fmaf(ok ? it.twt[t] : 0.f, ok ? dp : 0.f, acc[t]);
  }
}
template <int LPI>
__device__ __forceinline__ void dc_family_packed(const DcItem* items, int ib, int ie, int c,
                                                 const bf16_t* hl, int lane, const DcFamily& F,
                                                 int d, float (&acc)[kTokInline]) {
  constexpr int G = kWave / LPI, D = kDcLoads;
  const int rows = F.rows;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(F.down), (short)0, (int)((size_t)F.n_mats * F.rows * d * 2),
      kGfx9BufferDword3);
  u32x4_t buf[D];
  for (int i0 = ib - D * G; i0 < ie; i0 += D * G) {
#pragma unroll
    for (int q = 0; q < D; ++q) {
      dcp_consume<LPI>(items, i0 + q * G, ib, ie, hl, lane, buf[q], acc);
      dcp_load<LPI>(items, i0 + (q + D) * G, ie, c, lane, rs, rows, buf[q]);
    }
  }
}

// (built for 8 waves per SIMD -- four 8-wave blocks per CU -- which the
// register budget of 64 reaches without spills)
// NS0 > 0 (bf16): the first family takes dc_family<NS0>, and each wave
// requests its first groups' weight rows straight from the work descriptors
// before the group table is built, so their HBM latency overlaps the table
// and the staging of h instead of following them.
template <bool FP8, int NS0>
__global__ __launch_bounds__(kDcWaves * kWave) __attribute__((amdgpu_waves_per_eu(8, 8)))
void down_combine_kernel(DownCombineArgs a, bf16_t* __restrict__ y) {
  extern __shared__ __align__(16) unsigned char dc_lds[];
  bf16_t* hl = reinterpret_cast<bf16_t*>(dc_lds);
  DcItem* items =
      reinterpret_cast<DcItem*>(dc_lds + (((size_t)a.h_elems * 2 + 15) & ~(size_t)15));
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int T = a.T, d = a.d;
  constexpr int STEP = 8 * kWave;  // elements of a weight row per step
  constexpr bool PRE = !FP8 && NS0 > 0;
  constexpr int NSP = NS0 > 0 ? NS0 : 1;
  const int c = uni((int)(blockIdx.x * kDcWaves) + wid);  // wave-uniform: scalar resource base
  u32x4_t pre[dc_ahead<NSP>()][NSP];
  if constexpr (PRE) {
    // the descriptors first, then every row: one round trip for the
    // descriptors in all
    constexpr int DP = dc_ahead<NSP>();
    int mat[DP];
    if (a.f[0].work) {
      const auto wv = as_global<u32x4_t>(a.f[0].work);
      u32x4_t w[DP];
#pragma unroll
      for (int q = 0; q < DP; ++q) w[q] = wv[2 * q];
#pragma unroll
      for (int q = 0; q < DP; ++q) mat[q] = min(max(uni((int)w[q].x), 0), a.f[0].n_mats - 1);
    } else {
#pragma unroll
      for (int q = 0; q < DP; ++q) mat[q] = 0;
    }
#pragma unroll
    for (int q = 0; q < dc_ahead<NSP>(); ++q)
      dc_prefetch<NSP>(a.f[0], q, mat[q], d, min(c, d - 1), lane, pre[q]);
  }
  // The group table (descriptors checked against the family's bounds and the
  // rows of h in use), and the staging of the rows of h.  Nothing here waits
  // for anything else: the counts, every descriptor slot up to the host's
  // bound and every row of h the step can use (family f's rows [0,
  // max_hrows) are contiguous in global memory and go to hl + lds_off) are
  // all requested at once, and slots past the count are simply not consumed.
  // Family f's table entries start at fb[f] (the sum of the earlier
  // families' bounds) and end at fe[f].
  int fb[kDcFamilies], fe[kDcFamilies];
  int ib = 0;
#pragma unroll
  for (int fi = 0; fi < kDcFamilies; ++fi) {
    fb[fi] = fe[fi] = ib;
    if (fi < a.nf) {
      const DcFamily& F = a.f[fi];
      const int nh = F.n_hrows ? F.max_hrows : min(T, F.max_hrows);  // rows staged
      const int nmax = F.work ? F.max_items : 1;
      // (the count read back as a wave-uniform value: the group loop bounds
      // and the weight-row resources built from it stay scalar)
      const int nf = uni(F.work ? min(max(*F.n_items, 0), F.max_items) : 1);
      const int nu = uni(F.n_hrows ? min(max(*F.n_hrows, 0), F.max_hrows) : nh);  // rows in use
      const size_t ms = (size_t)d * F.rows;
      const int nch = nh * (F.rows / 8);  // 16-byte chunks of the rows staged
      const bf16_t* src = static_cast<const bf16_t*>(F.h);
      for (int q = wid; q * kWave < nch; q += kDcWaves) {
        const int ch = q * kWave + lane;
        if (ch < nch)
          __builtin_amdgcn_global_load_lds(src + (size_t)ch * 8,
                                           (lds_void_t*)(hl + F.lds_off + q * STEP), 16, 0, 0);
      }
      for (int i = tid; i < nmax; i += kDcWaves * kWave) {
        int mat = 0, r0 = 0, n = 0;
        int tk[kTokInline] = {0, 1, 2, 3};
        if (F.work) {
          // the descriptor as two 16-byte vectors (a struct copy would go
          // through the private stack)
          const u32x4_t* wv = reinterpret_cast<const u32x4_t*>(F.work + i);
          const u32x4_t w0 = wv[0], w1 = wv[1];
          const int dm = (int)w0.x, dr = (int)w0.y, dn = (int)w0.z;
          if (i < nf && dm >= 0 && dm < F.n_mats && dr >= 0 && dn >= 1 && dn <= kTokInline &&
              dn <= nu - dr) {
            mat = dm;
            r0 = dr;
            n = dn;
            tk[0] = (int)w0.w;
            tk[1] = (int)w1.x;
            tk[2] = (int)w1.y;
            tk[3] = (int)w1.z;
          }
        } else {
          n = min(min(T, kTokInline), nu);  // the shared expert: row t is token t
        }
        DcItem it;
        it.w = static_cast<const char*>(F.down) + (size_t)mat * ms * (FP8 ? 1 : 2);
        it.woff = (uint32_t)((size_t)mat * ms * (FP8 ? 1 : 2));
        it.scale = FP8 ? F.down_scale + (size_t)mat * d : nullptr;
        it.rows = F.rows;
        it.nsteps = (F.rows + dc_epl<FP8>() * kWave - 1) / (dc_epl<FP8>() * kWave);
        it.n = n;
#pragma unroll
        for (int j = 0; j < kTokInline; ++j) {
          it.hoff[j] = F.lds_off + (r0 + min(j, max(n - 1, 0))) * F.rows;
          it.tok[j] = min(max(tk[j], 0), T - 1);
          it.wt[j] = j < n ? (F.wrow ? F.wrow[r0 + j] : 1.f) : 0.f;
        }
        // the same by token (a group's rows belong to distinct tokens)
#pragma unroll
        for (int t = 0; t < kTokInline; ++t) {
          it.thoff[t] = it.hoff[0];
          it.twt[t] = 0.f;
#pragma unroll
          for (int j = 0; j < kTokInline; ++j)
            if (j < n && it.tok[j] == t) {
              it.thoff[t] = it.hoff[j];
              it.twt[t] = it.wt[j];
            }
        }
        items[ib + i] = it;
      }
      fe[fi] = ib + nf;
      ib += nmax;
    }
  }
  // every wave's staged rows have landed, and the table is complete, for the block
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (c >= d) return;
  float acc[kTokInline];
#pragma unroll
  for (int t = 0; t < kTokInline; ++t) acc[t] = 0.f;
#pragma unroll
  for (int fi = 0; fi < kDcFamilies; ++fi) {
    if (fi < a.nf && fb[fi] < fe[fi]) {
      constexpr int SE = dc_epl<FP8>() * kWave;  // elements per step
      const int ns = (a.f[fi].rows + SE - 1) / SE;
      const int rows = a.f[fi].rows;
      // (packed loads address the family's weights by 32-bit byte offsets)
      const bool packable = !FP8 && (size_t)a.f[fi].n_mats * rows * d * 2 < (size_t)kDcOob;
      if (PRE && fi == 0)
        dc_family<NSP, FP8, true>(items, fb[fi], fe[fi], c, hl, lane, acc, pre);
      else if (packable && rows == 16 * 8)
        dc_family_packed<16>(items, fb[fi], fe[fi], c, hl, lane, a.f[fi], d, acc);
      else if (packable && rows == 32 * 8)
        dc_family_packed<32>(items, fb[fi], fe[fi], c, hl, lane, a.f[fi], d, acc);
      else if (ns <= 1)
        dc_family<1, FP8>(items, fb[fi], fe[fi], c, hl, lane, acc);
      else if (ns == 2 || FP8)
        dc_family<2, FP8>(items, fb[fi], fe[fi], c, hl, lane, acc);
      else if (ns == 3)
        dc_family<3, FP8>(items, fb[fi], fe[fi], c, hl, lane, acc);
      else
        dc_family<kDcMaxSteps, FP8>(items, fb[fi], fe[fi], c, hl, lane, acc);
    }
  }
  // lane 16 t holds token t's sum
  float v[kTokInline];
#pragma unroll
  for (int j = 0; j < kTokInline; ++j) v[j] = acc[j];
  wave_reduce_scatter<kTokInline>(v, lane);
  const int t = lane >> 4;
  if ((lane & 15) == 0 && t < T) y[(size_t)t * d + c] = f32_to_bf16(v[0]);
}

// ---------------------------------------------------------------------------
// FP8 expert weights: OCP E4M3 codes with one fp32 scale per output row.
// A lane reads 16 codes (16 bytes) of a weight row per step.  Every E4M3
// value is exactly a bf16 value, so v_cvt_scalef32_pk_bf16_fp8 with scale 1
// widens each pair of codes to a bf16 pair and the packed bf16 dot
// instruction multiplies them with the bf16 activations, summing in fp32; the
// row's scale multiplies the finished sum.  Groups of any size are taken
// kTokInline tokens at a time, their activation rows (gate/up) or rows of h
// (down) staged in LDS once per chunk, so the weights of a group of more
// than kTokInline rows are re-read from the cache for each further chunk;
// larger batches take the matrix-core tiles further below instead.
// ---------------------------------------------------------------------------


// A buffer resource spanning one FP8 matrix: a load at a byte offset at or
// past `bytes` returns zeros without a memory access, so a lane past its
// row's end (or a row past the matrix end) takes an out-of-range offset
// instead of a branch, and every load is unconditional -- the compiler then
// waits for each step's own loads only, not for all loads in flight.
constexpr uint32_t kFp8Oob = 0x80000000u;  // beyond every FP8 matrix (< 2^31 bytes)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t fp8_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kGfx9BufferDword3);
}
// POL: cache policy -- non-temporal where every code is read once (the
// GEMVs: 7-9% faster steps at 1-16 tokens), the default where a 64-row tile
// may read its codes once per token pass (non-temporal there: DeepSeek-V3-
// shaped batch 128 1271 -> 1503 us).
template <int POL = 0>
__device__ __forceinline__ u32x4_t fp8_ld(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, POL));
}

// Gate and up rows i0 .. i0 + RPW - 1 (one wave) of matrix `mat` for every
// row of the group, kTokInline tokens a chunk: h[r0 + t][i] =
// SiLU(sg_i * g_t) * (su_i * u_t).  A wave takes RPW consecutive rows so that
// it streams as many bytes as a bf16 wave of one row; its loads run R steps
// ahead across the row boundaries (the steps after the last row are out of
// range).  Rows past the matrix end store nothing.
template <int RPW, int R>
__device__ __forceinline__ void gu_fp8(const Family& F, const Slot& sl, const bf16_t* __restrict__ x,
                                       int d, int i0, int nts, bf16_t* __restrict__ xl, int lane,
                                       int wid) {
  constexpr int NT = kTokInline, STEP = 16 * kWave;
  const int rows = F.rows, n = sl.n;
  const size_t ms = (size_t)rows * d;
  const __amdgpu_buffer_rsrc_t rsg =
      fp8_rsrc(static_cast<const uint8_t*>(F.gate) + (size_t)sl.mat * ms, (uint32_t)ms);
  const __amdgpu_buffer_rsrc_t rsu =
      fp8_rsrc(static_cast<const uint8_t*>(F.up) + (size_t)sl.mat * ms, (uint32_t)ms);
  const float* gsc = F.gate_scale + (size_t)sl.mat * rows;
  const float* usc = F.up_scale + (size_t)sl.mat * rows;
  const int nsteps = (d + STEP - 1) / STEP;
  const int nouter = (nsteps + R - 1) / R;
  const int spr = nouter * R;  // steps per row, padded to the ring
  // byte offset of flat step f = k * spr + s (row i0 + k) for this lane
  auto off = [&](int f) -> uint32_t {
    const int k = f / spr, e = lane * 16 + (f - k * spr) * STEP;
    return (k < RPW && i0 + k < rows && e < d) ? (uint32_t)((i0 + k) * d + e) : kFp8Oob;
  };
  const bf16_t* xg = F.x_gate ? static_cast<const bf16_t*>(F.x_gate) : x;
  bf16_t* h = static_cast<bf16_t*>(F.h);
#pragma unroll 1
  for (int tc = 0; tc < n; tc += nts) {
    const int nv = min(nts, n - tc);
    u32x4_t rg[R], ru[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      rg[r] = fp8_ld<kCpolNt>(rsg, off(r));
      ru[r] = fp8_ld<kCpolNt>(rsu, off(r));
    }
    // the chunk's activation rows, one 1 KB wave instruction at a time
    {
      constexpr int EPI = 8 * kWave;  // bf16 elements per wave instruction
      const int per_row = (d + EPI - 1) / EPI, total = nv * per_row;
      for (int q = wid; q < total; q += kWaves) {
        const int t = q / per_row, c0 = (q - t * per_row) * EPI;
        const int c = c0 + lane * 8;
        // row tc + t of the group (inline tokens are indexed from the
        // group's first row, so the chunk offset goes into the row index)
        const int tok = slot_token(sl, F.grp_token, 0, tc + t, n, F.in_rows);
        if (c < d)
          __builtin_amdgcn_global_load_lds(xg + (size_t)tok * d + c,
                                           (lds_void_t*)(xl + (size_t)t * d + c0), 16, 0, 0);
      }
    }
    stage_wait();
    float res[RPW], resu[RPW];
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
      float ag[NT], au[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) ag[t] = au[t] = 0.f;
      for (int o = 0; o < nouter; ++o) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int sidx = o * R + r;
          // past the row's end the weights are zero and x is read at the
          // row's last 16 elements (finite values)
          const int xo = min(lane * 16 + sidx * STEP, d - 16);
          uint32_t wg[8], wu[8];
          fp8x16_to_bf16(rg[r], wg);
          fp8x16_to_bf16(ru[r], wu);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            if (t < nv) {
              const bf16_t* xp = xl + (size_t)t * d + xo;
              ag[t] = dot16(wg, xp, ag[t]);
              au[t] = dot16(wu, xp, au[t]);
            }
          }
          const int f = k * spr + sidx + R;
          rg[r] = fp8_ld<kCpolNt>(rsg, off(f));
          ru[r] = fp8_ld<kCpolNt>(rsu, off(f));
        }
      }
      constexpr int N = 2 * NT;
      float v[N];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        v[t] = ag[t];
        v[NT + t] = au[t];
      }
      group_reduce_scatter<N, 64>(v, lane);
      res[k] = v[0];
      resu[k] = xor32(v[0], lane);  // gate index t and up index t + NT: lanes l, l ^ 32
    }
    constexpr int SH = 6 - Log2<2 * NT>::value;
    const int t = lane >> SH;
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
      const int i = i0 + k;
      if (t < NT && (lane & ((1 << SH) - 1)) == 0 && t < nv && i < rows)
        store_act(h + (size_t)(sl.r0 + tc + t) * rows + i,
                  silu(gsc[i] * res[k]) * (usc[i] * resu[k]));
    }
    __syncthreads();  // every wave is done with the staged rows before the next chunk
  }
}

// ---- FP8 layers at batches past kTokInline: 64-row (gate/up) or 64-column
// (down) matrix-core tiles, 16*NC tokens a pass, so each weight byte is read
// once per pass rather than once per kTokInline tokens.  A step covers 128 codes
// of K: lane group g = l/16 reads the 32 consecutive codes 32g .. 32g + 31 of
// its row (two 16-byte loads through the matrix's buffer resource) and widens
// them to four bf16 fragments; the activations are staged in the same k
// order (H = 4).  The row (gate/up) or column (down) scale multiplies the
// finished sum.
constexpr int kWideK8 = 128;

// Codes 8j .. 8j + 7 of a 16-byte load (j = 0, 1) as one bf16x8 fragment.
__device__ __forceinline__ u32x4_t fp8x8_frag(const u32x4_t& w, int j) {
  const uint32_t a = j == 0 ? w.x : w.z, b = j == 0 ? w.y : w.w;
  u32x4_t o;
  o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a, 1.0f, false));
  o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a, 1.0f, true));
  o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b, 1.0f, false));
  o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b, 1.0f, true));
  return o;
}

// Shared by both FP8 tiles: acc[m][c] += A_m (rows of codes, `rs[m]` at
// offsets aoff(k)) x B (16*NC inputs staged from `in`), over K in 128-code
// steps.
template <int NC, int NM, typename AOff>
__device__ __forceinline__ void fp8_wide_loop(const __amdgpu_buffer_rsrc_t (&rs)[NM], AOff aoff,
                                              const WideIn<NC, 1, 4>& in, int K, int g,
                                              int lane, WideLds<NC, 1, 4>& lds,
                                              f32x4_t (&acc)[NM][NC]) {
  constexpr int R = WideIn<NC, 1, 4>::R;
  u32x4_t rx[2][R], ra[2][NM][2];
  auto request = [&](auto S, int k0) {
    constexpr int s = decltype(S)::value;
    wide_load<NC, 1, 4>(rx[s], in, k0, K);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t o = aoff(k0 + 32 * g + 16 * j);
#pragma unroll
      for (int m = 0; m < NM; ++m) ra[s][m][j] = fp8_ld(rs[m], o);
    }
  };
  auto use = [&](auto S) {
    constexpr int s = decltype(S)::value;
    wide_stage<NC, 1, 4>(lds, s, rx[s]);
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      u32x4_t a[NM];
#pragma unroll
      for (int m = 0; m < NM; ++m) a[m] = fp8x8_frag(ra[s][m][hh >> 1], hh & 1);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u32x4_t b = lds.x[s][(c * 4 + hh) * kWave + lane];
#pragma unroll
        for (int m = 0; m < NM; ++m)
          acc[m][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[m]), as_bf16x8(b),
                                                              acc[m][c], 0, 0, 0);
      }
    }
  };
  const int nk = (K + kWideK8 - 1) / kWideK8;
  const Slot0 s0;
  const Slot1 s1;
  request(s0, 0);
  for (int it = 0; it < nk; it += 2) {
    if (it + 1 < nk) request(s1, (it + 1) * kWideK8);
    use(s0);
    if (it + 1 < nk) {
      if (it + 2 < nk) request(s0, (it + 2) * kWideK8);
      use(s1);
    }
  }
}

// 64 rows (i0..) of FP8 gate and up (matrix bases Wg, Wu; row scales gsc,
// usc) against 16*NC tokens (rows tc.. of the group [r0, r0 + n)):
// h[r0 + t][i] = SiLU(sg_i * g_t) * (su_i * u_t).
template <int NC>
__device__ __forceinline__ void gu_wide_fp8(
    const uint8_t* __restrict__ Wg, const uint8_t* __restrict__ Wu,
    const float* __restrict__ gsc, const float* __restrict__ usc, int d, int rows, int i0,
    const bf16_t* __restrict__ x, int in_rows, int r0, int n, const int* grp_token, int tc,
    bf16_t* __restrict__ h, int lane, int wid, WideLds<NC, 1, 4>& lds) {
  const int r16 = lane & 15, g = lane >> 4;
  const uint32_t ms = (uint32_t)((size_t)rows * d);
  const __amdgpu_buffer_rsrc_t rs[2] = {fp8_rsrc(Wg, ms), fp8_rsrc(Wu, ms)};
  const int wr = i0 + 16 * wid + r16;  // this lane's weight row
  auto aoff = [&](int k) -> uint32_t {
    return (wr < rows && k < d) ? (uint32_t)(wr * d + k) : kFp8Oob;
  };
  WideIn<NC, 1, 4> in;
  const bf16_t* const src[1] = {x};
  wide_inputs<NC, 1, 4>(in, src, d, tc, n, [&](int t) {
    const int tok = grp_token ? grp_token[r0 + t] : t;
    return min(max(tok, 0), in_rows - 1);
  });
  f32x4_t acc[2][NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[0][c] = acc[1][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  fp8_wide_loop<NC, 2>(rs, aoff, in, d, g, lane, lds, acc);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int t = tc + c * 16 + r16;
    if (t < n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = i0 + 16 * wid + 4 * g + i;
        if (rr < rows)
          store_act(h + (size_t)(r0 + t) * rows + rr,
                    silu(gsc[rr] * acc[0][c][i]) * (usc[rr] * acc[1][c][i]));
      }
    }
  }
  __syncthreads();  // the buffers are free for the next pass
}

// 64 output columns (c0..) of FP8 down (matrix base Wd, column scales dsc)
// against 16*NC rows of h (rows tc.. of the group):
// out[r0 + t][c] = sd_c * (W_down[c] . h[r0 + t]).
template <int NC>
__device__ __forceinline__ void dn_wide_fp8(const uint8_t* __restrict__ Wd,
                                                      const float* __restrict__ dsc, int d,
                                                      int rows, int c0,
                                                      const bf16_t* __restrict__ h, int r0,
                                                      int n, int tc, float* __restrict__ out,
                                                      int lane, int wid,
                                                      WideLds<NC, 1, 4>& lds) {
  const int r16 = lane & 15, g = lane >> 4;
  const __amdgpu_buffer_rsrc_t rs[1] = {fp8_rsrc(Wd, (uint32_t)((size_t)rows * d))};
  const int wc = c0 + 16 * wid + r16;  // this lane's weight row (output column)
  auto aoff = [&](int k) -> uint32_t {
    return (wc < d && k < rows) ? (uint32_t)(wc * rows + k) : kFp8Oob;
  };
  WideIn<NC, 1, 4> in;
  const bf16_t* const src[1] = {h};
  wide_inputs<NC, 1, 4>(in, src, rows, tc, n, [&](int t) { return r0 + t; });
  f32x4_t acc[1][NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[0][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  fp8_wide_loop<NC, 1>(rs, aoff, in, rows, g, lane, lds, acc);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int t = tc + c * 16 + r16;
    if (t < n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = c0 + 16 * wid + 4 * g + i;
        if (col < d) out[(size_t)(r0 + t) * d + col] = dsc[col] * acc[0][c][i];
      }
    }
  }
  __syncthreads();
}

constexpr size_t kFp8WideLds = sizeof(WideLds<2, 1, 4>);

constexpr int kFp8Rows = kFp8RowsPerWave;

// R: 16-code steps requested ahead per row (more for long rows, whose
// staged activations leave room for fewer waves per CU)
template <int R>
__global__ __launch_bounds__(kThreads) void gateup_fp8_kernel(FamilySet set,
                                                             const bf16_t* __restrict__ x, int T,
                                                             int d, int nts) {
  extern __shared__ __align__(16) unsigned char fp8_lds[];
  int tile;
  const Family& F = block_part(set, tile);
  Slot sl;
  if (!map_slot(F, T, sl, tile)) return;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  // the wave's first row, wave-uniform (the weight resources are scalar)
  const int i0 = __builtin_amdgcn_readfirstlane((tile * kWaves + wid) * kFp8Rows);
  gu_fp8<kFp8Rows, R>(F, sl, x, d, i0, nts, reinterpret_cast<bf16_t*>(fp8_lds), lane, wid);
}

// Down columns cb + q*G + g (lane group g of LPR lanes, column group q < CG,
// G = 64 / LPR) of matrix `mat` for every row of the group, kTokInline rows
// of h a chunk: out[r0 + t][c] = sd[c] * (W_down[c] . h[r0 + t]).  CG column
// groups per wave give it as many bytes as a bf16 wave.  Loads are
// unconditional (out-of-range offsets past a row's end), R steps ahead.
template <int LPR, int CG, int R>
__device__ __forceinline__ void dn_fp8(const Family& F, const Slot& sl, int d, int cb, int nts,
                                       bf16_t* __restrict__ hl, int lane, int wid) {
  constexpr int NT = kTokInline, STEP = 16 * LPR, G = 64 / LPR;
  const int rows = F.rows, n = sl.n;
  const int g = lane / LPR, j = lane - g * LPR;
  const size_t ms = (size_t)rows * d;
  const __amdgpu_buffer_rsrc_t rs =
      fp8_rsrc(static_cast<const uint8_t*>(F.down) + (size_t)sl.mat * ms, (uint32_t)ms);
  uint32_t cbase[CG];
  float sd[CG];
#pragma unroll
  for (int q = 0; q < CG; ++q) {
    const int c = cb + q * G + g;
    cbase[q] = c < d ? (uint32_t)(c * rows + j * 16) : kFp8Oob;
    sd[q] = F.down_scale[(size_t)sl.mat * d + min(c, d - 1)];
  }
  const int rl = rows - j * 16;  // this lane's codes: j*16 + k*STEP for k*STEP < rl
  const int nouter = ((rows + STEP - 1) / STEP + R - 1) / R;
  auto off = [&](int q, int sidx) -> uint32_t {
    return (sidx * STEP < rl && cbase[q] != kFp8Oob) ? cbase[q] + sidx * STEP : kFp8Oob;
  };
  const bf16_t* h = static_cast<const bf16_t*>(F.h);
#pragma unroll 1
  for (int tc = 0; tc < n; tc += nts) {
    const int nv = min(nts, n - tc);
    u32x4_t rw[R][CG];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int q = 0; q < CG; ++q) rw[r][q] = fp8_ld<kCpolNt>(rs, off(q, r));
    {
      constexpr int EPI = 8 * kWave;
      const int per_row = (rows + EPI - 1) / EPI, total = nv * per_row;
      for (int q = wid; q < total; q += kWaves) {
        const int t = q / per_row, c0 = (q - t * per_row) * EPI;
        const int e = c0 + lane * 8;
        if (e < rows)
          __builtin_amdgcn_global_load_lds(h + (size_t)(sl.r0 + tc + t) * rows + e,
                                           (lds_void_t*)(hl + (size_t)t * rows + c0), 16, 0, 0);
      }
    }
    stage_wait();
    float acc[CG][NT];
#pragma unroll
    for (int q = 0; q < CG; ++q)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[q][t] = 0.f;
    for (int o = 0; o < nouter; ++o) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int sidx = o * R + r;
        const int ho = min(j * 16 + sidx * STEP, rows - 16);
#pragma unroll
        for (int q = 0; q < CG; ++q) {
          uint32_t wb[8];
          fp8x16_to_bf16(rw[r][q], wb);
#pragma unroll
          for (int t = 0; t < NT; ++t)
            if (t < nv) acc[q][t] = dot16(wb, hl + (size_t)t * rows + ho, acc[q][t]);
          rw[r][q] = fp8_ld<kCpolNt>(rs, off(q, sidx + R));
        }
      }
    }
    constexpr int N = CG * NT;
    float v[N];
#pragma unroll
    for (int q = 0; q < CG; ++q)
#pragma unroll
      for (int t = 0; t < NT; ++t) v[q * NT + t] = acc[q][t];
    group_reduce_scatter<N, LPR>(v, lane);
    if constexpr (N >= LPR) {
      constexpr int PER = N / LPR;
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int idx = j * PER + p, q = idx / NT, t = idx - (idx / NT) * NT;
        const int c = cb + q * G + g;
        if (t < nv && c < d) F.out[(size_t)(sl.r0 + tc + t) * d + c] = sd[q] * v[p];
      }
    } else {
      // lane j of the group holds value index j / (LPR / N)
      constexpr int SPAN = LPR / N;
      const int idx = j / SPAN, q = idx / NT, t = idx - (idx / NT) * NT;
      const int c = cb + q * G + g;
      float sc = sd[0];
#pragma unroll
      for (int qq = 1; qq < CG; ++qq) sc = q == qq ? sd[qq] : sc;
      if (j % SPAN == 0 && t < nv && c < d) F.out[(size_t)(sl.r0 + tc + t) * d + c] = sc * v[0];
    }
    __syncthreads();
  }
}

constexpr int kFp8ColGroups = kFp8DownColGroups;

template <int LPR>
__global__ __launch_bounds__(kThreads) void down_fp8_kernel(FamilySet set, int T, int d, int nts) {
  extern __shared__ __align__(16) unsigned char fp8_lds[];
  int tile;
  const Family& F = block_part(set, tile);
  Slot sl;
  if (!map_slot(F, T, sl, tile)) return;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  constexpr int CPW = kFp8ColGroups * (64 / LPR);  // columns per wave
  const int cb = __builtin_amdgcn_readfirstlane(tile * (kWaves * CPW) + wid * CPW);
  dn_fp8<LPR, kFp8ColGroups, kFp8DnAhead>(F, sl, d, cb, nts, reinterpret_cast<bf16_t*>(fp8_lds),
                                          lane, wid);
}

// FP8 layers at larger batches: every group (small or large) on 64-row
// matrix-core tiles, the whole block on one tile.  Held to four waves per
// SIMD (128 registers, no spills; measured 0.2-1.7% faster than three).
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void gateup_fp8_wide_kernel(FamilySet set,
                                                                  const bf16_t* __restrict__ x,
                                                                  int T, int d) {
  __shared__ __align__(16) unsigned char fp8_lds[kFp8WideLds];
  int tile;
  const Family& F = block_part(set, tile);
  Slot sl;
  if (!map_slot(F, T, sl, tile)) return;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int i0 = tile * kWideRows;
  if (i0 >= F.rows) return;
  const size_t ms = (size_t)F.rows * d;
  const uint8_t* Wg = static_cast<const uint8_t*>(F.gate) + (size_t)sl.mat * ms;
  const uint8_t* Wu = static_cast<const uint8_t*>(F.up) + (size_t)sl.mat * ms;
  const float* gsc = F.gate_scale + (size_t)sl.mat * F.rows;
  const float* usc = F.up_scale + (size_t)sl.mat * F.rows;
  const bf16_t* xg = F.x_gate ? static_cast<const bf16_t*>(F.x_gate) : x;
  bf16_t* h = static_cast<bf16_t*>(F.h);
#pragma unroll 1
  for (int tc = 0; tc < sl.n; tc += 32) {
    if (sl.n - tc > 16)
      gu_wide_fp8<2>(Wg, Wu, gsc, usc, d, F.rows, i0, xg, F.in_rows, sl.r0, sl.n, F.grp_token,
                     tc, h, lane, wid, *reinterpret_cast<WideLds<2, 1, 4>*>(fp8_lds));
    else
      gu_wide_fp8<1>(Wg, Wu, gsc, usc, d, F.rows, i0, xg, F.in_rows, sl.r0, sl.n, F.grp_token,
                     tc, h, lane, wid, *reinterpret_cast<WideLds<1, 1, 4>*>(fp8_lds));
  }
}

// The same for the down projection, on 64-column tiles.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void down_fp8_wide_kernel(FamilySet set, int T, int d) {
  __shared__ __align__(16) unsigned char fp8_lds[kFp8WideLds];
  int tile;
  const Family& F = block_part(set, tile);
  Slot sl;
  if (!map_slot(F, T, sl, tile)) return;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int c0 = tile * kWideRows;
  if (c0 >= d) return;
  const uint8_t* Wd = static_cast<const uint8_t*>(F.down) + (size_t)sl.mat * F.rows * d;
  const float* dsc = F.down_scale + (size_t)sl.mat * d;
  const bf16_t* h = static_cast<const bf16_t*>(F.h);
#pragma unroll 1
  for (int tc = 0; tc < sl.n; tc += 32) {
    if (sl.n - tc > 16)
      dn_wide_fp8<2>(Wd, dsc, d, F.rows, c0, h, sl.r0, sl.n, tc, F.out, lane, wid,
                     *reinterpret_cast<WideLds<2, 1, 4>*>(fp8_lds));
    else
      dn_wide_fp8<1>(Wd, dsc, d, F.rows, c0, h, sl.r0, sl.n, tc, F.out, lane, wid,
                     *reinterpret_cast<WideLds<1, 1, 4>*>(fp8_lds));
  }
}

__global__ void zero_kernel(unsigned int* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <typename K, typename... A>
static void launch(K kernel, dim3 grid, dim3 block, hipStream_t st, const KernelEvents* ev,
                   A... args) {
  if (ev)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, ev->start, ev->stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
}

// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
template <typename T_>
static hipError_t launch_route_t(const RouteArgs& ra, const PlanArgs* pa, hipStream_t st,
                                 const KernelEvents* ev) {
  if constexpr (sizeof(T_) == 2) {
    // matrix cores: 16-expert tiles x ksplit K pieces
    const dim3 grid((ra.E + 15) / 16, ra.ksplit);
    if (ra.T > 16)
      launch(route_mfma_kernel<2>, grid, dim3(kThreads), st, ev, ra);
    else
      launch(route_mfma_kernel<1>, grid, dim3(kThreads), st, ev, ra);
  } else if (ra.E >= 256) {
    // two experts per block once there are enough blocks to cover the chip:
    // each activation chunk is then read once for both
    launch(route_kernel<T_, 2>, dim3((ra.E + 1) / 2), dim3(kThreads), st, ev, ra);
  } else {
    launch(route_kernel<T_, 1>, dim3(ra.E), dim3(kThreads), st, ev, ra);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  PlanArgs p{};
  if (pa) p = *pa;
  const int do_plan = pa != nullptr;
  const KernelEvents* ev2 = ev ? ev + 1 : nullptr;
  // department-limited top-k only where the cap binds or coverage is
  // enforced (its own instances)
  const bool grouped = ra.k_dept > 0 && (ra.k_dept < ra.m || ra.strict);
  const int npl = (ra.E + kWave - 1) / kWave;
  if (topk_in_one_block(ra.T, ra.E)) {
    // one block: a wave per token, then the plan from LDS
    const dim3 grid(1), block(kPlanThreads);
    auto go = [&](auto N) {
      constexpr int NPL = decltype(N)::value;
      if (grouped)
        launch(topk_plan_kernel<NPL, true>, grid, block, st, ev2, ra, p, do_plan);
      else
        launch(topk_plan_kernel<NPL, false>, grid, block, st, ev2, ra, p, do_plan);
    };
    if (npl <= 1)
      go(std::integral_constant<int, 1>{});
    else if (npl <= 2)
      go(std::integral_constant<int, 2>{});
    else
      go(std::integral_constant<int, 4>{});
    return hipGetLastError();
  }
  // many tokens, or many experts per lane: the tokens' selections side by
  // side in blocks of four waves, then (with a plan) the plan launch on the
  // ids they wrote
  const KernelEvents ea{ev2 ? ev2->start : nullptr, nullptr};
  const KernelEvents eb{nullptr, ev2 ? ev2->stop : nullptr};
  const dim3 grid(npl <= 4 ? (ra.T + kWaves - 1) / kWaves : ra.T), block(kThreads);
  auto go = [&](auto N) {
    constexpr int NPL = decltype(N)::value;
    const KernelEvents* e1 = ev2 ? (do_plan ? &ea : ev2) : nullptr;
    if (grouped)
      launch(topk_token_kernel<NPL, true>, grid, block, st, e1, ra);
    else
      launch(topk_token_kernel<NPL, false>, grid, block, st, e1, ra);
  };
  if (npl <= 1)
    go(std::integral_constant<int, 1>{});
  else if (npl <= 2)
    go(std::integral_constant<int, 2>{});
  else if (npl <= 4)
    go(std::integral_constant<int, 4>{});
  else if (npl <= 8)
    go(std::integral_constant<int, 8>{});
  else if (npl <= 16)
    go(std::integral_constant<int, 16>{});
  else
    go(std::integral_constant<int, 32>{});
  if (!do_plan) return hipGetLastError();
  if ((e = hipGetLastError()) != hipSuccess) return e;
  launch(dispatch_kernel<true>, dim3(1), dim3(kPlanThreads), st, ev2 ? &eb : nullptr,
         (const int32_t*)ra.ids_out, (const float*)ra.w_out, p);
  return hipGetLastError();
}

hipError_t launch_route(int w_dtype, const RouteArgs& ra, const PlanArgs* pa, hipStream_t st,
                        const KernelEvents* ev) {
  return w_dtype == MOE_BF16 ? launch_route_t<bf16_t>(ra, pa, st, ev)
                             : launch_route_t<float>(ra, pa, st, ev);
}

hipError_t launch_dispatch(const int32_t* ids, const float* w, const PlanArgs& pa,
                           hipStream_t st) {
  hipLaunchKernelGGL(dispatch_kernel<false>, dim3(1), dim3(kPlanThreads), 0, st, ids, w, pa);
  return hipGetLastError();
}

template <typename T_>
static hipError_t launch_gateup_t(const FamilySet& set, const T_* x, int T, int d, int rpw,
                                  int rw, hipStream_t st, const KernelEvents* ev) {
  const dim3 grid(set.blk_start[set.n]), block(kThreads);
  // a group holds at most T rows: wider token passes (more accumulators) only
  // where a group can use them
  const int ncmax = T > 32 ? 4 : T > 16 ? 2 : 1;
  // one row per wave and pass: measured fastest, and the register budget of
  // the capped-occupancy build leaves no room for more
  if (rpw != 1 || rw != 1) return hipErrorInvalidValue;
  const bool xl = d <= kXLds;
  // two-input launches (factorised private transforms) have every part so
  const bool dual = set.f[0].x_up != nullptr;
#define MOE_GU(W, X, D) launch(gateup_kernel<T_, 1, 1, W, X, D>, grid, block, st, ev, set, x, T, d)
  if (dual) {
    // the private transforms' groups seldom pass four rows: 16-token passes
    if (xl) MOE_GU(1, true, true); else MOE_GU(1, false, true);
  } else {
    if (T == 1 && xl)  // one token: one row per group
      launch(gateup_kernel<T_, 1, 1, 1, true, false, 1>, grid, block, st, ev, set, x, T, d);
    else if (ncmax == 4) { if (xl) MOE_GU(4, true, false); else MOE_GU(4, false, false); }
    else if (ncmax == 2) { if (xl) MOE_GU(2, true, false); else MOE_GU(2, false, false); }
    else if (xl) MOE_GU(1, true, false); else MOE_GU(1, false, false);
  }
#undef MOE_GU
  return hipGetLastError();
}

hipError_t launch_gateup(int w_dtype, const FamilySet& set, const void* x, int T, int d,
                         int rows_per_wave, int rows_per_pass, hipStream_t st,
                         const KernelEvents* ev) {
  if (set.blk_start[set.n] <= 0) return hipSuccess;
  return w_dtype == MOE_BF16 ? launch_gateup_t<bf16_t>(set, static_cast<const bf16_t*>(x), T, d,
                                                       rows_per_wave, rows_per_pass, st, ev)
                             : launch_gateup_t<float>(set, static_cast<const float*>(x), T, d,
                                                      rows_per_wave, rows_per_pass, st, ev);
}

template <typename T_>
static hipError_t launch_down_t(const FamilySet& set, int T, int d, int lpr, int cg,
                                hipStream_t st, const KernelEvents* ev) {
  const dim3 grid(set.blk_start[set.n]), block(kThreads);
  int max_rows = 0;
  for (int i = 0; i < set.n; ++i) max_rows = set.f[i].rows > max_rows ? set.f[i].rows : max_rows;
  const bool xl = max_rows <= kXLds;
#define MOE_DOWN(L, C)                                                    \
  (xl ? launch(down_kernel<T_, L, C, true>, grid, block, st, ev, set, T, d) \
      : launch(down_kernel<T_, L, C, false>, grid, block, st, ev, set, T, d))
  if (lpr == 16) {
    if (cg >= 4) MOE_DOWN(16, 4); else if (cg >= 2) MOE_DOWN(16, 2); else MOE_DOWN(16, 1);
  } else if (lpr == 32) {
    if (cg >= 4) MOE_DOWN(32, 4); else if (cg >= 2) MOE_DOWN(32, 2); else MOE_DOWN(32, 1);
  } else {
    if (cg >= 4) MOE_DOWN(64, 4); else if (cg >= 2) MOE_DOWN(64, 2); else MOE_DOWN(64, 1);
  }
#undef MOE_DOWN
  return hipGetLastError();
}

hipError_t launch_down(int w_dtype, const FamilySet& set, int T, int d, int lpr, int col_groups,
                       hipStream_t st, const KernelEvents* ev) {
  if (set.blk_start[set.n] <= 0) return hipSuccess;
  return w_dtype == MOE_BF16 ? launch_down_t<bf16_t>(set, T, d, lpr, col_groups, st, ev)
                             : launch_down_t<float>(set, T, d, lpr, col_groups, st, ev);
}

hipError_t launch_combine(int act_dtype, const CombineArgs& a, void* y, hipStream_t st,
                          const KernelEvents* ev) {
  const dim3 grid((a.d + kThreads - 1) / kThreads, a.T), block(kThreads);
  if (act_dtype == MOE_BF16)
    launch(combine_kernel<bf16_t>, grid, block, st, ev, a, static_cast<bf16_t*>(y));
  else
    launch(combine_kernel<float>, grid, block, st, ev, a, static_cast<float*>(y));
  return hipGetLastError();
}

hipError_t launch_down_combine(const DownCombineArgs& a, void* y, hipStream_t st,
                               const KernelEvents* ev) {
  const dim3 grid((a.d + kDcWaves - 1) / kDcWaves), block(kDcWaves * kWave);
  const size_t lds = down_combine_lds_bytes(a);
  bf16_t* yo = static_cast<bf16_t*>(y);
  auto go = [&](auto k) {
    if (ev)
      hipExtLaunchKernelGGL(k, grid, block, lds, st, ev->start, ev->stop, 0, a, yo);
    else
      hipLaunchKernelGGL(k, grid, block, lds, st, a, yo);
  };
  // the first family's path, as the kernel chooses it per family; its first
  // groups are requested ahead of the table only for wide layers (measured:
  // DeepSeek-V3-shaped batch 1 down 45.4 -> 43.6 us; at d = 2048 the early
  // requests delayed the table's own loads, 7.9 -> 8.4 us at batch 1)
  const int r0 = a.f[0].rows, ns0 = (r0 + 8 * kWave - 1) / (8 * kWave);
  const bool packable0 = (size_t)a.f[0].n_mats * r0 * a.d * 2 < (size_t)kDcOob;
  if (a.fp8)
    go(down_combine_kernel<true, 0>);
  else if ((packable0 && (r0 == 16 * 8 || r0 == 32 * 8)) || a.d <= kDcPrefetchMinD)
    go(down_combine_kernel<false, 0>);
  else if (ns0 <= 1)
    go(down_combine_kernel<false, 1>);
  else if (ns0 == 2)
    go(down_combine_kernel<false, 2>);
  else if (ns0 == 3)
    go(down_combine_kernel<false, 3>);
  else
    go(down_combine_kernel<false, kDcMaxSteps>);
  return hipGetLastError();
}

// Rows staged per token chunk of the FP8 kernels: at most kTokInline, at most
// T (a group has at most T rows), and few enough that a block's staged rows
// of `width` bf16 stay within kFp8StageBytes (long rows would otherwise leave
// room for only two blocks per CU).
constexpr int kFp8StageBytes = 32 * 1024;
static int fp8_chunk_tokens(int T, int width) {
  int n = T < kTokInline ? T : kTokInline;
  while (n > 1 && (size_t)n * width * sizeof(bf16_t) > (size_t)kFp8StageBytes) --n;
  return n;
}

hipError_t launch_gateup_fp8(const FamilySet& set, const void* x, int T, int d, hipStream_t st,
                             const KernelEvents* ev) {
  if (set.blk_start[set.n] <= 0) return hipSuccess;
  const dim3 grid(set.blk_start[set.n]), block(kThreads);
  const int nts = fp8_chunk_tokens(T, d);
  const size_t lds = (size_t)nts * d * sizeof(bf16_t);
  const bf16_t* xb = static_cast<const bf16_t*>(x);
  auto go = [&](auto kernel) {
    if (ev)
      hipExtLaunchKernelGGL(kernel, grid, block, lds, st, ev->start, ev->stop, 0, set, xb, T, d,
                            nts);
    else
      hipLaunchKernelGGL(kernel, grid, block, lds, st, set, xb, T, d, nts);
  };
  // measured: two steps ahead for rows of up to 2048 codes, four beyond
  if (d <= 2048)
    go(gateup_fp8_kernel<2>);
  else
    go(gateup_fp8_kernel<4>);
  return hipGetLastError();
}

hipError_t launch_down_fp8(const FamilySet& set, int T, int d, int lpr, hipStream_t st,
                           const KernelEvents* ev) {
  if (set.blk_start[set.n] <= 0) return hipSuccess;
  const dim3 grid(set.blk_start[set.n]), block(kThreads);
  int max_rows = 0;
  for (int i = 0; i < set.n; ++i) max_rows = set.f[i].rows > max_rows ? set.f[i].rows : max_rows;
  const int nts = fp8_chunk_tokens(T, max_rows);
  const size_t lds = (size_t)nts * max_rows * sizeof(bf16_t);
  auto go = [&](auto kernel) {
    if (ev)
      hipExtLaunchKernelGGL(kernel, grid, block, lds, st, ev->start, ev->stop, 0, set, T, d, nts);
    else
      hipLaunchKernelGGL(kernel, grid, block, lds, st, set, T, d, nts);
  };
  if (lpr == 16)
    go(down_fp8_kernel<16>);
  else if (lpr == 32)
    go(down_fp8_kernel<32>);
  else
    go(down_fp8_kernel<64>);
  return hipGetLastError();
}

hipError_t launch_fp8_wide(bool gateup, const FamilySet& set, const void* x, int T, int d,
                           hipStream_t st, const KernelEvents* ev) {
  if (set.blk_start[set.n] <= 0) return hipSuccess;
  const dim3 grid(set.blk_start[set.n]), block(kThreads);
  const bf16_t* xb = static_cast<const bf16_t*>(x);
  if (gateup) {
    if (ev)
      hipExtLaunchKernelGGL(gateup_fp8_wide_kernel, grid, block, 0, st, ev->start, ev->stop, 0,
                            set, xb, T, d);
    else
      hipLaunchKernelGGL(gateup_fp8_wide_kernel, grid, block, 0, st, set, xb, T, d);
  } else {
    if (ev)
      hipExtLaunchKernelGGL(down_fp8_wide_kernel, grid, block, 0, st, ev->start, ev->stop, 0,
                            set, T, d);
    else
      hipLaunchKernelGGL(down_fp8_wide_kernel, grid, block, 0, st, set, T, d);
  }
  return hipGetLastError();
}

// Streaming read for measurement: block b sums the 8192 bf16 values of bytes
// [16 KiB b, 16 KiB (b+1)), one 4 KiB row per wave, each lane 16 bytes per
// step with the next step requested before the current one is used.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const bf16_t* __restrict__ src,
                                                              float* __restrict__ sink) {
  __shared__ float part[kWaves];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const bf16_t* row = src + ((size_t)blockIdx.x * kWaves + wid) * 2048 + lane * 8;
  Raw8<bf16_t> cur, nxt;
  cur.load(row);
  float acc = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s + 1 < 4) nxt.load(row + (s + 1) * 512);
    float v[8];
    cur.to_f32(v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += v[i];
    cur = nxt;
  }
  acc = wave_sum(acc);
  if (lane == 0) part[wid] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = ((part[0] + part[1]) + part[2]) + part[3];
}

hipError_t launch_pair_combine(int act_dtype, const PairCombineArgs& a, void* zc, int max_pairs,
                               hipStream_t st) {
  if (max_pairs <= 0) return hipSuccess;
  const dim3 grid((a.cols + kThreads - 1) / kThreads, max_pairs), block(kThreads);
  if (act_dtype == MOE_BF16)
    hipLaunchKernelGGL(pair_combine_kernel<bf16_t>, grid, block, 0, st, a, static_cast<bf16_t*>(zc));
  else
    hipLaunchKernelGGL(pair_combine_kernel<float>, grid, block, 0, st, a, static_cast<float*>(zc));
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, size_t blocks, float* sink, hipStream_t st) {
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st,
                     static_cast<const bf16_t*>(src), sink);
  return hipGetLastError();
}

hipError_t launch_zero(unsigned int* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int blocks = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
  hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace moe
