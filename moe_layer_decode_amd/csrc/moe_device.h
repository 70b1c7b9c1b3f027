// Device helpers for the gfx950 MoE decode kernels: bf16 <-> fp32, global
// loads, and wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ void store_act(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_act(bf16_t* p, float v) { *p = f32_to_bf16(v); }

// Global-memory view of a generic pointer.  Loads through it compile to
// global loads, counted by vmcnt alone.  A load through a generic pointer the
// compiler cannot place (in an out-of-line function, say) becomes a flat
// load, which also counts against lgkmcnt, so the compiler then waits for
// every load in flight before the next LDS access or use -- a prefetch ring
// of weight loads collapses to one step.
template <typename V>
__device__ __forceinline__ const __attribute__((address_space(1))) V* as_global(const void* p) {
  return (const __attribute__((address_space(1))) V*)(p);
}

// 16-byte vectors of fp32 values and of raw 32-bit words.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Cross-lane moves by DPP (a modifier of the VALU operand, no round trip
// through the LDS crossbar as with ds_bpermute) inside 16-lane rows.
// Controls: quad_perm [1,0,3,2] and [2,3,0,1] (lane xor 1, xor 2), the
// half-row mirror (lane i <-> 7 - i in each 8 lanes), the row mirror (lane i
// <-> 15 - i in each 16), and row shifts right by 1, 2, 4, 8 (lanes without a
// source read 0).
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppRowMirror = 0x140;
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;
// Across rows: lane 15 of each row to the next row, and lane 31 to rows 2
// and 3; rows left out by the row mask keep their value.
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(dpp<CTRL>(__float_as_int(v)));
}

// Reduction of each 16-lane row, the result in every lane of the row:
// pairs of lanes, then quads, then the two halves of each 8 (mirror), then
// the two halves of the row (mirror).  OP(a, b) must be commutative.
template <typename V, typename Op>
__device__ __forceinline__ V row16_reduce(V v, Op op) {
  v = op(v, dpp<kDppXor1>(v));
  v = op(v, dpp<kDppXor2>(v));
  v = op(v, dpp<kDppHalfMirror>(v));
  return op(v, dpp<kDppRowMirror>(v));
}

// Whole-wave reductions (wave-uniform result): each row reduced by row16_reduce,
// then row 1 takes row 0 and row 3 takes row 2 (lane 15 / 47 broadcast), and
// row 3 takes row 1 (lane 31): lane 63 holds (r3 + r2) + (r1 + r0) in a fixed
// order, read once into a scalar.  All on the vector unit but the final read.
template <typename Op>
__device__ __forceinline__ int wave_reduce_i(int v, Op op) {
  v = row16_reduce(v, op);
  v = op(v, __builtin_amdgcn_update_dpp(v, v, kDppBcast15, 0xA, 0xF, false));
  v = op(v, __builtin_amdgcn_update_dpp(v, v, kDppBcast31, 0xC, 0xF, false));
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ float wave_sum(float v) {
  return __int_as_float(wave_reduce_i(__float_as_int(v), [](int a, int b) {
    return __float_as_int(__int_as_float(a) + __int_as_float(b));
  }));
}
__device__ __forceinline__ float wave_max(float v) {
  return __int_as_float(wave_reduce_i(__float_as_int(v), [](int a, int b) {
    return __float_as_int(fmaxf(__int_as_float(a), __int_as_float(b)));
  }));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return (uint32_t)wave_reduce_i((int)v, [](int a, int b) {
    return (uint32_t)a > (uint32_t)b ? a : b;
  });
}

// Inclusive prefix sum over the wave's lanes: a scan inside each 16-lane row
// by DPP row shifts, then each row adds the totals of the rows before it.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
  v += dpp<kDppShr1>(v);
  v += dpp<kDppShr2>(v);
  v += dpp<kDppShr4>(v);
  v += dpp<kDppShr8>(v);
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
            r2 = __builtin_amdgcn_readlane(v, 47);
  const int q = lane >> 4;
  return v + (q >= 1 ? r0 : 0) + (q >= 2 ? r1 : 0) + (q >= 3 ? r2 : 0);
}

template <int N> struct Log2 { static constexpr int value = 1 + Log2<N / 2>::value; };
template <> struct Log2<1> { static constexpr int value = 0; };

// The value of lane l ^ 32 (the other half of the wave), by the gfx950
// half swap: swapping the upper half of a copy with the lower half of
// another leaves each lane's partner value in one of the two.
__device__ __forceinline__ float xor32(float v, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

// a + (the same value of the partner lane) for one butterfly step across lane
// bit 5 or 4, from one gfx950 half / row swap: swapping the upper halves of a
// with the lower halves of b gives, in every lane, the sum of the pair it
// keeps (lower lanes a + partner's a, upper lanes b + partner's b).
template <int O>
__device__ __forceinline__ float swap_pair_sum(float a, float b) {
  const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
  if constexpr (O == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(ua, ub, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    static_assert(O == 16, "row swaps pair lanes 16 or 32 apart");
    const auto r = __builtin_amdgcn_permlane16_swap(ua, ub, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}

// DPP control of a butterfly partner across lane bit log2(O), O <= 8: a
// permutation inside the 16-lane row that flips that bit (and possibly lower
// ones) and keeps every higher bit, which is all a reduce-scatter step needs.
template <int O>
constexpr int butterfly_dpp() {
  return O == 8 ? kDppRowMirror : O == 4 ? kDppHalfMirror : O == 2 ? kDppXor2 : kDppXor1;
}

// Reduce N per-lane values over the L lanes of an aligned lane group (lanes
// differing only in bits below log2 L; L a power of two, 2 .. 64).  Butterfly
// steps from lane bit log2(L) - 1 down to bit 0; at each step a lane keeps the
// half of its live values that its bit selects (upper lanes the upper half)
// and adds its partner's copy of that half, so each step halves the live
// values.  Afterwards lane j of the group holds, in v[0 .. max(N/L, 1)), the
// sums of value indices (N/L) * j + i when N >= L, or of index j / (L/N) when
// N < L.  Partners across bits 5 and 4 come from the gfx950 half / row swaps,
// the others from DPP row permutations: no LDS traffic.
template <int N, int L>
__device__ __forceinline__ void group_reduce_scatter(float (&v)[N], int lane) {
  static_assert(L >= 2 && L <= 64 && (L & (L - 1)) == 0, "L must be a power of two <= 64");
  int n = N;
#pragma unroll
  for (int o = L / 2; o >= 1; o >>= 1) {
    const int half = n > 1 ? n >> 1 : 1;
#pragma unroll
    for (int i = 0; i < (N > 1 ? N / 2 : 1); ++i) {
      if (i < half) {
        const float lo = v[i], hi = n > 1 ? v[i + half] : v[i];
        if (o >= 16) {
          v[i] = o == 32 ? swap_pair_sum<32>(lo, hi) : swap_pair_sum<16>(lo, hi);
        } else {
          const bool upper = (lane & o) != 0;
          const float send = upper ? lo : hi, keep = upper ? hi : lo;
          v[i] = keep + (o == 8 ? dpp<butterfly_dpp<8>()>(send)
                         : o == 4 ? dpp<butterfly_dpp<4>()>(send)
                         : o == 2 ? dpp<butterfly_dpp<2>()>(send)
                                  : dpp<butterfly_dpp<1>()>(send));
        }
      }
    }
    n = half;
  }
}

// group_reduce_scatter over the whole wave: lane l holds the full sum of value
// index (l >> (6 - log2 N)) & (N - 1); the top index bit sits in lane bit 5.
template <int N>
__device__ __forceinline__ float wave_reduce_scatter(float (&v)[N], int lane) {
  static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "N must be a power of two <= 64");
  group_reduce_scatter<N, 64>(v, lane);
  return v[0];
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

}  // namespace moe
