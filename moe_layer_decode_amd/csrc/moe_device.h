// Device helpers for the gfx950 MoE decode kernels: bf16 <-> fp32, 8-wide
// vector loads, and wave64 reductions.
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

// Eight consecutive elements widened to fp32.  p must be 16-byte aligned.
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8(const bf16_t* p, float (&v)[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
  v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z); v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
}

// Streaming (read-once) weight loads: same values, non-temporal cache hint.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void load8_stream(const float* p, float (&v)[8]) {
  const f32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  const f32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p + 4));
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8_stream(const bf16_t* p, float (&v)[8]) {
  const u32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
  v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z); v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
}

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

// Reduce N per-lane values (N a power of two, <= 64) over the 64 lanes of a
// wave.  Each butterfly step halves the live values, so the whole reduction
// costs N - 1 + (6 - log2 N) shuffles instead of 6 N.  On return lane l holds
// the full sum of value index (l >> (6 - log2 N)) & (N - 1); the top index bit
// always sits in lane bit 5.
template <int N>
__device__ __forceinline__ float wave_reduce_scatter(float (&v)[N], int lane) {
  static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "N must be a power of two <= 64");
  int n = N;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    if (n > 1) {
      const int half = n >> 1;
      const bool upper = (lane & o) != 0;
#pragma unroll
      for (int i = 0; i < N / 2; ++i) {
        if (i < half) {
          const float send = upper ? v[i] : v[i + half];
          const float keep = upper ? v[i + half] : v[i];
          v[i] = keep + __shfl_xor(send, o, kWave);
        }
      }
      n = half;
    } else {
      v[0] += __shfl_xor(v[0], o, kWave);
    }
  }
  return v[0];
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

}  // namespace moe
