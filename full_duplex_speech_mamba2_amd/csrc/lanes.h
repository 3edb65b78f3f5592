// Cross-lane reductions of a wave64 in VALU instructions: DPP row rotations, the half-row
// mirror and quad permutes within 16-lane rows, and the gfx950 permlane16/permlane32 swaps
// across rows, in place of LDS permutes (ds_bpermute), whose round trips through the LDS
// unit sit on the critical path of short reductions.
#pragma once

#include <hip/hip_runtime.h>

namespace m2d {
namespace {

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <bool MAX>
__device__ __forceinline__ float combine2(float a, float b) {
  return MAX ? fmaxf(a, b) : a + b;
}

// Lanes 16r..16r+15 exchange with lanes 16(r^1)..: the pair of a permlane16 swap of v with
// itself holds v of both rows (elements copied out before use).
template <bool MAX>
__device__ __forceinline__ float xrow16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const unsigned a = r[0], b = r[1];
  return combine2<MAX>(__uint_as_float(a), __uint_as_float(b));
}

template <bool MAX>
__device__ __forceinline__ float xrow32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const unsigned a = r[0], b = r[1];
  return combine2<MAX>(__uint_as_float(a), __uint_as_float(b));
}

// Every lane receives the sum (or maximum) over its group of G consecutive lanes, G = 8, 16
// or 64: within a 16-lane row by rotations of 8 and 4 (or the half-row mirror for G = 8)
// and quad permutes, then across rows by permlane swaps.
template <int G, bool MAX = false>
__device__ __forceinline__ float group_reduce(float v) {
  static_assert(G == 8 || G == 16 || G == 64, "group");
  if (G == 8) {
    v = combine2<MAX>(v, dpp<0x141>(v));           // row_half_mirror: lanes i, 7 - i
  } else {
    v = combine2<MAX>(v, dpp<0x128>(v));           // row_ror:8
    v = combine2<MAX>(v, dpp<0x124>(v));           // row_ror:4
  }
  v = combine2<MAX>(v, dpp<0x4E>(v));              // quad_perm [2,3,0,1]
  v = combine2<MAX>(v, dpp<0xB1>(v));              // quad_perm [1,0,3,2]
  if (G == 64) {
    v = xrow16<MAX>(v);
    v = xrow32<MAX>(v);
  }
  return v;
}

// Sum over the lanes that share lane % LPP (LPP = 8 or 16): the position groups of a wave.
template <int LPP>
__device__ __forceinline__ float across_groups_sum(float v) {
  if (LPP == 8) v += dpp<0x128>(v);                // row_ror:8 pairs lanes i and i + 8 of a row
  v = xrow16<false>(v);
  return xrow32<false>(v);
}

// group_reduce for a group size known only at run time (uniform over the wave): 1 .. 64.
__device__ __forceinline__ float group_sum_rt(float v, int g) {
  switch (g) {
    case 64: return group_reduce<64>(v);
    case 32: {
      v = group_reduce<16>(v);
      return xrow16<false>(v);
    }
    case 16: return group_reduce<16>(v);
    case 8: return group_reduce<8>(v);
    case 4:
      v += dpp<0x4E>(v);
      return v + dpp<0xB1>(v);
    case 2: return v + dpp<0xB1>(v);
    default: return v;
  }
}

}  // namespace
}  // namespace m2d
