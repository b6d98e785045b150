// Sums over the 64 lanes of a wave for gfx950, without LDS: the lane swaps
// v_permlane32_swap / v_permlane16_swap for lane bits 5 and 4, DPP
// row_mirror / row_half_mirror / quad_perm for bits 3, 2, 1, 0.
//
// A butterfly over lane bit b pairs every lane with one in the other half of
// its 2^(b+1)-lane group.  Plain xor partners are not needed: a mirror pairs
// lane i with lane (2^(b+1) - 1) - i of its group, which is lane i xor a mask
// whose top set bit is b, and masks with distinct top bits are independent,
// so after one step per bit every lane has gathered all 64 lanes.
#pragma once

#include "devmath.h"

namespace mhc {

template <int CTRL>
MHC_DEV float wave_dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                              0xF, 0xF, true));
}

// DPP controls: partner across lane bit 3, 2, 1, 0
constexpr int kDppBit3 = 0x140;  // row_mirror: i <-> 15 - i within 16 lanes
constexpr int kDppBit2 = 0x141;  // row_half_mirror: i <-> 7 - i within 8 lanes
constexpr int kDppBit1 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppBit0 = 0xB1;   // quad_perm [1,0,3,2]

// One halving step over lane bit 5: lanes 0-31 get lo[l] + lo[l+32], lanes
// 32-63 get hi[l-32] + hi[l].  permlane32_swap(x, y) returns (x[0..31] with
// y[0..31]) and (x[32..63] with y[32..63]).
MHC_DEV float halve_bit5(float lo, float hi)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The same over lane bit 4 (rows of 16 lanes): even rows get the lo sums,
// odd rows the hi sums.
MHC_DEV float halve_bit4(float lo, float hi)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Full sums over one lane bit: every lane gets v[l] + v[partner] for the
// partner across bit 5 (lane l ^ 32) or bit 4 (l ^ 16), from a swap of the
// register with itself.
MHC_DEV float sum_bit5(float v) { return halve_bit5(v, v); }
MHC_DEV float sum_bit4(float v) { return halve_bit4(v, v); }

// One halving step over lane bit b <= 3 with the DPP partner CTRL: lanes with
// bit b clear keep (and receive) the lower half of the values, the others the
// upper half.
template <int CTRL, int BIT, int H>
MHC_DEV void halve_dpp(float* v)
{
    const bool up = (threadIdx.x >> BIT) & 1;
#pragma unroll
    for (int k = 0; k < H; ++k) {
        const float lo = mhc_opaque(v[k]), hi = mhc_opaque(v[k + H]);
        const float keep = up ? hi : lo;
        const float send = up ? lo : hi;
        v[k] = keep + wave_dpp<CTRL>(send);
    }
}

// Sum N (16 or 32) per-lane partials v[0..N-1] over the wave by butterfly
// halving: each step over a lane bit sends half of the remaining values to
// the partner lane and keeps the other half, then the bits left over are
// summed whole.  Afterwards lane l holds the total of value
// (l >> (6 - log2 N)) & (N - 1); v is overwritten.
template <int N>
MHC_DEV float wave_sum_halving(float* v)
{
    static_assert(N == 16 || N == 32, "16 or 32 partials");
#pragma unroll
    for (int k = 0; k < N / 2; ++k) v[k] = halve_bit5(v[k], v[k + N / 2]);
#pragma unroll
    for (int k = 0; k < N / 4; ++k) v[k] = halve_bit4(v[k], v[k + N / 4]);
    halve_dpp<kDppBit3, 3, N / 8>(v);
    halve_dpp<kDppBit2, 2, N / 16>(v);
    float s = v[0];
    if constexpr (N == 32) {
        halve_dpp<kDppBit1, 1, 1>(v);
        s = v[0];
    } else {
        s += wave_dpp<kDppBit1>(s);
    }
    return s + wave_dpp<kDppBit0>(s);
}

}  // namespace mhc
