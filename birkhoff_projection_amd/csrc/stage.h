// Moving a wave's 64 consecutive records (R floats each) between global
// memory and one record per lane, through a per-wave LDS tile.
//
// A lane that loads or stores its own record directly makes every memory
// instruction touch 64 records R*4 bytes apart; at R = 16 (4x4 matrices)
// each store instruction then writes 16 bytes into each of 64 different
// 64-byte records, and with streaming stores those partial lines reached
// HBM as 37 % extra write traffic.  Going through LDS, every instruction
// covers one contiguous piece of the wave's block instead, and the lanes
// then exchange records through the tile (pitch R rounded up to odd, so the
// per-lane record reads are free of bank conflicts).
//
// Records at or past B read as zeros and are not stored.  A wave reads all
// of its inputs before it writes, so an output may be the same buffer as an
// input.  Only lanes of one wave share a tile, so the exchanges need no
// barrier, only a compiler fence (the compiler models lanes as threads).
// All accesses are streaming (nontemporal): every record is moved once.
//
// The wave's position (`first`) must be the same in every lane; kernels take
// the wave index from wave_index(), which the compiler then knows to be
// uniform, so the full-wave tests below are scalar branches and a full wave
// (the common case) runs no per-lane bounds arithmetic.
#pragma once

#include "devmath.h"

namespace mhc {

// Index of the calling wave in its workgroup, as a wave-uniform value.
MHC_DEV int wave_index() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

template <int R>
constexpr int record_pitch()
{
    return R | 1;
}

template <int R>
constexpr int stage_tile_floats()
{
    return 64 * record_pitch<R>();
}

// 4-byte elements: any R, base 4-byte aligned.  All R loads are issued
// before the first is used (addresses past the batch are clamped to its last
// element and the value replaced by zero).
template <int R>
MHC_DEV void load_records(const float* __restrict__ g, int64_t first, int64_t B, float* tile,
                          float* out, int lane)
{
    constexpr int kP = record_pitch<R>();
    const int64_t have = B - first;
    const int64_t last = R * B - 1;
    float v[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int64_t idx = R * first + lane + 64 * i;
        v[i] = __builtin_nontemporal_load(g + (idx < last ? idx : last));
    }
    mhc_wave_lds_fence();  // earlier reads of the tile by other lanes come first
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int e = lane + 64 * i;
        const int rec = e / R, col = e % R;
        tile[rec * kP + col] = rec < have ? v[i] : 0.f;
    }
    mhc_wave_lds_fence();  // the reads below see the other lanes' writes
#pragma unroll
    for (int k = 0; k < R; ++k) out[k] = tile[lane * kP + k];
}

template <int R>
MHC_DEV void store_records(float* __restrict__ g, int64_t first, int64_t B, float* tile,
                           const float* in, int lane)
{
    constexpr int kP = record_pitch<R>();
    const int64_t have = B - first;
    mhc_wave_lds_fence();
#pragma unroll
    for (int k = 0; k < R; ++k) tile[lane * kP + k] = in[k];
    mhc_wave_lds_fence();
    if (have >= 64) {  // a full wave: no per-element checks
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int e = lane + 64 * i;
            __builtin_nontemporal_store(tile[(e / R) * kP + e % R], g + R * first + e);
        }
    } else {
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int e = lane + 64 * i;
            const int rec = e / R;
            if (rec < have) __builtin_nontemporal_store(tile[rec * kP + e % R], g + R * first + e);
        }
    }
}

// 16-byte elements: R a multiple of 4 and a 16-byte aligned base.  The load
// is split in two so that a caller can issue the loads of several record
// sets before it moves any of them through the tile: issue_records_v4 starts
// the wave's R/4 float4 loads (clamped past the batch), scatter_records_v4
// moves them through the tile to one record per lane (zeros past B).
template <int R>
MHC_DEV void issue_records_v4(const float* __restrict__ g, int64_t first, int64_t B,
                              float4 (&v)[R / 4], int lane)
{
    static_assert(R % 4 == 0, "records of whole float4s");
    constexpr int kQ = R / 4;  // float4 loads per lane
    const float4* g4 = reinterpret_cast<const float4*>(g);
    if (B - first >= 64) {
#pragma unroll
        for (int i = 0; i < kQ; ++i) v[i] = mhc_load_stream(g4 + kQ * first + lane + 64 * i);
        return;
    }
    const int64_t last = kQ * B - 1;
#pragma unroll
    for (int i = 0; i < kQ; ++i) {
        const int64_t idx = kQ * first + lane + 64 * i;
        v[i] = mhc_load_stream(g4 + (idx < last ? idx : last));
    }
}

template <int R>
MHC_DEV void scatter_records_v4(const float4 (&v)[R / 4], int64_t first, int64_t B, float* tile,
                                float* out, int lane)
{
    constexpr int kP = record_pitch<R>();
    constexpr int kQ = R / 4;
    const int64_t have = B - first;
    mhc_wave_lds_fence();
    if (have >= 64) {
#pragma unroll
        for (int i = 0; i < kQ; ++i) {
            const int e = 4 * (lane + 64 * i);
            float* t = tile + (e / R) * kP + e % R;
            t[0] = v[i].x;
            t[1] = v[i].y;
            t[2] = v[i].z;
            t[3] = v[i].w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < kQ; ++i) {
            const int e = 4 * (lane + 64 * i);
            const int rec = e / R, col = e % R;
            const bool in = rec < have;
            float* t = tile + rec * kP + col;
            t[0] = in ? v[i].x : 0.f;
            t[1] = in ? v[i].y : 0.f;
            t[2] = in ? v[i].z : 0.f;
            t[3] = in ? v[i].w : 0.f;
        }
    }
    mhc_wave_lds_fence();
#pragma unroll
    for (int k = 0; k < R; ++k) out[k] = tile[lane * kP + k];
}

template <int R>
MHC_DEV void load_records_v4(const float* __restrict__ g, int64_t first, int64_t B, float* tile,
                             float* out, int lane)
{
    float4 v[R / 4];
    issue_records_v4<R>(g, first, B, v, lane);
    scatter_records_v4<R>(v, first, B, tile, out, lane);
}

template <int R>
MHC_DEV void store_records_v4(float* __restrict__ g, int64_t first, int64_t B, float* tile,
                              const float* in, int lane)
{
    static_assert(R % 4 == 0, "records of whole float4s");
    constexpr int kP = record_pitch<R>();
    constexpr int kQ = R / 4;
    const int64_t have = B - first;
    float4* g4 = reinterpret_cast<float4*>(g);
    mhc_wave_lds_fence();
#pragma unroll
    for (int k = 0; k < R; ++k) tile[lane * kP + k] = in[k];
    mhc_wave_lds_fence();
#pragma unroll
    for (int i = 0; i < kQ; ++i) {
        const int e = 4 * (lane + 64 * i);
        const int rec = e / R, col = e % R;
        const float* t = tile + rec * kP + col;
        const float4 q = make_float4(t[0], t[1], t[2], t[3]);
        if (have >= 64 || rec < have) mhc_store_stream(g4 + kQ * first + lane + 64 * i, q);
    }
}

// store_records_v4 for records that are already in the tile (lane l's record
// at tile + l * record_pitch<R>(), each written by its own lane): only the
// coalesced global stores.
template <int R>
MHC_DEV void store_tile_v4(float* __restrict__ g, int64_t first, int64_t B, const float* tile,
                           int lane)
{
    static_assert(R % 4 == 0, "records of whole float4s");
    constexpr int kP = record_pitch<R>();
    constexpr int kQ = R / 4;
    const int64_t have = B - first;
    float4* g4 = reinterpret_cast<float4*>(g);
    mhc_wave_lds_fence();  // the reads below see the other lanes' writes
#pragma unroll
    for (int i = 0; i < kQ; ++i) {
        const int e = 4 * (lane + 64 * i);
        const int rec = e / R, col = e % R;
        const float* t = tile + rec * kP + col;
        const float4 q = make_float4(t[0], t[1], t[2], t[3]);
        if (have >= 64 || rec < have) mhc_store_stream(g4 + kQ * first + lane + 64 * i, q);
    }
}

}  // namespace mhc
