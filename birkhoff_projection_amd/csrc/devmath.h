// Device math used by the gfx950 kernels: the hardware transcendental
// instructions, called through clang's amdgcn builtins.
//
//   mhc_exp2(x)  v_exp_f32   2^x      (about 1 ulp)
//   mhc_log2(x)  v_log_f32   log2(x)  (about 1 ulp)
//   mhc_rcp(x)   v_rcp_f32   1/x      (about 1 ulp)
//
// The solver works in base 2: logits are multiplied by log2(e) once at load,
// so exp(a) = 2^(a log2 e) and a log-sum-exp becomes a log2-sum-exp2.  The
// caller always shifts the argument of mhc_exp2 to be <= 0 (a row max-shift),
// so there is no overflow and the result lies in (0, 1].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MHC_DEV __device__ __forceinline__

MHC_DEV float mhc_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
MHC_DEV float mhc_log2(float x) { return __builtin_amdgcn_logf(x); }
MHC_DEV float mhc_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
MHC_DEV float mhc_max(float a, float b) { return __builtin_fmaxf(a, b); }
MHC_DEV float mhc_min(float a, float b) { return __builtin_fminf(a, b); }
MHC_DEV float mhc_abs(float a) { return __builtin_fabsf(a); }

// Makes a value opaque to the optimizer; emits no instruction.  The butterfly
// reductions pass both candidates of a per-lane select through it, so the
// select is not folded into one dynamically indexed array load (which the
// backend lowers to a compare-and-select chain over the whole array).
MHC_DEV float mhc_opaque(float x)
{
    asm("" : "+v"(x));
    return x;
}

// Like mhc_opaque, but the value is materialised on every path: a volatile
// statement cannot be sunk into one arm of a branch, so a select between
// pinned values stays a v_cndmask instead of becoming an if/else.
MHC_DEV float mhc_pin(float x)
{
    asm volatile("" : "+v"(x));
    return x;
}

// Compiler barrier for LDS data that lanes of one wave exchange.  A wave's LDS
// instructions execute in order, so the hardware needs no wait; but the
// optimizer models each lane as a separate thread, and without this it may
// reuse a value the lane read from LDS earlier (or move an LDS access across
// the exchange) when it can prove that the lane's own writes did not touch
// that address -- other lanes' writes are invisible to it.
MHC_DEV void mhc_wave_lds_fence()
{
    asm volatile("" ::: "memory");
}

// Workgroup barrier that orders LDS traffic only: waits for this wave's LDS
// operations, then s_barrier.  Unlike __syncthreads it does not drain the
// wave's outstanding global loads and stores, so a streaming loop keeps its
// HBM requests in flight across the barrier.  The memory clobber keeps the
// compiler from moving memory accesses across it.
MHC_DEV void mhc_lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// bf16 <-> fp32.  A bf16 is the top half of an fp32, so widening is a shift.
// Streaming 16-byte load and store for data that is moved exactly once
// (nontemporal hint: not kept in the caches).  Where reads and writes
// stream together it helps: the stream-mix passes measured 4 % faster and
// the projection backward 11 % (hinting only the reads or only the writes
// made no difference).
typedef unsigned int mhc_u32x4 __attribute__((ext_vector_type(4)));
MHC_DEV uint4 mhc_load_stream(const uint4* p)
{
    const mhc_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const mhc_u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
MHC_DEV void mhc_store_stream(uint4* p, const uint4& q)
{
    const mhc_u32x4 v = {q.x, q.y, q.z, q.w};
    __builtin_nontemporal_store(v, reinterpret_cast<mhc_u32x4*>(p));
}
typedef float mhc_f32x4 __attribute__((ext_vector_type(4)));
MHC_DEV float4 mhc_load_stream(const float4* p)
{
    const mhc_f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const mhc_f32x4*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
MHC_DEV void mhc_store_stream(float4* p, const float4& q)
{
    const mhc_f32x4 v = {q.x, q.y, q.z, q.w};
    __builtin_nontemporal_store(v, reinterpret_cast<mhc_f32x4*>(p));
}

MHC_DEV float mhc_bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
MHC_DEV float mhc_bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// Cross-lane reads inside a quad of 4 lanes (DPP quad_perm, no LDS).  With
// bound_ctrl set, the compiler folds the move into the consuming VALU
// instruction (v_add_f32_dpp), so a 4-lane sum costs two instructions.
MHC_DEV float mhc_quad_xor1(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                              0xB1 /* quad_perm [1,0,3,2] */,
                                                              0xF, 0xF, true));
}
MHC_DEV float mhc_quad_xor2(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                              0x4E /* quad_perm [2,3,0,1] */,
                                                              0xF, 0xF, true));
}
// Sum over the 4 lanes of a quad; every lane of the quad gets the total.
MHC_DEV float mhc_quad_sum(float v)
{
    v += mhc_quad_xor1(v);
    return v + mhc_quad_xor2(v);
}
