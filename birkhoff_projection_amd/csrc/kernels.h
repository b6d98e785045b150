// Kernel launchers behind the C ABI (internal; see include/mhc.h for the
// public contract).  Each returns hipGetLastError() after enqueueing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "proj4.h"

namespace mhc {

hipError_t launch_birkhoff_fwd(const float* logits, float* P, uint8_t* iters, int64_t B,
                               const SolverOpts& o, hipStream_t stream);
hipError_t launch_birkhoff_bwd(const float* P, const float* G, float* dA, int64_t B,
                               hipStream_t stream);
hipError_t launch_birkhoff_bwd_recompute(const float* logits, const float* G, float* dA, int64_t B,
                                         const SolverOpts& o, hipStream_t stream);
hipError_t launch_birkhoff_fwd_bwd(const float* logits, const float* G, float* P, float* dA,
                                   uint8_t* iters, int64_t B, const SolverOpts& o,
                                   hipStream_t stream);
// Forward of (logits, P, B) and backward of (Pb, Gb -> dAb, Bb) in one launch.
hipError_t launch_birkhoff_pipeline(const float* logits, float* P, uint8_t* iters, int64_t B,
                                   const SolverOpts& o, const float* Pb, const float* Gb,
                                   float* dAb, int64_t Bb, hipStream_t stream);
// n x n projection for n in {1, 2, 3, 5, 6, 7, 8} (4 has its own kernels).
hipError_t launch_birkhoff_fwd_n(const float* logits, float* P, uint8_t* iters, int64_t B, int n,
                                 const SolverOpts& o, hipStream_t stream);
hipError_t launch_birkhoff_bwd_n(const float* P, const float* G, float* dA, int64_t B, int n,
                                 hipStream_t stream);
hipError_t launch_stream_mix_fwd(const void* x, const float* Hl, float* H_out, void* out,
                                 int64_t T, int64_t C, const SolverOpts* proj,
                                 hipStream_t stream);
hipError_t launch_stream_mix_bwd(const void* x, const float* H, const void* gout, void* gx,
                                 float* gH, int64_t T, int64_t C, hipStream_t stream);

// Device pointers of one layer step (see mhc_layer_args in include/mhc.h).
struct LayerPtrs {
    const void* x;
    const void* W;
    const void* f;
    void* u;
    void* x_out;
    float* rms;
    float* logits;
    float* H_pre;
    float* H_post;
    float* H_res;
    const void* grad_x_out;
    const void* grad_u;
    void* grad_x;
    void* grad_f;
    float* grad_W;
    float* grad_logits;
    void* workspace;
};

// Backward workspace layout: s[Tp] fp32 | dl^T hi [24][Tp] bf16 | dl^T lo
// [24][Tp] bf16 | W^T [4C][24] bf16 | grad_W partials [groups][24][4C] fp32
// (each 256-byte aligned).
struct LayerPlan {
    int64_t Tp;            // T rounded up to 64
    int64_t group_tokens;  // tokens per grad_W partial
    int64_t groups;
    int64_t off_s, off_hi, off_lo, off_wt, off_partial;
    int64_t bytes;
};

LayerPlan layer_plan(int64_t T, int64_t C);

// Size of the device array that mhc_layer_bwd_noalloc uses as its workspace
// (one per GPU, for the life of the process): shapes whose layer_plan bytes
// exceed it are refused.
constexpr int64_t kLayerNoAllocScratchBytes = (int64_t)64 << 20;
// Device address of that array on `device`, which must be the current device
// (looked up once per device, then cached; thread-safe).
hipError_t layer_noalloc_scratch(int device, void** ptr);
hipError_t launch_layer_fwd(const LayerPtrs& a, int64_t T, int64_t C, float eps,
                            const SolverOpts& o, hipStream_t stream);
hipError_t launch_layer_bwd(const LayerPtrs& a, int64_t T, int64_t C, hipStream_t stream);

}  // namespace mhc
