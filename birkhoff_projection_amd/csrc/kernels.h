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
hipError_t launch_stream_mix_fwd(const void* x, const float* Hl, float* H_out, void* out,
                                 int64_t T, int64_t C, const SolverOpts* proj,
                                 hipStream_t stream);
hipError_t launch_stream_mix_bwd(const void* x, const float* H, const void* gout, void* gx,
                                 float* gH, int64_t T, int64_t C, hipStream_t stream);

}  // namespace mhc
