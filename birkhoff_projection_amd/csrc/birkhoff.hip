// Batched 4x4 Birkhoff projection kernels for gfx950: forward (Newton or
// Sinkhorn-Knopp) and backward (implicit differentiation).
//
// Layout: one lane per matrix, 64 matrices per wave64, 256 per workgroup.
// A lane reads its matrix as four 16-byte loads (64 contiguous bytes), keeps
// the whole solve in VGPRs (proj4.h) and writes four 16-byte stores.  There is
// no cross-lane communication, so a tail wave simply masks off the lanes past
// B.  The forward is bound by VALU work (exp2/log2/rcp and the Newton solve);
// the backward is straight-line and bound by HBM traffic (192 bytes/matrix),
// so it uses one row per lane instead (see birkhoff_bwd_kernel).
#include "kernels.h"
#include "proj4.h"

namespace mhc {

namespace {

constexpr int kBlock = 256;

MHC_DEV void load16(const float* src, float* v)
{
    const float4* p = reinterpret_cast<const float4*>(src);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float4 q = p[k];
        v[4 * k + 0] = q.x;
        v[4 * k + 1] = q.y;
        v[4 * k + 2] = q.z;
        v[4 * k + 3] = q.w;
    }
}

MHC_DEV void store16(float* dst, const float* v)
{
    float4* p = reinterpret_cast<float4*>(dst);
#pragma unroll
    for (int k = 0; k < 4; ++k) p[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
}

// logits and P may be the same buffer: each lane reads its whole matrix
// before it writes it, and no lane touches another lane's matrix.
template <int SOLVER>
__global__ __launch_bounds__(kBlock) void birkhoff_fwd_kernel(const float* logits, float* P,
                                                              uint8_t* __restrict__ iters,
                                                              int64_t B, SolverOpts o)
{
    const int64_t b = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (b >= B) return;
    float a[16], p[16];
    load16(logits + 16 * b, a);
    const uint32_t it = SOLVER == 0 ? project_newton(a, p, o) : project_sinkhorn(a, p, o);
    store16(P + 16 * b, p);
    if (iters != nullptr) iters[b] = (uint8_t)it;
}

// Backward: one row per lane (quad = one matrix, 64 matrices per 256-lane
// workgroup), so loads and stores are contiguous 16-byte rows across lanes
// and a launch has four times the waves of the forward.  Quads past B load
// zeros (all-zero rows give a zero gradient) and skip the store, keeping every
// quad fully active for the DPP reductions.
__global__ __launch_bounds__(kBlock) void birkhoff_bwd_kernel(const float4* __restrict__ P,
                                                              const float4* G, float4* dA,
                                                              int64_t B)
{
    const int64_t r = (int64_t)blockIdx.x * kBlock + threadIdx.x;  // row 4 b + i
    const bool ok = (r >> 2) < B;
    const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 p4 = ok ? P[r] : zero;
    const float4 g4 = ok ? G[r] : zero;
    const float p[4] = {p4.x, p4.y, p4.z, p4.w};
    const float g[4] = {g4.x, g4.y, g4.z, g4.w};
    float d[4];
    project_bwd_row(p, g, d);
    if (ok) dA[r] = make_float4(d[0], d[1], d[2], d[3]);
}

}  // namespace

hipError_t launch_birkhoff_fwd(const float* logits, float* P, uint8_t* iters, int64_t B,
                               const SolverOpts& o, hipStream_t stream)
{
    const dim3 grid((unsigned)((B + kBlock - 1) / kBlock));
    if (o.solver == 0)
        hipLaunchKernelGGL(birkhoff_fwd_kernel<0>, grid, dim3(kBlock), 0, stream, logits, P,
                           iters, B, o);
    else
        hipLaunchKernelGGL(birkhoff_fwd_kernel<1>, grid, dim3(kBlock), 0, stream, logits, P,
                           iters, B, o);
    return hipGetLastError();
}

hipError_t launch_birkhoff_bwd(const float* P, const float* G, float* dA, int64_t B,
                               hipStream_t stream)
{
    const dim3 grid((unsigned)((4 * B + kBlock - 1) / kBlock));
    hipLaunchKernelGGL(birkhoff_bwd_kernel, grid, dim3(kBlock), 0, stream,
                       reinterpret_cast<const float4*>(P), reinterpret_cast<const float4*>(G),
                       reinterpret_cast<float4*>(dA), B);
    return hipGetLastError();
}

}  // namespace mhc
