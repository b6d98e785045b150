// Batched 4x4 Birkhoff projection kernels for gfx950: forward (Newton or
// Sinkhorn-Knopp) and backward (implicit differentiation).
//
// Forward layout: one lane per matrix, 64 matrices per wave64, 256 per
// workgroup.  A wave moves its 64 consecutive matrices (4 KB) through a
// per-wave LDS tile (stage.h), so its global loads and stores are contiguous
// 1 KB pieces, and each lane keeps its whole solve in VGPRs (proj4.h).  There
// is no other cross-lane communication; lanes past B solve a zero matrix and
// store nothing.  The forward is bound by VALU work (exp2/log2/rcp and the
// Newton solve); the backward is straight-line and bound by HBM traffic
// (192 bytes/matrix), so it uses one row per lane instead (see
// birkhoff_bwd_kernel).
#include "kernels.h"
#include "proj4.h"
#include "stage.h"

namespace mhc {

namespace {

constexpr int kBlock = 256;

// logits and P may be the same buffer: a wave reads all of its matrices
// before it writes any, and no wave touches another wave's matrices.
template <int SOLVER>
__global__ __launch_bounds__(kBlock) void birkhoff_fwd_kernel(const float* logits, float* P,
                                                              uint8_t* __restrict__ iters,
                                                              int64_t B, SolverOpts o)
{
    __shared__ float tiles[kBlock / 64][stage_tile_floats<16>()];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t first = (int64_t)blockIdx.x * kBlock + 64 * w;
    if (first >= B) return;  // the whole wave is past the batch
    float a[16], p[16];
    load_records_v4<16>(logits, first, B, tiles[w], a, lane);
    const uint32_t it = SOLVER == 0 ? project_newton(a, p, o) : project_sinkhorn(a, p, o);
    store_records_v4<16>(P, first, B, tiles[w], p, lane);
    if (iters != nullptr && first + lane < B) iters[first + lane] = (uint8_t)it;
}

// Backward: one row per lane (quad = one matrix), so loads and stores are
// contiguous 16-byte rows across lanes.  A single generation of waves would
// load everything, compute, then store everything, leaving reads and writes
// in separate phases; instead a grid of kBwdWgPerCu workgroups per CU strides
// over the rows, and the rows of the next stride are loaded (into the other
// of two register sets) before the current ones are reduced and stored, so
// one stride's stores overlap the next one's loads.  Quads past B load a
// clamped row, compute on zeros and skip the store, which keeps every quad
// whole for the DPP reductions (the stride is a multiple of 4).
constexpr int kBwdWgPerCu = 2;
constexpr int kCus = 256;

struct BwdRows {
    float4 p, g;
};

MHC_DEV void bwd_issue(const float4* P, const float4* G, int64_t r, int64_t rows, BwdRows& d)
{
    const int64_t rc = r < rows ? r : rows - 1;
    d.p = mhc_load_stream(P + rc);
    d.g = mhc_load_stream(G + rc);
}

MHC_DEV void bwd_consume(const BwdRows& d, float4* dA, int64_t r)
{
    const float p[4] = {d.p.x, d.p.y, d.p.z, d.p.w};
    const float g[4] = {d.g.x, d.g.y, d.g.z, d.g.w};
    float o[4];
    project_bwd_row(p, g, o);
    mhc_store_stream(dA + r, make_float4(o[0], o[1], o[2], o[3]));
}

MHC_DEV void bwd_consume_tail(const BwdRows& d, float4* dA, int64_t r, int64_t rows)
{
    const bool ok = r < rows;
    const float p[4] = {ok ? d.p.x : 0.f, ok ? d.p.y : 0.f, ok ? d.p.z : 0.f, ok ? d.p.w : 0.f};
    const float g[4] = {ok ? d.g.x : 0.f, ok ? d.g.y : 0.f, ok ? d.g.z : 0.f, ok ? d.g.w : 0.f};
    float o[4];
    project_bwd_row(p, g, o);
    if (ok) mhc_store_stream(dA + r, make_float4(o[0], o[1], o[2], o[3]));
}

__global__ __launch_bounds__(kBlock) void birkhoff_bwd_kernel(const float4* __restrict__ P,
                                                              const float4* G, float4* dA,
                                                              int64_t B)
{
    const int64_t rows = 4 * B;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    int64_t r = (int64_t)blockIdx.x * kBlock + threadIdx.x;  // row 4 b + i
    // Pairs of strides that lie wholly inside the batch store without a
    // check (a conditional store would make the compiler's wait for the next
    // loads also wait for that store); the last, partial pair is checked.
    const int64_t full = rows / (2 * stride);
    BwdRows d0, d1;
    bwd_issue(P, G, r, rows, d0);
    for (int64_t k = 0; k < full; ++k) {
        bwd_issue(P, G, r + stride, rows, d1);
        __builtin_amdgcn_sched_barrier(0);
        bwd_consume(d0, dA, r);
        __builtin_amdgcn_sched_barrier(0);
        bwd_issue(P, G, r + 2 * stride, rows, d0);
        __builtin_amdgcn_sched_barrier(0);
        bwd_consume(d1, dA, r + stride);
        __builtin_amdgcn_sched_barrier(0);
        r += 2 * stride;
    }
    if (full * 2 * stride < rows) {
        bwd_issue(P, G, r + stride, rows, d1);
        bwd_consume_tail(d0, dA, r, rows);
        bwd_consume_tail(d1, dA, r + stride, rows);
    }
}

// Recompute backward: lane per matrix, the forward solve redone in
// registers and the implicit-differentiation gradient formed from that P
// (matrix-per-lane form of the backward), records staged as in the forward.
// logits or G may be the same buffer as dA: a wave reads all of its matrices
// from both before writing.
template <int SOLVER>
__global__ __launch_bounds__(kBlock) void birkhoff_bwd_recompute_kernel(const float* logits,
                                                                        const float* G,
                                                                        float* dA, int64_t B,
                                                                        SolverOpts o)
{
    __shared__ float tiles[kBlock / 64][stage_tile_floats<16>()];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t first = (int64_t)blockIdx.x * kBlock + 64 * w;
    if (first >= B) return;
    float a[16], g[16], p[16], d[16];
    load_records_v4<16>(logits, first, B, tiles[w], a, lane);
    load_records_v4<16>(G, first, B, tiles[w], g, lane);
    if (SOLVER == 0)
        project_newton(a, p, o);
    else
        project_sinkhorn(a, p, o);
    project_bwd(p, g, d);
    store_records_v4<16>(dA, first, B, tiles[w], d, lane);
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
    const int64_t need = (4 * B + kBlock - 1) / kBlock;
    const int64_t cap = (int64_t)kCus * kBwdWgPerCu;
    const dim3 grid((unsigned)(need < cap ? need : cap));
    hipLaunchKernelGGL(birkhoff_bwd_kernel, grid, dim3(kBlock), 0, stream,
                       reinterpret_cast<const float4*>(P), reinterpret_cast<const float4*>(G),
                       reinterpret_cast<float4*>(dA), B);
    return hipGetLastError();
}

hipError_t launch_birkhoff_bwd_recompute(const float* logits, const float* G, float* dA, int64_t B,
                                         const SolverOpts& o, hipStream_t stream)
{
    const dim3 grid((unsigned)((B + kBlock - 1) / kBlock));
    if (o.solver == 0)
        hipLaunchKernelGGL(birkhoff_bwd_recompute_kernel<0>, grid, dim3(kBlock), 0, stream,
                           logits, G, dA, B, o);
    else
        hipLaunchKernelGGL(birkhoff_bwd_recompute_kernel<1>, grid, dim3(kBlock), 0, stream,
                           logits, G, dA, B, o);
    return hipGetLastError();
}

}  // namespace mhc
