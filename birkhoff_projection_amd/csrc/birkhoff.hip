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

using FwdTiles = float[kBlock / 64][stage_tile_floats<16>()];

// One forward workgroup: matrices block*256 .. block*256+255.  logits and P
// may be the same buffer: a wave reads all of its matrices before it writes
// any, and no wave touches another wave's matrices.
template <int SOLVER>
MHC_DEV void fwd_block(const float* logits, float* P, uint8_t* __restrict__ iters, int64_t B,
                       const SolverOpts& o, FwdTiles& tiles, int64_t block)
{
    const int lane = threadIdx.x & 63, w = wave_index();
    const int64_t first = block * kBlock + 64 * w;
    if (first >= B) return;  // the whole wave is past the batch
    float a[16];
    load_records_v4<16>(logits, first, B, tiles[w], a, lane);
    // each lane's slot of the tile keeps its logits for the start's row
    // reads, then receives its P (Newton); the store reads the tile
    float* rec = tiles[w] + lane * record_pitch<16>();
    uint32_t it;
    if (SOLVER == 0) {
        it = project_newton_lds(a, rec, o);
        store_tile_v4<16>(P, first, B, tiles[w], lane);
    } else {
        float p[16];
        it = project_sinkhorn(a, p, o);
        store_records_v4<16>(P, first, B, tiles[w], p, lane);
    }
    if (iters != nullptr && first + lane < B) iters[first + lane] = (uint8_t)it;
}

template <int SOLVER>
__global__ __launch_bounds__(kBlock) void birkhoff_fwd_kernel(const float* logits, float* P,
                                                              uint8_t* __restrict__ iters,
                                                              int64_t B, SolverOpts o)
{
    __shared__ FwdTiles tiles;
    fwd_block<SOLVER>(logits, P, iters, B, o, tiles, blockIdx.x);
}

// Backward: one row per lane (quad = one matrix), so loads and stores are
// contiguous 16-byte rows across lanes, with the streaming hint, and one
// generation of waves covers the batch: each lane loads its P and G rows,
// the quad reduces them (DPP) and solves, and each lane stores its dA row.
// Lanes past the batch load a clamped row, compute on zeros and skip the
// store, which keeps every quad whole for the reductions (rows come in
// fours).  A grid-stride pipeline that loads the next rows before storing
// the current ones was faster when the accesses were plain; with streaming
// loads and stores this form is within 0.3 us of a copy-only kernel of the
// same pattern at 131072 matrices (5.9 against 6.4 us for the pipeline).
// dA may alias G exactly: a lane reads its rows before any lane of its quad
// exchanges values, and stores only its own row.
__global__ __launch_bounds__(kBlock) void birkhoff_bwd_kernel(const float4* __restrict__ P,
                                                              const float4* G, float4* dA,
                                                              int64_t B)
{
    const int64_t rows = 4 * B;
    const int64_t r = (int64_t)blockIdx.x * kBlock + threadIdx.x;  // row 4 b + i
    const bool ok = r < rows;
    const int64_t rc = ok ? r : rows - 1;
    const float4 pv = mhc_load_stream(P + rc);
    const float4 gv = mhc_load_stream(G + rc);
    const float p[4] = {ok ? pv.x : 0.f, ok ? pv.y : 0.f, ok ? pv.z : 0.f, ok ? pv.w : 0.f};
    const float g[4] = {ok ? gv.x : 0.f, ok ? gv.y : 0.f, ok ? gv.z : 0.f, ok ? gv.w : 0.f};
    float o[4];
    project_bwd_row(p, g, o);
    if (ok) mhc_store_stream(dA + r, make_float4(o[0], o[1], o[2], o[3]));
}

// The backward for the workgroups of birkhoff_pipeline_kernel: one lane per
// matrix, as in birkhoff_solve_bwd_kernel, so the 3x3 solve runs once per
// matrix instead of in every lane of a quad (about half the VALU
// instructions of birkhoff_bwd_kernel, which matters here: beside the
// forward, the two halves share the SIMDs' issue slots).  A wave issues the
// loads of its 64 P records and 64 G records first, then moves each set
// through its LDS tile to one record per lane; dA goes back the same way.
// The result is bit for bit what birkhoff_solve_bwd_kernel's project_bwd
// gives for the same P and G.
MHC_DEV void bwd_block_lanes(const float* P, const float* G, float* dA, int64_t B,
                             FwdTiles& tiles, int64_t block)
{
    const int lane = threadIdx.x & 63, w = wave_index();
    const int64_t first = block * kBlock + 64 * w;
    if (first >= B) return;  // the whole wave is past the batch
    float4 vp[4], vg[4];
    issue_records_v4<16>(P, first, B, vp, lane);
    issue_records_v4<16>(G, first, B, vg, lane);
    float p[16], g[16], d[16];
    scatter_records_v4<16>(vp, first, B, tiles[w], p, lane);
    scatter_records_v4<16>(vg, first, B, tiles[w], g, lane);
    project_bwd(p, g, d);
    store_records_v4<16>(dA, first, B, tiles[w], d, lane);
}

// Forward of one batch and backward of another in one launch: workgroups
// below fwd_blocks run birkhoff_fwd_kernel's work, the rest the backward
// (bwd_block_lanes, 256 matrices per workgroup).  The two halves complement
// each other on the chip: the forward is bound by the latency of its solve at
// two waves per SIMD and leaves HBM mostly idle, the backward is bound by HBM,
// so the backward's workgroups fill the SIMD slots the forward leaves free
// (at 131072 matrices two forward and two backward waves per SIMD, all
// resident at once).  Forward workgroups come first, so they are dispatched
// first and spread evenly over the CUs (orders that mix backward workgroups
// in among them, round-robin or in rounds of eight, one per XCD, left some
// SIMDs with more forward waves and measured 25-30 % slower at 131072
// matrices).  The batches are independent (the ABI rejects overlaps between
// them), as when a trainer runs micro-batch k's forward while micro-batch
// k-1 goes backward, or recomputes one layer's projection during another
// layer's backward.  grad_logits may be grad_P itself: a wave reads all of its
// records before it writes any.
template <int SOLVER>
__global__ __launch_bounds__(kBlock) void birkhoff_pipeline_kernel(
    const float* logits, float* P, uint8_t* __restrict__ iters, int64_t B, SolverOpts o,
    const float* __restrict__ Pb, const float* Gb, float* dAb, int64_t Bb, unsigned fwd_blocks)
{
    __shared__ FwdTiles tiles;
    if (blockIdx.x < fwd_blocks)
        fwd_block<SOLVER>(logits, P, iters, B, o, tiles, blockIdx.x);
    else
        bwd_block_lanes(Pb, Gb, dAb, Bb, tiles, (int64_t)(blockIdx.x - fwd_blocks));
}

// Solve and differentiate in one pass: lane per matrix, the projection
// solved in registers and the implicit-differentiation gradient formed from
// that P while it is still there (matrix-per-lane form of the backward),
// records staged as in the forward.  Two entry points use it:
//  * the recompute backward (WRITE_P false): P is not stored at all, the
//    forward solve is simply redone;
//  * the fused forward + backward (WRITE_P true), for when dL/dP is known
//    when the projection is computed: P (and the iteration codes) are
//    stored as well, 256 bytes per matrix in one launch instead of 320 in
//    two.
// A wave reads all of its matrices from logits and G before writing any, so
// P may be the logits buffer and dA the G buffer (the ABI rejects the other
// overlaps).
template <int SOLVER, bool WRITE_P>
__global__ __launch_bounds__(kBlock) void birkhoff_solve_bwd_kernel(const float* logits,
                                                                    const float* G, float* P,
                                                                    float* dA,
                                                                    uint8_t* __restrict__ iters,
                                                                    int64_t B, SolverOpts o)
{
    // G goes through a tile of its own, so the logits' tile is intact for
    // the start's row reads (the same start as birkhoff_fwd_kernel's)
    __shared__ float tiles[kBlock / 64][stage_tile_floats<16>()];
    __shared__ float gtiles[kBlock / 64][stage_tile_floats<16>()];
    const int lane = threadIdx.x & 63, w = wave_index();
    const int64_t first = (int64_t)blockIdx.x * kBlock + 64 * w;
    if (first >= B) return;
    float a[16], g[16], p[16], d[16];
    load_records_v4<16>(logits, first, B, tiles[w], a, lane);
    load_records_v4<16>(G, first, B, gtiles[w], g, lane);
    float* rec = tiles[w] + lane * record_pitch<16>();
    uint32_t it;
    if (SOLVER == 0) {
        // P is left in the lane's own slot of the tile (no cross-lane data)
        it = project_newton_lds(a, rec, o);
#pragma unroll
        for (int k = 0; k < 16; ++k) p[k] = rec[k];
        if (WRITE_P) store_tile_v4<16>(P, first, B, tiles[w], lane);
    } else {
        it = project_sinkhorn(a, p, o);
        if (WRITE_P) store_records_v4<16>(P, first, B, tiles[w], p, lane);
    }
    project_bwd(p, g, d);
    store_records_v4<16>(dA, first, B, tiles[w], d, lane);
    if (WRITE_P && iters != nullptr && first + lane < B) iters[first + lane] = (uint8_t)it;
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
    // 4 B rows, one per lane; B <= 2^36 keeps the grid below 2^30
    const dim3 grid((unsigned)((4 * B + kBlock - 1) / kBlock));
    hipLaunchKernelGGL(birkhoff_bwd_kernel, grid, dim3(kBlock), 0, stream,
                       reinterpret_cast<const float4*>(P), reinterpret_cast<const float4*>(G),
                       reinterpret_cast<float4*>(dA), B);
    return hipGetLastError();
}

hipError_t launch_birkhoff_pipeline(const float* logits, float* P, uint8_t* iters, int64_t B,
                                   const SolverOpts& o, const float* Pb, const float* Gb,
                                   float* dAb, int64_t Bb, hipStream_t stream)
{
    const int64_t fwd_blocks = (B + kBlock - 1) / kBlock;
    const int64_t bwd_blocks = (Bb + kBlock - 1) / kBlock;
    const dim3 grid((unsigned)(fwd_blocks + bwd_blocks));
    if (o.solver == 0)
        hipLaunchKernelGGL(birkhoff_pipeline_kernel<0>, grid, dim3(kBlock), 0, stream, logits, P,
                           iters, B, o, Pb, Gb, dAb, Bb, (unsigned)fwd_blocks);
    else
        hipLaunchKernelGGL(birkhoff_pipeline_kernel<1>, grid, dim3(kBlock), 0, stream, logits, P,
                           iters, B, o, Pb, Gb, dAb, Bb, (unsigned)fwd_blocks);
    return hipGetLastError();
}

hipError_t launch_birkhoff_bwd_recompute(const float* logits, const float* G, float* dA, int64_t B,
                                         const SolverOpts& o, hipStream_t stream)
{
    const dim3 grid((unsigned)((B + kBlock - 1) / kBlock));
    if (o.solver == 0)
        hipLaunchKernelGGL((birkhoff_solve_bwd_kernel<0, false>), grid, dim3(kBlock), 0, stream,
                           logits, G, nullptr, dA, nullptr, B, o);
    else
        hipLaunchKernelGGL((birkhoff_solve_bwd_kernel<1, false>), grid, dim3(kBlock), 0, stream,
                           logits, G, nullptr, dA, nullptr, B, o);
    return hipGetLastError();
}

hipError_t launch_birkhoff_fwd_bwd(const float* logits, const float* G, float* P, float* dA,
                                   uint8_t* iters, int64_t B, const SolverOpts& o,
                                   hipStream_t stream)
{
    const dim3 grid((unsigned)((B + kBlock - 1) / kBlock));
    if (o.solver == 0)
        hipLaunchKernelGGL((birkhoff_solve_bwd_kernel<0, true>), grid, dim3(kBlock), 0, stream,
                           logits, G, P, dA, iters, B, o);
    else
        hipLaunchKernelGGL((birkhoff_solve_bwd_kernel<1, true>), grid, dim3(kBlock), 0, stream,
                           logits, G, P, dA, iters, B, o);
    return hipGetLastError();
}

}  // namespace mhc
