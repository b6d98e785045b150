// n x n Birkhoff projection kernels for n = 1..8 other than 4 (the 4x4 case
// has its own kernels in birkhoff.hip).  One lane per matrix, solved in
// registers (projn.h).  A matrix is n*n floats, generally not 16-byte
// aligned and, at n = 8, 256 bytes, so each wave moves its 64 consecutive
// matrices through a padded LDS tile (stage.h): the wave's global loads and
// stores are contiguous 256-byte runs.  A wave reads all of its inputs before
// it writes, so P may be the logits' buffer and dA the gradient's.
#include "kernels.h"
#include "projn.h"
#include "stage.h"

namespace mhc {

namespace {

constexpr int kBlockN = 256;

// store_records for records that are already in the tile (lane l's record
// at tile + l * record_pitch<R>(), each written by its own lane): only the
// coalesced global stores.
template <int R>
MHC_DEV void store_tile(float* __restrict__ g, int64_t first, int64_t B, const float* tile,
                        int lane)
{
    constexpr int kP = record_pitch<R>();
    const int64_t have = B - first;
    mhc_wave_lds_fence();  // the reads below see the other lanes' writes
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

// At least two waves per SIMD: left to itself the compiler gives the 7x7 and
// 8x8 Newton solves 276 and 306 registers (all 256 VGPRs plus AGPRs), one
// wave per SIMD, so 131072 matrices run in two generations of lone waves.
// Held to 256 the 7x7 solve needed no spill and the 8x8 one spilled 204
// bytes to scratch (20 in the current solver), and still: 7x7 51.7 -> 41.1
// us, 8x8 74.6 -> 62.7 us at 131072 matrices (same-process A/B, bit-identical
// output).  Smaller n already fit.
template <int N, int SOLVER>
__global__ __launch_bounds__(kBlockN) __attribute__((amdgpu_waves_per_eu(2))) void birkhoff_fwd_n_kernel(const float* logits, float* P,
                                                                 uint8_t* __restrict__ iters,
                                                                 int64_t B, SolverOpts o)
{
    constexpr int R = N * N;
    __shared__ float tiles[kBlockN / 64][stage_tile_floats<R>()];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t first = (int64_t)blockIdx.x * kBlockN + 64 * w;
    if (first >= B) return;  // the whole wave is past the batch
    float a[R];
    load_records<R>(logits, first, B, tiles[w], a, lane);
    uint32_t it;
    if (SOLVER == 0) {
        // the lane's slot of the tile is free once its logits are in
        // registers; the solve leaves P there and the store reads the tile
        it = project_newton_lds_n<N>(a, tiles[w] + lane * record_pitch<R>(), o);
        store_tile<R>(P, first, B, tiles[w], lane);
    } else {
        float p[R];
        it = project_sinkhorn_n<N>(a, p, o);
        store_records<R>(P, first, B, tiles[w], p, lane);
    }
    if (iters != nullptr && first + lane < B) iters[first + lane] = (uint8_t)it;
}

template <int N>
__global__ __launch_bounds__(kBlockN) void birkhoff_bwd_n_kernel(const float* P, const float* G,
                                                                 float* dA, int64_t B)
{
    constexpr int R = N * N;
    __shared__ float tiles[kBlockN / 64][stage_tile_floats<R>()];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t first = (int64_t)blockIdx.x * kBlockN + 64 * w;
    if (first >= B) return;
    float p[R], g[R], d[R];
    load_records<R>(P, first, B, tiles[w], p, lane);
    load_records<R>(G, first, B, tiles[w], g, lane);
    project_bwd_n<N>(p, g, d);
    store_records<R>(dA, first, B, tiles[w], d, lane);
}

// n = 2 in closed form.  A 2x2 doubly stochastic matrix is [[p, 1-p], [1-p, p]]
// and diag(u) exp(A) diag(v) has that form exactly when
// p / (1-p) = sqrt(K11 K22 / (K12 K21)), i.e. p = sigmoid(s / 2) with
// s = a11 + a22 - a12 - a21 -- the unique scaling the Newton solve converges to
// (used for the Newton solver; Sinkhorn keeps its own iterates).  1 - p is
// formed as sigmoid(-s / 2), without cancellation.  The gradient through it is
// dA = (G11 - G12 - G21 + G22) p (1-p) / 2 [[1, -1], [-1, 1]].
MHC_DEV float sigmoid_half(float s)
{
    return mhc_rcp(1.f + mhc_exp2(-0.5f * kLog2e * s));
}

__global__ __launch_bounds__(kBlockN) void birkhoff_fwd_2_closed_kernel(const float* logits,
                                                                        float* P,
                                                                        uint8_t* __restrict__ iters,
                                                                        int64_t B)
{
    const int64_t b = (int64_t)blockIdx.x * kBlockN + threadIdx.x;
    if (b >= B) return;
    const float4 a = reinterpret_cast<const float4*>(logits)[b];
    const float s = (a.x + a.w) - (a.y + a.z);
    const float p = sigmoid_half(s), q = sigmoid_half(-s);
    reinterpret_cast<float4*>(P)[b] = make_float4(p, q, q, p);
    if (iters != nullptr) iters[b] = 0;
}

__global__ __launch_bounds__(kBlockN) void birkhoff_bwd_2_closed_kernel(const float* __restrict__ P,
                                                                        const float* G, float* dA,
                                                                        int64_t B)
{
    const int64_t b = (int64_t)blockIdx.x * kBlockN + threadIdx.x;
    if (b >= B) return;
    const float4 p = reinterpret_cast<const float4*>(P)[b];
    const float4 g = reinterpret_cast<const float4*>(G)[b];
    // p (1-p) from the two entries of a row (they sum to 1)
    const float h = 0.5f * p.x * p.y * ((g.x - g.y) - (g.z - g.w));
    reinterpret_cast<float4*>(dA)[b] = make_float4(h, -h, -h, h);
}

// n = 1: the only doubly stochastic 1x1 matrix is [1]; its gradient is 0.
__global__ __launch_bounds__(kBlockN) void birkhoff_one_kernel(float* out, uint8_t* iters,
                                                               float value, int64_t B)
{
    const int64_t b = (int64_t)blockIdx.x * kBlockN + threadIdx.x;
    if (b >= B) return;
    out[b] = value;
    if (iters != nullptr) iters[b] = 0;
}

template <int N>
hipError_t fwd_n(const float* logits, float* P, uint8_t* iters, int64_t B, const SolverOpts& o,
                 hipStream_t stream)
{
    const dim3 grid((unsigned)((B + kBlockN - 1) / kBlockN));
    if (o.solver == 0)
        hipLaunchKernelGGL((birkhoff_fwd_n_kernel<N, 0>), grid, dim3(kBlockN), 0, stream, logits,
                           P, iters, B, o);
    else
        hipLaunchKernelGGL((birkhoff_fwd_n_kernel<N, 1>), grid, dim3(kBlockN), 0, stream, logits,
                           P, iters, B, o);
    return hipGetLastError();
}

template <int N>
hipError_t bwd_n(const float* P, const float* G, float* dA, int64_t B, hipStream_t stream)
{
    const dim3 grid((unsigned)((B + kBlockN - 1) / kBlockN));
    hipLaunchKernelGGL(birkhoff_bwd_n_kernel<N>, grid, dim3(kBlockN), 0, stream, P, G, dA, B);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_birkhoff_fwd_n(const float* logits, float* P, uint8_t* iters, int64_t B, int n,
                                 const SolverOpts& o, hipStream_t stream)
{
    switch (n) {
    case 1:
        hipLaunchKernelGGL(birkhoff_one_kernel, dim3((unsigned)((B + kBlockN - 1) / kBlockN)),
                           dim3(kBlockN), 0, stream, P, iters, 1.f, B);
        return hipGetLastError();
    case 2:
        if (o.solver == 0 && ((uintptr_t)logits & 15u) == 0 && ((uintptr_t)P & 15u) == 0) {
            hipLaunchKernelGGL(birkhoff_fwd_2_closed_kernel, dim3((unsigned)((B + kBlockN - 1) / kBlockN)),
                               dim3(kBlockN), 0, stream, logits, P, iters, B);
            return hipGetLastError();
        }
        return fwd_n<2>(logits, P, iters, B, o, stream);
    case 3: return fwd_n<3>(logits, P, iters, B, o, stream);
    case 5: return fwd_n<5>(logits, P, iters, B, o, stream);
    case 6: return fwd_n<6>(logits, P, iters, B, o, stream);
    case 7: return fwd_n<7>(logits, P, iters, B, o, stream);
    case 8: return fwd_n<8>(logits, P, iters, B, o, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_birkhoff_bwd_n(const float* P, const float* G, float* dA, int64_t B, int n,
                                 hipStream_t stream)
{
    switch (n) {
    case 1:
        hipLaunchKernelGGL(birkhoff_one_kernel, dim3((unsigned)((B + kBlockN - 1) / kBlockN)),
                           dim3(kBlockN), 0, stream, dA, nullptr, 0.f, B);
        return hipGetLastError();
    case 2:
        if (((uintptr_t)P & 15u) == 0 && ((uintptr_t)G & 15u) == 0 && ((uintptr_t)dA & 15u) == 0) {
            hipLaunchKernelGGL(birkhoff_bwd_2_closed_kernel, dim3((unsigned)((B + kBlockN - 1) / kBlockN)),
                               dim3(kBlockN), 0, stream, P, G, dA, B);
            return hipGetLastError();
        }
        return bwd_n<2>(P, G, dA, B, stream);
    case 3: return bwd_n<3>(P, G, dA, B, stream);
    case 5: return bwd_n<5>(P, G, dA, B, stream);
    case 6: return bwd_n<6>(P, G, dA, B, stream);
    case 7: return bwd_n<7>(P, G, dA, B, stream);
    case 8: return bwd_n<8>(P, G, dA, B, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace mhc
