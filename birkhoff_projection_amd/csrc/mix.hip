// n = 4 stream mix kernels for gfx950.
//
// Forward:  out[t,i,:] = sum_j H[t,i,j] x[t,j,:]   (optionally projecting H's
//           logits in the same kernel first)
// Backward: grad_x[t,j,:] = sum_i H[t,i,j] grad_out[t,i,:]
//           grad_H[t,i,j] = <grad_out[t,i,:], x[t,j,:]>
//
// Both are HBM-streaming: per token the forward reads 4 C bf16 and writes
// 4 C bf16 (64 KiB at C = 4096); the mix itself is 2 flop per byte.  Every
// lane moves 16-byte chunks (8 bf16 columns of one stream row), consecutive
// lanes take consecutive chunks, so each wave-level load or store covers a
// contiguous kilobyte.  Arithmetic is fp32 FMA; results are rounded to bf16
// by the hardware round-to-nearest-even conversion.  There is no reuse of
// stream data, so nothing is staged through LDS; LDS only holds the per-token
// 4x4 matrices that all lanes of a workgroup share.
#include "kernels.h"
#include "proj4.h"
#include "wave.h"

namespace mhc {

namespace {

constexpr int kBlock = 256;
constexpr int kTokensPerBlock = 16;  // forward: tokens sharing one workgroup

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

MHC_DEV uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2_t r;
    r.x = (__bf16)lo;
    r.y = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}

// 8 bf16 (one uint4) -> 8 fp32
MHC_DEV void unpack8(const uint4& q, float* f)
{
    f[0] = mhc_bf16_lo(q.x);
    f[1] = mhc_bf16_hi(q.x);
    f[2] = mhc_bf16_lo(q.y);
    f[3] = mhc_bf16_hi(q.y);
    f[4] = mhc_bf16_lo(q.z);
    f[5] = mhc_bf16_hi(q.z);
    f[6] = mhc_bf16_lo(q.w);
    f[7] = mhc_bf16_hi(q.w);
}

MHC_DEV uint4 pack8(const float* f)
{
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                      pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
}

// out rows for one 8-column chunk: o_i = sum_j M[i][j] x_j  (M row-major 4x4)
MHC_DEV void mix_chunk(const float* M, const uint4* xin, uint4* oout)
{
    float x[4][8];
#pragma unroll
    for (int j = 0; j < 4; ++j) unpack8(xin[j], x[j]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float o[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float s = M[4 * i + 0] * x[0][c];
            s = __builtin_fmaf(M[4 * i + 1], x[1][c], s);
            s = __builtin_fmaf(M[4 * i + 2], x[2][c], s);
            s = __builtin_fmaf(M[4 * i + 3], x[3][c], s);
            o[c] = s;
        }
        oout[i] = pack8(o);
    }
}

// Forward.  Workgroup b of a grid of G takes up to kTokensPerBlock tokens
// b, b + G, b + 2G, ...: at any moment the workgroups stream neighbouring
// tokens, a contiguous front of the tensors, which HBM serves faster than
// G separate runs of consecutive tokens (T = 16384, C = 4096: 190 against
// 202 us; 2-9 % on most shapes measured).  Lanes 0..15 of wave 0 first
// obtain the tokens' 4x4 matrices -- projecting the logits (PROJ = 1 Newton,
// 2 Sinkhorn) or loading H (PROJ = 0) -- into LDS; then all 256 lanes stream
// the tokens' chunks.  H_out may be the logits buffer itself (a lane reads its
// token's logits before it writes that token's H), so neither pointer is
// declared restrict.
template <int PROJ>
__global__ __launch_bounds__(kBlock) void stream_mix_fwd_kernel(
    const uint4* __restrict__ x, const float* Hl, float* H_out, uint4* __restrict__ out,
    int64_t T, int64_t C8, SolverOpts o)
{
    __shared__ float sH[kTokensPerBlock][16];
    const int64_t b = blockIdx.x, G = gridDim.x;
    const int tid = threadIdx.x;
    // tokens b + G l for l < nt (the grid is ceil(T / kTokensPerBlock), so
    // every token belongs to exactly one workgroup)
    const int64_t per = (T - b + G - 1) / G;
    const int nt = (int)(per < kTokensPerBlock ? per : kTokensPerBlock);
    if (tid < nt) {
        const int64_t t = b + G * tid;
        float a[16], h[16];
        const float4* src = reinterpret_cast<const float4*>(Hl + 16 * t);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float4 q = src[k];
            a[4 * k] = q.x;
            a[4 * k + 1] = q.y;
            a[4 * k + 2] = q.z;
            a[4 * k + 3] = q.w;
        }
        if (PROJ == 0) {
#pragma unroll
            for (int k = 0; k < 16; ++k) h[k] = a[k];
        } else {
            if (PROJ == 1)
                project_newton(a, h, o);
            else
                project_sinkhorn(a, h, o);
            if (H_out != nullptr) {
                float4* dst = reinterpret_cast<float4*>(H_out + 16 * t);
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    dst[k] = make_float4(h[4 * k], h[4 * k + 1], h[4 * k + 2], h[4 * k + 3]);
            }
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) sH[tid][k] = h[k];
    }
    __syncthreads();

    for (int tl = 0; tl < nt; ++tl) {
        float M[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) M[k] = sH[tl][k];
        const int64_t row = (b + G * tl) * 4 * C8;  // first chunk of stream 0
        for (int64_t c = tid; c < C8; c += kBlock) {
            uint4 xin[4], oo[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) xin[j] = mhc_load_stream(&x[row + j * C8 + c]);
            mix_chunk(M, xin, oo);
#pragma unroll
            for (int i = 0; i < 4; ++i) mhc_store_stream(&out[row + i * C8 + c], oo[i]);
        }
    }
}

// Backward.  One wave per token at a time (grid-stride); a lane accumulates
// its chunks' contribution to grad_H in 16 registers, the wave reduces them
// once per token.
__global__ __launch_bounds__(kBlock) void stream_mix_bwd_kernel(
    const uint4* __restrict__ x, const float* __restrict__ H, const uint4* __restrict__ gout,
    uint4* __restrict__ gx, float* __restrict__ gH, int64_t T, int64_t C8)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * (kBlock / 64);
    for (int64_t t = wave; t < T; t += nwaves) {
        float Mt[16];  // H transposed: grad_x_j = sum_i H_ij g_i
        const float4* hp = reinterpret_cast<const float4*>(H + 16 * t);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float4 q = hp[k];
            Mt[k] = q.x;
            Mt[4 + k] = q.y;
            Mt[8 + k] = q.z;
            Mt[12 + k] = q.w;
        }
        float acc[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) acc[k] = 0.f;
        const int64_t row = t * 4 * C8;
        for (int64_t c = lane; c < C8; c += 64) {
            uint4 xin[4], gin[4], oo[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                xin[j] = mhc_load_stream(&x[row + j * C8 + c]);
                gin[j] = mhc_load_stream(&gout[row + j * C8 + c]);
            }
            mix_chunk(Mt, gin, oo);
#pragma unroll
            for (int j = 0; j < 4; ++j) mhc_store_stream(&gx[row + j * C8 + c], oo[j]);
            float xf[4][8], gf[4][8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                unpack8(xin[j], xf[j]);
                unpack8(gin[j], gf[j]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int cc = 0; cc < 8; ++cc)
                        acc[4 * i + j] = __builtin_fmaf(gf[i][cc], xf[j][cc], acc[4 * i + j]);
        }
        const float s = wave_sum_halving<16>(acc);
        if ((lane & 3) == 0) gH[16 * t + (lane >> 2)] = s;
    }
}

}  // namespace

hipError_t launch_stream_mix_fwd(const void* x, const float* Hl, float* H_out, void* out,
                                 int64_t T, int64_t C, const SolverOpts* proj,
                                 hipStream_t stream)
{
    const dim3 grid((unsigned)((T + kTokensPerBlock - 1) / kTokensPerBlock));
    const int64_t C8 = C / 8;
    const uint4* xv = static_cast<const uint4*>(x);
    uint4* ov = static_cast<uint4*>(out);
    if (proj == nullptr) {
        hipLaunchKernelGGL(stream_mix_fwd_kernel<0>, grid, dim3(kBlock), 0, stream, xv, Hl,
                           nullptr, ov, T, C8, SolverOpts{});
    } else if (proj->solver == 0) {
        hipLaunchKernelGGL(stream_mix_fwd_kernel<1>, grid, dim3(kBlock), 0, stream, xv, Hl,
                           H_out, ov, T, C8, *proj);
    } else {
        hipLaunchKernelGGL(stream_mix_fwd_kernel<2>, grid, dim3(kBlock), 0, stream, xv, Hl,
                           H_out, ov, T, C8, *proj);
    }
    return hipGetLastError();
}

hipError_t launch_stream_mix_bwd(const void* x, const float* H, const void* gout, void* gx,
                                 float* gH, int64_t T, int64_t C, hipStream_t stream)
{
    // enough waves to fill the chip several times over, each looping on tokens
    const int64_t waves_wanted = T < 8192 ? T : 8192;
    const dim3 grid((unsigned)((waves_wanted + 3) / 4));
    hipLaunchKernelGGL(stream_mix_bwd_kernel, grid, dim3(kBlock), 0, stream,
                       static_cast<const uint4*>(x), H, static_cast<const uint4*>(gout),
                       static_cast<uint4*>(gx), gH, T, C / 8);
    return hipGetLastError();
}

}  // namespace mhc
