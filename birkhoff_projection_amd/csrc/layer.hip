// One mHC residual-layer step for n = 4 streams on gfx950 (forward and
// backward), per token t:
//
//   r      = sqrt(mean(x_t^2) + eps) over the flattened 4C stream values
//   l      = (x_t W^T) / r                     W [24, 4C], rows pre|post|res
//   H_pre  = sigmoid(l[0:4]),  H_post = sigmoid(l[4:8]),  H_res = P(l[8:24])
//   u      = sum_j H_pre[j] x_j                (read-mix, the layer input)
//   x_out_i = H_post[i] f + sum_j H_res[i,j] x_j   (write-back)
//
// (forpes.ru mHC explainer, "Hyper-Connections" and "mHC" sections: n
// parallel streams, projection to the model width before the layer function
// and expansion after, sigmoid on the pre/post maps; kimiseek V4-Flash
// article: the maps are generated from the input; neo-ai mHC summary: fused
// RMSNorm + matmul + activation kernels, mixed precision.)
//
// Kernels (all HBM-streaming except the small solves):
//   maps   x W^T on bf16 MFMA with the per-token sum of squares in the same
//          pass; epilogue: 1/r scaling, sigmoids, Birkhoff projection
//   mix    read-mix and write-back
//   dots   per-token reductions dH_pre, dH_post, dH_res (read only); epilogue:
//          sigmoid derivative and projection backward -> grad_logits
//   wt     W transposed to [4C][24] for the dx pass
//   dx     grad_x = H_res^T grad_x_out + H_pre grad_u + RMSNorm backward of
//          grad_logits W, the latter on MFMA; grad_f = H_post^T grad_x_out
//   dw     grad_W partials = (grad_logits / r)^T x on MFMA, x transposed
//          through LDS; then a fixed-order reduction over token groups
//
// Mixed precision: MFMA operands are bf16.  x and W are bf16 already (exact);
// grad_logits is fp32 and enters MFMA as the sum of two bf16 halves (hi +
// lo, about 16 significant bits), so its products keep fp32-level accuracy.
// Accumulation is fp32 throughout.
#include <atomic>
#include <mutex>

#include "kernels.h"
#include "proj4.h"
#include "wave.h"

namespace mhc {

namespace {

constexpr int kBlock = 256;
constexpr int kMaps = 24;            // n*n + 2n for n = 4

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

MHC_DEV uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2_t r;
    r.x = (__bf16)lo;
    r.y = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}

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

MHC_DEV uint32_t word(const uint4& q, int i)
{
    return i == 0 ? q.x : (i == 1 ? q.y : (i == 2 ? q.z : q.w));
}

MHC_DEV float sigmoid(float z) { return 1.f / (1.f + expf(-z)); }

MHC_DEV bf16x8 as_bf16x8(const uint4& q) { return __builtin_bit_cast(bf16x8, q); }

// Split 8 fp32 values into bf16 hi and lo parts with v ~= hi + lo.
MHC_DEV void split8(const float* v, bf16x8& hi, bf16x8& lo)
{
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const __bf16 h = (__bf16)v[e];
        hi[e] = h;
        lo[e] = (__bf16)(v[e] - (float)h);
    }
}

// ---------------------------------------------------------------------------
// maps: 64 tokens per workgroup; wave w handles stream w, i.e. the K range
// [w C, (w+1) C) of the flattened token vector, in stages of 64 k.
// MFMA 16x16x32 bf16:
//   A (16 tokens x 32 k): lane l holds x[token 16*tile + l%16][k0 + 8*(l/16) ..+7]
//   B (32 k x 16 maps):   lane l holds W[map 16*ot + l%16][k0 + 8*(l/16) ..+7]
//   D (16 x 16):          lane l, v -> token 4*(l/16)+v, map l%16
// Loading A straight from HBM in that layout would make every load
// instruction touch 16 rows with 64 bytes each; instead each stage of x
// (64 tokens x 128 bytes) is loaded with 8 rows x 128 contiguous bytes per
// instruction into the wave's own LDS tile and A is read from there.  The
// tile is private to the wave, so the K loop needs no workgroup barrier.
// Every workgroup reads all of W as B fragments (from L2), so 64 tokens per
// workgroup keeps that traffic at half the x traffic.
// Pipeline as in the dx pass: stage i+1's loads (W fragments, x rows) are
// issued into the other register set before stage i is consumed.
// ---------------------------------------------------------------------------
constexpr int kMapTok = 64;                 // tokens per workgroup
constexpr int kMapTiles = kMapTok / 16;     // MFMA token tiles
constexpr int kMapK = 64;                   // k per stage
constexpr int kMapSteps = kMapK / 32;       // MFMA k-steps per stage
constexpr int kMapPitch = kMapK + 8;        // bf16 per LDS row (bank spread)
constexpr int kMapRowPieces = kMapK / 8;    // 16-byte pieces per row per stage
constexpr int kMapRowsPerLoad = 64 / kMapRowPieces;
constexpr int kMapPieces = kMapTok / kMapRowsPerLoad;  // x pieces per lane per stage

struct MapLoads {
    uint4 b[kMapSteps][2];  // W fragments
    uint4 xr[kMapPieces];   // x rows: piece q -> token 8q + lane/8, 16 bytes at lane%8
};

struct MapLane {
    const uint16_t* xrow[kMapPieces];  // stream-w row start of the piece's token (clamped)
    const uint16_t* wrow[2];           // W row of map 16 ot + row (clamped), stream w
    int64_t C;
    int row, kq, pc, pr;               // piece column (lane % 8) and row (lane / 8)
};

MHC_DEV void maps_issue(const MapLane& L, MapLoads& d, int64_t k0)
{
    // k past C (ragged last stage) is clamped; those k-steps are skipped
#pragma unroll
    for (int s = 0; s < kMapSteps; ++s) {
        int64_t k = k0 + 32 * s + 8 * L.kq;
        k = k < L.C ? k : L.C - 8;
#pragma unroll
        for (int ot = 0; ot < 2; ++ot) d.b[s][ot] = *reinterpret_cast<const uint4*>(L.wrow[ot] + k);
    }
    int64_t k = k0 + 8 * L.pc;
    k = k < L.C ? k : L.C - 8;
#pragma unroll
    for (int q = 0; q < kMapPieces; ++q) d.xr[q] = *reinterpret_cast<const uint4*>(L.xrow[q] + k);
}

MHC_DEV void maps_consume(const MapLane& L, const MapLoads& d, uint16_t (*sX)[kMapPitch],
                          floatx4 (&acc)[kMapTiles][2], float (&ssq)[kMapTiles], int64_t k0)
{
    mhc_wave_lds_fence();  // the previous stage's reads of the tile come first
#pragma unroll
    for (int q = 0; q < kMapPieces; ++q)
        *reinterpret_cast<uint4*>(&sX[kMapRowsPerLoad * q + L.pr][8 * L.pc]) = d.xr[q];
    // the tile is this wave's own and LDS is in order within a wave; the
    // fence keeps the compiler from reusing earlier reads of it
    mhc_wave_lds_fence();
    const int64_t left = (L.C - k0) / 32;
    const int ns = left < kMapSteps ? (int)left : kMapSteps;
#pragma unroll
    for (int s = 0; s < kMapSteps; ++s) {
        if (s < ns) {
#pragma unroll
            for (int tile = 0; tile < kMapTiles; ++tile) {
                const uint4 a = *reinterpret_cast<const uint4*>(&sX[16 * tile + L.row][32 * s + 8 * L.kq]);
#pragma unroll
                for (int ot = 0; ot < 2; ++ot)
                    acc[tile][ot] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        as_bf16x8(a), as_bf16x8(d.b[s][ot]), acc[tile][ot], 0, 0, 0);
                float f[8];
                unpack8(a, f);
#pragma unroll
                for (int e = 0; e < 8; ++e) ssq[tile] = __builtin_fmaf(f[e], f[e], ssq[tile]);
            }
        }
    }
}

template <int SOLVER>
__global__ __launch_bounds__(kBlock) void layer_maps_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, float* __restrict__ logits,
    float* __restrict__ rms, float* __restrict__ Hpre, float* __restrict__ Hpost,
    float* __restrict__ Hres, int64_t T, int64_t C, float eps, SolverOpts o)
{
    __shared__ __attribute__((aligned(16))) uint16_t sX[4][kMapTok][kMapPitch];
    __shared__ float sRed[4][kMapTok][kMaps + 1];
    __shared__ float sSsq[4][kMapTok];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * kMapTok;
    const int64_t D = 4 * C;
    MapLane L;
    L.C = C;
    L.row = lane & 15;
    L.kq = lane >> 4;
    L.pc = lane % kMapRowPieces;
    L.pr = lane / kMapRowPieces;
#pragma unroll
    for (int q = 0; q < kMapPieces; ++q) {
        int64_t t = t0 + kMapRowsPerLoad * q + L.pr;
        t = t < T ? t : T - 1;
        L.xrow[q] = x + (t * 4 + w) * C;
    }
#pragma unroll
    for (int ot = 0; ot < 2; ++ot) {
        const int m = 16 * ot + L.row;
        L.wrow[ot] = W + (int64_t)(m < kMaps ? m : kMaps - 1) * D + (int64_t)w * C;
    }
    floatx4 acc[kMapTiles][2];
    float ssq[kMapTiles];
#pragma unroll
    for (int tile = 0; tile < kMapTiles; ++tile) {
        ssq[tile] = 0.f;
#pragma unroll
        for (int ot = 0; ot < 2; ++ot) acc[tile][ot] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    // branch-free ping-pong over an even number of stages; a stage past C
    // loads clamped addresses and does no MFMA
    const int64_t n = (C + kMapK - 1) / kMapK;
    MapLoads d0, d1;
    maps_issue(L, d0, 0);
    for (int64_t si = 0; si < n; si += 2) {
        maps_issue(L, d1, (si + 1) * kMapK);
        __builtin_amdgcn_sched_barrier(0);
        maps_consume(L, d0, sX[w], acc, ssq, si * kMapK);
        __builtin_amdgcn_sched_barrier(0);
        maps_issue(L, d0, (si + 2) * kMapK);
        __builtin_amdgcn_sched_barrier(0);
        maps_consume(L, d1, sX[w], acc, ssq, (si + 1) * kMapK);
        __builtin_amdgcn_sched_barrier(0);
    }
    const int row = L.row, kq = L.kq;
#pragma unroll
    for (int tile = 0; tile < kMapTiles; ++tile) {
#pragma unroll
        for (int ot = 0; ot < 2; ++ot) {
            const int m = 16 * ot + row;
            if (m < kMaps) {
#pragma unroll
                for (int v = 0; v < 4; ++v) sRed[w][16 * tile + 4 * kq + v][m] = acc[tile][ot][v];
            }
        }
        const float s = sum_bit5(sum_bit4(ssq[tile]));
        if (kq == 0) sSsq[w][16 * tile + row] = s;
    }
    __syncthreads();
    if (w != 0) return;
    const int64_t t = t0 + lane;
    if (t >= T) return;
    float l[kMaps];
#pragma unroll
    for (int m = 0; m < kMaps; ++m)
        l[m] = (sRed[0][lane][m] + sRed[1][lane][m]) + (sRed[2][lane][m] + sRed[3][lane][m]);
    const float ss = (sSsq[0][lane] + sSsq[1][lane]) + (sSsq[2][lane] + sSsq[3][lane]);
    const float r = sqrtf(ss / (float)D + eps);
    const float inv = 1.f / r;
#pragma unroll
    for (int m = 0; m < kMaps; ++m) l[m] *= inv;
    rms[t] = r;
    float4* lo = reinterpret_cast<float4*>(logits + kMaps * t);
#pragma unroll
    for (int q = 0; q < kMaps / 4; ++q) lo[q] = make_float4(l[4 * q], l[4 * q + 1], l[4 * q + 2], l[4 * q + 3]);
    reinterpret_cast<float4*>(Hpre)[t] = make_float4(sigmoid(l[0]), sigmoid(l[1]), sigmoid(l[2]), sigmoid(l[3]));
    reinterpret_cast<float4*>(Hpost)[t] = make_float4(sigmoid(l[4]), sigmoid(l[5]), sigmoid(l[6]), sigmoid(l[7]));
    float h[16];
    if (SOLVER == 0)
        project_newton(l + 8, h, o);
    else
        project_sinkhorn(l + 8, h, o);
    float4* ho = reinterpret_cast<float4*>(Hres + 16 * t);
#pragma unroll
    for (int q = 0; q < 4; ++q) ho[q] = make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
}

// ---------------------------------------------------------------------------
// mix: read-mix u and write-back x_out, 16 tokens per workgroup (spaced by
// the grid size).
// ---------------------------------------------------------------------------
constexpr int kMixTokens = 16;

__global__ __launch_bounds__(kBlock) void layer_mix_kernel(
    const uint4* __restrict__ x, const uint4* __restrict__ f, const float* __restrict__ Hpre,
    const float* __restrict__ Hpost, const float* __restrict__ Hres, uint4* __restrict__ u,
    uint4* __restrict__ xo, int64_t T, int64_t C8)
{
    __shared__ float sM[kMixTokens][kMaps];
    // tokens b + G l for l < nt, as in the stream mix forward: the
    // workgroups stream neighbouring tokens at any moment
    const int64_t b = blockIdx.x, G = gridDim.x;
    const int tid = threadIdx.x;
    const int64_t per = (T - b + G - 1) / G;
    const int nt = (int)(per < kMixTokens ? per : kMixTokens);
    for (int p = tid; p < nt * kMaps; p += kBlock) {
        const int tl = p / kMaps, m = p % kMaps;
        const int64_t t = b + G * tl;
        sM[tl][m] = m < 4 ? Hpre[4 * t + m] : (m < 8 ? Hpost[4 * t + m - 4] : Hres[16 * t + m - 8]);
    }
    __syncthreads();
    for (int tl = 0; tl < nt; ++tl) {
        float M[kMaps];
#pragma unroll
        for (int m = 0; m < kMaps; ++m) M[m] = sM[tl][m];
        const int64_t t = b + G * tl;
        for (int64_t c = tid; c < C8; c += kBlock) {
            float xs[4][8], ff[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) unpack8(mhc_load_stream(&x[(t * 4 + j) * C8 + c]), xs[j]);
            unpack8(mhc_load_stream(&f[t * C8 + c]), ff);
            float uu[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float s = M[0] * xs[0][e];
                s = __builtin_fmaf(M[1], xs[1][e], s);
                s = __builtin_fmaf(M[2], xs[2][e], s);
                uu[e] = __builtin_fmaf(M[3], xs[3][e], s);
            }
            mhc_store_stream(&u[t * C8 + c], pack8(uu));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float o8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float s = M[4 + i] * ff[e];
                    s = __builtin_fmaf(M[8 + 4 * i + 0], xs[0][e], s);
                    s = __builtin_fmaf(M[8 + 4 * i + 1], xs[1][e], s);
                    s = __builtin_fmaf(M[8 + 4 * i + 2], xs[2][e], s);
                    o8[e] = __builtin_fmaf(M[8 + 4 * i + 3], xs[3][e], s);
                }
                mhc_store_stream(&xo[(t * 4 + i) * C8 + c], pack8(o8));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// dots: wave w of workgroup b handles tokens 64 b + 16 w + [0, 16), one token
// at a time across the wave; lanes stride over the 8-column chunks.  (Tokens
// spaced by the grid's wave count, the order that speeds up the mix passes,
// made the backward 1 % slower here.)  The pass
// only reads (grad_f, which needs grad_x_out alone, is written by the dx pass:
// a small write stream mixed into this read stream costs far more than its
// bytes).  The
// (token, chunk) steps of a wave form one software pipeline: step i+1's loads
// are issued into the other register set before step i is consumed, across
// token boundaries too.  At a token's last chunk the 24 partial dots are
// wave-reduced into LDS; then lanes 0..15 each finish one token: sigmoid
// derivative, projection backward, the RMSNorm coefficient s = <dl, l> / (4C),
// and the transposed, r-scaled bf16 hi/lo copy of dl that the dW pass uses as
// an MFMA operand.
// ---------------------------------------------------------------------------
struct DotsLoads {
    uint4 x[4], g[4], f, u;
};

struct DotsLane {
    const uint4* x;
    const uint4* f;
    const uint4* gxo;
    const uint4* gu;
    int64_t T, C8, nch, tb;
    int lane;
};

MHC_DEV void dots_issue(const DotsLane& L, DotsLoads& d, int64_t i)
{
    // steps past the wave's last one read clamped addresses and are never consumed
    int64_t tl = i / L.nch;
    tl = tl < 16 ? tl : 15;
    int64_t t = L.tb + tl;
    t = t < L.T ? t : L.T - 1;
    int64_t c = L.lane + 64 * (i % L.nch);
    c = c < L.C8 ? c : L.C8 - 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        d.x[j] = L.x[(t * 4 + j) * L.C8 + c];
        d.g[j] = L.gxo[(t * 4 + j) * L.C8 + c];
    }
    d.f = L.f[t * L.C8 + c];
    d.u = L.gu[t * L.C8 + c];
}

MHC_DEV void dots_consume(const DotsLane& L, const DotsLoads& d, int64_t i, float (&acc)[32],
                          float (*sDots)[kMaps])
{
    const int64_t tl = i / L.nch, ci = i % L.nch;
    const int64_t t = L.tb + tl;
    const int64_t c = L.lane + 64 * ci;
    if (t < L.T && c < L.C8) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {  // one 32-bit word = 2 columns
            float xs[4][2], gs[4][2], ff[2], uu[2];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                xs[j][0] = mhc_bf16_lo(word(d.x[j], q));
                xs[j][1] = mhc_bf16_hi(word(d.x[j], q));
                gs[j][0] = mhc_bf16_lo(word(d.g[j], q));
                gs[j][1] = mhc_bf16_hi(word(d.g[j], q));
            }
            ff[0] = mhc_bf16_lo(word(d.f, q));
            ff[1] = mhc_bf16_hi(word(d.f, q));
            uu[0] = mhc_bf16_lo(word(d.u, q));
            uu[1] = mhc_bf16_hi(word(d.u, q));
#pragma unroll
            for (int e = 0; e < 2; ++e) {
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j] = __builtin_fmaf(uu[e], xs[j][e], acc[j]);
#pragma unroll
                for (int k = 0; k < 4; ++k) acc[4 + k] = __builtin_fmaf(gs[k][e], ff[e], acc[4 + k]);
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[8 + 4 * k + j] = __builtin_fmaf(gs[k][e], xs[j][e], acc[8 + 4 * k + j]);
            }
        }
    }
    if (ci == L.nch - 1) {  // the token's last chunk: reduce its dots
        const float sm = wave_sum_halving<32>(acc);
        const int idx = (L.lane >> 1) & 31;
        if ((L.lane & 1) == 0 && idx < kMaps) sDots[tl][idx] = sm;
#pragma unroll
        for (int k = 0; k < 32; ++k) acc[k] = 0.f;
    }
}

__global__ __launch_bounds__(kBlock) void layer_dots_kernel(
    const uint4* __restrict__ x, const uint4* __restrict__ f, const uint4* __restrict__ gxo,
    const uint4* __restrict__ gu, const float* __restrict__ Hpre, const float* __restrict__ Hpost,
    const float* __restrict__ Hres, const float* __restrict__ logits, const float* __restrict__ rms,
    float* __restrict__ glogits, float* __restrict__ svec, __bf16* __restrict__ dlT_hi,
    __bf16* __restrict__ dlT_lo, int64_t T, int64_t Tp, int64_t C8)
{
    __shared__ float sDots[4][16][kMaps];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t tb = (int64_t)blockIdx.x * 64 + 16 * w;
    DotsLane L;
    L.x = x; L.f = f; L.gxo = gxo; L.gu = gu;
    L.T = T; L.C8 = C8; L.nch = (C8 + 63) / 64; L.tb = tb; L.lane = lane;
    float acc[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) acc[k] = 0.f;
    // 16 tokens x nch chunks: always an even number of steps
    const int64_t steps = 16 * L.nch;
    DotsLoads d0, d1;
    dots_issue(L, d0, 0);
    for (int64_t i = 0; i < steps; i += 2) {
        dots_issue(L, d1, i + 1);
        __builtin_amdgcn_sched_barrier(0);
        dots_consume(L, d0, i, acc, sDots[w]);
        __builtin_amdgcn_sched_barrier(0);
        dots_issue(L, d0, i + 2);
        __builtin_amdgcn_sched_barrier(0);
        dots_consume(L, d1, i + 1, acc, sDots[w]);
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    if (lane >= 16) return;
    const int64_t t = tb + lane;
    if (t >= Tp) return;
    float dl[kMaps];
    if (t < T) {
        float d[kMaps];
#pragma unroll
        for (int m = 0; m < kMaps; ++m) d[m] = sDots[w][lane][m];
        const float4 pq = reinterpret_cast<const float4*>(Hpre)[t];
        const float4 oq = reinterpret_cast<const float4*>(Hpost)[t];
        const float hp[4] = {pq.x, pq.y, pq.z, pq.w};
        const float ho[4] = {oq.x, oq.y, oq.z, oq.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            dl[j] = d[j] * hp[j] * (1.f - hp[j]);
            dl[4 + j] = d[4 + j] * ho[j] * (1.f - ho[j]);
        }
        float H[16];
        const float4* hr = reinterpret_cast<const float4*>(Hres + 16 * t);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 v = hr[q];
            H[4 * q] = v.x;
            H[4 * q + 1] = v.y;
            H[4 * q + 2] = v.z;
            H[4 * q + 3] = v.w;
        }
        project_bwd(H, d + 8, dl + 8);
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < kMaps; ++m) s = __builtin_fmaf(dl[m], logits[kMaps * t + m], s);
        svec[t] = s / (float)(32 * C8);
        float4* go = reinterpret_cast<float4*>(glogits + kMaps * t);
#pragma unroll
        for (int q = 0; q < kMaps / 4; ++q) go[q] = make_float4(dl[4 * q], dl[4 * q + 1], dl[4 * q + 2], dl[4 * q + 3]);
        const float inv = 1.f / rms[t];
#pragma unroll
        for (int m = 0; m < kMaps; ++m) dl[m] *= inv;
    } else {
#pragma unroll
        for (int m = 0; m < kMaps; ++m) dl[m] = 0.f;
    }
#pragma unroll
    for (int m = 0; m < kMaps; ++m) {
        const __bf16 h = (__bf16)dl[m];
        dlT_hi[m * Tp + t] = h;
        dlT_lo[m * Tp + t] = (__bf16)(dl[m] - (float)h);
    }
}

// ---------------------------------------------------------------------------
// Wt = W transposed to [4C][24] bf16 (48 bytes per k), so that an MFMA
// fragment of 8 maps at one k is a single 16-byte load in the dx pass.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void layer_wt_kernel(const uint16_t* __restrict__ W,
                                                          uint4* __restrict__ Wt, int64_t D)
{
    const int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (k >= D) return;
    uint32_t v[kMaps / 2];
#pragma unroll
    for (int q = 0; q < kMaps / 2; ++q)
        v[q] = (uint32_t)W[(2 * q) * D + k] | ((uint32_t)W[(2 * q + 1) * D + k] << 16);
#pragma unroll
    for (int q = 0; q < 3; ++q) Wt[3 * k + q] = make_uint4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
}

// ---------------------------------------------------------------------------
// dx: workgroup = 16 tokens x all columns, in chunks of 128 columns of every
// stream (512 flattened k).  Per chunk:
//  1. wave w forms dxn = dl W for stream w on MFMA, transposed so that the
//     tokens are the N dimension:
//       dxn^T (16 k x 16 tokens) = Wt (16 k x 32 maps) * dl^T (32 maps x 16 tokens)
//     A is a 16-byte load of Wt (lanes of maps 24..31 supply zeros), B is dl
//     split into bf16 hi + lo and fixed for the workgroup.  A lane's D holds
//     4 consecutive k of one token and goes to LDS as one 16-byte write.
//  2. element-wise pass: wave w takes tokens 4w..4w+3 with lane = (token,
//     8 columns); it also writes grad_f = sum_i H_post[i] grad_x_out_i from
//     the same grad_x_out loads.  Each global access covers 4 rows x 256
//     contiguous bytes
//     (row-contiguous access runs much closer to the HBM peak than many short
//     row segments per instruction, which is what the MFMA layout would give).
// Software pipeline: the vector-memory counter retires in order, so waiting
// for any load also waits for every older load and store.  All loads of
// chunk i+1 (Wt fragments and stream rows) are therefore issued before chunk
// i is consumed, into the other of two register sets, and the LDS buffer is
// double-buffered so that one barrier per chunk suffices.
// ---------------------------------------------------------------------------
constexpr int kDxTok = 16;                    // tokens per workgroup (MFMA N)
constexpr int kDxChunk = 128;                 // columns per stream per chunk
constexpr int kDxTiles = kDxChunk / 16;       // k-tiles per wave per chunk
constexpr int kDxPitch = 4 * kDxChunk + 4;    // floats per LDS row (bank spread)

struct DxLoads {
    uint4 a[kDxTiles];  // Wt fragments of this wave's k-tiles
    uint4 g[4], x[4], u;  // grad_x_out, x, grad_u of the lane's token and columns
};

struct DxLane {
    const uint4* x;
    const uint4* gxo;
    const uint4* gu;
    const uint4* Wt;
    uint4* gx;
    uint4* gf;
    int64_t C, C8;
    int64_t tr;      // token row of the element-wise lane (clamped into range)
    bool tok;        // that token exists
    int w, row, kq, cl;
    float H[16], hp[4], ho[4], inv, sr;
    bf16x8 bhi, blo;
};

MHC_DEV void dx_issue(const DxLane& L, DxLoads& d, int64_t c0)
{
    // Wt rows past C (a ragged last chunk) are clamped; their products land
    // in LDS columns that the element-wise pass never reads.  Lanes kq = 3
    // (maps 24..31, which do not exist) load the piece of maps 0..7.
    const int kqc = L.kq < 3 ? L.kq : 0;
#pragma unroll
    for (int s = 0; s < kDxTiles; ++s) {
        int64_t c = c0 + 16 * s + L.row;
        c = c < L.C ? c : L.C - 1;
        d.a[s] = L.Wt[3 * (L.w * L.C + c) + kqc];
    }
    const bool col = c0 + 8 * L.cl < L.C;
    const int64_t c8 = col ? c0 / 8 + L.cl : L.C8 - 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        d.g[i] = L.gxo[(L.tr * 4 + i) * L.C8 + c8];
        d.x[i] = L.x[(L.tr * 4 + i) * L.C8 + c8];
    }
    d.u = L.gu[L.tr * L.C8 + c8];
}

MHC_DEV void dx_consume(const DxLane& L, const DxLoads& d, float (*sD)[kDxPitch], int64_t c0)
{
#pragma unroll
    for (int s = 0; s < kDxTiles; ++s) {
        // lanes kq = 3 hold a finite piece of another map range: their B
        // (maps 24..31) is zero, so they add nothing
        const bf16x8 a = as_bf16x8(d.a[s]);
        floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, L.bhi, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, L.blo, acc, 0, 0, 0);
        *reinterpret_cast<floatx4*>(&sD[L.row][L.w * kDxChunk + 16 * s + 4 * L.kq]) = acc;
    }
    mhc_lds_barrier();
    const bool col = c0 + 8 * L.cl < L.C;
    if (!(L.tok && col)) return;
    const int tl = 4 * L.w + (L.kq);  // element-wise token of this lane (lane >> 4)
    const int64_t c8 = c0 / 8 + L.cl;
    float gs[4][8], uu[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) unpack8(d.g[i], gs[i]);
    unpack8(d.u, uu);
    {
        float g8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float sm = L.ho[0] * gs[0][e];
            sm = __builtin_fmaf(L.ho[1], gs[1][e], sm);
            sm = __builtin_fmaf(L.ho[2], gs[2][e], sm);
            g8[e] = __builtin_fmaf(L.ho[3], gs[3][e], sm);
        }
        mhc_store_stream(&L.gf[L.tr * L.C8 + c8], pack8(g8));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float xs[8], dn[8], o8[8];
        unpack8(d.x[j], xs);
        const floatx4 d0 = *reinterpret_cast<const floatx4*>(&sD[tl][j * kDxChunk + 8 * L.cl]);
        const floatx4 d1 = *reinterpret_cast<const floatx4*>(&sD[tl][j * kDxChunk + 8 * L.cl + 4]);
        dn[0] = d0[0]; dn[1] = d0[1]; dn[2] = d0[2]; dn[3] = d0[3];
        dn[4] = d1[0]; dn[5] = d1[1]; dn[6] = d1[2]; dn[7] = d1[3];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float sm = L.H[j] * gs[0][e];
            sm = __builtin_fmaf(L.H[4 + j], gs[1][e], sm);
            sm = __builtin_fmaf(L.H[8 + j], gs[2][e], sm);
            sm = __builtin_fmaf(L.H[12 + j], gs[3][e], sm);
            sm = __builtin_fmaf(L.hp[j], uu[e], sm);
            o8[e] = __builtin_fmaf(__builtin_fmaf(-xs[e], L.sr, dn[e]), L.inv, sm);
        }
        mhc_store_stream(&L.gx[(L.tr * 4 + j) * L.C8 + c8], pack8(o8));
    }
}

__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void layer_dx_kernel(
    const uint4* __restrict__ x, const uint4* __restrict__ gxo, const uint4* __restrict__ gu,
    const uint4* __restrict__ Wt, const float* __restrict__ Hpre, const float* __restrict__ Hpost,
    const float* __restrict__ Hres, const float* __restrict__ rms, const float* __restrict__ glogits,
    const float* __restrict__ svec, uint4* __restrict__ gx, uint4* __restrict__ gf, int64_t T,
    int64_t C)
{
    __shared__ __attribute__((aligned(16))) float sD[2][kDxTok][kDxPitch];
    DxLane L;
    const int lane = threadIdx.x & 63;
    L.x = x; L.gxo = gxo; L.gu = gu; L.Wt = Wt; L.gx = gx; L.gf = gf;
    L.C = C; L.C8 = C / 8;
    L.w = threadIdx.x >> 6;
    L.row = lane & 15;
    L.kq = lane >> 4;
    L.cl = lane & 15;
    const int64_t t0 = (int64_t)blockIdx.x * kDxTok;
    // B operand: dl[token t0 + row][maps 8 kq ..+7], split hi / lo
    {
        float b8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) b8[e] = 0.f;
        if (t0 + L.row < T && L.kq < 3) {
            const float4* src = reinterpret_cast<const float4*>(glogits + kMaps * (t0 + L.row) + 8 * L.kq);
            const float4 v0 = src[0], v1 = src[1];
            b8[0] = v0.x; b8[1] = v0.y; b8[2] = v0.z; b8[3] = v0.w;
            b8[4] = v1.x; b8[5] = v1.y; b8[6] = v1.z; b8[7] = v1.w;
        }
        split8(b8, L.bhi, L.blo);
    }
    // element-wise token of this lane: 4w + (lane >> 4)
    {
        const int64_t t = t0 + 4 * L.w + L.kq;
        L.tok = t < T;
        L.tr = L.tok ? t : T - 1;
        const float4* hr = reinterpret_cast<const float4*>(Hres + 16 * L.tr);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float4 v = hr[k];
            L.H[4 * k] = v.x;
            L.H[4 * k + 1] = v.y;
            L.H[4 * k + 2] = v.z;
            L.H[4 * k + 3] = v.w;
        }
        const float4 pq = reinterpret_cast<const float4*>(Hpre)[L.tr];
        L.hp[0] = pq.x; L.hp[1] = pq.y; L.hp[2] = pq.z; L.hp[3] = pq.w;
        const float4 oq = reinterpret_cast<const float4*>(Hpost)[L.tr];
        L.ho[0] = oq.x; L.ho[1] = oq.y; L.ho[2] = oq.z; L.ho[3] = oq.w;
        L.inv = 1.f / rms[L.tr];
        L.sr = svec[L.tr] * L.inv;
    }
    // Branch-free pipeline (a conditional issue would make the compiler's
    // wait at the join drain every load): the chunk count is padded to even,
    // chunks past C load clamped addresses and do no element-wise work.
    const int64_t n = (C + kDxChunk - 1) / kDxChunk;
    DxLoads d0, d1;
    // (the scheduling barriers keep the compiler from starting a chunk's
    // consumption, and with it the waits, before the next chunk is issued)
    dx_issue(L, d0, 0);
    for (int64_t ci = 0; ci < n; ci += 2) {
        dx_issue(L, d1, (ci + 1) * kDxChunk);
        __builtin_amdgcn_sched_barrier(0);
        dx_consume(L, d0, sD[0], ci * kDxChunk);
        __builtin_amdgcn_sched_barrier(0);
        dx_issue(L, d0, (ci + 2) * kDxChunk);
        __builtin_amdgcn_sched_barrier(0);
        dx_consume(L, d1, sD[1], (ci + 1) * kDxChunk);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// ---------------------------------------------------------------------------
// dw: workgroup = 128 flattened k x one token group; wave w takes every 4th
// 32-token chunk of the group.  Per chunk the x tile is staged in the wave's
// own LDS region ([token][k], loaded as 4 rows x 256 bytes per instruction)
// and read back transposed for the MFMA B operand:
//   dW^T tile (32 maps x 16 k) += dlT (32 maps x 32 tokens) * x (32 tokens x 16 k)
// The chunk's dlT fragments (A, from L2) and x rows are issued together, one
// chunk ahead, into the other of two register sets (the vector-memory
// counter retires in order, so A loads issued after a prefetch would make
// the MFMA wait for the prefetch).  The four waves' partials are summed in
// LDS and one partial per token group is written; layer_dw_reduce adds the
// groups in a fixed order.
// ---------------------------------------------------------------------------
constexpr int kDwK = 128;                   // flattened k per workgroup
constexpr int kDwNt = kDwK / 16;            // 16-column MFMA tiles
constexpr int kXPitch = kDwK + 8;           // bf16 per LDS row
constexpr int kDwPieces = 32 * kDwK / 8 / 64;  // 16-byte x pieces per lane per chunk

struct DwLoads {
    uint4 ahi[2], alo[2];  // dlT fragments: maps 16 mt + row, tokens 8 kq ..+7
    uint4 xr[kDwPieces];   // x: piece q -> token 4q + lane/16, 16 bytes at lane%16
};

MHC_DEV void dw_issue(DwLoads& d, const uint16_t* __restrict__ x, const __bf16* __restrict__ dlT_hi,
                      const __bf16* __restrict__ dlT_lo, int64_t tc, int64_t T, int64_t Tp,
                      int64_t D, int64_t k0, int lane)
{
    const int row = lane & 15, kq = lane >> 4;
    // chunks past the group read a clamped chunk; their A is zeroed on use
    const int64_t ta = tc + 32 < Tp ? tc : Tp - 32;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const int m = 16 * mt + row < kMaps ? 16 * mt + row : kMaps - 1;
        d.ahi[mt] = *reinterpret_cast<const uint4*>(dlT_hi + m * Tp + ta + 8 * kq);
        d.alo[mt] = *reinterpret_cast<const uint4*>(dlT_lo + m * Tp + ta + 8 * kq);
    }
#pragma unroll
    for (int q = 0; q < kDwPieces; ++q) {
        int64_t t = tc + 4 * q + (lane >> 4);
        t = t < T ? t : T - 1;
        d.xr[q] = *reinterpret_cast<const uint4*>(x + t * D + k0 + 8 * (lane & 15));
    }
}

MHC_DEV void dw_consume(const DwLoads& d, uint16_t (*sX)[kXPitch], floatx4 (&acc)[2][kDwNt],
                        bool live, int lane)
{
    const int row = lane & 15, kq = lane >> 4;
    mhc_wave_lds_fence();  // the previous chunk's reads of the region come first
#pragma unroll
    for (int q = 0; q < kDwPieces; ++q)
        *reinterpret_cast<uint4*>(&sX[4 * q + (lane >> 4)][8 * (lane & 15)]) = d.xr[q];
    // the region is this wave's own and LDS is in order within a wave; the
    // fence keeps the compiler from reusing earlier reads of it
    mhc_wave_lds_fence();
    if (!live) return;
    bf16x8 ahi[2], alo[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        // A rows 24..31 repeat map 23 (clamped load); they only feed D rows
        // 24..31, which are never stored
        ahi[mt] = as_bf16x8(d.ahi[mt]);
        alo[mt] = as_bf16x8(d.alo[mt]);
    }
#pragma unroll
    for (int nt = 0; nt < kDwNt; ++nt) {
        bf16x8 b;
#pragma unroll
        for (int e = 0; e < 8; ++e) b[e] = __builtin_bit_cast(__bf16, sX[8 * kq + e][16 * nt + row]);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[mt], b, acc[mt][nt], 0, 0, 0);
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[mt], b, acc[mt][nt], 0, 0, 0);
        }
    }
}

__global__ __launch_bounds__(kBlock) void layer_dw_kernel(
    const uint16_t* __restrict__ x, const __bf16* __restrict__ dlT_hi,
    const __bf16* __restrict__ dlT_lo, float* __restrict__ partial, int64_t T, int64_t Tp,
    int64_t C, int64_t group_tokens)
{
    __shared__ __attribute__((aligned(16))) uint16_t sX[4][32][kXPitch];
    __shared__ float sR[32][kDwK + 1];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int row = lane & 15, kq = lane >> 4;
    const int64_t D = 4 * C;
    const int64_t k0 = (int64_t)blockIdx.x * kDwK;
    const int64_t g = blockIdx.y;
    const int64_t tg0 = g * group_tokens;
    int64_t tg1 = tg0 + group_tokens;
    if (tg1 > Tp) tg1 = Tp;
    floatx4 acc[2][kDwNt];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < kDwNt; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    // wave w: chunks tg0 + 32 (w + 4 i); the pair loop is branch-free (a chunk
    // past the group loads clamped addresses and is not accumulated), so the
    // compiler's waits stay one chunk behind the issue
    DwLoads d0, d1;
    const int64_t first = tg0 + 32 * w;
    dw_issue(d0, x, dlT_hi, dlT_lo, first, T, Tp, D, k0, lane);
    for (int64_t tc = first; tc < tg1; tc += 256) {
        dw_issue(d1, x, dlT_hi, dlT_lo, tc + 128, T, Tp, D, k0, lane);
        __builtin_amdgcn_sched_barrier(0);
        dw_consume(d0, sX[w], acc, true, lane);
        __builtin_amdgcn_sched_barrier(0);
        dw_issue(d0, x, dlT_hi, dlT_lo, tc + 256, T, Tp, D, k0, lane);
        __builtin_amdgcn_sched_barrier(0);
        dw_consume(d1, sX[w], acc, tc + 128 < tg1, lane);
        __builtin_amdgcn_sched_barrier(0);
    }
    // sum the four waves' partials: wave 0 writes, the others add in turn
    for (int ww = 0; ww < 4; ++ww) {
        if (w == ww) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < kDwNt; ++nt)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        float& dst = sR[16 * mt + 4 * kq + v][16 * nt + row];
                        dst = (ww == 0 ? 0.f : dst) + acc[mt][nt][v];
                    }
        }
        __syncthreads();
    }
    float* out = partial + g * (int64_t)kMaps * D;
    for (int p = threadIdx.x; p < kMaps * kDwK; p += kBlock) {
        const int m = p / kDwK, kk = p % kDwK;
        out[m * D + k0 + kk] = sR[m][kk];
    }
}

__global__ __launch_bounds__(kBlock) void layer_dw_reduce_kernel(const float4* __restrict__ partial,
                                                                 float4* __restrict__ gW,
                                                                 int64_t n4, int64_t groups)
{
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n4; i += (int64_t)gridDim.x * kBlock) {
        float4 s = partial[i];
        for (int64_t g = 1; g < groups; ++g) {
            const float4 v = partial[g * n4 + i];
            s.x += v.x;
            s.y += v.y;
            s.z += v.z;
            s.w += v.w;
        }
        gW[i] = s;
    }
}

}  // namespace

LayerPlan layer_plan(int64_t T, int64_t C)
{
    LayerPlan p;
    p.Tp = (T + 63) / 64 * 64;
    const int64_t want_groups = 16;
    int64_t gt = (p.Tp + want_groups - 1) / want_groups;
    gt = (gt + 127) / 128 * 128;  // whole 4-wave x 32-token rounds
    if (gt < 128) gt = 128;
    p.group_tokens = gt;
    p.groups = (p.Tp + gt - 1) / gt;
    const int64_t D = 4 * C;
    p.off_s = 0;
    p.off_hi = (p.Tp * 4 + 255) / 256 * 256;
    p.off_lo = p.off_hi + (p.Tp * kMaps * 2 + 255) / 256 * 256;
    p.off_wt = p.off_lo + (p.Tp * kMaps * 2 + 255) / 256 * 256;
    p.off_partial = p.off_wt + (D * kMaps * 2 + 255) / 256 * 256;
    p.bytes = p.off_partial + p.groups * kMaps * D * 4;
    return p;
}

hipError_t launch_layer_fwd(const LayerPtrs& a, int64_t T, int64_t C, float eps,
                            const SolverOpts& o, hipStream_t stream)
{
    const dim3 g1((unsigned)((T + kMapTok - 1) / kMapTok));
    if (o.solver == 0)
        hipLaunchKernelGGL(layer_maps_kernel<0>, g1, dim3(kBlock), 0, stream,
                           (const uint16_t*)a.x, (const uint16_t*)a.W, a.logits, a.rms, a.H_pre,
                           a.H_post, a.H_res, T, C, eps, o);
    else
        hipLaunchKernelGGL(layer_maps_kernel<1>, g1, dim3(kBlock), 0, stream,
                           (const uint16_t*)a.x, (const uint16_t*)a.W, a.logits, a.rms, a.H_pre,
                           a.H_post, a.H_res, T, C, eps, o);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 g2((unsigned)((T + kMixTokens - 1) / kMixTokens));
    hipLaunchKernelGGL(layer_mix_kernel, g2, dim3(kBlock), 0, stream, (const uint4*)a.x,
                       (const uint4*)a.f, a.H_pre, a.H_post, a.H_res, (uint4*)a.u,
                       (uint4*)a.x_out, T, C / 8);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free backward (mhc_layer_bwd_noalloc): the same
// workspace layout as layer_plan's, held in this file-scope device array
// instead of caller memory.  Every GPU the library runs on holds its own copy
// (kLayerNoAllocScratchBytes, allocated when the code object is loaded and
// kept until the process ends).  In host code `scratch` names a host-side
// stand-in, not device memory, so its device address is looked up once per
// device with hipGetSymbolAddress and only that address is ever passed on.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kLayerNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;
}  // namespace

hipError_t layer_noalloc_scratch(int device, void** ptr)
{
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_ptr[device].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_ptr[device].load(std::memory_order_relaxed);
        if (p == nullptr) {
            // the caller has made `device` current
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (p == nullptr) return hipErrorInvalidSymbol;
            g_scratch_ptr[device].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_layer_bwd(const LayerPtrs& a, int64_t T, int64_t C, hipStream_t stream)
{
    const LayerPlan p = layer_plan(T, C);
    char* ws = static_cast<char*>(a.workspace);
    float* svec = reinterpret_cast<float*>(ws + p.off_s);
    __bf16* dhi = reinterpret_cast<__bf16*>(ws + p.off_hi);
    __bf16* dlo = reinterpret_cast<__bf16*>(ws + p.off_lo);
    float* partial = reinterpret_cast<float*>(ws + p.off_partial);
    const int64_t C8 = C / 8;
    hipLaunchKernelGGL(layer_dots_kernel, dim3((unsigned)(p.Tp / 64)), dim3(kBlock), 0, stream,
                       (const uint4*)a.x, (const uint4*)a.f, (const uint4*)a.grad_x_out,
                       (const uint4*)a.grad_u, a.H_pre, a.H_post, a.H_res, a.logits, a.rms,
                       a.grad_logits, svec, dhi, dlo, T, p.Tp, C8);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    uint4* wt = reinterpret_cast<uint4*>(ws + p.off_wt);
    hipLaunchKernelGGL(layer_wt_kernel, dim3((unsigned)((4 * C + kBlock - 1) / kBlock)), dim3(kBlock),
                       0, stream, (const uint16_t*)a.W, wt, 4 * C);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(layer_dx_kernel, dim3((unsigned)((T + kDxTok - 1) / kDxTok)), dim3(kBlock), 0,
                       stream, (const uint4*)a.x, (const uint4*)a.grad_x_out, (const uint4*)a.grad_u,
                       (const uint4*)wt, a.H_pre, a.H_post, a.H_res, a.rms, a.grad_logits, svec,
                       (uint4*)a.grad_x, (uint4*)a.grad_f, T, C);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 gdw((unsigned)(4 * C / kDwK), (unsigned)p.groups);
    hipLaunchKernelGGL(layer_dw_kernel, gdw, dim3(kBlock), 0, stream, (const uint16_t*)a.x, dhi,
                       dlo, partial, T, p.Tp, C, p.group_tokens);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n4 = (int64_t)kMaps * 4 * C / 4;
    hipLaunchKernelGGL(layer_dw_reduce_kernel, dim3((unsigned)((n4 + kBlock - 1) / kBlock)),
                       dim3(kBlock), 0, stream, (const float4*)partial, (float4*)a.grad_W, n4,
                       p.groups);
    return hipGetLastError();
}

}  // namespace mhc
