// C ABI entry points: argument checks on the host, then one kernel launch on
// the caller's stream.  Nothing is allocated and no state is kept between
// calls except the calling thread's last error message.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/mhc.h"
#include "kernels.h"

namespace {

thread_local char g_last_error[256] = "";

mhc_status fail(mhc_status s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

mhc_status ok()
{
    g_last_error[0] = '\0';
    return MHC_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// [a, a+na) and [b, b+nb) share at least one byte
bool overlap(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// Largest batch / token count one call accepts.  A launch's grid may hold
// fewer than 2^32 work-items in total, and the widest launches use 4 lanes per
// matrix (the 4x4 backward) and 16 per token (the stream-mix forward and the
// layer's mix and dx passes), so these keep every grid below that.
constexpr int64_t kMaxBatch = MHC_MAX_BATCH;
constexpr int64_t kMaxTokens = MHC_MAX_TOKENS;
static_assert(4 * kMaxBatch <= ((int64_t)1 << 32) - 256, "4x4 backward grid");
static_assert(16 * kMaxTokens <= ((int64_t)1 << 32) - 256, "token grids");

// Solver limits when mhc_proj_opts.max_iters is -1.
constexpr int kDefaultNewtonIters = 30;
constexpr int kDefaultSinkhornSweeps = 1000;

mhc_status check_opts(const mhc_proj_opts* in, mhc::SolverOpts* out)
{
    mhc_proj_opts o;
    mhc_proj_opts_default(&o);
    if (in != nullptr) o = *in;
    if (o.solver != MHC_SOLVER_NEWTON && o.solver != MHC_SOLVER_SINKHORN)
        return fail(MHC_ERR_INVALID_ARGUMENT, "opts.solver must be 0 (Newton) or 1 (Sinkhorn)");
    if (o.max_iters == -1)
        o.max_iters = o.solver == MHC_SOLVER_NEWTON ? kDefaultNewtonIters : kDefaultSinkhornSweeps;
    if (o.max_iters < 1 || o.max_iters > 10000)
        return fail(MHC_ERR_INVALID_ARGUMENT,
                    "opts.max_iters must be -1 (the solver's default) or in 1..10000");
    if (!(o.tol >= 0.f) || o.tol > 1.f)
        return fail(MHC_ERR_INVALID_ARGUMENT, "opts.tol must be in [0, 1]");
    if (o.warm_sweeps < -1 || o.warm_sweeps > 64)
        return fail(MHC_ERR_INVALID_ARGUMENT, "opts.warm_sweeps must be -1 (default) or in 0..64");
    *out = mhc::SolverOpts{o.solver, o.max_iters, o.tol, o.warm_sweeps};
    return MHC_OK;
}

mhc_status launched(hipError_t e, const char* what)
{
    if (e != hipSuccess) return fail(MHC_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// The buffers of a 4x4 forward (B > 0).
mhc_status check_fwd_buffers(const float* logits, const float* P, const uint8_t* iters, int64_t B)
{
    if (logits == nullptr || P == nullptr) return fail(MHC_ERR_INVALID_ARGUMENT, "logits and P must not be NULL");
    if (!aligned16(logits) || !aligned16(P)) return fail(MHC_ERR_INVALID_ARGUMENT, "logits and P must be 16-byte aligned");
    const size_t bytes = (size_t)B * 64;
    if (logits != P && overlap(logits, bytes, P, bytes))
        return fail(MHC_ERR_INVALID_ARGUMENT, "P partially overlaps logits");
    if (iters != nullptr && (overlap(iters, (size_t)B, logits, bytes) || overlap(iters, (size_t)B, P, bytes)))
        return fail(MHC_ERR_INVALID_ARGUMENT, "iters overlaps logits or P");
    return MHC_OK;
}

// The buffers of a 4x4 backward from P (B > 0).
mhc_status check_bwd_buffers(const float* P, const float* grad_P, const float* grad_logits,
                             int64_t B)
{
    if (P == nullptr || grad_P == nullptr || grad_logits == nullptr)
        return fail(MHC_ERR_INVALID_ARGUMENT, "P, grad_P and grad_logits must not be NULL");
    if (!aligned16(P) || !aligned16(grad_P) || !aligned16(grad_logits))
        return fail(MHC_ERR_INVALID_ARGUMENT, "P, grad_P and grad_logits must be 16-byte aligned");
    const size_t bytes = (size_t)B * 64;
    if (overlap(P, bytes, grad_logits, bytes))
        return fail(MHC_ERR_INVALID_ARGUMENT, "grad_logits overlaps P");
    if (grad_P != grad_logits && overlap(grad_P, bytes, grad_logits, bytes))
        return fail(MHC_ERR_INVALID_ARGUMENT, "grad_logits partially overlaps grad_P");
    return MHC_OK;
}

}  // namespace

extern "C" {

mhc_status mhc_proj_opts_default(mhc_proj_opts* opts)
{
    if (opts == nullptr) return fail(MHC_ERR_INVALID_ARGUMENT, "opts is NULL");
    opts->solver = MHC_SOLVER_NEWTON;
    opts->max_iters = -1;
    opts->tol = 1e-6f;
    opts->warm_sweeps = -1;
    return MHC_OK;
}

mhc_status mhc_birkhoff_fwd(const float* logits, float* P, int64_t B, const mhc_proj_opts* opts,
                            uint8_t* iters, void* stream)
{
    if (B < 0 || B > kMaxBatch) return fail(MHC_ERR_INVALID_ARGUMENT, "B=%lld out of range", (long long)B);
    mhc::SolverOpts o;
    mhc_status s = check_opts(opts, &o);
    if (s != MHC_OK) return s;
    if (B == 0) return ok();
    if ((s = check_fwd_buffers(logits, P, iters, B)) != MHC_OK) return s;
    return launched(mhc::launch_birkhoff_fwd(logits, P, iters, B, o, (hipStream_t)stream),
                    "birkhoff_fwd launch");
}

mhc_status mhc_birkhoff_bwd(const float* P, const float* grad_P, float* grad_logits, int64_t B,
                            void* stream)
{
    if (B < 0 || B > kMaxBatch) return fail(MHC_ERR_INVALID_ARGUMENT, "B=%lld out of range", (long long)B);
    if (B == 0) return ok();
    const mhc_status s = check_bwd_buffers(P, grad_P, grad_logits, B);
    if (s != MHC_OK) return s;
    return launched(mhc::launch_birkhoff_bwd(P, grad_P, grad_logits, B, (hipStream_t)stream),
                    "birkhoff_bwd launch");
}

mhc_status mhc_birkhoff_pipeline_step(const float* logits, float* P, int64_t B,
                                      const mhc_proj_opts* opts, uint8_t* iters,
                                      const float* P_bwd, const float* grad_P,
                                      float* grad_logits, int64_t B_bwd, void* stream)
{
    if (B < 0 || B > kMaxBatch) return fail(MHC_ERR_INVALID_ARGUMENT, "B=%lld out of range", (long long)B);
    if (B_bwd < 0 || B_bwd > kMaxBatch)
        return fail(MHC_ERR_INVALID_ARGUMENT, "B_bwd=%lld out of range", (long long)B_bwd);
    mhc::SolverOpts o;
    mhc_status s = check_opts(opts, &o);
    if (s != MHC_OK) return s;
    if (B == 0 && B_bwd == 0) return ok();
    if (B > 0 && (s = check_fwd_buffers(logits, P, iters, B)) != MHC_OK) return s;
    if (B_bwd > 0 && (s = check_bwd_buffers(P_bwd, grad_P, grad_logits, B_bwd)) != MHC_OK) return s;
    if (B > 0 && B_bwd > 0) {
        // the forward's outputs against every backward array, and the
        // backward's output against every forward array; the inputs of the
        // two halves may share memory (both only read it)
        const size_t fb = (size_t)B * 64, bb = (size_t)B_bwd * 64;
        if (overlap(P, fb, P_bwd, bb) || overlap(P, fb, grad_P, bb) || overlap(P, fb, grad_logits, bb))
            return fail(MHC_ERR_INVALID_ARGUMENT, "P overlaps P_bwd, grad_P or grad_logits");
        if (overlap(grad_logits, bb, logits, fb))
            return fail(MHC_ERR_INVALID_ARGUMENT, "grad_logits overlaps logits");
        if (iters != nullptr && (overlap(iters, (size_t)B, P_bwd, bb) ||
                                 overlap(iters, (size_t)B, grad_P, bb) ||
                                 overlap(iters, (size_t)B, grad_logits, bb)))
            return fail(MHC_ERR_INVALID_ARGUMENT, "iters overlaps P_bwd, grad_P or grad_logits");
    }
    return launched(mhc::launch_birkhoff_pipeline(logits, P, iters, B, o, P_bwd, grad_P,
                                                  grad_logits, B_bwd, (hipStream_t)stream),
                    "birkhoff_pipeline_step launch");
}

mhc_status mhc_birkhoff_bwd_recompute(const float* logits, const float* grad_P,
                                      float* grad_logits, int64_t B,
                                      const mhc_proj_opts* opts, void* stream)
{
    if (B < 0 || B > kMaxBatch) return fail(MHC_ERR_INVALID_ARGUMENT, "B=%lld out of range", (long long)B);
    mhc::SolverOpts o;
    const mhc_status s = check_opts(opts, &o);
    if (s != MHC_OK) return s;
    if (B == 0) return ok();
    if (logits == nullptr || grad_P == nullptr || grad_logits == nullptr)
        return fail(MHC_ERR_INVALID_ARGUMENT, "logits, grad_P and grad_logits must not be NULL");
    if (!aligned16(logits) || !aligned16(grad_P) || !aligned16(grad_logits))
        return fail(MHC_ERR_INVALID_ARGUMENT, "logits, grad_P and grad_logits must be 16-byte aligned");
    const size_t bytes = (size_t)B * 64;
    if (grad_logits != logits && overlap(logits, bytes, grad_logits, bytes))
        return fail(MHC_ERR_INVALID_ARGUMENT, "grad_logits partially overlaps logits");
    if (grad_logits != grad_P && overlap(grad_P, bytes, grad_logits, bytes))
        return fail(MHC_ERR_INVALID_ARGUMENT, "grad_logits partially overlaps grad_P");
    return launched(mhc::launch_birkhoff_bwd_recompute(logits, grad_P, grad_logits, B, o,
                                                      (hipStream_t)stream),
                    "birkhoff_bwd_recompute launch");
}

mhc_status mhc_birkhoff_fwd_bwd(const float* logits, const float* grad_P, float* P,
                                float* grad_logits, int64_t B, const mhc_proj_opts* opts,
                                uint8_t* iters, void* stream)
{
    if (B < 0 || B > kMaxBatch) return fail(MHC_ERR_INVALID_ARGUMENT, "B=%lld out of range", (long long)B);
    mhc::SolverOpts o;
    const mhc_status s = check_opts(opts, &o);
    if (s != MHC_OK) return s;
    if (B == 0) return ok();
    if (logits == nullptr || grad_P == nullptr || P == nullptr || grad_logits == nullptr)
        return fail(MHC_ERR_INVALID_ARGUMENT, "logits, grad_P, P and grad_logits must not be NULL");
    if (!aligned16(logits) || !aligned16(grad_P) || !aligned16(P) || !aligned16(grad_logits))
        return fail(MHC_ERR_INVALID_ARGUMENT,
                    "logits, grad_P, P and grad_logits must be 16-byte aligned");
    const size_t bytes = (size_t)B * 64;
    if (P != logits && overlap(logits, bytes, P, bytes))
        return fail(MHC_ERR_INVALID_ARGUMENT, "P partially overlaps logits");
    if (grad_logits != grad_P && overlap(grad_P, bytes, grad_logits, bytes))
        return fail(MHC_ERR_INVALID_ARGUMENT, "grad_logits partially overlaps grad_P");
    if (overlap(P, bytes, grad_P, bytes) || overlap(P, bytes, grad_logits, bytes))
        return fail(MHC_ERR_INVALID_ARGUMENT, "P overlaps grad_P or grad_logits");
    if (overlap(grad_logits, bytes, logits, bytes))
        return fail(MHC_ERR_INVALID_ARGUMENT, "grad_logits overlaps logits");
    if (iters != nullptr &&
        (overlap(iters, (size_t)B, logits, bytes) || overlap(iters, (size_t)B, grad_P, bytes) ||
         overlap(iters, (size_t)B, P, bytes) || overlap(iters, (size_t)B, grad_logits, bytes)))
        return fail(MHC_ERR_INVALID_ARGUMENT, "iters overlaps logits, grad_P, P or grad_logits");
    return launched(mhc::launch_birkhoff_fwd_bwd(logits, grad_P, P, grad_logits, iters, B, o,
                                                (hipStream_t)stream),
                    "birkhoff_fwd_bwd launch");
}

static bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

mhc_status mhc_birkhoff_fwd_n(const float* logits, float* P, int64_t B, int32_t n,
                              const mhc_proj_opts* opts, uint8_t* iters, void* stream)
{
    if (n < 1 || n > 8)
        return fail(MHC_ERR_UNSUPPORTED, "n must be in 1..8 (got %d)", n);
    if (n == 4) return mhc_birkhoff_fwd(logits, P, B, opts, iters, stream);
    if (B < 0 || B > kMaxBatch) return fail(MHC_ERR_INVALID_ARGUMENT, "B=%lld out of range", (long long)B);
    mhc::SolverOpts o;
    const mhc_status s = check_opts(opts, &o);
    if (s != MHC_OK) return s;
    if (B == 0) return ok();
    if (logits == nullptr || P == nullptr)
        return fail(MHC_ERR_INVALID_ARGUMENT, "logits and P must not be NULL");
    if (!aligned4(logits) || !aligned4(P))
        return fail(MHC_ERR_INVALID_ARGUMENT, "logits and P must be 4-byte aligned");
    const size_t bytes = (size_t)B * n * n * 4;
    if (logits != P && overlap(logits, bytes, P, bytes))
        return fail(MHC_ERR_INVALID_ARGUMENT, "P partially overlaps logits");
    if (iters != nullptr && (overlap(iters, (size_t)B, logits, bytes) || overlap(iters, (size_t)B, P, bytes)))
        return fail(MHC_ERR_INVALID_ARGUMENT, "iters overlaps logits or P");
    return launched(mhc::launch_birkhoff_fwd_n(logits, P, iters, B, n, o, (hipStream_t)stream),
                    "birkhoff_fwd_n launch");
}

mhc_status mhc_birkhoff_bwd_n(const float* P, const float* grad_P, float* grad_logits, int64_t B,
                              int32_t n, void* stream)
{
    if (n < 1 || n > 8)
        return fail(MHC_ERR_UNSUPPORTED, "n must be in 1..8 (got %d)", n);
    if (n == 4) return mhc_birkhoff_bwd(P, grad_P, grad_logits, B, stream);
    if (B < 0 || B > kMaxBatch) return fail(MHC_ERR_INVALID_ARGUMENT, "B=%lld out of range", (long long)B);
    if (B == 0) return ok();
    if (P == nullptr || grad_P == nullptr || grad_logits == nullptr)
        return fail(MHC_ERR_INVALID_ARGUMENT, "P, grad_P and grad_logits must not be NULL");
    if (!aligned4(P) || !aligned4(grad_P) || !aligned4(grad_logits))
        return fail(MHC_ERR_INVALID_ARGUMENT, "P, grad_P and grad_logits must be 4-byte aligned");
    const size_t bytes = (size_t)B * n * n * 4;
    if (overlap(P, bytes, grad_logits, bytes))
        return fail(MHC_ERR_INVALID_ARGUMENT, "grad_logits overlaps P");
    if (grad_P != grad_logits && overlap(grad_P, bytes, grad_logits, bytes))
        return fail(MHC_ERR_INVALID_ARGUMENT, "grad_logits partially overlaps grad_P");
    return launched(mhc::launch_birkhoff_bwd_n(P, grad_P, grad_logits, B, n, (hipStream_t)stream),
                    "birkhoff_bwd_n launch");
}

mhc_status mhc_stream_mix(const void* x, const float* H_or_logits, float* H_out, void* out,
                          int64_t T, int32_t n, int64_t C, const mhc_proj_opts* proj,
                          void* stream)
{
    if (n != 4) return fail(MHC_ERR_UNSUPPORTED, "only n = 4 streams are supported (got %d)", n);
    if (T < 0 || T > kMaxTokens) return fail(MHC_ERR_INVALID_ARGUMENT, "T=%lld out of range", (long long)T);
    if (C < 8 || C % 8 != 0 || C > ((int64_t)1 << 30))
        return fail(MHC_ERR_INVALID_ARGUMENT, "C must be a positive multiple of 8 (got %lld)", (long long)C);
    mhc::SolverOpts o{};
    if (proj != nullptr) {
        const mhc_status s = check_opts(proj, &o);
        if (s != MHC_OK) return s;
    }
    if (T == 0) return ok();
    if (x == nullptr || H_or_logits == nullptr || out == nullptr)
        return fail(MHC_ERR_INVALID_ARGUMENT, "x, H_or_logits and out must not be NULL");
    if (!aligned16(x) || !aligned16(H_or_logits) || !aligned16(out) || (H_out && !aligned16(H_out)))
        return fail(MHC_ERR_INVALID_ARGUMENT, "tensors must be 16-byte aligned");
    const size_t xbytes = (size_t)T * 4 * (size_t)C * 2, hbytes = (size_t)T * 64;
    if (overlap(x, xbytes, out, xbytes) || overlap(H_or_logits, hbytes, out, xbytes))
        return fail(MHC_ERR_INVALID_ARGUMENT, "out overlaps an input");
    if (proj != nullptr && H_out != nullptr &&
        (overlap(H_out, hbytes, x, xbytes) || overlap(H_out, hbytes, out, xbytes) ||
         (H_out != H_or_logits && overlap(H_out, hbytes, H_or_logits, hbytes))))
        return fail(MHC_ERR_INVALID_ARGUMENT, "H_out overlaps another tensor");
    return launched(mhc::launch_stream_mix_fwd(x, H_or_logits, proj ? H_out : nullptr, out, T, C,
                                               proj ? &o : nullptr, (hipStream_t)stream),
                    "stream_mix launch");
}

mhc_status mhc_stream_mix_bwd(const void* x, const float* H, const void* grad_out, void* grad_x,
                              float* grad_H, int64_t T, int32_t n, int64_t C, void* stream)
{
    if (n != 4) return fail(MHC_ERR_UNSUPPORTED, "only n = 4 streams are supported (got %d)", n);
    if (T < 0 || T > kMaxTokens) return fail(MHC_ERR_INVALID_ARGUMENT, "T=%lld out of range", (long long)T);
    if (C < 8 || C % 8 != 0 || C > ((int64_t)1 << 30))
        return fail(MHC_ERR_INVALID_ARGUMENT, "C must be a positive multiple of 8 (got %lld)", (long long)C);
    if (T == 0) return ok();
    if (!x || !H || !grad_out || !grad_x || !grad_H)
        return fail(MHC_ERR_INVALID_ARGUMENT, "x, H, grad_out, grad_x and grad_H must not be NULL");
    if (!aligned16(x) || !aligned16(H) || !aligned16(grad_out) || !aligned16(grad_x) || !aligned16(grad_H))
        return fail(MHC_ERR_INVALID_ARGUMENT, "tensors must be 16-byte aligned");
    const size_t xbytes = (size_t)T * 4 * (size_t)C * 2, hbytes = (size_t)T * 64;
    if (overlap(grad_x, xbytes, x, xbytes) || overlap(grad_x, xbytes, grad_out, xbytes) ||
        overlap(grad_x, xbytes, H, hbytes) || overlap(grad_x, xbytes, grad_H, hbytes) ||
        overlap(grad_H, hbytes, x, xbytes) || overlap(grad_H, hbytes, grad_out, xbytes) ||
        overlap(grad_H, hbytes, H, hbytes))
        return fail(MHC_ERR_INVALID_ARGUMENT, "an output overlaps another tensor");
    return launched(mhc::launch_stream_mix_bwd(x, H, grad_out, grad_x, grad_H, T, C,
                                               (hipStream_t)stream),
                    "stream_mix_bwd launch");
}

static mhc_status check_layer_shape(int64_t T, int32_t n, int64_t C)
{
    if (n != 4) return fail(MHC_ERR_UNSUPPORTED, "only n = 4 streams are supported (got %d)", n);
    if (T < 0 || T > kMaxTokens) return fail(MHC_ERR_INVALID_ARGUMENT, "T=%lld out of range", (long long)T);
    if (C < 64 || C % 64 != 0 || C > ((int64_t)1 << 24))
        return fail(MHC_ERR_INVALID_ARGUMENT, "C must be a positive multiple of 64 (got %lld)", (long long)C);
    return MHC_OK;
}

int64_t mhc_layer_workspace_bytes(int64_t T, int32_t n, int64_t C)
{
    if (check_layer_shape(T, n, C) != MHC_OK) return -1;
    return mhc::layer_plan(T, C).bytes;
}

namespace {

struct Buf {
    const void* p;
    size_t bytes;
    const char* name;
};

// every pointer non-NULL and 16-byte aligned; no two buffers overlap
static mhc_status check_buffers(const Buf* b, int nb)
{
    for (int i = 0; i < nb; ++i) {
        if (b[i].p == nullptr) return fail(MHC_ERR_INVALID_ARGUMENT, "%s must not be NULL", b[i].name);
        if (!aligned16(b[i].p)) return fail(MHC_ERR_INVALID_ARGUMENT, "%s must be 16-byte aligned", b[i].name);
    }
    for (int i = 0; i < nb; ++i)
        for (int j = i + 1; j < nb; ++j)
            if (overlap(b[i].p, b[i].bytes, b[j].p, b[j].bytes))
                return fail(MHC_ERR_INVALID_ARGUMENT, "%s overlaps %s", b[i].name, b[j].name);
    return MHC_OK;
}

}  // namespace

mhc_status mhc_layer_fwd(const mhc_layer_args* a, void* stream)
{
    if (a == nullptr) return fail(MHC_ERR_INVALID_ARGUMENT, "args is NULL");
    mhc_status s = check_layer_shape(a->T, a->n, a->C);
    if (s != MHC_OK) return s;
    if (!(a->eps > 0.f) || !(a->eps < 1.f)) return fail(MHC_ERR_INVALID_ARGUMENT, "eps must be in (0, 1)");
    mhc::SolverOpts o;
    s = check_opts(a->proj, &o);
    if (s != MHC_OK) return s;
    if (a->T == 0) return ok();
    const size_t T = (size_t)a->T, C = (size_t)a->C;
    const Buf b[] = {{a->x, T * 4 * C * 2, "x"},          {a->W, 24 * 4 * C * 2, "W"},
                     {a->f, T * C * 2, "f"},              {a->u, T * C * 2, "u"},
                     {a->x_out, T * 4 * C * 2, "x_out"},  {a->rms, T * 4, "rms"},
                     {a->logits, T * 96, "logits"},       {a->H_pre, T * 16, "H_pre"},
                     {a->H_post, T * 16, "H_post"},       {a->H_res, T * 64, "H_res"}};
    s = check_buffers(b, sizeof(b) / sizeof(b[0]));
    if (s != MHC_OK) return s;
    const mhc::LayerPtrs p{a->x,   a->W,      a->f,     a->u,     a->x_out, a->rms,
                           a->logits, a->H_pre, a->H_post, a->H_res, nullptr, nullptr,
                           nullptr, nullptr,  nullptr,  nullptr,  nullptr};
    return launched(mhc::launch_layer_fwd(p, a->T, a->C, a->eps, o, (hipStream_t)stream),
                    "layer_fwd launch");
}

// The backward's pointer checks: NULL, alignment, overlaps.  `ws`/`ws_bytes`
// is the workspace to include in the overlap test (NULL: none, as for
// mhc_layer_bwd_noalloc, whose workspace is the library's own).
static mhc_status check_layer_bwd(const mhc_layer_args* a, const void* ws, size_t ws_bytes)
{
    const size_t T = (size_t)a->T, C = (size_t)a->C;
    const Buf b[] = {{a->x, T * 4 * C * 2, "x"},
                     {a->W, 24 * 4 * C * 2, "W"},
                     {a->f, T * C * 2, "f"},
                     {a->rms, T * 4, "rms"},
                     {a->logits, T * 96, "logits"},
                     {a->H_pre, T * 16, "H_pre"},
                     {a->H_post, T * 16, "H_post"},
                     {a->H_res, T * 64, "H_res"},
                     {a->grad_x_out, T * 4 * C * 2, "grad_x_out"},
                     {a->grad_u, T * C * 2, "grad_u"},
                     {a->grad_x, T * 4 * C * 2, "grad_x"},
                     {a->grad_f, T * C * 2, "grad_f"},
                     {a->grad_W, 24 * 4 * C * 4, "grad_W"},
                     {a->grad_logits, T * 96, "grad_logits"},
                     {ws, ws_bytes, "workspace"}};
    return check_buffers(b, sizeof(b) / sizeof(b[0]) - (ws == nullptr ? 1 : 0));
}

static mhc::LayerPtrs layer_bwd_ptrs(const mhc_layer_args* a, void* ws)
{
    return mhc::LayerPtrs{a->x,         a->W,      a->f,      nullptr,       nullptr,
                          a->rms,       a->logits, a->H_pre,  a->H_post,     a->H_res,
                          a->grad_x_out, a->grad_u, a->grad_x, a->grad_f,    a->grad_W,
                          a->grad_logits, ws};
}

mhc_status mhc_layer_bwd(const mhc_layer_args* a, void* stream)
{
    if (a == nullptr) return fail(MHC_ERR_INVALID_ARGUMENT, "args is NULL");
    mhc_status s = check_layer_shape(a->T, a->n, a->C);
    if (s != MHC_OK) return s;
    if (a->T == 0) return ok();
    const int64_t need = mhc::layer_plan(a->T, a->C).bytes;
    if (a->workspace_bytes < need)
        return fail(MHC_ERR_INVALID_ARGUMENT, "workspace_bytes=%lld < %lld required",
                    (long long)a->workspace_bytes, (long long)need);
    if (((uintptr_t)a->workspace & 255u) != 0)
        return fail(MHC_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    s = check_layer_bwd(a, a->workspace, (size_t)need);
    if (s != MHC_OK) return s;
    return launched(mhc::launch_layer_bwd(layer_bwd_ptrs(a, a->workspace), a->T, a->C,
                                          (hipStream_t)stream),
                    "layer_bwd launch");
}

static_assert(MHC_LAYER_NOALLOC_SCRATCH_BYTES == mhc::kLayerNoAllocScratchBytes,
              "header and library agree on the no-alloc scratch size");

mhc_status mhc_layer_bwd_noalloc(const mhc_layer_args* a, void* stream)
{
    if (a == nullptr) return fail(MHC_ERR_INVALID_ARGUMENT, "args is NULL");
    mhc_status s = check_layer_shape(a->T, a->n, a->C);
    if (s != MHC_OK) return s;
    if (a->T == 0) return ok();
    const int64_t need = mhc::layer_plan(a->T, a->C).bytes;
    if (need > mhc::kLayerNoAllocScratchBytes)
        return fail(MHC_ERR_INVALID_ARGUMENT,
                    "T=%lld, C=%lld needs %lld bytes of scratch; mhc_layer_bwd_noalloc holds "
                    "%lld (use mhc_layer_bwd with a workspace)",
                    (long long)a->T, (long long)a->C, (long long)need,
                    (long long)mhc::kLayerNoAllocScratchBytes);
    s = check_layer_bwd(a, nullptr, 0);
    if (s != MHC_OK) return s;
    // the scratch array of the device the work runs on, which must be current
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return launched(e, "layer_bwd_noalloc: hipGetDevice");
    if (stream != nullptr) {
        int sdev = -1;
        e = hipStreamGetDevice((hipStream_t)stream, &sdev);
        if (e != hipSuccess) return launched(e, "layer_bwd_noalloc: hipStreamGetDevice");
        if (sdev != dev)
            return fail(MHC_ERR_INVALID_ARGUMENT,
                        "stream belongs to device %d but device %d is current", sdev, dev);
    }
    void* ws = nullptr;
    e = mhc::layer_noalloc_scratch(dev, &ws);
    if (e != hipSuccess) return launched(e, "layer_bwd_noalloc: scratch address");
    return launched(mhc::launch_layer_bwd(layer_bwd_ptrs(a, ws), a->T, a->C, (hipStream_t)stream),
                    "layer_bwd_noalloc launch");
}

const char* mhc_status_string(mhc_status s)
{
    switch (s) {
    case MHC_OK: return "ok";
    case MHC_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MHC_ERR_UNSUPPORTED: return "unsupported";
    case MHC_ERR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

const char* mhc_last_error(void) { return g_last_error; }

int32_t mhc_abi_version(void) { return MHC_ABI_VERSION; }

}  // extern "C"
