// Per-lane n x n Birkhoff projection for 2 <= n <= 8 (forward and backward),
// the same method as proj4.h written for any n.  The pages build the 4x4 case
// ("Accelerating Birkhoff projection for mHC", gist.science summary, section
// 2.1: the dual has one redundant direction, leaving n - 1 free potentials);
// nothing in the method depends on n = 4:
//   * forward: Newton on the column potentials g_0..g_{n-2} (g_{n-1} = 0) of
//     psi(g) = sum_i logsumexp_j(a_ij + g_j) - sum_j g_j, gradient c - 1,
//     Hessian = graph Laplacian with weights W_jk = sum_i P_ij P_ik, solved
//     by Kron reduction (eliminating vertices in turn; every term is
//     non-negative); globalisation, noise floor and step growth as in
//     proj4.h, except that growth does not wait for the residual to halve;
//     for 3 <= n <= 6 the start comes from the assignment problem as in
//     proj4.h (n = 7, 8 start from g = 0), followed by one Sinkhorn sweep;
//   * backward (section 2.2): dA = P o (G - alpha 1^T - 1 beta^T) with the
//     same Laplacian for beta, in the cancellation-free centred forms.
// Everything is fully unrolled; a lane holds O(n^2) registers (about 250
// VGPRs at n = 8).
#pragma once

#include "proj4.h"

namespace mhc {

template <int N>
struct EvalN {
    float P[N * N];
    float c[N];
    float res;
};

template <int N>
MHC_DEV void finish_residual(EvalN<N>& E)
{
    float r = 0.f;
#pragma unroll
    for (int j = 0; j < N; ++j) r = mhc_max(r, mhc_abs(E.c[j] - 1.f));
    E.res = r;
}

// Row softmax of a + 1 g^T (g_{n-1} = 0), rows shifted by their maximum.
template <int N>
MHC_DEV void evaluate_shifted_n(const float* a, const float* g, EvalN<N>& E)
{
#pragma unroll
    for (int j = 0; j < N; ++j) E.c[j] = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float z[N], m = -3.4028235e38f;
#pragma unroll
        for (int j = 0; j < N; ++j) {
            z[j] = a[N * i + j] + (j < N - 1 ? g[j] : 0.f);
            m = mhc_max(m, z[j]);
        }
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < N; ++j) {
            z[j] = mhc_exp2(z[j] - m);
            s += z[j];
        }
        const float r = mhc_rcp(s);
#pragma unroll
        for (int j = 0; j < N; ++j) {
            E.P[N * i + j] = z[j] * r;
            E.c[j] += E.P[N * i + j];
        }
    }
    finish_residual(E);
}

// The same from k = 2^a and u_j = 2^g_j (see evaluate_factored in proj4.h
// for when this is exact to rounding); false when a row sum is out of range.
template <int N>
MHC_DEV bool evaluate_factored_n(const float* k, const float* g, EvalN<N>& E)
{
    float u[N];
#pragma unroll
    for (int j = 0; j < N - 1; ++j) u[j] = mhc_exp2(g[j]);
    u[N - 1] = 1.f;
#pragma unroll
    for (int j = 0; j < N; ++j) E.c[j] = 0.f;
    bool ok = true;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float e[N], s = 0.f;
#pragma unroll
        for (int j = 0; j < N; ++j) {
            e[j] = k[N * i + j] * u[j];
            s += e[j];
        }
        ok = ok & (s >= kRowLo) & (s <= kRowHi);
        const float r = mhc_rcp(s);
#pragma unroll
        for (int j = 0; j < N; ++j) {
            E.P[N * i + j] = e[j] * r;
            E.c[j] += E.P[N * i + j];
        }
    }
    finish_residual(E);
    return ok;
}

template <int N>
MHC_DEV void evaluate_n(const float* a, const float* k, bool kfast, const float* g, EvalN<N>& E)
{
    if (!(kfast && evaluate_factored_n<N>(k, g, E))) evaluate_shifted_n<N>(a, g, E);
}

// Edge weights W_jk = sum_i P_ij P_ik (j < k) of the Hessian's Laplacian.
template <int N>
MHC_DEV void laplacian_weights_n(const float* P, float (&w)[N][N])
{
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
        for (int k = j + 1; k < N; ++k) {
            float s = P[j] * P[k];
#pragma unroll
            for (int i = 1; i < N; ++i) s = __builtin_fmaf(P[N * i + j], P[N * i + k], s);
            w[j][k] = s;
        }
}

// Relative ridge: 8 eps times the trace of the reduced (grounded) Hessian.
template <int N>
MHC_DEV float ridge_n(const float (&w)[N][N])
{
    float tr = 0.f;
#pragma unroll
    for (int j = 0; j < N - 1; ++j)
#pragma unroll
        for (int k = j + 1; k < N; ++k) tr += (k < N - 1 ? 2.f : 1.f) * w[j][k];
    return __builtin_fmaf(8.f * kFltEps, tr, 1e-30f);
}

// Solve L d = b for the Laplacian of the complete graph on n vertices with
// weights w (upper triangle), vertex n-1 grounded (d_{n-1} = 0), plus a ridge
// lam on the edges from the free vertices to the grounded one.  Gaussian
// elimination of a vertex is Kron reduction: the remaining weights become
// w_ij + w_ki w_kj / deg(k), sums of non-negative terms, so no cancellation
// occurs however small some weights are.  w is overwritten.
template <int N>
MHC_DEV void laplacian_solve_n(float (&w)[N][N], float lam, float (&b)[N], float (&d)[N])
{
#pragma unroll
    for (int i = 0; i < N - 1; ++i) w[i][N - 1] += lam;
    float inv[N];
#pragma unroll
    for (int k = 0; k < N - 1; ++k) {
        float deg = 0.f;
#pragma unroll
        for (int j = k + 1; j < N; ++j) deg += w[k][j];
        inv[k] = mhc_rcp(deg);
#pragma unroll
        for (int i = k + 1; i < N; ++i) {
            const float f = w[k][i] * inv[k];
#pragma unroll
            for (int j = i + 1; j < N; ++j) w[i][j] = __builtin_fmaf(f, w[k][j], w[i][j]);
            if (i < N - 1) b[i] = __builtin_fmaf(f, b[k], b[i]);
        }
    }
    d[N - 1] = 0.f;
#pragma unroll
    for (int k = N - 2; k >= 0; --k) {
        float s = b[k];
#pragma unroll
        for (int j = k + 1; j < N - 1; ++j) s = __builtin_fmaf(w[k][j], d[j], s);
        d[k] = s * inv[k];
    }
}

template <int N>
struct NewtonLaneN {
    float a[N * N];      // base-2 logits, rows shifted to max 0
    float k[N * N];      // 2^a
    float g[N - 1];      // accepted potentials (g_{n-1} = 0)
    float d[N - 1];      // direction (base 2)
    float t, res, slope, grow;
    int newton, trials;
    uint32_t code;
    bool done, slow, kfast;
    bool stored;  // P is in the lane's sink (SINK solvers)
};

// Lane-private slot of N*N floats (LDS) that receives P where the lane's
// solve ends, as sink_store for the 4x4 solver.
template <int N>
MHC_DEV void sink_store_n(float* sink, const float* P)
{
#pragma unroll
    for (int e = 0; e < N * N; ++e) sink[e] = P[e];
}

// Newton direction at E in base-2 units, slope psi'(0) along it, and the
// longest first step kMaxStep / max|d|.
template <int N>
MHC_DEV void newton_direction_n(const EvalN<N>& E, float* d, float& slope, float& tcap)
{
    float w[N][N], b[N], x[N];
    laplacian_weights_n<N>(E.P, w);
    const float lam = ridge_n<N>(w);
#pragma unroll
    for (int j = 0; j < N; ++j) b[j] = 1.f - E.c[j];
    laplacian_solve_n<N>(w, lam, b, x);
    slope = 0.f;
    float dmax = 0.f;
#pragma unroll
    for (int j = 0; j < N - 1; ++j) {
        d[j] = x[j] * kLog2e;
        slope = __builtin_fmaf(E.c[j] - 1.f, d[j], slope);
        dmax = mhc_max(dmax, mhc_abs(d[j]));
    }
    tcap = kMaxStep * mhc_rcp(dmax);
}

// Largest n whose start comes from the assignment problem (the 4x4 start of
// proj4.h, assignment_start, for any n): the best permutation by dynamic
// programming over column subsets, two layers of which are live at a time
// (at most 20 + 15 states at n = 6, each a value and its permutation packed
// 3 bits per row); larger n would need more registers than a lane has left.
constexpr int kAssignStartMaxN = 6;

// Step-growth threshold of the general-n solver (see kFar in proj4.h).  It
// stays at 0.25 for every n: from g = 0 (n = 7, 8) drifts are long and a
// lower threshold catches them a step earlier, and after the assignment
// start the 4x4 value 0.35 measured no better (5x5 forward 13.94 against
// 13.96 us) or worse (6x6: 20.23 against 19.88 us).
constexpr float kFarN = 0.25f;

constexpr int popcount_c(int m) { return m == 0 ? 0 : (m & 1) + popcount_c(m >> 1); }

// Starting potentials g_0..g_{n-2} (base 2, g_{n-1} = 0) from the assignment
// problem on the base-2 logits a: the optimal permutation, the middle of each
// column potential's range over the optimal LP duals (shortest paths to and
// from column n-1 in the permutation's exchange graph, n-2 Bellman-Ford
// rounds after the direct edges), then two max-balancing sweeps; g = 0 if the
// result is not finite.  See assignment_start in proj4.h for the reasoning.
template <int N>
MHC_DEV void assignment_start_n(const float* a, float* g)
{
    static_assert(N >= 3 && N <= kAssignStartMaxN, "assignment start: 3 <= n <= 6");
    // best[mask]: largest sum of a[r][sigma(r)] over rows r < popcount(mask)
    // assigned to the columns in mask; code[mask]: those columns, 3 bits a row
    float best[1 << N];
    uint32_t code[1 << N];
    best[0] = 0.f;
    code[0] = 0u;
#pragma unroll
    for (int row = 0; row < N; ++row) {
#pragma unroll
        for (int mask = 1; mask < (1 << N); ++mask) {
            if (popcount_c(mask) != row + 1) continue;
            float v = -__builtin_inff();
            uint32_t c = 0u;
            bool first = true;
#pragma unroll
            for (int j = 0; j < N; ++j) {
                if (!(mask & (1 << j))) continue;
                const int prev = mask ^ (1 << j);
                const float cand = best[prev] + a[N * row + j];
                const uint32_t cc = code[prev] | ((uint32_t)j << (3 * row));
                const bool take = first | (cand > v);
                v = take ? cand : v;
                c = take ? cc : c;
                first = false;
            }
            best[mask] = v;
            code[mask] = c;
        }
    }
    const uint32_t perm = code[(1 << N) - 1];
    // w[c][j]: length of the edge c -> j (the row owning column c moves to j)
    float w[N][N];
#pragma unroll
    for (int c = 0; c < N; ++c) {
        float row[N];
#pragma unroll
        for (int j = 0; j < N; ++j) row[j] = a[N * (N - 1) + j];
#pragma unroll
        for (int r = N - 2; r >= 0; --r) {
            const bool owns = ((perm >> (3 * r)) & 7u) == (uint32_t)c;
#pragma unroll
            for (int j = 0; j < N; ++j) row[j] = owns ? a[N * r + j] : row[j];
        }
#pragma unroll
        for (int j = 0; j < N; ++j) w[c][j] = row[c] - row[j];
    }
    float to[N - 1], from[N - 1];
#pragma unroll
    for (int j = 0; j < N - 1; ++j) {
        to[j] = w[N - 1][j];
        from[j] = w[j][N - 1];
    }
#pragma unroll
    for (int round = 0; round < N - 2; ++round) {
#pragma unroll
        for (int j = 0; j < N - 1; ++j) {
#pragma unroll
            for (int k = 0; k < N - 1; ++k) {
                if (k == j) continue;
                to[j] = mhc_min(to[j], to[k] + w[k][j]);
                from[j] = mhc_min(from[j], w[j][k] + from[k]);
            }
        }
    }
    float h[N];
#pragma unroll
    for (int j = 0; j < N - 1; ++j) h[j] = 0.5f * (to[j] - from[j]);
    h[N - 1] = 0.f;
#pragma unroll
    for (int sweep = 0; sweep < kBalanceSweeps; ++sweep) {
#pragma unroll
        for (int j = 0; j < N; ++j) {
            float in = __builtin_inff(), out = __builtin_inff();
#pragma unroll
            for (int k = 0; k < N; ++k) {
                if (k == j) continue;
                in = mhc_min(in, w[k][j] + h[k]);
                out = mhc_min(out, w[j][k] - h[k]);
            }
            h[j] = 0.5f * (in - out);
        }
    }
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < N - 1; ++j) {
        h[j] -= h[N - 1];
        sum += mhc_abs(h[j]);
    }
    const bool finite = sum < __builtin_inff();  // NaN, +-inf, overflow: g = 0
#pragma unroll
    for (int j = 0; j < N - 1; ++j) g[j] = finite ? h[j] : 0.f;
}

template <int N, bool SINK>
MHC_DEV void newton_init_n(NewtonLaneN<N>& s, const float* a_nat, const SolverOpts& o, float* sink)
{
    float amin = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float m = a_nat[N * i];
#pragma unroll
        for (int j = 1; j < N; ++j) m = mhc_max(m, a_nat[N * i + j]);
#pragma unroll
        for (int j = 0; j < N; ++j) {
            s.a[N * i + j] = (a_nat[N * i + j] - m) * kLog2e;
            amin = mhc_min(amin, s.a[N * i + j]);
        }
    }
    s.kfast = amin >= kMinLogit;
    s.slow = !s.kfast;
#pragma unroll
    for (int e = 0; e < N * N; ++e) s.k[e] = mhc_exp2(s.a[e]);
    if constexpr (N >= 3 && N <= kAssignStartMaxN) {
        assignment_start_n<N>(s.a, s.g);
    } else {
#pragma unroll
        for (int j = 0; j < N - 1; ++j) s.g[j] = 0.f;
    }
    s.newton = 0;
    s.trials = 0;
    s.grow = 1.f;
    EvalN<N> E;
    evaluate_n<N>(s.a, s.k, s.kfast, s.g, E);
    s.res = E.res;
    s.done = s.res <= o.tol;
    s.code = 0;
    // -1: one sweep, after either start.  After the assignment start it
    // still pays for small logits (6x6 N(0,1): slowest lane of a wave 3.9
    // Newton trials without it, 3.0 with it), unlike for n = 4.
    const int warm = o.warm_sweeps < 0 ? 1 : o.warm_sweeps;
    for (int sw = 0; sw < warm; ++sw) {
        // a lane that is done re-evaluates its own point (bit for bit the same
        // E), so that E is overwritten in place and one evaluation is live here
        const float ln = mhc_log2(mhc_max(E.c[N - 1], kMinMass));
        float ng[N - 1];
#pragma unroll
        for (int j = 0; j < N - 1; ++j)
            ng[j] = s.done ? s.g[j] : s.g[j] + (ln - mhc_log2(mhc_max(E.c[j], kMinMass)));
        evaluate_n<N>(s.a, s.k, s.kfast, ng, E);
        if (!s.done) {
#pragma unroll
            for (int j = 0; j < N - 1; ++j) s.g[j] = ng[j];
            s.res = E.res;
            s.done = s.res <= o.tol;
        }
    }
    float tcap = 0.f;
#pragma unroll
    for (int j = 0; j < N - 1; ++j) s.d[j] = 0.f;
    s.slope = 0.f;
    if (!SINK || wave_any(!s.done)) newton_direction_n<N>(E, s.d, s.slope, tcap);
    s.t = mhc_min(1.f, tcap);
    if (!s.done && o.max_iters < 1) {
        s.done = true;
        s.code = kNotConverged;
    }
    s.newton = 1;
    s.stored = false;
    if (SINK && s.done && s.code != kNotConverged) {
        sink_store_n<N>(sink, E.P);
        s.stored = true;
    }
}

// One trial (see newton_step in proj4.h: same tests, branch-free update
// except that the next direction is computed only if some lane of the wave
// goes on from an accepted point; with SINK a lane that converges writes
// this trial's P to `sink`).
template <int N, bool FACTORED, bool SINK>
MHC_DEV void newton_step_n(NewtonLaneN<N>& s, const SolverOpts& o, float* sink)
{
    float tg[N - 1];
#pragma unroll
    for (int j = 0; j < N - 1; ++j) tg[j] = __builtin_fmaf(s.t, s.d[j], s.g[j]);
    EvalN<N> E;
    bool ok = true;
    if (FACTORED)
        ok = evaluate_factored_n<N>(s.k, tg, E);
    else
        evaluate_shifted_n<N>(s.a, tg, E);
    float dphi = 0.f;
#pragma unroll
    for (int j = 0; j < N - 1; ++j) dphi = __builtin_fmaf(E.c[j] - 1.f, s.d[j], dphi);

    const bool near_floor = s.res <= kNoiseFloor;
    const bool lower = E.res < s.res;
    const bool curved = dphi <= kCurvature * mhc_abs(s.slope);
    const bool conv_t = E.res <= o.tol;
    const bool pass = conv_t | (near_floor & lower) | (!near_floor & curved);
    const bool accept = ok & pass;
    const bool reject = ok & !pass;
    // (no residual-progress condition here: with more columns the residual
    // stalls in the drift too, and at n = 8 the condition cost convergence)
    const bool first = (s.trials == 0) & (s.t >= s.grow);
    const bool far = first & (dphi <= kFarN * s.slope);
    const bool short_of_min = first & (dphi < 0.f);
    const float grow_far = mhc_pin(mhc_min(2.f * s.grow, kMaxGrow));
    const float grow_else = mhc_pin(short_of_min ? s.grow : 1.f);
    const float grow = far ? grow_far : grow_else;
    const bool conv = accept & conv_t;
    const bool maxed = accept & !conv & (s.newton >= o.max_iters);
    const int trials = s.trials + 1;
    const bool stuck = reject & ((near_floor & (s.t <= 1.f)) | (trials > 30));
    const bool done = s.done | conv | maxed | stuck;

    // (P goes to the sink before the direction, which is the last use of E)
    if (SINK && conv) {
        sink_store_n<N>(sink, E.P);
        s.stored = true;
    }
    // The direction, its slope and the next trial length change only here:
    // a lane that accepts while no lane of its wave goes on is done.
    if (wave_any(accept & !done)) {
        float nd[N - 1], nslope, ncap;
        newton_direction_n<N>(E, nd, nslope, ncap);
#pragma unroll
        for (int j = 0; j < N - 1; ++j) s.d[j] = accept ? nd[j] : s.d[j];
        s.slope = accept ? nslope : s.slope;
        s.t = accept ? mhc_min(grow, ncap) : s.t;
    }
#pragma unroll
    for (int j = 0; j < N - 1; ++j) s.g[j] = accept ? tg[j] : s.g[j];
    s.res = accept ? E.res : s.res;
    s.grow = accept ? grow : s.grow;
    s.t = reject ? 0.5f * s.t : s.t;
    s.trials = accept ? 0 : (reject ? trials : s.trials);
    s.newton += (accept & !conv & !maxed) ? 1 : 0;
    s.code = conv ? iters_code(s.newton) : ((maxed | stuck) ? kNotConverged : s.code);
    s.done = done;
    s.slow = s.slow | !ok;
}

template <int N>
MHC_DEV uint32_t project_newton_n(const float* a_nat, float* P_out, const SolverOpts& o)
{
    NewtonLaneN<N> s;
    newton_init_n<N, false>(s, a_nat, o, nullptr);
    while (!s.done && !s.slow) newton_step_n<N, true, false>(s, o, nullptr);
    while (!s.done) newton_step_n<N, false, false>(s, o, nullptr);
    EvalN<N> E;
    evaluate_n<N>(s.a, s.k, s.kfast, s.g, E);
#pragma unroll
    for (int e = 0; e < N * N; ++e) P_out[e] = E.P[e];
    return s.code;
}

// The same projection leaving P in the lane's N*N-float LDS slot `rec`
// (free once the logits are in registers): a lane writes P there from the
// evaluation that converged, so only lanes that stop without converging
// (flag 255) evaluate again at their last accepted point.
template <int N>
MHC_DEV uint32_t project_newton_lds_n(const float* a_nat, float* rec, const SolverOpts& o)
{
    NewtonLaneN<N> s;
    newton_init_n<N, true>(s, a_nat, o, rec);
    while (!s.done && !s.slow) newton_step_n<N, true, true>(s, o, rec);
    while (!s.done) newton_step_n<N, false, true>(s, o, rec);
    if (!s.stored) {
        EvalN<N> E;
        evaluate_n<N>(s.a, s.k, s.kfast, s.g, E);
        sink_store_n<N>(rec, E.P);
    }
    return s.code;
}

// Sinkhorn-Knopp sweeps (rows, then columns), as project_sinkhorn.
template <int N>
MHC_DEV uint32_t project_sinkhorn_n(const float* a_nat, float* K, const SolverOpts& o)
{
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float m = a_nat[N * i];
#pragma unroll
        for (int j = 1; j < N; ++j) m = mhc_max(m, a_nat[N * i + j]);
#pragma unroll
        for (int j = 0; j < N; ++j) K[N * i + j] = mhc_exp2((a_nat[N * i + j] - m) * kLog2e);
    }
    float r[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        r[i] = 0.f;
#pragma unroll
        for (int j = 0; j < N; ++j) r[i] += K[N * i + j];
    }
    int sweeps = 0;
    bool done = false;
    while (sweeps < o.max_iters) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const float inv = mhc_rcp(r[i]);
#pragma unroll
            for (int j = 0; j < N; ++j) K[N * i + j] *= inv;
        }
#pragma unroll
        for (int j = 0; j < N; ++j) {
            float c = 0.f;
#pragma unroll
            for (int i = 0; i < N; ++i) c += K[N * i + j];
            const float inv = mhc_rcp(c);
#pragma unroll
            for (int i = 0; i < N; ++i) K[N * i + j] *= inv;
        }
        ++sweeps;
        float rr = 0.f;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            r[i] = 0.f;
#pragma unroll
            for (int j = 0; j < N; ++j) r[i] += K[N * i + j];
            rr = mhc_max(rr, mhc_abs(r[i] - 1.f));
        }
        if (o.tol > 0.f && rr <= o.tol) {
            done = true;
            break;
        }
    }
    if (o.tol > 0.f && !done) return kNotConverged;
    return iters_code(sweeps);
}

// out_j = sum_k p_k (x_j - x_k) for one row p of P (sum_k p_k = 1): x_j minus
// the p-weighted mean of the row, as a weighted sum of differences.
template <int N>
MHC_DEV void centred_row_n(const float* p, const float* x, float* out)
{
#pragma unroll
    for (int j = 0; j < N; ++j) {
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < N; ++k)
            if (k != j) s = __builtin_fmaf(p[k], x[j] - x[k], s);
        out[j] = s;
    }
}

// Backward of the projection (section 2.2), as project_bwd in proj4.h:
//   (b - P^T a)_j = sum_i P_ij sum_k P_ik (G_ij - G_ik),
//   Laplacian(W) beta = that (beta_{n-1} = 0),
//   dA_ij = P_ij sum_k P_ik (H_ij - H_ik),   H = G - 1 beta^T.
template <int N>
MHC_DEV void project_bwd_n(const float* P, const float* G, float* dA)
{
    float rhs[N];
#pragma unroll
    for (int j = 0; j < N; ++j) rhs[j] = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float gc[N];
        centred_row_n<N>(P + N * i, G + N * i, gc);
#pragma unroll
        for (int j = 0; j < N; ++j) rhs[j] = __builtin_fmaf(P[N * i + j], gc[j], rhs[j]);
    }
    float w[N][N], beta[N];
    laplacian_weights_n<N>(P, w);
    const float lam = ridge_n<N>(w);
    laplacian_solve_n<N>(w, lam, rhs, beta);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float h[N], hc[N];
#pragma unroll
        for (int j = 0; j < N; ++j) h[j] = G[N * i + j] - beta[j];
        centred_row_n<N>(P + N * i, h, hc);
#pragma unroll
        for (int j = 0; j < N; ++j) dA[N * i + j] = P[N * i + j] * hc[j];
    }
}

}  // namespace mhc
