// Per-lane 4x4 Birkhoff projection: forward (Newton on the column potentials,
// or Sinkhorn-Knopp) and backward (implicit differentiation).
//
// One lane owns one matrix.  All 16 entries, the potentials and the solver
// state stay in VGPRs, with no cross-lane traffic; the staged kernels also
// give each lane a private LDS slot, from which the start reads rows of its
// logits and into which the solve leaves P.  Every loop below is fully
// unrolled so that array indices are compile-time constants.
//
// Method ("Accelerating Birkhoff projection for mHC", gist.science summary):
//  * section 2 -- the projection of A is the entropy-regularised transport
//    plan P = diag(u) exp(A) diag(v), the unique doubly stochastic scaling;
//  * section 2.1 -- the dual has one redundant direction (a common shift), so
//    for 4x4 it is a three-variable unconstrained convex problem solved by
//    Newton's method with closed-form gradient and Hessian; rows are shifted
//    by their maximum before the softmax;
//  * section 2.2 -- the gradient comes from the implicit function theorem,
//    with no forward state kept, and the last Newton Hessian is the matrix
//    the backward needs.
//
// Reading taken here: the row potentials are eliminated in closed form by a
// row softmax, leaving column potentials g = (g0, g1, g2, 0):
//     P(g)_ij = exp(A_ij + g_j) / sum_k exp(A_ik + g_k)
//     psi(g)  = sum_i logsumexp_j(A_ij + g_j) - sum_j g_j        (convex)
//     grad    = c - 1,   c_j = sum_i P_ij (column sums)
//     Hessian = diag(c) - P^T P  =  graph Laplacian with edge weights
//               W_jk = sum_i P_ij P_ik  (because rows of P sum to 1)
// Rows of P(g) are stochastic by construction; g solves the problem when the
// columns are too.  At the solution the Hessian is I - P^T P, the matrix of
// the implicit-differentiation system -- the "Hessian reuse" of section 2.2.
//
// Everything is computed in base 2 (a = A log2 e, g in log2 units):
// 2^(a + g) = e^(A + g ln 2).  The Newton direction of the base-2 objective is
// the natural-units direction times log2 e, which the solve yields directly
// from the column defects scaled by log2 e (Eval::b).
#pragma once

#include "devmath.h"

namespace mhc {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kFltEps = 1.1920928955078125e-07f;
// Longest first trial step of a Newton iteration, in base-2 potential units
// (a factor 2^8 in a column's scaling).  Far from the solution the Newton
// model of the exponential objective can propose steps of thousands of
// units; starting the backtracking at this length instead saves the many
// halvings that would otherwise be spent getting back down.
constexpr float kMaxStep = 8.f;
// Below this column residual (about 4x the fp32 rounding floor of a column
// sum of four row-softmax entries) a trial is judged by the residual alone,
// and one that does not lower it marks the noise floor and ends the solve.
constexpr float kNoiseFloor = 4e-6f;
constexpr float kNoiseFloor2 = kNoiseFloor * kLog2e;  // the same in Eval::res units
// Curvature test of the line search: accept a trial whose directional
// derivative is at most this fraction of the initial one's magnitude.
constexpr float kCurvature = 0.9f;
// Step growth.  Where some entries of P are tending to zero the objective is
// exponential, not quadratic, along the Newton direction d: its directional
// derivative decays like e^-t in units of the Newton step, so each full step
// gains only a factor e and the potentials drift a constant distance per
// iteration.  An accepted full first trial whose directional derivative
// still has at least kFar of its initial magnitude doubles the next
// iteration's first trial (up to kMaxGrow Newton steps), provided the trial
// cut the residual by at least kGrowProgress: when the drift ends, the
// directional derivative keeps looking far while the residual stalls, and
// longer trials there only overshoot.  Every other outcome returns to the
// plain Newton step.  (Keeping a grown multiple after a trial that merely
// stopped short of the line minimum paid when drifts were long; from the
// assignment start they last a trial or two, and the kept multiple then
// overshoots once the iteration is quadratic: on 131072 N(0,10^2) matrices
// it left 45 waves needing a fifth trial, against 11 without it.)
// A drift step keeps about e^-1 = 0.37 of the directional derivative.  From
// the assignment start long drifts are rare, and a first full step that
// keeps 0.25-0.35 of it is mostly mild curvature change near the solution,
// where a doubled trial overshoots; kFar sits just below e^-1 (on 131072
// N(0,10^2) matrices any value in 0.34-0.36 gives the same waves; 0.25 left
// 4.5x as many waves needing a fifth trial).  (The general-n solver keeps
// its own threshold, kFarN.)
constexpr float kFar = 0.35f;
constexpr float kMaxGrow = 64.f;
constexpr float kGrowProgress = 0.5f;
// Floor on a column mass before its logarithm is taken.
constexpr float kMinMass = 7.8886091e-31f;  // 2^-100

// Solver selection and limits (mirrors mhc_proj_opts of the public header).
struct SolverOpts {
    int solver;       // 0 = Newton, 1 = Sinkhorn
    int max_iters;    // Newton iterations / Sinkhorn sweeps
    float tol;        // stop when max_j |c_j - 1| <= tol
    int warm_sweeps;  // log-domain Sinkhorn sweeps before Newton (-1: the solver's choice)
};

// Column sums and row-softmax matrix of the semi-dual at g.
struct Eval {
    float P[16];
    float c[4];
    float b[4];  // (1 - c_j) log2 e
    float res;   // max_j |b_j| = max_j |c_j - 1| log2 e
};

// Column sums of E.P, their defects and the residual.  The defects are kept
// in the base-2 units of the potentials, b_j = (1 - c_j) log2 e (one fused
// multiply-add, a single rounding), so that the Newton system solved with
// them gives the base-2 direction directly; the residual is in the same
// units, and every tolerance it is compared with is scaled by log2 e
// (kLog2e * o.tol, kNoiseFloor2).  Contraction is off so that the sums add
// the stored entries (which the Hessian weights use too) instead of
// re-multiplying them.
MHC_DEV void column_sums(Eval& E)
{
#pragma clang fp contract(off)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        E.c[j] = (E.P[j] + E.P[4 + j]) + (E.P[8 + j] + E.P[12 + j]);
        E.b[j] = __builtin_fmaf(-kLog2e, E.c[j], kLog2e);
    }
    E.res = mhc_max(mhc_max(mhc_abs(E.b[0]), mhc_abs(E.b[1])),
                    mhc_max(mhc_abs(E.b[2]), mhc_abs(E.b[3])));
}

// Row softmax of a + 1 g^T (g3 = 0) with the row max-shift before exp2.
MHC_DEV void evaluate_shifted(const float* a, float g0, float g1, float g2, Eval& E)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float z0 = a[4 * i + 0] + g0;
        const float z1 = a[4 * i + 1] + g1;
        const float z2 = a[4 * i + 2] + g2;
        const float z3 = a[4 * i + 3];
        const float m = mhc_max(mhc_max(z0, z1), mhc_max(z2, z3));
        const float e0 = mhc_exp2(z0 - m);
        const float e1 = mhc_exp2(z1 - m);
        const float e2 = mhc_exp2(z2 - m);
        const float e3 = mhc_exp2(z3 - m);
        const float r = mhc_rcp((e0 + e1) + (e2 + e3));
        E.P[4 * i + 0] = e0 * r;
        E.P[4 * i + 1] = e1 * r;
        E.P[4 * i + 2] = e2 * r;
        E.P[4 * i + 3] = e3 * r;
    }
    column_sums(E);
}

// The same row softmax from k = 2^a (a's rows have maximum 0, so k <= 1 with
// one entry 1 per row): P_ij = k_ij u_j / sum_l k_il u_l with u_j = 2^g_j,
// three exponentials instead of sixteen and no max-shift.  It is used when
//  * every a_ij >= -126 (kfast, fixed per matrix): each k_ij is a normal
//    float, so each product k_ij u_j carries the relative accuracy of its
//    factors whatever u_j is, or under/overflows outright; and
//  * every row sum is finite and at least 2^-60: a product that underflowed
//    (2^(a+g) < 2^-126, since k <= 1) is then below 2^-66 of its row, and an
//    overflow or a NaN shows up in the sum.
// Otherwise the lane takes the max-shifted form.
constexpr float kRowLo = 8.6736174e-19f;  // 2^-60
constexpr float kRowHi = 3.4028235e38f;   // largest finite float
constexpr float kMinLogit = -126.f;

// Factored form only; returns false (E then unusable) when a row sum is out
// of range.
MHC_DEV bool evaluate_factored(const float* k, float g0, float g1, float g2, Eval& E)
{
    const float u0 = mhc_exp2(g0), u1 = mhc_exp2(g1), u2 = mhc_exp2(g2);
    bool ok = true;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float e0 = k[4 * i + 0] * u0;
        const float e1 = k[4 * i + 1] * u1;
        const float e2 = k[4 * i + 2] * u2;
        const float e3 = k[4 * i + 3];
        const float sum = (e0 + e1) + (e2 + e3);
        ok = ok && sum >= kRowLo && sum <= kRowHi;
        const float r = mhc_rcp(sum);
        E.P[4 * i + 0] = e0 * r;
        E.P[4 * i + 1] = e1 * r;
        E.P[4 * i + 2] = e2 * r;
        E.P[4 * i + 3] = e3 * r;
    }
    column_sums(E);
    return ok;
}

// Factored form where it applies, max-shifted form otherwise.
MHC_DEV void evaluate(const float* a, const float* k, bool kfast, float g0, float g1, float g2,
                      Eval& E)
{
    if (!(kfast && evaluate_factored(k, g0, g1, g2, E))) evaluate_shifted(a, g0, g1, g2, E);
}

// Solve L d = b for the Laplacian L of the complete graph on {0,1,2,3} with
// edge weights w01..w23, vertex 3 grounded (d3 = 0), plus a ridge lam on the
// three free vertices (an extra edge of weight lam from each to vertex 3).
//
// Gaussian elimination of a Laplacian vertex is Kron reduction: removing
// vertex k leaves a Laplacian whose weights are w_ij + w_ik w_jk / deg(k).
// Every quantity below is a sum of non-negative terms, so there is no
// cancellation however small some weights are; the pivots are the vertex
// degrees, which the ridge keeps positive.
MHC_DEV void laplacian_solve(float w01, float w02, float w03, float w12, float w13,
                             float w23, float lam, float b0, float b1, float b2,
                             float& d0, float& d1, float& d2)
{
    w03 += lam;
    w13 += lam;
    w23 += lam;
    // eliminate vertex 0
    const float inv0 = mhc_rcp((w01 + w02) + w03);
    const float k1 = w01 * inv0;
    const float k2 = w02 * inv0;
    const float w12r = w12 + w01 * k2;
    const float w13r = w13 + w03 * k1;
    const float w23r = w23 + w03 * k2;
    const float b1r = b1 + k1 * b0;
    const float b2r = b2 + k2 * b0;
    // eliminate vertex 1
    const float inv1 = mhc_rcp(w12r + w13r);
    const float m2 = w12r * inv1;
    const float w23rr = w23r + w13r * m2;
    const float b2rr = b2r + m2 * b1r;
    // vertex 2 is tied only to the grounded vertex now
    d2 = b2rr * mhc_rcp(w23rr);
    d1 = (b1r + w12r * d2) * inv1;
    d0 = ((b0 + w01 * d1) + w02 * d2) * inv0;
}

// Edge weights W_jk = sum_i P_ij P_ik of the Hessian's Laplacian.
struct Weights {
    float w01, w02, w03, w12, w13, w23;
};

MHC_DEV Weights laplacian_weights(const float* P)
{
    Weights w;
    w.w01 = P[0] * P[1];
    w.w02 = P[0] * P[2];
    w.w03 = P[0] * P[3];
    w.w12 = P[1] * P[2];
    w.w13 = P[1] * P[3];
    w.w23 = P[2] * P[3];
#pragma unroll
    for (int i = 1; i < 4; ++i) {
        const float* p = P + 4 * i;
        w.w01 = __builtin_fmaf(p[0], p[1], w.w01);
        w.w02 = __builtin_fmaf(p[0], p[2], w.w02);
        w.w03 = __builtin_fmaf(p[0], p[3], w.w03);
        w.w12 = __builtin_fmaf(p[1], p[2], w.w12);
        w.w13 = __builtin_fmaf(p[1], p[3], w.w13);
        w.w23 = __builtin_fmaf(p[2], p[3], w.w23);
    }
    return w;
}

// Relative ridge: 8 eps times the trace of the reduced Hessian, plus a floor
// that only matters when every off-diagonal weight underflowed.
MHC_DEV float ridge(const Weights& w)
{
    const float tr = 2.f * (w.w01 + w.w02 + w.w12) + (w.w03 + w.w13 + w.w23);
    return __builtin_fmaf(8.f * kFltEps, tr, 1e-30f);
}

// Ridge of the forward's Newton solve: a constant kDirRidge on the degree of
// every free vertex.  A computed column residual carries rounding noise of a
// couple of ulps of 1, so along a direction whose curvature is below that
// (a column tied to the others only by weights of 1e-12, as near a
// permutation matrix) the plain solve turns noise into steps of hundreds of
// units; the cap on the trial length then shrinks the whole step, and the
// useful part of the direction with it, to a few percent.  With the floor such
// a direction moves about noise / kDirRidge, under a unit.  Directions with
// curvature well above it are unchanged, so the final quadratic convergence
// is kept.  The relative part of ridge() (8 eps times the trace, at most
// about 6e-6 here) changed no iteration count on the benchmark batches and
// costs six instructions per direction, so the forward does without it.
// (The backward solves the exact system and keeps ridge().)
constexpr float kDirRidge = 2.f * kFltEps;

// Iteration counter encoding for the optional per-matrix output.
constexpr uint32_t kNotConverged = 255u;
MHC_DEV uint32_t iters_code(int n) { return n > 254 ? 254u : (uint32_t)n; }

// True if `pred` holds on any active lane of the wave (wave-uniform).
MHC_DEV bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }

// Lane-private 16-float slot in LDS that receives P when the lane's solve
// ends (SINK solvers); the lane's logits occupied it until the start read them.
MHC_DEV void sink_store(float* sink, const float* P)
{
#pragma unroll
    for (int k = 0; k < 16; ++k) sink[k] = P[k];
}

// Newton's method on the semi-dual for one matrix, as a state machine:
//
//   init():  base-2 logits with each row shifted to maximum 0; evaluate at
//            the assignment start; warm_sweeps log-domain Sinkhorn sweeps
//            (none by default; g_j -= log c_j, re-gauged so g3 = 0; a column
//            whose entries all underflowed has its mass floored so the step
//            stays finite); first Newton direction.
//   step():  one trial point g + t d.  psi is convex along the line, so its
//            derivative psi'(s) = (c(s) - 1) . d rises monotonically from
//            psi'(0) = slope < 0; a trial is accepted when
//            psi'(t) <= kCurvature |slope| (it has not overshot the line
//            minimum by much), which needs only the column sums the
//            evaluation already has -- no logarithms.  Near the fp32 noise
//            floor (column residual <= kNoiseFloor) a trial is accepted only if it
//            lowers the residual, and a rejected trial no longer than the
//            Newton step ends the solve.  A rejected trial halves t.  Every
//            trial reaching the tolerance is accepted.
// The Newton direction solves the Laplacian system of the Hessian with a
// ridge (kDirRidge, Kron reduction); its first trial step is capped at
// kMaxStep.
struct NewtonLane {
    float a[16];         // base-2 logits, rows shifted to max 0
    float k[16];         // 2^a
    bool kfast;          // every a_ij >= kMinLogit: the factored evaluation applies
    bool slow;           // the lane has left the factored evaluation for good
    float g0, g1, g2;    // accepted potentials (g3 = 0)
    float d0, d1, d2;    // direction (base 2)
    float t, res, slope; // step length, residual and psi'(0) along d (Eval::res units)
    float grow;          // first-trial multiple of the Newton step (>= 1)
    int newton, trials;  // Newton directions taken, halvings this step
    bool failed;         // stopped without converging (iteration code 255)
    bool done;
    bool stored;         // P already written to the lane's LDS sink
};

// Newton direction at E in base-2 units (the Laplacian solve with the
// defects already in those units, Eval::b), the slope psi'(0) along it (in
// the same scaled units as Eval::res), and the longest first step
// kMaxStep / max|d|.
MHC_DEV void newton_direction(const Eval& E, float& d0, float& d1, float& d2, float& slope,
                              float& tcap)
{
    const Weights w = laplacian_weights(E.P);
    laplacian_solve(w.w01, w.w02, w.w03, w.w12, w.w13, w.w23, kDirRidge, E.b[0], E.b[1], E.b[2], d0,
                    d1, d2);
    slope = -(E.b[0] * d0 + E.b[1] * d1 + E.b[2] * d2);
    const float dmax = mhc_max(mhc_max(mhc_abs(d0), mhc_abs(d1)), mhc_abs(d2));
    tcap = kMaxStep * mhc_rcp(dmax);
}

MHC_DEV void newton_take(NewtonLane& s, const Eval& E) { s.res = E.res; }

// Iteration code of a finished lane: the Newton directions it took before
// converging (0 at the start), or kNotConverged.
MHC_DEV uint32_t newton_code(const NewtonLane& s)
{
    return s.failed ? kNotConverged : iters_code(s.newton);
}

// Starting potentials from the assignment problem.  A doubly stochastic
// matrix is a convex combination of permutation matrices (neo-ai news
// summary of mHC, passage on the properties of doubly stochastic matrices),
// and with large logits the projection is close to the best permutation: as
// the logits grow, the potentials approach an optimal dual of the linear
// assignment problem max over sigma of sum_i a_i,sigma(i).  The optimal duals
// form a polytope; with g3 = 0 each column potential g_j ranges over an
// interval whose ends are shortest-path distances between columns j and 3 in
// the exchange graph of the optimal permutation (an edge c -> j of length
// a_oc - a_oj for the row o that sigma assigns to column c: moving row o from
// column c to j).  The middle of each interval is a dual-feasible point with
// slack on both sides; two sweeps of max-balancing (below) then move it
// towards the entropic solution.  On N(0,10^2) logits the result lies 0.27
// natural units from the solution on average and 4.3 at most (the middle of
// the intervals: 1.7 and 14; one Sinkhorn sweep from g = 0: 6.8 and 30).
// The permutation is found by brute force: rows 2 and 3 take the better
// orientation of each of the 6 column pairs, rows 0 and 1 each of the 12
// ordered pairs of the other two columns.  Shortest paths have at most 3
// edges; one round of Bellman-Ford after the direct edges finds those of up
// to 2, and a second round (exact) changed no iteration count on N(0,10^2)
// or mixed batches once the balancing sweeps follow, so it is left out.
// The search works in the base-2 units of a.  The exchange lengths take the
// owner rows either from a by select chains (ROWS_IN_LDS false) or, when the
// caller still holds the lane's raw logits in LDS (rec: 16 floats,
// row-major), by indexed LDS reads: a row's max-shift cancels in every length,
// so those lengths, the paths and the balancing are in natural units and the
// result is scaled by log2 e at the end.  A non-finite result (a NaN or
// infinite logit) falls back to g = 0.
constexpr int kBalanceSweeps = 2;
template <bool ROWS_IN_LDS>
MHC_DEV void assignment_start(const float* a, const float* rec, float& g0, float& g1, float& g2)
{
    // column pairs (k, l), k < l, and the pair left over by each ordered
    // (j0, j1)
    constexpr int pk[6] = {0, 0, 0, 1, 1, 2};
    constexpr int pl[6] = {1, 2, 3, 2, 3, 3};
    float m23[6];
    uint32_t r2bits = 0;  // 2 bits per pair p: column of row 2 in its better orientation
#pragma unroll
    for (int p = 0; p < 6; ++p) {
        const float v1 = a[8 + pk[p]] + a[12 + pl[p]];
        const float v2 = a[8 + pl[p]] + a[12 + pk[p]];
        m23[p] = mhc_max(v1, v2);
        r2bits |= (v2 > v1 ? (uint32_t)pl[p] : (uint32_t)pk[p]) << (2 * p);
    }
    // The 12 ordered pairs (j0, j1) of rows 0 and 1, numbered q in loop
    // order.  Each candidate sum carries q in its 4 lowest mantissa bits, so
    // one max over the tagged sums gives the best one and its number
    // (candidates within 2^-19 of each other, relatively, are not told
    // apart; either is a valid start).  A -inf sum turns into a NaN, which
    // the max skips.  kJ0 and kJ1 hold j0 and j1 of each q (2 bits each), kPq
    // the leftover pair p (3 bits each); q is clamped to the table in case
    // every candidate was skipped.
    constexpr uint32_t kJ0 = 0xfea540u, kJ1 = 0x934e39u;
    constexpr uint64_t kPq = 0x5850aae5ull;  // 36 bits (the top entry is 0)
    float best = -__builtin_inff();
    int q = 0;
#pragma unroll
    for (int j0 = 0; j0 < 4; ++j0) {
#pragma unroll
        for (int j1 = 0; j1 < 4; ++j1) {
            if (j1 == j0) continue;
            const int lo = (j0 != 0 && j1 != 0) ? 0 : ((j0 != 1 && j1 != 1) ? 1 : 2);
            const int hi = (j0 != 3 && j1 != 3) ? 3 : ((j0 != 2 && j1 != 2) ? 2 : 1);
            const int p = lo == 0 ? hi - 1 : (lo == 1 ? hi + 1 : 5);
            const float v = a[j0] + a[4 + j1] + m23[p];
            best = mhc_max(best, __uint_as_float((__float_as_uint(v) & ~15u) | (uint32_t)q));
            ++q;
        }
    }
    const uint32_t qb = __float_as_uint(best) & 15u;
    const uint32_t qi = qb < 11u ? qb : 11u;
    const int c0 = (int)((kJ0 >> (2 * qi)) & 3u);  // columns of rows 0, 1, 2
    const int c1 = (int)((kJ1 >> (2 * qi)) & 3u);
    const int c2 = (int)((r2bits >> (2 * (uint32_t)((kPq >> (3 * qi)) & 7u))) & 3u);
    // w[c][j]: length of the edge c -> j (row owning column c moves to j)
    float w[4][4];
    if constexpr (ROWS_IN_LDS) {
        // owner row of every column, two bits per column (row 0's are zero)
        const int c3 = 6 - c0 - c1 - c2;
        const uint32_t own = (1u << (2 * c1)) | (2u << (2 * c2)) | (3u << (2 * c3));
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float* r = rec + 4 * ((own >> (2 * c)) & 3u);
            float row[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) row[j] = r[j];
#pragma unroll
            for (int j = 0; j < 4; ++j) w[c][j] = row[c] - row[j];
        }
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bool o0 = c0 == c, o1 = c1 == c, o2 = c2 == c;
            float row[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                row[j] = o0 ? a[j] : (o1 ? a[4 + j] : (o2 ? a[8 + j] : a[12 + j]));
#pragma unroll
            for (int j = 0; j < 4; ++j) w[c][j] = row[c] - row[j];
        }
    }
    // to[j]: shortest 3 -> j (upper end of g_j); from[j]: shortest j -> 3
    // (minus the lower end)
    float to[3], from[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        to[j] = w[3][j];
        from[j] = w[j][3];
    }
#pragma unroll
    for (int round = 0; round < 1; ++round) {
#pragma unroll
        for (int j = 0; j < 3; ++j) {
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                if (k == j) continue;
                to[j] = mhc_min(to[j], to[k] + w[k][j]);
                from[j] = mhc_min(from[j], w[j][k] + from[k]);
            }
        }
    }
    float h[4] = {0.5f * (to[0] - from[0]), 0.5f * (to[1] - from[1]),
                  0.5f * (to[2] - from[2]), 0.f};
    // Max-balancing: column j moves to where its cheapest incoming exchange
    // and its cheapest outgoing one have equal slack (slack of c -> j:
    // w[c][j] - h_j + h_c).  Near a permutation an off-assignment entry of P
    // is about e^-slack and a column balances when what flows in equals what
    // flows out, so this is the solution's balance with each sum replaced by
    // its largest term.  Two Gauss-Seidel sweeps.
#pragma unroll
    for (int sweep = 0; sweep < kBalanceSweeps; ++sweep) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float in = __builtin_inff(), out = __builtin_inff();
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (k == j) continue;
                in = mhc_min(in, w[k][j] + h[k]);
                out = mhc_min(out, w[j][k] - h[k]);
            }
            h[j] = 0.5f * (in - out);
        }
    }
    const float unit = ROWS_IN_LDS ? kLog2e : 1.f;
    const float m0 = (h[0] - h[3]) * unit, m1 = (h[1] - h[3]) * unit, m2 = (h[2] - h[3]) * unit;
    // NaN, +-inf (or overflow of the sum) fall back to g = 0
    const bool finite = (mhc_abs(m0) + mhc_abs(m1)) + mhc_abs(m2) < __builtin_inff();
    g0 = finite ? m0 : 0.f;
    g1 = finite ? m1 : 0.f;
    g2 = finite ? m2 : 0.f;
}

template <bool ROWS_IN_LDS, bool SINK>
MHC_DEV void newton_init(NewtonLane& s, const float* a_nat, const float* rec, const SolverOpts& o,
                         float* sink)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float m = mhc_max(mhc_max(a_nat[4 * i], a_nat[4 * i + 1]),
                                mhc_max(a_nat[4 * i + 2], a_nat[4 * i + 3]));
#pragma unroll
        for (int j = 0; j < 4; ++j) s.a[4 * i + j] = (a_nat[4 * i + j] - m) * kLog2e;
    }
    float amin = s.a[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) amin = mhc_min(amin, s.a[j]);
    s.kfast = amin >= kMinLogit;  // (a NaN entry fails the row-sum test instead)
    s.slow = !s.kfast;
#pragma unroll
    for (int j = 0; j < 16; ++j) s.k[j] = mhc_exp2(s.a[j]);
    assignment_start<ROWS_IN_LDS>(s.a, rec, s.g0, s.g1, s.g2);
    s.newton = 0;
    s.trials = 0;
    Eval E;
    evaluate(s.a, s.k, s.kfast, s.g0, s.g1, s.g2, E);
    newton_take(s, E);
    const float tol2 = kLog2e * o.tol;
    s.done = s.res <= tol2;
    s.failed = false;
    const int warm = o.warm_sweeps < 0 ? 0 : o.warm_sweeps;  // -1: none after this start
    for (int w = 0; w < warm; ++w) {
        // A lane that is done re-evaluates its own point (bit for bit the
        // same E), so that the sweep can overwrite E in place: holding two
        // whole evaluations across this loop set the register count of every
        // forward kernel, the default (no sweeps) included.
        const float l3 = mhc_log2(mhc_max(E.c[3], kMinMass));
        const float n0 = s.done ? s.g0 : s.g0 + (l3 - mhc_log2(mhc_max(E.c[0], kMinMass)));
        const float n1 = s.done ? s.g1 : s.g1 + (l3 - mhc_log2(mhc_max(E.c[1], kMinMass)));
        const float n2 = s.done ? s.g2 : s.g2 + (l3 - mhc_log2(mhc_max(E.c[2], kMinMass)));
        evaluate(s.a, s.k, s.kfast, n0, n1, n2, E);
        if (!s.done) {
            s.g0 = n0;
            s.g1 = n1;
            s.g2 = n2;
            newton_take(s, E);
            s.done = s.res <= tol2;
        }
    }
    float tcap = 0.f;
    s.d0 = s.d1 = s.d2 = s.slope = 0.f;
    if (!SINK || wave_any(!s.done)) newton_direction(E, s.d0, s.d1, s.d2, s.slope, tcap);
    s.grow = 1.f;
    s.t = mhc_min(1.f, tcap);
    s.newton = s.done ? 0 : 1;  // a lane converged at the start reports 0
    if (!s.done && o.max_iters < 1) {
        s.done = true;
        s.failed = true;
    }
    s.stored = false;
    if (SINK && s.done && !s.failed) {
        sink_store(sink, E.P);
        s.stored = true;
    }
}

// One trial of a lane that is not done (the caller guarantees !s.done and,
// for FACTORED, !s.slow).  Written without branches, except that the next
// Newton direction is computed only if some lane of the wave goes on from an
// accepted point: a wave's last trial, where every remaining lane converges
// or stops, skips it.  With FACTORED a trial whose factored evaluation is out
// of range changes nothing but s.slow; the lane then repeats it, and
// continues, with the max-shifted form.  With SINK a lane that converges
// writes its P (this trial's evaluation) to `sink` and sets s.stored.
template <bool FACTORED, bool SINK>
MHC_DEV void newton_step(NewtonLane& s, const SolverOpts& o, float* sink)
{
    const float t0 = s.g0 + s.t * s.d0, t1 = s.g1 + s.t * s.d1, t2 = s.g2 + s.t * s.d2;
    Eval E;
    bool ok = true;
    if (FACTORED)
        ok = evaluate_factored(s.k, t0, t1, t2, E);
    else
        evaluate_shifted(s.a, t0, t1, t2, E);

    const float dphi = -(E.b[0] * s.d0 + E.b[1] * s.d1 + E.b[2] * s.d2);
    // (bitwise & and | on bools: no short-circuit branches)
    const bool near_floor = s.res <= kNoiseFloor2;
    const bool lower = E.res < s.res;
    const bool curved = dphi <= kCurvature * mhc_abs(s.slope);
    const bool conv_t = E.res <= kLog2e * o.tol;
    // On the max-shifted path (lanes whose logits span more than ~87 natural
    // units, where the potentials reach the hundreds) two fp32 stalls are
    // cut short; the factored loop, all ordinary inputs, skips both tests.
    // A trial that takes the residual from above the noise floor into it is
    // judged by the residual (the directional derivative is quantised there
    // and can read as an overshoot).
    const bool to_floor = !FACTORED && (E.res <= kNoiseFloor2);
    // (above_floor is its own comparison rather than !near_floor, so that
    // the test stays a combination of lane masks instead of a per-lane
    // select, which costs five vector instructions)
    const bool above_floor = s.res > kNoiseFloor2;
    const bool pass = conv_t | ((near_floor | to_floor) & lower) | (above_floor & curved);
    const bool accept = ok & pass;
    const bool reject = ok & !pass;
    // next first trial: doubled after a full first trial that at least
    // halved the residual and stayed far from the line minimum; the Newton
    // step otherwise.  (A first trial has t = min(grow, cap) <= grow and a
    // rejection halves t, so t >= grow holds only on an uncapped first trial.)
    const bool first = (s.t >= s.grow) & (E.res < kGrowProgress * s.res);
    const bool far = first & (dphi <= kFar * s.slope);
    const float grow = mhc_pin(far ? mhc_min(2.f * s.grow, kMaxGrow) : 1.f);
    const bool conv = accept & conv_t;
    const bool maxed = accept & !conv & (s.newton >= o.max_iters);
    const int trials = s.trials + 1;
    // A trial point equal to the accepted one (t d below the fp32 resolution
    // of every potential) changes nothing, and the next iteration from that
    // point would repeat it: the solve is at its fp32 limit.  Without these
    // two tests such lanes spent up to 340 evaluations on N(0,100^2) logits
    // (5 at most otherwise; the forward there ran 3.7x longer).  Applied to
    // every trial they cost 3 % of the ordinary forward, hence this path only.
    const bool still = !FACTORED && ((t0 == s.g0) & (t1 == s.g1) & (t2 == s.g2) & !conv_t);
    const bool stuck = (reject & ((near_floor & (s.t <= 1.f)) | (trials > 30))) | (ok & still);
    const bool done = s.done | conv | maxed | stuck;

    // The direction, its slope and the next trial length change only here:
    // a lane that accepts while no lane of its wave goes on is done, and
    // its direction is never read again.
    if (wave_any(accept & !done)) {
        float nd0, nd1, nd2, nslope, ncap;
        newton_direction(E, nd0, nd1, nd2, nslope, ncap);
        s.d0 = accept ? nd0 : s.d0;
        s.d1 = accept ? nd1 : s.d1;
        s.d2 = accept ? nd2 : s.d2;
        s.slope = accept ? nslope : s.slope;
        s.t = accept ? mhc_min(grow, ncap) : s.t;
    }
    if (SINK && conv) {
        sink_store(sink, E.P);
        s.stored = true;
    }

    s.g0 = accept ? t0 : s.g0;
    s.g1 = accept ? t1 : s.g1;
    s.g2 = accept ? t2 : s.g2;
    s.res = accept ? E.res : s.res;
    s.grow = accept ? grow : s.grow;
    s.t = reject ? 0.5f * s.t : s.t;
    s.trials = accept ? 0 : (reject ? trials : s.trials);
    s.newton += (accept & !conv & !maxed) ? 1 : 0;
    s.failed = s.failed | maxed | stuck;
    s.done = done;
    s.slow = s.slow | !ok;
}

// Forward projection of one matrix by Newton's method on the semi-dual.
//   a_nat : the 16 logits (natural units), row-major
//   P_out : the projected matrix (row-stochastic; doubly stochastic to tol)
//   returns the Newton iteration count (warm sweeps not counted), or
//   kNotConverged when max_iters, the noise floor or the line search stopped it.
//
// rec, with ROWS_IN_LDS: the same 16 logits in LDS, left unchanged until this
// returns (the start reads rows of it by a per-lane index).
template <bool ROWS_IN_LDS = false>
MHC_DEV uint32_t project_newton(const float* a_nat, float* P_out, const SolverOpts& o,
                                const float* rec = nullptr)
{
    NewtonLane s;
    newton_init<ROWS_IN_LDS, false>(s, a_nat, rec, o, nullptr);
    while (!s.done && !s.slow) newton_step<true, false>(s, o, nullptr);
    while (!s.done) newton_step<false, false>(s, o, nullptr);
    // P of the accepted point (the same arithmetic as when it was accepted)
    Eval E;
    evaluate(s.a, s.k, s.kfast, s.g0, s.g1, s.g2, E);
#pragma unroll
    for (int k = 0; k < 16; ++k) P_out[k] = E.P[k];
    return newton_code(s);
}

// The same projection for a lane whose logits sit in its own 16-float LDS
// slot `rec` (as the staged kernels hold them): the start reads rows of it,
// and P is left in it.  A lane writes its P there from the evaluation that
// converged, so only lanes that stop without converging (flag 255) evaluate
// again at their last accepted point; the others skip that evaluation.
MHC_DEV uint32_t project_newton_lds(const float* a_nat, float* rec, const SolverOpts& o)
{
    NewtonLane s;
    newton_init<true, true>(s, a_nat, rec, o, rec);
    while (!s.done && !s.slow) newton_step<true, true>(s, o, rec);
    while (!s.done) newton_step<false, true>(s, o, rec);
    if (!s.stored) {
        Eval E;
        evaluate(s.a, s.k, s.kfast, s.g0, s.g1, s.g2, E);
        sink_store(rec, E.P);
    }
    return newton_code(s);
}

// Forward projection of one matrix by Sinkhorn-Knopp sweeps (each sweep:
// divide rows by their sums, then columns by theirs; Deep Signal mHC article,
// section on Sinkhorn-Knopp).  With tol > 0 it stops once the row sums after
// a sweep are within tol of 1 (column sums are 1 to rounding right after the
// column step); with tol == 0 it runs exactly max_iters sweeps, the
// fixed-count practice the summary's section 1 describes.
MHC_DEV uint32_t project_sinkhorn(const float* a_nat, float* K, const SolverOpts& o)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float m = mhc_max(mhc_max(a_nat[4 * i], a_nat[4 * i + 1]),
                                mhc_max(a_nat[4 * i + 2], a_nat[4 * i + 3]));
#pragma unroll
        for (int j = 0; j < 4; ++j) K[4 * i + j] = mhc_exp2((a_nat[4 * i + j] - m) * kLog2e);
    }
    float r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (K[4 * i] + K[4 * i + 1]) + (K[4 * i + 2] + K[4 * i + 3]);
    int s = 0;
    bool done = false;
    while (s < o.max_iters) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float inv = mhc_rcp(r[i]);
#pragma unroll
            for (int j = 0; j < 4; ++j) K[4 * i + j] *= inv;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float inv = mhc_rcp((K[j] + K[4 + j]) + (K[8 + j] + K[12 + j]));
#pragma unroll
            for (int i = 0; i < 4; ++i) K[4 * i + j] *= inv;
        }
        ++s;
        float rr = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            r[i] = (K[4 * i] + K[4 * i + 1]) + (K[4 * i + 2] + K[4 * i + 3]);
            rr = mhc_max(rr, mhc_abs(r[i] - 1.f));
        }
        if (o.tol > 0.f && rr <= o.tol) {
            done = true;
            break;
        }
    }
    if (o.tol > 0.f && !done) return kNotConverged;
    return iters_code(s);
}

// Row-centred differences: out_j = sum_k p_k (x_j - x_k) for one row p of P
// (sum_k p_k = 1), i.e. x_j minus the p-weighted mean of the row, written as
// a weighted sum of differences so that no large terms cancel.
MHC_DEV void centred_row(const float* p, const float* x, float* out)
{
    const float x01 = x[0] - x[1], x02 = x[0] - x[2], x03 = x[0] - x[3];
    const float x12 = x[1] - x[2], x13 = x[1] - x[3], x23 = x[2] - x[3];
    out[0] = __builtin_fmaf(p[3], x03, __builtin_fmaf(p[2], x02, p[1] * x01));
    out[1] = __builtin_fmaf(p[3], x13, __builtin_fmaf(p[2], x12, -(p[0] * x01)));
    out[2] = __builtin_fmaf(p[3], x23, __builtin_fmaf(-p[1], x12, -(p[0] * x02)));
    out[3] = __builtin_fmaf(-p[2], x23, __builtin_fmaf(-p[1], x13, -(p[0] * x03)));
}

// Backward of the projection for one matrix (summary, section 2.2).
// Implicit differentiation of the scaling conditions gives
//   dA = P o (G - alpha 1^T - 1 beta^T),   (I - P^T P) beta = b - P^T a,
//   alpha = a - P beta,   a = (P o G) 1,   b = (P o G)^T 1,   beta3 = 0,
// and I - P^T P is the Newton Hessian at the solution (its Laplacian form,
// rebuilt from P).  With unit row sums the same quantities are
//   (b - P^T a)_j          = sum_i P_ij sum_k P_ik (G_ij - G_ik)
//   G_ij - alpha_i - beta_j = sum_k P_ik (H_ij - H_ik),   H = G - 1 beta^T,
// which are what is evaluated here: in fp32 the first forms cancel
// catastrophically when P is close to a permutation (b and P^T a agree to
// about the size of the true gradient), the second forms do not.
MHC_DEV void project_bwd(const float* P, const float* G, float* dA)
{
    float rhs0 = 0.f, rhs1 = 0.f, rhs2 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float gc[4];
        centred_row(P + 4 * i, G + 4 * i, gc);
        rhs0 = __builtin_fmaf(P[4 * i + 0], gc[0], rhs0);
        rhs1 = __builtin_fmaf(P[4 * i + 1], gc[1], rhs1);
        rhs2 = __builtin_fmaf(P[4 * i + 2], gc[2], rhs2);
    }
    const Weights w = laplacian_weights(P);
    const float lam = ridge(w);
    float be0, be1, be2;
    laplacian_solve(w.w01, w.w02, w.w03, w.w12, w.w13, w.w23, lam, rhs0, rhs1, rhs2,
                    be0, be1, be2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float h[4] = {G[4 * i + 0] - be0, G[4 * i + 1] - be1, G[4 * i + 2] - be2,
                            G[4 * i + 3]};
        float hc[4];
        centred_row(P + 4 * i, h, hc);
#pragma unroll
        for (int j = 0; j < 4; ++j) dA[4 * i + j] = P[4 * i + j] * hc[j];
    }
}

// The same backward with one ROW per lane: the 4 lanes of a quad hold the 4
// rows of one matrix (p, g = row i of P and G), column sums over rows are
// quad DPP reductions, and the 3x3 solve is repeated in the 4 lanes.  Returns
// row i of dA.  All four lanes of a quad must be active.
MHC_DEV void project_bwd_row(const float* p, const float* g, float* da)
{
    float gc[4];
    centred_row(p, g, gc);
    const float rhs0 = mhc_quad_sum(p[0] * gc[0]);
    const float rhs1 = mhc_quad_sum(p[1] * gc[1]);
    const float rhs2 = mhc_quad_sum(p[2] * gc[2]);
    Weights w;
    w.w01 = mhc_quad_sum(p[0] * p[1]);
    w.w02 = mhc_quad_sum(p[0] * p[2]);
    w.w03 = mhc_quad_sum(p[0] * p[3]);
    w.w12 = mhc_quad_sum(p[1] * p[2]);
    w.w13 = mhc_quad_sum(p[1] * p[3]);
    w.w23 = mhc_quad_sum(p[2] * p[3]);
    const float lam = ridge(w);
    float be0, be1, be2;
    laplacian_solve(w.w01, w.w02, w.w03, w.w12, w.w13, w.w23, lam, rhs0, rhs1, rhs2, be0, be1,
                    be2);
    const float h[4] = {g[0] - be0, g[1] - be1, g[2] - be2, g[3]};
    float hc[4];
    centred_row(p, h, hc);
#pragma unroll
    for (int j = 0; j < 4; ++j) da[j] = p[j] * hc[j];
}

}  // namespace mhc
