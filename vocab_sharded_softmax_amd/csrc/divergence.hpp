// divergence.hpp -- per-element divergence terms and the per-row finish shared by the
// two-pass and the fused JSD forwards, so both do identical arithmetic.
//
// [JSD-PR] DeepSpeed PR #8958 "[VocabTP] Add vocabulary-parallel generalized JSD with
// Triton kernels", sections Motivation and Changes: the generalized JSD as two
// KL-to-mixture expectations reduced together; beta = 0 / 1 as forward / reverse KL.
//
// Base-2 row algebra.  With u = x*ks - c (ks = log2 e / T, c = fl32(m*ks)), e = 2^u,
// Z = sum e:
//   M = beta p_t + (1-beta) p_s = (beta e_t + gamma e_s) / Z_t,  gamma = (1-beta) Z_t / Z_s
//   L = log2(beta e_t + gamma e_s),  r = log2(Z_s / Z_t)
//   log2(p_t / M) = u_t - L,  log2(p_s / M) = (u_s - L) - r
//   KT / ln2 = (1/Z_t) sum e_t (u_t - L),  KS / ln2 = (1/Z_s) sum e_s ((u_s - L) - r)
// so the per-element work touches only O(1)-sized quantities, never log Z; u - L and
// (u_s - L) - r are differences of nearby numbers and come out (nearly) exact.
// For the endpoints: log2(p_t / p_s) = (u_t - u_s) + r and log2(p_s / p_t) = (u_s - u_t) - r.
#pragma once

#include "device.hpp"

namespace vjsd {

enum Mode { INTERIOR = 0, FWD_KL = 1, REV_KL = 2 };

// Row constants of the divergence pass and one element's contribution.
template <int MODE>
struct DivTerm {
    float cs, ct, bf, gam, rf;
    float ks = L2E;  // log2 e / temperature

    // adds the element (xs, xt) to the running sums; F tracks max(u_t - u_s) (forward
    // KL) or max(u_s - u_t) (reverse KL) over raw values: +inf flags target mass on a
    // masked token
    __device__ __forceinline__ void add(float xs, float xt, float &At, float &As,
                                        float &F) const {
        const float usr = fmaf(xs, ks, -cs);
        const float utr = fmaf(xt, ks, -ct);
        const float us = fmaxf(usr, U_FLOOR), ut = fmaxf(utr, U_FLOOR);
        if constexpr (MODE == INTERIOR) {
            const float es = ex2(us), et = ex2(ut);
            const float L = lg2(fmaf(bf, et, fmaf(gam, es, W_FLOOR)));
            At = fmaf(et, ut - L, At);
            As = fmaf(es, (us - L) - rf, As);
        } else if constexpr (MODE == FWD_KL) {
            F = fmaxf(F, utr - usr);
            At = fmaf(ex2(ut), (ut - us) + rf, At);
        } else {
            F = fmaxf(F, usr - utr);
            As = fmaf(ex2(us), (us - ut) - rf, As);
        }
    }
};

// ---- the interior divergence, 0 < beta < 1 -------------------------------------------
//
// With u = x ks - c (c the statistics' reference point of that side) and e = 2^u, the
// mixture scaled by Z_t is M Z_t = beta e_t + (1 - beta) (Z_t / Z_s) e_s.  The ratio
// Z_t / Z_s goes into the student's exponent reference: v_s = x_s ks - c'_s with
// c'_s = fl32(c_s + r), r = log2(Z_s / Z_t), so f_s = 2^v_s = 2^(c_s - c'_s) e_s, and
//   delta = (c_s - c'_s) + r          (the rounding of c'_s: at most half its ulp)
//   W = beta e_t + k_s f_s = M Z_t,   k_s = fl32((1 - beta) 2^-delta),   L = log2 W
//   u_t - L = log2(p_t / M),          v_s - L = log2(p_s / M) + delta
//   KL(p_t || M) / ln 2 = (1 / Z_t) sum e_t (u_t - L)
//   KL(p_s || M) / ln 2 = (1 / (2^delta Z_t)) sum f_s (v_s - L) - delta
// (2^(c_s - c'_s) Z_s = 2^delta Z_t).  Both log-ratios come out of one subtraction of
// nearby numbers, free of any row offset.  Per element pair: two FMAs for the
// exponents, two exp2, a multiply and an FMA for the mixture, one log2, two
// subtractions and two FMAs into the sums.  SAFE adds what a row with masked (-inf)
// tokens, or with logits so spread that both exponentials of a pair underflow, needs: u
// and v clamped at U_FLOOR (so 0 * -inf never forms) and W_FLOOR inside the logarithm
// (so log2 never sees 0).  A row takes the plain form when its statistics sweep found
// every logit of both sides within FAST_RANGE (base 2) of the row's maximum: then
// e_t >= 2^-FAST_RANGE and W > 0, and every term is finite.
constexpr float FAST_RANGE = 96.0f;

template <bool SAFE>
struct MixTerm {
    float ks = L2E;  // log2 e / temperature
    float ct, cs, bt, ksc;  // references (c_t, c'_s) and mixture weights (beta, k_s)

    __device__ __forceinline__ void add(float xs, float xt, float &at, float &as) const {
        float ut = fmaf(xt, ks, -ct);
        float vs = fmaf(xs, ks, -cs);
        if constexpr (SAFE) {
            ut = fmaxf(ut, U_FLOOR);
            vs = fmaxf(vs, U_FLOOR);
        }
        const float et = ex2(ut), fs = ex2(vs);
        const float L = lg2(fmaf(bt, et, SAFE ? fmaf(ksc, fs, W_FLOOR) : ksc * fs));
        at = fmaf(et, ut - L, at);
        as = fmaf(fs, vs - L, as);
    }
};

// Row constants of the interior divergence, from the row's statistics: reference
// points and sums of 2^u relative to them (both sides defined: zs, zt > 0).
struct MixRow {
    float ct, cs, ksc;   // c_t, c'_s, k_s
    double izt, izs;     // 1 / Z_t and 1 / (2^delta Z_t)
    double delta;
};

__device__ __forceinline__ MixRow mix_row(double beta, float cs, double zs, float ct,
                                          double zt) {
    MixRow k;
    const double r = log2(zs / zt);
    k.ct = ct;
    k.cs = (float)((double)cs + r);
    k.delta = ((double)cs - (double)k.cs) + r;
    const double e = exp2(k.delta);
    k.ksc = (float)((1.0 - beta) / e);
    k.izt = 1.0 / zt;
    k.izs = 1.0 / (e * zt);
    return k;
}

// KL(p_t || M) / ln 2 and KL(p_s || M) / ln 2 from the row's two sums.
__device__ __forceinline__ void mix_finish(const MixRow &k, double at, double as, double &kt2,
                                           double &ks2) {
    kt2 = at * k.izt;
    ks2 = as * k.izs - k.delta;
}

// Sweep op of the interior divergence: four independent accumulators per side.
template <bool SAFE>
struct OpMix : MixTerm<SAFE> {
    float at[4] = {0, 0, 0, 0}, as[4] = {0, 0, 0, 0};

    __device__ __forceinline__ void set(const MixRow &k, float beta, float ks) {
        this->ks = ks;
        this->ct = k.ct;
        this->cs = k.cs;
        this->bt = beta;
        this->ksc = k.ksc;
    }
    template <int NV, int W>
    __device__ __forceinline__ void run(const float (&x)[NV][W], const float (&y)[NV][W],
                                        const int64_t (&)[NV]) {
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int i = 0; i < W; ++i) this->add(x[j][i], y[j][i], at[j], as[j]);
    }
    __device__ __forceinline__ float sum_t() const { return (at[0] + at[1]) + (at[2] + at[3]); }
    __device__ __forceinline__ float sum_s() const { return (as[0] + as[1]) + (as[2] + as[3]); }
};

// Sweep op of the two-pass divergence kernel: four independent accumulators.
template <int MODE>
struct OpDiv : DivTerm<MODE> {
    float At[4] = {0, 0, 0, 0}, As[4] = {0, 0, 0, 0};
    float F = NINF;

    template <int NV, int W>
    __device__ __forceinline__ void run(const float (&x)[NV][W], const float (&y)[NV][W],
                                        const int64_t (&)[NV]) {
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int i = 0; i < W; ++i) this->add(x[j][i], y[j][i], At[j], As[j], F);
    }
};

// Register op of the fused forward: one accumulator per side.
template <int MODE>
struct OpDivRegs : DivTerm<MODE> {
    float At = 0.0f, As = 0.0f, F = NINF;

    template <int V>
    __device__ __forceinline__ void add(const float (&x)[V], const float (&y)[V]) {
#pragma unroll
        for (int i = 0; i < V; ++i) DivTerm<MODE>::add(x[i], y[i], At, As, F);
    }
};

// Final per-token values from the part-summed partials (base 2, fp64).  The loss is
// multiplied by lscale (T^2 for a temperature-scaled loss, else 1); kl is not.
__device__ __forceinline__ void finalize_row(int mode, double beta, bool undefined, double pt,
                                             double ps, float F, float *kl, float *loss,
                                             float lscale = 1.0f) {
    double KT, KS, l;
    if (undefined) {
        KT = KS = l = __builtin_nan("");
    } else if (mode == INTERIOR) {
        KT = pt * LN2_D;
        KS = ps * LN2_D;
        l = beta * KT + (1.0 - beta) * KS;
    } else if (mode == FWD_KL) {
        KT = F == __builtin_huge_valf() ? __builtin_inf() : pt * LN2_D;
        KS = 0.0;
        l = KT;
    } else {
        KS = F == __builtin_huge_valf() ? __builtin_inf() : ps * LN2_D;
        KT = 0.0;
        l = KS;
    }
    kl[0] = (float)KT;
    kl[1] = (float)KS;
    *loss = (float)(l * (double)lscale);
}

// A row the caller's mask drops: nothing evaluated, loss and KL pair 0.
__device__ __forceinline__ void masked_row(float *kl, float *loss) {
    kl[0] = 0.0f;
    kl[1] = 0.0f;
    *loss = 0.0f;
}
// The same from a one-pass forward, which also owns the row's statistics: they read
// as a row with no distribution, so a backward gives it exactly zero gradients.
__device__ __forceinline__ void dropped_row(double *st, float *kl, float *loss) {
    if (threadIdx.x == 0) {
        st[0] = st[1] = st[2] = st[3] = -__builtin_inf();
        masked_row(kl, loss);
    }
}

}  // namespace vjsd
