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
