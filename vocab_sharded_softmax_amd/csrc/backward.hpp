// backward.hpp -- the closed-form gradient of the JSD and of its KL endpoints, shared by
// the streaming backward and the fused forward-and-backward kernel so that both do
// identical arithmetic: per-row constants from the forward's statistics and KL pair,
// then one element's two gradients.
//
// [JSD-PR] DeepSpeed PR #8958 "[VocabTP] Add vocabulary-parallel generalized JSD with
// Triton kernels", section Changes: the backward recomputes the probabilities from the
// saved global statistics and forms the gradients to both inputs (or one) in closed
// form; beta = 0 / 1 are the forward / reverse KL branches.
//
// With u = x ks - c, e = 2^u, L = log2(beta e_t + gamma e_s), r = log2(Z_s / Z_t) and the
// forward's per-token KL(p_t || M) = KT, KL(p_s || M) = KS (nats), the interior loss
// l = beta KT + (1 - beta) KS has, for an upstream gradient g,
//   dl/dx_s = g (1 - beta) p_s (log p_s - log M - KS)
//           = g (1 - beta) ln2 / Z_s * e_s * ((u_s - L) - (r + KS / ln2))
//   dl/dx_t = g beta p_t (log p_t - log M - KT)
//           = g beta ln2 / Z_t * e_t * ((u_t - L) - KT / ln2)
// (the terms from M's own dependence on the logits drop out, since
// beta p_t / M + (1 - beta) p_s / M = 1 at every token).  The endpoints are
// the plain KL gradients: forward KL(p_t || p_s) gives g (p_s - p_t) to the student and
// g p_t (log p_t - log p_s - KT) to the teacher; reverse KL the mirror image.
#pragma once

#include <type_traits>

#include "device.hpp"
#include "divergence.hpp"

namespace vjsd {

// Per-row constants of a two-input pass, rebuilt from the fp64 statistics.
struct RowConst {
    bool undefined;
    float cs, ct;    // reference points
    float izs, izt;  // 1 / Z
    double Zs, Zt;
    double r;        // log2(Z_s / Z_t)
};

__device__ __forceinline__ RowConst row_const(const double *__restrict__ stats, int64_t r,
                                              float ks = L2E) {
    RowConst k;
    const double *st = stats + r * 4;
    const float ms = (float)st[0], mt = (float)st[2];
    k.undefined = (ms == NINF) || (mt == NINF);
    k.cs = refc(ms, ks);
    k.ct = refc(mt, ks);
    k.Zs = k.undefined ? 1.0 : z_from_stats(ms, st[1], ks);
    k.Zt = k.undefined ? 1.0 : z_from_stats(mt, st[3], ks);
    k.izs = (float)(1.0 / k.Zs);
    k.izt = (float)(1.0 / k.Zt);
    k.r = log2(k.Zs / k.Zt);
    return k;
}

// Row r's upstream gradient scale under GradOpts (grad NULL: a unit gradient).
__device__ __forceinline__ double upstream_g(const float *grad, const GradOpts &go, int64_t r) {
    double g = grad == nullptr ? 1.0 : (go.scalar ? (double)grad[0] : (double)grad[r]);
    if (go.count) g /= fmax((double)*go.count, 1.0);
    return g * go.gmul;
}

// One row's backward constants o[0..ROWC): cs, ct, beta, gamma, Cs, Ct, Hs, Ht, Gs, Gt
// (slots 0..9), the exponent scale in slot ROWC_KS and, in slot ROWC_UNDEFINED, 1.0f
// when the row's gradients are exactly zero (`zero`: no distribution, or a dropped
// row).  g is the row's upstream gradient scale, klr its forward KL pair.
__device__ __forceinline__ void bwd_constants(int mode, const RowConst &k, const float *klr,
                                              double beta, double g, float ks, bool zero,
                                              float *o) {
    const double KT2 = (double)klr[0] * L2E_D, KS2 = (double)klr[1] * L2E_D;
    double Cs = 0.0, Ct = 0.0, Hs = 0.0, Ht = 0.0;
    if (mode == INTERIOR) {
        Cs = g * (1.0 - beta) * LN2_D / k.Zs;
        Ct = g * beta * LN2_D / k.Zt;
        Hs = k.r + KS2;
        Ht = KT2;
    } else if (mode == FWD_KL) {  // d/dt = g p_t (lp_t - lp_s - KT), lp2_t - lp2_s = u_t - u_s + r
        Ct = g * LN2_D / k.Zt;
        Ht = KT2 - k.r;
    } else {  // d/ds = g p_s (lp_s - lp_t - KS), lp2_s - lp2_t = u_s - u_t - r
        Cs = g * LN2_D / k.Zs;
        Hs = KS2 + k.r;
    }
    o[0] = k.cs;
    o[1] = k.ct;
    o[2] = (float)beta;
    o[3] = (float)((1.0 - beta) * k.Zt / k.Zs);
    o[4] = (float)Cs;
    o[5] = (float)Ct;
    o[6] = (float)Hs;
    o[7] = (float)Ht;
    o[8] = (float)(g / k.Zs);
    o[9] = (float)(g / k.Zt);
    o[ROWC_KS] = ks;
    o[ROWC_UNDEFINED] = zero ? 1.0f : 0.0f;
}

// The element op of the gradient sweeps: both gradients of NV vectors (or single
// elements) of W values.  DG: storage of the gradients (the input's, or bf16 for fp32
// input: the logit gradient the fused-linear products consume).  CLAMP = false drops the
// U_FLOOR clamps, for rows whose every logit lies within FAST_RANGE of its maximum:
// there u >= -FAST_RANGE > U_FLOOR, the clamps return u unchanged and the results are
// the same bit for bit.
template <class D, int MODE, bool WS, bool WT, class DG = D, bool CLAMP = true>
struct OpBwd {
    using T = typename D::T;
    using TG = typename DG::T;
    TG *gs, *gt;
    float ks;  // log2 e / temperature
    float cs, ct, bf, gam;
    float Cs, Ct;  // gradient scales
    float Hs, Ht;  // per-side offsets subtracted from the log-ratio
    float Gs, Gt;  // g / Z for the p_s - p_t terms of the endpoints

    // the constants of one row, as bwd_constants lays them out
    __device__ __forceinline__ void set(const float *k) {
        ks = k[ROWC_KS];
        cs = k[0];
        ct = k[1];
        bf = k[2];
        gam = k[3];
        Cs = k[4];
        Ct = k[5];
        Hs = k[6];
        Ht = k[7];
        Gs = k[8];
        Gt = k[9];
    }

    template <int NV, int W>
    __device__ __forceinline__ void run(const float (&x)[NV][W], const float (&y)[NV][W],
                                        const int64_t (&col)[NV]) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            float os[W], ot[W];
#pragma unroll
            for (int i = 0; i < W; ++i) {
                const float us = CLAMP ? fmaxf(fmaf(x[j][i], ks, -cs), U_FLOOR)
                                       : fmaf(x[j][i], ks, -cs);
                const float ut = CLAMP ? fmaxf(fmaf(y[j][i], ks, -ct), U_FLOOR)
                                       : fmaf(y[j][i], ks, -ct);
                const float es = ex2(us), et = ex2(ut);
                if constexpr (MODE == INTERIOR) {
                    const float L = lg2(fmaf(bf, et, fmaf(gam, es, W_FLOOR)));
                    os[i] = (Cs * es) * ((us - L) - Hs);
                    ot[i] = (Ct * et) * ((ut - L) - Ht);
                } else if constexpr (MODE == FWD_KL) {
                    os[i] = fmaf(Gs, es, -(Gt * et));
                    ot[i] = (Ct * et) * ((ut - us) - Ht);
                } else {
                    os[i] = (Cs * es) * ((us - ut) - Hs);
                    ot[i] = fmaf(Gt, et, -(Gs * es));
                }
            }
            if constexpr (W == D::VEC && std::is_same<D, DG>::value) {
                if (WS) store_vec<D, true>(gs + col[j], os);
                if (WT) store_vec<D, true>(gt + col[j], ot);
            } else if constexpr (W == D::VEC) {  // four fp32 values as 8 bytes of bf16
                if (WS) st_bf16x4(gs + col[j], os);
                if (WT) st_bf16x4(gt + col[j], ot);
            } else {
#pragma unroll
                for (int i = 0; i < W; ++i) {
                    if (WS) store1<DG>(gs + col[j] + i, os[i]);
                    if (WT) store1<DG>(gt + col[j] + i, ot[i]);
                }
            }
        }
    }
};

}  // namespace vjsd
