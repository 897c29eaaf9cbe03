// jsd.hip -- input passes 2 and 3 of the generalized JSD and of its KL endpoints.
//
// [JSD-PR] DeepSpeed PR #8958 "[VocabTP] Add vocabulary-parallel generalized JSD with
// Triton kernels": section Motivation (the interior 0 < beta < 1 generalized JSD of
// GKD-style distillation), section Changes (global normalisation reused, the two
// KL-to-mixture expectations reduced together, probabilities recomputed in registers
// in the backward, gradients to both inputs or one, beta = 0 / 1 as explicit forward /
// reverse KL branches), section Scope and limitations (statistics and divergence are
// two input passes).  [OPS-PR] DeepSpeed PR #8791 "Add vocabulary-parallel logprobs,
// entropy and KL ops", section How (closed-form local backward; -inf tokens add
// nothing) and section Tests (KL is +inf when target mass meets a masked token).
//
// Base-2 row algebra.  With u = x*L2E - c (c = fl32(m*L2E)), e = 2^u, Z = sum e:
//   M = beta p_t + (1-beta) p_s = (beta e_t + gamma e_s) / Z_t,  gamma = (1-beta) Z_t / Z_s
//   L = log2(beta e_t + gamma e_s),  r = log2(Z_s / Z_t)
//   log2(p_t / M) = u_t - L,  log2(p_s / M) = u_s - L - r
//   KT / ln2 = (1/Z_t) sum e_t (u_t - L),  KS / ln2 = (1/Z_s) sum e_s ((u_s - L) - r)
// so the per-element work touches only O(1)-sized quantities, never log Z; u - L and
// (u_s - L) - r are differences of nearby numbers and come out (nearly) exact.
#include "backward.hpp"
#include "divergence.hpp"
#include <type_traits>

#include "kernels.hpp"
#include "sweep.hpp"

namespace vjsd {

namespace {

template <class D, int MODE>
__global__ __launch_bounds__(BLOCK) void k_div(RowView sv, RowView tv, int64_t w,
                                               const double *__restrict__ stats, double beta,
                                               float *__restrict__ part_k, float *__restrict__ kl,
                                               float *__restrict__ loss, RowOpts o) {
    using T = typename D::T;
    __shared__ float red[3 * NWAVE];
    const int64_t r = blockIdx.x;
    const RowConst k = row_const(stats, r, o.ks);
    // interior: (KL(p_t||M), KL(p_s||M)) / ln 2 of this shard before the row's offset
    // (mix_finish); endpoints: base-2 partial KL sums scaled by 1 / Z
    double pt = 0.0, ps = 0.0;
    float F = NINF;
    MixRow mx{};
    // a dropped row has statistics (-inf, ...) and so counts as undefined here
    if (!k.undefined) {
        if constexpr (MODE == INTERIOR) mx = mix_row(beta, k.cs, k.Zs, k.ct, k.Zt);
    }
    if (!k.undefined && w > 0) {
        const T *s = row_ptr<T>(sv, r), *t = row_ptr<T>(tv, r);
        float v[2];
        if constexpr (MODE == INTERIOR) {
            // no row minimum in this pass: masked tokens admitted throughout
            OpMix<true> op;
            op.set(mx, (float)beta, o.ks);
            sweep<D, 4, true, BLOCK, true>(s, t, w, head_len<T>(w, s, t), op);
            v[0] = op.sum_t();
            v[1] = op.sum_s();
        } else {
            OpDiv<MODE> op;
            op.ks = o.ks;
            op.cs = k.cs;
            op.ct = k.ct;
            op.bf = (float)beta;
            op.gam = (float)((1.0 - beta) * k.Zt / k.Zs);
            op.rf = (float)k.r;
            sweep<D, 4, true, BLOCK, true>(s, t, w, head_len<T>(w, s, t), op);
            v[0] = (op.At[0] + op.At[1]) + (op.At[2] + op.At[3]);
            v[1] = (op.As[0] + op.As[1]) + (op.As[2] + op.As[3]);
            F = op.F;
        }
        block_sum<2>(v, red);
        const float f = wave_max(F);
        if ((threadIdx.x & 63) == 0) red[2 * NWAVE + (threadIdx.x >> 6)] = f;
        __syncthreads();
        if (threadIdx.x == 0) {
            if constexpr (MODE == INTERIOR) {
                pt = v[0] * mx.izt;
                ps = v[1] * mx.izs;
            } else {
                pt = v[0] * k.izt;
                ps = v[1] * k.izs;
            }
            for (int q = 0; q < NWAVE; ++q) F = fmaxf(F, red[2 * NWAVE + q]);
        }
    }
    if (threadIdx.x == 0) {
        if (loss) {
            if (row_dropped(o, r)) {
                masked_row(kl + 2 * r, loss + r);
            } else {
                if (MODE == INTERIOR && !k.undefined) ps -= mx.delta;
                finalize_row(MODE, beta, k.undefined, pt, ps, F, kl + 2 * r, loss + r, o.lscale);
            }
        } else {
            float *o = part_k + r * PART_STRIDE;
            o[0] = (float)pt;
            o[1] = (float)ps;
            o[2] = F;
        }
    }
}

__global__ void k_div_finalize(int mode, const float *__restrict__ part, int S, int64_t N,
                               const double *__restrict__ stats, double beta,
                               float *__restrict__ kl, float *__restrict__ loss, RowOpts o) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= N) return;
    if (row_dropped(o, r)) {
        masked_row(kl + 2 * r, loss + r);
        return;
    }
    const RowConst k = row_const(stats, r, o.ks);
    double pt = 0.0, ps = 0.0;
    float F = NINF;
    for (int q = 0; q < S; ++q) {
        const float *p = part + ((int64_t)q * N + r) * PART_STRIDE;
        pt += p[0];
        ps += p[1];
        F = fmaxf(F, p[2]);
    }
    if (mode == INTERIOR && !k.undefined) ps -= mix_row(beta, k.cs, k.Zs, k.ct, k.Zt).delta;
    finalize_row(mode, beta, k.undefined, pt, ps, F, kl + 2 * r, loss + r, o.lscale);
}

// ---- backward ---------------------------------------------------------------------
//
// The constants and the element op are those of backward.hpp, which the one-launch
// forward and backward (fused.hip) shares.

// Per-row constants of the backward, computed once per call from the fp64 statistics
// (bwd_constants: rowc[r*ROWC + i] = cs, ct, beta, gamma, Cs, Ct, Hs, Ht, Gs, Gt for
// i = 0..9, the exponent scale in slot ROWC_KS and the zero-gradient flag, no
// distribution or a row the mask drops, in slot ROWC_UNDEFINED).
__global__ void k_bwd_prep(int mode, int64_t N, const double *__restrict__ stats,
                           const float *__restrict__ kl, double beta,
                           const float *__restrict__ grad, float *__restrict__ rowc,
                           GradOpts go) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= N) return;
    const RowConst k = row_const(stats, r, go.ks);
    const bool dropped = go.mask != nullptr && go.mask[r] == 0;
    bwd_constants(mode, k, kl + 2 * r, beta, upstream_g(grad, go, r), go.ks,
                  k.undefined || dropped, rowc + r * ROWC);
}

// One workgroup of LANES lanes per row chunk of up to cw columns (chunk_span), one
// 16-byte vector per lane; the chunks of a row are consecutive workgroups, so the whole
// grid streams through memory in order.  Measured on MI355X: one wave per chunk when
// both gradients are written (two waves: 1.68-1.69 against 1.63-1.69 ms at full
// vocabulary), two waves when one is (0.131-0.133 against 0.142-0.145 ms at 16032
// columns; even at full vocabulary).
template <int WS, int WT>
constexpr int bwd_lanes() { return WS && WT ? GRAD_BLOCK : 2 * GRAD_BLOCK; }

// Chunk q of row r of one shard (srow: the row of its first input).
template <class D, int MODE, bool WS, bool WT, class DG, int LANES>
__device__ __forceinline__ void bwd_chunk(const typename D::T *srow, const RowView &tv,
                                          const RowMView &gsv, const RowMView &gtv, int64_t w,
                                          int64_t cw, int64_t q, int64_t r,
                                          const float *__restrict__ rowc) {
    using T = typename D::T;
    using TG = typename DG::T;
    int64_t c0, n;
    chunk_span<true>(srow, w, cw, q, c0, n);
    if (n <= 0) return;
    const float *k = rowc + r * ROWC;
    TG *gs = WS ? row_ptr<TG>(gsv, r) + c0 : nullptr;
    TG *gt = WT ? row_ptr<TG>(gtv, r) + c0 : nullptr;
    if (k[ROWC_UNDEFINED] != 0.0f) {  // no distribution, or dropped: exactly zero gradient
        if (WS) zero_span<DG, LANES>(gs, n);
        if (WT) zero_span<DG, LANES>(gt, n);
        return;
    }
    const T *s = srow + c0, *t = row_ptr<T>(tv, r) + c0;
    OpBwd<D, MODE, WS, WT, DG> op;
    op.gs = gs;
    op.gt = gt;
    op.set(k);
    // the vector path needs every view of the chunk at the same offset inside 16 bytes;
    // inputs and gradients are touched once, so loads and stores stream
    // (a bf16 gradient of fp32 input sits at the same element offsets, 8-byte aligned
    // where the input is 16-byte aligned: the inputs alone fix the head)
    const int64_t h = std::is_same<D, DG>::value ? head_len<T>(n, s, t, gs, gt)
                                                 : head_len<T>(n, s, t);
    sweep<D, 1, true, LANES, true>(s, t, n, h, op);
}

template <class D, int MODE, bool WS, bool WT, class DG = D, int LANES = bwd_lanes<WS, WT>()>
__global__ __launch_bounds__(LANES) void k_bwd(RowView sv, RowView tv, RowMView gsv,
                                                    RowMView gtv, int64_t w, int64_t cw,
                                                    int64_t nchunk, const float *__restrict__ rowc,
                                                    int64_t items) {
    const int64_t b = xcd_item(blockIdx.x, items);
    if (b >= items) return;
    const int64_t r = b / nchunk;
    bwd_chunk<D, MODE, WS, WT, DG, LANES>(row_ptr<typename D::T>(sv, r), tv, gsv, gtv, w, cw,
                                          b - r * nchunk, r, rowc);
}

// Up to FUSED_SHARDS shards of a row in one launch: a row's chunks run through its
// shards in order (c0[k] is shard k's first chunk within the row), so column-slice
// shards of one tensor stream through memory as one row does.  Measured on MI355X at
// 4096 x 128256 fp32 in shards 60000/0/40000/28256: one launch per shard took 1.50 ms
// of kernel time, the same data as one shard 1.32 ms.
struct ShardGrads {
    int S;
    int64_t w[FUSED_SHARDS];
    int64_t c0[FUSED_SHARDS + 1];
    RowView s[FUSED_SHARDS], t[FUSED_SHARDS];
    RowMView gs[FUSED_SHARDS], gt[FUSED_SHARDS];
};

template <class D, int MODE, bool WS, bool WT, int LANES = bwd_lanes<WS, WT>()>
__global__ __launch_bounds__(LANES) void k_bwd_shards(ShardGrads g, int64_t cw, int64_t nchunk,
                                                       const float *__restrict__ rowc,
                                                       int64_t items) {
    const int64_t b = xcd_item(blockIdx.x, items);
    if (b >= items) return;
    const int64_t r = b / nchunk;
    const int64_t j = b - r * nchunk;
    int k = 0;
    while (k + 1 < g.S && j >= g.c0[k + 1]) ++k;
    bwd_chunk<D, MODE, WS, WT, D, LANES>(row_ptr<typename D::T>(g.s[k], r), g.t[k], g.gs[k],
                                         g.gt[k], g.w[k], cw, j - g.c0[k], r, rowc);
}

template <class D, int MODE>
hipError_t div_dt(const Shard &sh, int64_t N, const double *stats, double beta, float *part_k,
                  float *kl, float *loss, hipStream_t st, const RowOpts &o) {
    hipLaunchKernelGGL((k_div<D, MODE>), dim3((unsigned)N), dim3(BLOCK), 0, st, sh.s, sh.t,
                       sh.width, stats, beta, part_k, kl, loss, o);
    return hipGetLastError();
}

template <class D>
hipError_t div_mode(int mode, const Shard &sh, int64_t N, const double *stats, double beta,
                    float *part_k, float *kl, float *loss, hipStream_t st, const RowOpts &o) {
    if (mode == INTERIOR) return div_dt<D, INTERIOR>(sh, N, stats, beta, part_k, kl, loss, st, o);
    if (mode == FWD_KL) return div_dt<D, FWD_KL>(sh, N, stats, beta, part_k, kl, loss, st, o);
    return div_dt<D, REV_KL>(sh, N, stats, beta, part_k, kl, loss, st, o);
}

template <class D, int MODE, bool WS, bool WT>
hipError_t bwd_k(const Shard &sh, int64_t N, const float *rowc, hipStream_t st) {
    constexpr int L = bwd_lanes<WS, WT>();
    const Chunks ch = grad_chunks<true, L>(N, sh.width, sizeof(typename D::T));
    if (ch.nchunk == 0) return hipSuccess;
    hipLaunchKernelGGL((k_bwd<D, MODE, WS, WT>), dim3((unsigned)(N * ch.nchunk)),
                       dim3(L), 0, st, sh.s, sh.t, sh.gs, sh.gt, sh.width, ch.cw,
                       ch.nchunk, rowc, N * ch.nchunk);
    return hipGetLastError();
}

template <int MODE>
hipError_t bwd_g16(const Shard &sh, int64_t N, const float *rowc, hipStream_t st) {
    constexpr int L = bwd_lanes<true, false>();
    const Chunks ch = grad_chunks<true, L>(N, sh.width, sizeof(float));
    if (ch.nchunk == 0) return hipSuccess;
    hipLaunchKernelGGL((k_bwd<F32, MODE, true, false, BF16>),
                       dim3((unsigned)(N * ch.nchunk)), dim3(L), 0, st, sh.s, sh.t, sh.gs,
                       sh.gt, sh.width, ch.cw, ch.nchunk, rowc, N * ch.nchunk);
    return hipGetLastError();
}

template <class D, int MODE>
hipError_t bwd_want(const Shard &sh, int64_t N, const float *rowc, hipStream_t st) {
    const bool ws = sh.gs.p != nullptr, wt = sh.gt.p != nullptr;
    if (ws && wt) return bwd_k<D, MODE, true, true>(sh, N, rowc, st);
    if (ws) return bwd_k<D, MODE, true, false>(sh, N, rowc, st);
    if (wt) return bwd_k<D, MODE, false, true>(sh, N, rowc, st);
    return hipSuccess;
}

template <class D>
hipError_t bwd_mode(int mode, const Shard &sh, int64_t N, const float *rowc, hipStream_t st) {
    if (mode == INTERIOR) return bwd_want<D, INTERIOR>(sh, N, rowc, st);
    if (mode == FWD_KL) return bwd_want<D, FWD_KL>(sh, N, rowc, st);
    return bwd_want<D, REV_KL>(sh, N, rowc, st);
}

template <class D, int MODE, bool WS, bool WT>
hipError_t bwd_shards_k(const Shard *sh, int S, int64_t N, const float *rowc, hipStream_t st) {
    constexpr int L = bwd_lanes<WS, WT>();
    const int64_t vec = 16 / (int64_t)sizeof(typename D::T);
    auto count = [](int64_t w, int64_t c) { return w > 0 ? (w + 2 * c - 2) / c : (int64_t)0; };
    int64_t cw = L * vec, total = 0;
    for (;;) {  // the chunk width of grad_chunks, over all shards' chunks of a row
        total = 0;
        for (int k = 0; k < S; ++k) total += count(sh[k].width, cw);
        if (N * total <= 0x7fffffffLL) break;
        cw *= 2;
    }
    if (total == 0) return hipSuccess;
    ShardGrads g{};
    g.S = S;
    g.c0[0] = 0;
    for (int k = 0; k < S; ++k) {
        g.w[k] = sh[k].width;
        g.c0[k + 1] = g.c0[k] + count(sh[k].width, cw);
        g.s[k] = sh[k].s;
        g.t[k] = sh[k].t;
        g.gs[k] = sh[k].gs;
        g.gt[k] = sh[k].gt;
    }
    hipLaunchKernelGGL((k_bwd_shards<D, MODE, WS, WT>), dim3((unsigned)(N * total)),
                       dim3(L), 0, st, g, cw, total, rowc, N * total);
    return hipGetLastError();
}

template <class D, int MODE>
hipError_t bwd_shards_want(const Shard *sh, int S, int64_t N, const float *rowc, hipStream_t st,
                           bool ws, bool wt) {
    if (ws && wt) return bwd_shards_k<D, MODE, true, true>(sh, S, N, rowc, st);
    if (ws) return bwd_shards_k<D, MODE, true, false>(sh, S, N, rowc, st);
    if (wt) return bwd_shards_k<D, MODE, false, true>(sh, S, N, rowc, st);
    return hipSuccess;
}

template <class D>
hipError_t bwd_shards_mode(int mode, const Shard *sh, int S, int64_t N, const float *rowc,
                           hipStream_t st, bool ws, bool wt) {
    if (mode == INTERIOR) return bwd_shards_want<D, INTERIOR>(sh, S, N, rowc, st, ws, wt);
    if (mode == FWD_KL) return bwd_shards_want<D, FWD_KL>(sh, S, N, rowc, st, ws, wt);
    return bwd_shards_want<D, REV_KL>(sh, S, N, rowc, st, ws, wt);
}

}  // namespace

hipError_t launch_div(int dtype, int mode, const Shard &sh, int64_t N, const double *stats,
                      double beta, float *part_k, float *kl, float *loss, hipStream_t st,
                      const RowOpts &o) {
    switch (dtype) {
        case 0: return div_mode<F32>(mode, sh, N, stats, beta, part_k, kl, loss, st, o);
        case 1: return div_mode<F16>(mode, sh, N, stats, beta, part_k, kl, loss, st, o);
        default: return div_mode<BF16>(mode, sh, N, stats, beta, part_k, kl, loss, st, o);
    }
}

hipError_t launch_div_finalize(int mode, const float *part, int S, int64_t N,
                               const double *stats, double beta, float *kl, float *loss,
                               hipStream_t st, const RowOpts &o) {
    const int threads = 256;
    hipLaunchKernelGGL(k_div_finalize, dim3((unsigned)((N + threads - 1) / threads)),
                       dim3(threads), 0, st, mode, part, S, N, stats, beta, kl, loss, o);
    return hipGetLastError();
}

hipError_t launch_bwd_prep(int mode, int64_t N, const double *stats, const float *kl,
                           double beta, const float *grad, float *rowc, hipStream_t st,
                           const GradOpts &g) {
    hipLaunchKernelGGL(k_bwd_prep, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, st, mode, N,
                       stats, kl, beta, grad, rowc, g);
    return hipGetLastError();
}

hipError_t launch_bwd_f32_to_bf16(int mode, const Shard &sh, int64_t N, const float *rowc,
                                  hipStream_t st) {
    if (mode == INTERIOR) return bwd_g16<INTERIOR>(sh, N, rowc, st);
    if (mode == FWD_KL) return bwd_g16<FWD_KL>(sh, N, rowc, st);
    return bwd_g16<REV_KL>(sh, N, rowc, st);
}

hipError_t launch_bwd(int dtype, int mode, const Shard &sh, int64_t N, const float *rowc,
                      hipStream_t st) {
    switch (dtype) {
        case 0: return bwd_mode<F32>(mode, sh, N, rowc, st);
        case 1: return bwd_mode<F16>(mode, sh, N, rowc, st);
        default: return bwd_mode<BF16>(mode, sh, N, rowc, st);
    }
}

hipError_t launch_bwd_shards(int dtype, int mode, const Shard *sh, int S, int64_t N,
                             const float *rowc, hipStream_t st) {
    // one launch when every non-empty shard asks for the same gradients, else one per shard
    bool one = S >= 2 && S <= FUSED_SHARDS, seen = false, ws = false, wt = false;
    for (int k = 0; one && k < S; ++k) {
        if (sh[k].width == 0) continue;
        const bool a = sh[k].gs.p != nullptr, b = sh[k].gt.p != nullptr;
        if (seen && (a != ws || b != wt)) one = false;
        ws = a;
        wt = b;
        seen = true;
    }
    if (!one) {
        for (int k = 0; k < S; ++k) {
            const hipError_t e = launch_bwd(dtype, mode, sh[k], N, rowc, st);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    switch (dtype) {
        case 0: return bwd_shards_mode<F32>(mode, sh, S, N, rowc, st, ws, wt);
        case 1: return bwd_shards_mode<F16>(mode, sh, S, N, rowc, st, ws, wt);
        default: return bwd_shards_mode<BF16>(mode, sh, S, N, rowc, st, ws, wt);
    }
}

}  // namespace vjsd
