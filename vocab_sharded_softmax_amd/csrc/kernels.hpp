// kernels.hpp -- host-side launchers of libvjsd's kernels (one call per shard or per
// row set).  Each returns the launch status; argument checking happens in api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"
#include "divergence.hpp"

namespace vjsd {

struct Shard {
    int64_t start, width;
    RowView s, t;
    RowMView gs, gt;
};

// pass 1: per-shard (max, sum-exp) of the inputs selected by `which` (1 s, 2 t, 3 both)
hipError_t launch_stats(int dtype, int which, const Shard &sh, int64_t N, float *part_k,
                        hipStream_t st, const RowOpts &o = RowOpts());
// cross-shard merge of pass-1 partials into stats[N][4]
hipError_t launch_merge(const float *part, int S, int64_t N, int which, double *stats,
                        hipStream_t st, float ks = L2E);
// pass 2 of the JSD (and its endpoint branches): per-shard divergence partials; with
// `kl`/`loss` non-null (single shard) the row is finalised in the same launch
hipError_t launch_div(int dtype, int mode, const Shard &sh, int64_t N, const double *stats,
                      double beta, float *part_k, float *kl, float *loss, hipStream_t st,
                      const RowOpts &o = RowOpts());
// shard-ordered sum of pass-2 partials into kl[N][2], loss[N]
hipError_t launch_div_finalize(int mode, const float *part, int S, int64_t N,
                               const double *stats, double beta, float *kl, float *loss,
                               hipStream_t st, const RowOpts &o = RowOpts());
// Interior JSD forward (0 < beta < 1) of a single shard in one launch: statistics,
// then divergence, one workgroup per row (held in registers when the row fits).
hipError_t launch_fwd_fused(int dtype, const Shard &sh, int64_t N, double beta, double *stats,
                            float *kl, float *loss, hipStream_t st, const RowOpts &o = RowOpts());
// Interior JSD forward and backward of a single shard in one launch: launch_fwd_fused's
// outputs, then the gradients into sh.gs / sh.gt (a NULL view is not written) for the
// upstream gradient grad under go, as launch_bwd_prep + launch_bwd compute them.
// hipErrorNotSupported (nothing launched) for register-held rows whose gradient views
// are not 16-byte aligned like the inputs.
hipError_t launch_fwd_bwd_fused(int dtype, const Shard &sh, int64_t N, double beta,
                                const float *grad, double *stats, float *kl, float *loss,
                                hipStream_t st, const RowOpts &o, const GradOpts &go);
// The same for fp32 rows and their student gradient stored in bf16 (sh.gs; sh.gt NULL),
// always the two-sweep kernel, with a unit upstream gradient under go: the fused-linear
// loss's logit block and its gradient G in one launch.  The gradient rows sit at the
// inputs' element offsets.
hipError_t launch_fwd_bwd_f32_bf16(const Shard &sh, int64_t N, double beta, double *stats,
                                   float *kl, float *loss, hipStream_t st, const RowOpts &o,
                                   const GradOpts &go);
// interior JSD forward of 2..FUSED_SHARDS shards in one launch (stats, merge, divergence)
constexpr int FUSED_SHARDS = 8;
struct ShardRows {
    int S;
    int64_t w[FUSED_SHARDS];
    RowView s[FUSED_SHARDS], t[FUSED_SHARDS];
};
hipError_t launch_fwd_shards(int dtype, const Shard *sh, int S, int64_t N, double beta,
                             double *stats, float *kl, float *loss, hipStream_t st,
                             const RowOpts &o = RowOpts());

// Row chunks of the streaming gradient kernels: cw columns per workgroup (GRAD_BLOCK
// vectors times a power of two, so a power of two), nchunk chunks per row, N * nchunk
// workgroups in all.  With ALIGNED, chunk boundaries sit at multiples of cw elements of
// the address space (chunk_span), not of the row start, so a row may need one chunk
// more than ceil(w / cw); a chunk past a row's end is empty.
struct Chunks {
    int64_t cw, nchunk;
};

// The dispatcher hands workgroups to the eight XCDs in turn (workgroup i to XCD i % 8).
// The streaming backwards renumber their work items so that each XCD takes runs of
// XCD_RUN consecutive row chunks: on MI355X the both-gradient backward at 8192 x 151936
// bf16 ran 1-2 % faster than with consecutive chunks on eight XCDs, the student-only
// one 6 %, and at 16032 columns 3 % (runs of 32 chunks lost 5 % at full width; runs
// of 1024 gained more there but lost 3 % at 16032 columns).  Only whole rounds of
// 8 * XCD_RUN items are renumbered; the items of a last partial round keep their
// order, so they spread over all eight XCDs (a small batch is all partial round).
constexpr int64_t XCD_RUN = 256;
__device__ __forceinline__ int64_t xcd_item(int64_t i, int64_t items) {
    constexpr int64_t R = 8 * XCD_RUN;
    if (i >= items / R * R) return i;
    const int64_t round = i / R, k = i - round * R;
    return round * R + (k & 7) * XCD_RUN + (k >> 3);
}
template <bool ALIGNED, int LANES = GRAD_BLOCK>
inline Chunks grad_chunks(int64_t N, int64_t w, int esize) {
    const int64_t vec = 16 / esize;
    int64_t cw = LANES * vec;
    auto count = [w](int64_t c) {
        return w <= 0 ? (int64_t)0 : ALIGNED ? (w + 2 * c - 2) / c : (w + c - 1) / c;
    };
    while (N * count(cw) > 0x7fffffffLL) cw *= 2;  // grid.x limit
    return {cw, count(cw)};
}

// pass 3: per-row constants of the backward (once per call), then the closed-form
// gradients of the JSD / KL for one shard
hipError_t launch_bwd_prep(int mode, int64_t N, const double *stats, const float *kl,
                           double beta, const float *grad, float *rowc, hipStream_t st,
                           const GradOpts &g = GradOpts());
hipError_t launch_bwd(int dtype, int mode, const Shard &sh, int64_t N, const float *rowc,
                      hipStream_t st);
// the same over all S shards of a call: one launch for 2..FUSED_SHARDS shards that ask
// for the same gradients, else launch_bwd per shard
hipError_t launch_bwd_shards(int dtype, int mode, const Shard *sh, int S, int64_t N,
                             const float *rowc, hipStream_t st);
// the same for fp32 logits, writing only the student gradient, in bf16 (nearest even);
// the gradient view must be 8-byte aligned wherever the input view is 16-byte aligned
hipError_t launch_bwd_f32_to_bf16(int mode, const Shard &sh, int64_t N, const float *rowc,
                                  hipStream_t st);

// single-pass KL forward: per-shard online partials, then the merge into stats/kl/loss
hipError_t launch_kl1(int dtype, int reverse, const Shard &sh, int64_t N, float *part_k,
                      hipStream_t st, const RowOpts &o = RowOpts());
hipError_t launch_kl1_merge(int reverse, const float *part, int S, int64_t N, double *stats,
                            float *kl, float *loss, hipStream_t st, const RowOpts &o = RowOpts());

// fixed-order masked reduction of per-row losses: out[0] = sum (mean: sum / max(count,
// 1)) over the rows `sel` keeps; *count = kept rows (rows may be null to count only)
hipError_t launch_reduce_rows(const float *rows, const RowOpts &sel, int64_t N, bool mean,
                              float *out, double *count, hipStream_t st);
// single-pass entropy forward and its backward
hipError_t launch_ent1(int dtype, const Shard &sh, int64_t N, float *part_k, hipStream_t st);
hipError_t launch_ent1_merge(const float *part, int S, int64_t N, double *stats, float *ent,
                             hipStream_t st);
hipError_t launch_ent_bwd_prep(int64_t N, const double *stats, const float *ent,
                               const float *grad, float *rowc, hipStream_t st);
hipError_t launch_ent_bwd(int dtype, const Shard &sh, int64_t N, const float *rowc,
                          hipStream_t st);

// log-probabilities: gather of K ids per row, and the backward (stream + id fix-up)
constexpr int LP_TABLE = 16;  // shards per gather launch
struct LpTable {
    int n;
    int64_t start[LP_TABLE], width[LP_TABLE];
    RowView x[LP_TABLE];
};
// out = sign * lp (sign -1: cross-entropy); ignored ids give exactly 0
hipError_t launch_lp_gather(int dtype, const LpTable &tab, bool first, int64_t N,
                            int64_t vocab_global, const int64_t *ids, int K, int64_t ignore,
                            const double *stats, float *out, int32_t *dev_err, hipStream_t st,
                            float sign = 1.0f);
// Upstream gradient of each (row, slot) of the log-probability backward: grad[r*K+k]
// for log-probabilities; -grow[r] * exp(tlogp[r*K+k]) (0 where tlogp is -inf) for the
// teacher top-k forward KL, whose value depends on lp_s(id_k) through that weight.
// For cross-entropy (rows = -lp(label)): -g_r, g_r = grow[r] or grow[0] (scalar),
// divided by max(*count, 1) for a mean.
struct LpWeights {
    const float *grad = nullptr;
    const float *tlogp = nullptr;
    const float *grow = nullptr;
    bool scalar = false;
    const double *count = nullptr;
};
__device__ __forceinline__ float lp_weight(const LpWeights &w, int64_t r, int K, int k) {
    if (w.tlogp != nullptr) {
        const float t = w.tlogp[r * K + k];
        return t > -__builtin_huge_valf() ? -w.grow[r] * expf(t) : 0.0f;
    }
    if (w.grow != nullptr) {
        double g = w.scalar ? (double)w.grow[0] : (double)w.grow[r];
        if (w.count) g /= fmax(*w.count, 1.0);
        return (float)-g;
    }
    return w.grad[r * K + k];
}

hipError_t launch_lp_bwd_prep(int64_t N, int64_t vocab_global, const double *stats,
                              const int64_t *ids, int K, int64_t ignore, const LpWeights &w,
                              float *rowc, hipStream_t st);
hipError_t launch_lp_bwd(int dtype, const Shard &sh, int64_t N, const int64_t *ids, int K,
                         int64_t ignore, const LpWeights &w, const float *rowc, hipStream_t st);
// teacher top-k forward KL: per row, sum over the ids this table of shards owns of
// exp(t) (t - lp_s(id)); the first launch writes, later launches add
hipError_t launch_topk_kl(int dtype, const LpTable &tab, bool first, int64_t N,
                          int64_t vocab_global, const int64_t *ids, const float *tlogp, int K,
                          int64_t ignore, const double *stats, float *kl, int32_t *dev_err,
                          hipStream_t st);

// Matrix-core GEMM of the fused-linear loss: C[i][j] (+)= sum_k A(i, k) * B(j, k), bf16
// products (fp32 A rounded to bf16 when staged), fp32 accumulation.  A(i, k) is at
// a[i*lda + k] (a_kmajor) or a[k*lda + i]; B(j, k) at b[j*ldb + k] (b_kmajor) or
// b[k*ldb + j], bf16.  Pointers 16-byte aligned, leading dimensions multiples of 8
// elements (fp32 A: 4).
enum GemmOut {
    GEMM_F32 = 0,      // fp32 C = A B^T
    GEMM_F32_ACC = 1,  // fp32 C += A B^T
    GEMM_BF16 = 2,     // bf16 C = A B^T (nearest even)
    GEMM_BF16_ACC = 3  // bf16 C = addend + A B^T (addend fp32)
};
struct GemmArgs {
    int64_t M = 0, N = 0, K = 0;
    const void *a = nullptr;
    int64_t lda = 0;
    int a_f32 = 0, a_kmajor = 1;
    const void *b = nullptr;
    int64_t ldb = 0;
    int b_kmajor = 1;
    void *c = nullptr;
    int64_t ldc = 0;
    int out = GEMM_F32;
    const float *addend = nullptr;  // GEMM_BF16_ACC: fp32, element (i, j) at addend[i*ldadd + j]
    int64_t ldadd = 0;
    int n_fastest = 0;  // tile order (set by launch_gemm)
    // split of K over `ksplit` work items per tile (the direct-to-LDS kernel only): item s
    // writes the fp32 product of its K range to c + s * split_stride (out GEMM_F32)
    int ksplit = 1;
    int64_t split_stride = 0;
};
hipError_t launch_gemm(const GemmArgs &g, hipStream_t st);
// out[i][j] = bf16(sum_{s < S} part[s * stride + i * ldp + j]) (fixed order), i < M, j < N
hipError_t launch_sum_partials(const float *part, int S, int64_t stride, int64_t M, int64_t N,
                               int64_t ldp, uint16_t *out, int64_t ldo, hipStream_t st);
// dst[c][r] = src[r][c], 16-bit elements, r < R, c < C; row strides multiples of 8
// elements, bases 16-byte aligned
hipError_t launch_transpose16(const uint16_t *src, int64_t lds, int64_t R, int64_t C,
                              uint16_t *dst, int64_t ldd, hipStream_t st);
// p[i] *= g[0] over n values of dtype 0 (fp32), 1 (fp16) or 2 (bf16); p 16-byte aligned;
// nothing is read or written past g[0] when g[0] == 1
hipError_t launch_scale(int dtype, void *p, int64_t n, const float *g, hipStream_t st);

}  // namespace vjsd
