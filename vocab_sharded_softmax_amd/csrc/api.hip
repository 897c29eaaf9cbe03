// api.hip -- the extern "C" entry points of libvjsd: argument validation on the host,
// then one launch per shard per pass on the caller's stream.  The library allocates
// nothing and keeps no state, except the device array of vjsd_bwd_noalloc (below).
// The operations and their citations are documented in include/vjsd.h.
#include <math.h>
#include <string.h>

#include <atomic>

#include "kernels.hpp"
#include "vjsd.h"

using vjsd::Shard;

namespace {

constexpr int MAX_SHARDS = 4096;
constexpr int64_t MAX_ROWS = 0x7fffffff;  // one workgroup per row: grid.x limit

int esize(int dt) { return dt == VJSD_F32 ? 4 : 2; }

// A view is valid when its rows are element-aligned and do not overlap.
bool view_ok(const void *p, int64_t rs, int64_t rpb, int64_t bs, int64_t N, int64_t w, int es) {
    if (N == 0 || w == 0) return true;
    if (!p || (reinterpret_cast<uintptr_t>(p) % es) != 0) return false;
    if (rs < 0 || rpb < 0 || bs < 0) return false;
    const int64_t rows_in_batch = rpb > 0 ? (rpb < N ? rpb : N) : N;
    if (rows_in_batch > 1 && rs < w) return false;
    if (rpb > 0 && N > rpb && bs < (rpb - 1) * rs + w) return false;
    return true;
}

int check_common(const vjsd_shard *shards, int S, int64_t N, int dtype) {
    if (dtype != VJSD_F32 && dtype != VJSD_F16 && dtype != VJSD_BF16) return VJSD_ERR_DTYPE;
    if (N < 0 || N > MAX_ROWS || S < 1 || S > MAX_SHARDS || !shards) return VJSD_ERR_ARG;
    for (int k = 0; k < S; ++k) {
        if (shards[k].width < 0 || shards[k].vocab_start < 0) return VJSD_ERR_ARG;
        if (k > 0 && shards[k].vocab_start != shards[k - 1].vocab_start + shards[k - 1].width)
            return VJSD_ERR_LAYOUT;
    }
    return VJSD_OK;
}

// Inputs: student always, teacher when `two`; gradients when `grads` (a NULL gradient
// pointer means "not wanted" and is allowed).
int check_views(const vjsd_shard *shards, int S, int64_t N, int dtype, bool two, bool grads) {
    const int es = esize(dtype);
    for (int k = 0; k < S; ++k) {
        const vjsd_shard &h = shards[k];
        const int64_t w = h.width;
        if (!view_ok(h.s.p, h.s.row_stride, h.s.rows_per_batch, h.s.batch_stride, N, w, es))
            return VJSD_ERR_ARG;
        if (two && !view_ok(h.t.p, h.t.row_stride, h.t.rows_per_batch, h.t.batch_stride, N, w, es))
            return VJSD_ERR_ARG;
        if (grads) {
            if (h.gs.p && !view_ok(h.gs.p, h.gs.row_stride, h.gs.rows_per_batch,
                                   h.gs.batch_stride, N, w, es))
                return VJSD_ERR_ARG;
            if (two && h.gt.p && !view_ok(h.gt.p, h.gt.row_stride, h.gt.rows_per_batch,
                                          h.gt.batch_stride, N, w, es))
                return VJSD_ERR_ARG;
        }
    }
    return VJSD_OK;
}

Shard convert(const vjsd_shard &h, bool two, bool grads) {
    Shard s;
    s.start = h.vocab_start;
    s.width = h.width;
    s.s = {h.s.p, h.s.row_stride, h.s.rows_per_batch, h.s.batch_stride};
    if (two) s.t = {h.t.p, h.t.row_stride, h.t.rows_per_batch, h.t.batch_stride};
    else s.t = s.s;
    if (grads) {
        s.gs = {h.gs.p, h.gs.row_stride, h.gs.rows_per_batch, h.gs.batch_stride};
        if (two) s.gt = {h.gt.p, h.gt.row_stride, h.gt.rows_per_batch, h.gt.batch_stride};
        else s.gt = {nullptr, 0, 0, 0};
    } else {
        s.gs = {nullptr, 0, 0, 0};
        s.gt = {nullptr, 0, 0, 0};
    }
    return s;
}

int hip_status(hipError_t e) { return e == hipSuccess ? VJSD_OK : VJSD_ERR_HIP; }

// Workspace: N * ROWC floats of per-row constants, then S * N * PART_STRIDE partials.
float *part_of(float *part, int k, int64_t N) {
    return part + (size_t)N * vjsd::ROWC + (size_t)k * (size_t)N * vjsd::PART_STRIDE;
}
const float *part_of(const float *part, int k, int64_t N) {
    return part + (size_t)N * vjsd::ROWC + (size_t)k * (size_t)N * vjsd::PART_STRIDE;
}

// After the partials: one double holding the kept-row count of a masked mean.
double *count_of(float *part, int S, int64_t N) {
    return reinterpret_cast<double *>(part + (size_t)N * vjsd::ROWC +
                                      (size_t)S * (size_t)N * vjsd::PART_STRIDE);
}

// Options of the loss forms, validated; NULL means T = 1, no T^2, no mask, no reduction.
struct LossCfg {
    double T = 1.0;
    bool t2 = false;
    const uint8_t *mask = nullptr;
    int red = VJSD_REDUCE_NONE;
};
int loss_cfg(const vjsd_loss_opts *o, LossCfg *c) {
    *c = LossCfg();
    if (!o) return VJSD_OK;
    if (!(o->temperature > 0.0 && o->temperature <= 1e30)) return VJSD_ERR_ARG;  // NaN too
    if (o->reduction < VJSD_REDUCE_NONE || o->reduction > VJSD_REDUCE_MEAN) return VJSD_ERR_ARG;
    c->T = o->temperature;
    c->t2 = o->scale_t2 != 0;
    c->mask = o->mask;
    c->red = o->reduction;
    return VJSD_OK;
}
vjsd::RowOpts row_opts(const LossCfg &c) {
    vjsd::RowOpts o;
    o.ks = (float)(vjsd::L2E_D / c.T);
    o.lscale = c.t2 ? (float)(c.T * c.T) : 1.0f;
    o.mask = c.mask;
    return o;
}

// The backward's upstream-gradient options for the loss form c.
vjsd::GradOpts grad_opts(const LossCfg &c) {
    vjsd::GradOpts go;
    go.ks = row_opts(c).ks;
    go.gmul = (c.t2 ? c.T * c.T : 1.0) / c.T;
    go.scalar = c.red != VJSD_REDUCE_NONE;
    go.mask = c.mask;
    return go;
}

int mode_of(double beta) {
    return beta == 0.0 ? vjsd::FWD_KL : (beta == 1.0 ? vjsd::REV_KL : vjsd::INTERIOR);
}

// The student views of up to LP_TABLE shards starting at shard k0.
vjsd::LpTable lp_table(const vjsd_shard *shards, int S, int k0) {
    vjsd::LpTable tab;
    memset(&tab, 0, sizeof tab);
    tab.n = (S - k0) < vjsd::LP_TABLE ? (S - k0) : vjsd::LP_TABLE;
    for (int q = 0; q < tab.n; ++q) {
        const vjsd_shard &h = shards[k0 + q];
        tab.start[q] = h.vocab_start;
        tab.width[q] = h.width;
        tab.x[q] = {h.s.p, h.s.row_stride, h.s.rows_per_batch, h.s.batch_stride};
    }
    return tab;
}

// Log-probability backward with per-slot upstream weights (validated arguments).
int lp_backward(const vjsd_shard *shards, int S, int64_t N, int dtype, int64_t vocab_global,
                const double *stats, const int64_t *ids, int K, int64_t ignore_index,
                const vjsd::LpWeights &w, float *part, hipStream_t st) {
    int e;
    if ((e = hip_status(vjsd::launch_lp_bwd_prep(N, vocab_global, stats, ids, K, ignore_index, w,
                                                 part, st))))
        return e;
    for (int k = 0; k < S; ++k) {
        if (!shards[k].gs.p) continue;
        Shard sh = convert(shards[k], false, true);
        if ((e = hip_status(vjsd::launch_lp_bwd(dtype, sh, N, ids, K, ignore_index, w, part, st))))
            return e;
    }
    return VJSD_OK;
}


// ---- fused linear + JSD ------------------------------------------------------------

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of vljsd.  Tokens go C at a time (C = min(chunk, N); when that leaves more
// than one chunk, rounded down to a multiple of 8, at least 8, so that each chunk's
// columns of the transposed buffers below start 16 bytes apart) through two fp32 logit
// blocks (student, teacher; row stride ldl = V rounded up to 8) and the chunk's bf16
// logit gradient G, which feeds the chunk's hidden-gradient product at once.  For the
// head gradient, G and the student hidden states of a group of NG tokens (whole chunks:
// `group` rounded up, or with group 0 as many as fit LIN_G_BUDGET bytes, at least one
// chunk) are kept transposed, tokens contiguous; the group's product then runs at once,
// summed across groups in an fp32 accumulator when there is more than one.  Then the
// per-token losses, the chunk's statistics, KL pair and pass workspace, the kept-token
// count.  Measured on MI355X at N=8192, V=151936, D=3584 (fp32 logit blocks 8 C V bytes,
// G 2 C V, the group's transposed G 2 NG V, the transposed head 2 D V): C = 4096 held
// 11.1 GB when G was kept for the whole group; now C = 2048 with one group holds 6.8 GB,
// against 7.5 GB for the bf16 logits and logit gradient of the unfused route.
constexpr size_t LIN_G_BUDGET = (size_t)4 << 30;

struct LinLayout {
    int64_t C = 0, NG = 0, ldl = 0, ldt = 0, ldv = 0;
    int splits = 1;  // K split of the hidden-gradient product
    size_t ls = 0, lt = 0, g = 0, gt = 0, ht = 0, wt = 0, hp = 0, rows = 0, stats = 0, kl = 0,
           part = 0, count = 0, gw = 0;
    size_t total = 0;
    bool has_gw = false;
};

// The hidden-gradient product of a chunk (c x dim tiles of 256 x 256 over a K of V) may
// have fewer tiles than the 256 CUs: then its K is split, when V allows the
// direct-to-LDS kernel (V a multiple of 64), into the number of parts s that minimises
// the time, taken as (rounds of 256 work items) / s plus 2 % per extra part for the
// fp32 partials' write and sum.  112 tiles (2048 tokens at D = 3584) split 2 ways: one
// round at half the K, where 3 ways needed two rounds of a third each.  A round of
// tiles or more is not split (measured: 448 tiles split three ways ran 11 % slower than
// unsplit).
int lin_splits(int64_t ng, int64_t V, int64_t dim) {
    if (V % 64 != 0 || ng <= 0) return 1;
    const int64_t tiles = ((ng + 255) / 256) * ((dim + 255) / 256);
    if (tiles >= 256) return 1;
    const int64_t stages = V / 64;
    int best = 1;
    double best_t = 1.0;
    for (int s = 2; s <= 8 && stages / s >= 8; ++s) {  // at least 8 stages of k per item
        const double t = (double)((tiles * s + 255) / 256) / s + 0.02 * (s - 1);
        if (t < best_t - 1e-12) {
            best = s;
            best_t = t;
        }
    }
    return best;
}
LinLayout lin_layout(int64_t N, int64_t V, int64_t dim, int64_t chunk, int64_t group) {
    LinLayout L;
    L.C = chunk < N ? chunk : N;
    if (L.C < N) {  // several chunks: whole multiples of 8 tokens
        L.C = L.C >= 8 ? L.C / 8 * 8 : 8;
        if (L.C > N) L.C = N;
    }
    L.ldl = (V + 7) / 8 * 8;
    int64_t per = 1;  // chunks per group
    if (L.C > 0) {
        per = group > 0 ? (group + L.C - 1) / L.C
                        : (int64_t)(LIN_G_BUDGET / ((size_t)L.ldl * 2)) / L.C;
        if (per < 1) per = 1;
    }
    const int64_t ng = per * L.C;
    L.NG = ng < N ? ng : N;
    size_t o = 0;
    auto take = [&o](size_t bytes) {
        const size_t at = o;
        o = align256(o + bytes);
        return at;
    };
    const size_t blk = (size_t)L.C * (size_t)L.ldl * sizeof(float);
    L.ls = take(blk);
    L.lt = take(blk);
    L.g = take((size_t)L.C * (size_t)L.ldl * 2);
    // the group's G and student hidden states transposed (tokens contiguous), so that the
    // head-gradient product reads both operands k-major
    L.ldt = (L.NG + 7) / 8 * 8;
    L.gt = take((size_t)V * (size_t)L.ldt * 2);
    L.ht = take((size_t)dim * (size_t)L.ldt * 2);
    // the student head transposed (vocabulary contiguous) for the hidden-gradient
    // product, and that product's fp32 partials when its K is split
    L.ldv = (V + 7) / 8 * 8;
    L.wt = take((size_t)dim * (size_t)L.ldv * 2);
    L.splits = lin_splits(L.C, V, dim);
    L.hp = take(L.splits > 1 ? (size_t)L.splits * (size_t)L.C * (size_t)dim * 4 : 0);
    L.rows = take((size_t)N * sizeof(float));
    L.stats = take((size_t)L.C * 4 * sizeof(double));
    L.kl = take((size_t)L.C * 2 * sizeof(float));
    L.part = take(vjsd_workspace_bytes(L.C > 0 ? L.C : 1, 1));
    L.count = take(sizeof(double));
    L.has_gw = L.NG < N;
    L.gw = take(L.has_gw ? (size_t)V * (size_t)dim * sizeof(float) : 0);
    L.total = o;
    return L;
}

// A vlin_gemm operand of `rows` rows and K reduction steps.
int check_operand(const vlin_operand &o, int64_t rows, int64_t K, bool allow_f32) {
    if (o.dtype != VJSD_BF16 && !(allow_f32 && o.dtype == VJSD_F32)) return VJSD_ERR_DTYPE;
    if (o.kmajor != 0 && o.kmajor != 1) return VJSD_ERR_ARG;
    if (rows == 0 || K == 0) return VJSD_OK;  // never read
    if (!o.p || reinterpret_cast<uintptr_t>(o.p) % 16 != 0) return VJSD_ERR_ARG;
    const int64_t q = o.dtype == VJSD_F32 ? 4 : 8;
    if (o.ld <= 0 || o.ld % q != 0) return VJSD_ERR_ARG;
    if (o.kmajor ? o.ld < K : o.ld < rows) return VJSD_ERR_ARG;
    return VJSD_OK;
}

constexpr int64_t GEMM_TILES_MAX = 0x7fffff00LL;  // one workgroup per 128 x 128 tile

bool gemm_size_ok(int64_t M, int64_t N) {
    return ((M + 127) / 128) * ((N + 127) / 128) <= GEMM_TILES_MAX;
}

// One LM-head side: hidden [N][dim] and head [V][dim], bf16.
int check_head(const vlin_head *h, int64_t N, int64_t V) {
    if (!h || h->dim < 1) return VJSD_ERR_ARG;
    if (N > 0 && (!h->h || reinterpret_cast<uintptr_t>(h->h) % 16 != 0 || h->ldh < h->dim ||
                  h->ldh % 8 != 0))
        return VJSD_ERR_ARG;
    if (!h->w || reinterpret_cast<uintptr_t>(h->w) % 16 != 0 || h->ldw < h->dim ||
        h->ldw % 8 != 0)
        return VJSD_ERR_ARG;
    (void)V;
    return VJSD_OK;
}

// The backward of every shard of a call (one launch for up to eight shards).
int bwd_all(const vjsd_shard *shards, int S, int64_t N, int dtype, int mode, const float *rowc,
            hipStream_t st) {
    Shard sh[vjsd::FUSED_SHARDS];
    if (S <= vjsd::FUSED_SHARDS) {
        for (int k = 0; k < S; ++k) sh[k] = convert(shards[k], true, true);
        return hip_status(vjsd::launch_bwd_shards(dtype, mode, sh, S, N, rowc, st));
    }
    for (int k = 0; k < S; ++k) {
        Shard one = convert(shards[k], true, true);
        const int e = hip_status(vjsd::launch_bwd(dtype, mode, one, N, rowc, st));
        if (e) return e;
    }
    return VJSD_OK;
}

// Per-row constants of vjsd_bwd_noalloc: a file-scope device array.  In host code the
// name `scratch` is a host-side stand-in; kernels get the per-device address that
// hipGetSymbolAddress returns, kept in scratch_ptr.
static __device__ __align__(256) float scratch[(size_t)VJSD_NOALLOC_MAX_ROWS * vjsd::ROWC];
constexpr int SCRATCH_DEVICES = 64;
std::atomic<float *> scratch_ptr[SCRATCH_DEVICES];

// This device's address of `scratch`, looked up on the first call on the device (a
// second thread racing through the lookup stores the same address).  The stream must
// belong to the current device.
int scratch_of(hipStream_t st, float **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return VJSD_ERR_HIP;
    if (dev < 0 || dev >= SCRATCH_DEVICES) return VJSD_ERR_ARG;
    if (st) {
        hipDevice_t sd = 0;
        if (hipStreamGetDevice(st, &sd) != hipSuccess) return VJSD_ERR_HIP;
        if (sd != dev) return VJSD_ERR_ARG;
    }
    float *p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        void *q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return VJSD_ERR_HIP;
        p = static_cast<float *>(q);
        scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return VJSD_OK;
}

}  // namespace

extern "C" {

const char *vjsd_strerror(int code) {
    switch (code) {
        case VJSD_OK: return "success";
        case VJSD_ERR_ARG: return "invalid argument (null pointer, size, stride or alignment)";
        case VJSD_ERR_DTYPE: return "unsupported dtype";
        case VJSD_ERR_BETA: return "beta must be a number in [0, 1]";
        case VJSD_ERR_LAYOUT: return "shards must be ordered and contiguous in the vocabulary";
        case VJSD_ERR_EMPTY_SHARD: return "log-probabilities need every vocabulary shard non-empty";
        case VJSD_ERR_HIP: return "HIP kernel launch failed";
        case VJSD_ERR_SCRATCH:
            return "more rows than the no-allocation backward's scratch holds "
                   "(VJSD_NOALLOC_MAX_ROWS = 65536)";
        default: return "unknown vjsd status";
    }
}

size_t vjsd_workspace_bytes(int64_t N, int S) {
    if (N <= 0 || S <= 0) return 0;
    const size_t floats = (size_t)N * vjsd::ROWC + (size_t)N * (size_t)S * vjsd::PART_STRIDE;
    return floats * sizeof(float) + 64;  // + the scalar tail (kept-row count)
}

int vjsd_stats(const vjsd_shard *shards, int S, int64_t N, int dtype, int which, float *part,
               void *stream) {
    int e = check_common(shards, S, N, dtype);
    if (e) return e;
    if (which < 1 || which > 3) return VJSD_ERR_ARG;
    for (int k = 0; k < S; ++k) {  // only the selected inputs are read
        const vjsd_shard &h = shards[k];
        if ((which & 1) && !view_ok(h.s.p, h.s.row_stride, h.s.rows_per_batch, h.s.batch_stride,
                                    N, h.width, esize(dtype)))
            return VJSD_ERR_ARG;
        if ((which & 2) && !view_ok(h.t.p, h.t.row_stride, h.t.rows_per_batch, h.t.batch_stride,
                                    N, h.width, esize(dtype)))
            return VJSD_ERR_ARG;
    }
    if (N == 0) return VJSD_OK;
    if (!part) return VJSD_ERR_ARG;
    for (int k = 0; k < S; ++k) {
        Shard sh = convert(shards[k], true, false);
        if ((e = hip_status(vjsd::launch_stats(dtype, which, sh, N, part_of(part, k, N),
                                               (hipStream_t)stream))))
            return e;
    }
    return VJSD_OK;
}

int vjsd_merge(const float *part, int S, int64_t N, int which, double *stats, void *stream) {
    if (N < 0 || N > MAX_ROWS || S < 1 || S > MAX_SHARDS || which < 1 || which > 3)
        return VJSD_ERR_ARG;
    if (N == 0) return VJSD_OK;
    if (!part || !stats) return VJSD_ERR_ARG;
    return hip_status(
        vjsd::launch_merge(part_of(part, 0, N), S, N, which, stats, (hipStream_t)stream));
}

int vjsd_fwd(const vjsd_shard *shards, int S, int64_t N, int dtype, const double *stats,
             double beta, float *part, float *kl, float *loss, void *stream) {
    int e = check_common(shards, S, N, dtype);
    if (e) return e;
    if (!(beta >= 0.0 && beta <= 1.0)) return VJSD_ERR_BETA;
    if ((e = check_views(shards, S, N, dtype, true, false))) return e;
    if (N == 0) return VJSD_OK;
    if (!stats || !kl || !loss || (S > 1 && !part)) return VJSD_ERR_ARG;
    const int mode = mode_of(beta);
    hipStream_t st = (hipStream_t)stream;
    if (S == 1) {
        Shard sh = convert(shards[0], true, false);
        return hip_status(vjsd::launch_div(dtype, mode, sh, N, stats, beta, nullptr, kl, loss, st));
    }
    for (int k = 0; k < S; ++k) {
        Shard sh = convert(shards[k], true, false);
        if ((e = hip_status(vjsd::launch_div(dtype, mode, sh, N, stats, beta, part_of(part, k, N),
                                             nullptr, nullptr, st))))
            return e;
    }
    return hip_status(
        vjsd::launch_div_finalize(mode, part_of(part, 0, N), S, N, stats, beta, kl, loss, st));
}

int vjsd_forward(const vjsd_shard *shards, int S, int64_t N, int dtype, double beta, float *part,
                 double *stats, float *kl, float *loss, void *stream) {
    // the loss form without options: T = 1, no T^2, no mask, per-token losses
    return vjsd_loss_forward(shards, S, N, dtype, beta, nullptr, part, stats, kl, loss, nullptr,
                             stream);
}

int vjsd_loss_forward(const vjsd_shard *shards, int S, int64_t N, int dtype, double beta,
                      const vjsd_loss_opts *opts, float *part, double *stats, float *kl,
                      float *rows, float *out, void *stream) {
    int e = check_common(shards, S, N, dtype);
    if (e) return e;
    if (!(beta >= 0.0 && beta <= 1.0)) return VJSD_ERR_BETA;
    LossCfg c;
    if ((e = loss_cfg(opts, &c))) return e;
    if ((e = check_views(shards, S, N, dtype, true, false))) return e;
    if (c.red != VJSD_REDUCE_NONE && !out) return VJSD_ERR_ARG;
    hipStream_t st = (hipStream_t)stream;
    if (N == 0) {
        if (c.red != VJSD_REDUCE_NONE)
            return hip_status(
                vjsd::launch_reduce_rows(nullptr, vjsd::RowOpts(), 0, false, out, nullptr, st));
        return VJSD_OK;
    }
    if (!part || !stats || !kl || !rows) return VJSD_ERR_ARG;
    const vjsd::RowOpts ro = row_opts(c);
    const int mode = mode_of(beta);
    if (mode != vjsd::INTERIOR) {  // the endpoints are plain KL divergences: one input pass
        const int rev = mode == vjsd::REV_KL;
        for (int k = 0; k < S; ++k) {
            Shard sh = convert(shards[k], true, false);
            if ((e = hip_status(vjsd::launch_kl1(dtype, rev, sh, N, part_of(part, k, N), st, ro))))
                return e;
        }
        if ((e = hip_status(vjsd::launch_kl1_merge(rev, part_of(part, 0, N), S, N, stats, kl,
                                                   rows, st, ro))))
            return e;
    } else if (S == 1) {
        Shard sh = convert(shards[0], true, false);
        if ((e = hip_status(vjsd::launch_fwd_fused(dtype, sh, N, beta, stats, kl, rows, st, ro))))
            return e;
    } else if (S <= vjsd::FUSED_SHARDS) {
        Shard sh[vjsd::FUSED_SHARDS];
        for (int k = 0; k < S; ++k) sh[k] = convert(shards[k], true, false);
        if ((e = hip_status(vjsd::launch_fwd_shards(dtype, sh, S, N, beta, stats, kl, rows, st, ro))))
            return e;
    } else {
        for (int k = 0; k < S; ++k) {
            Shard sh = convert(shards[k], true, false);
            if ((e = hip_status(vjsd::launch_stats(dtype, 3, sh, N, part_of(part, k, N), st, ro))))
                return e;
        }
        if ((e = hip_status(vjsd::launch_merge(part_of(part, 0, N), S, N, 3, stats, st, ro.ks))))
            return e;
        for (int k = 0; k < S; ++k) {
            Shard sh = convert(shards[k], true, false);
            if ((e = hip_status(vjsd::launch_div(dtype, mode, sh, N, stats, beta,
                                                 part_of(part, k, N), nullptr, nullptr, st, ro))))
                return e;
        }
        if ((e = hip_status(vjsd::launch_div_finalize(mode, part_of(part, 0, N), S, N, stats, beta,
                                                      kl, rows, st, ro))))
            return e;
    }
    if (c.red == VJSD_REDUCE_NONE) return VJSD_OK;
    return hip_status(vjsd::launch_reduce_rows(rows, ro, N, c.red == VJSD_REDUCE_MEAN, out,
                                               nullptr, st));
}

int vjsd_loss_backward(const vjsd_shard *shards, int S, int64_t N, int dtype, double beta,
                       const vjsd_loss_opts *opts, const double *stats, const float *kl,
                       const float *grad, float *part, void *stream) {
    int e = check_common(shards, S, N, dtype);
    if (e) return e;
    if (!(beta >= 0.0 && beta <= 1.0)) return VJSD_ERR_BETA;
    LossCfg c;
    if ((e = loss_cfg(opts, &c))) return e;
    if ((e = check_views(shards, S, N, dtype, true, true))) return e;
    if (N == 0) return VJSD_OK;
    if (!stats || !kl || !grad || !part) return VJSD_ERR_ARG;
    const int mode = mode_of(beta);
    hipStream_t st = (hipStream_t)stream;
    vjsd::GradOpts go = grad_opts(c);
    if (c.red == VJSD_REDUCE_MEAN) {
        double *cnt = count_of(part, S, N);
        if ((e = hip_status(
                 vjsd::launch_reduce_rows(nullptr, row_opts(c), N, false, nullptr, cnt, st))))
            return e;
        go.count = cnt;
    }
    if ((e = hip_status(vjsd::launch_bwd_prep(mode, N, stats, kl, beta, grad, part, st, go))))
        return e;
    return bwd_all(shards, S, N, dtype, mode, part, st);
}

int vjsd_loss_forward_backward(const vjsd_shard *shards, int S, int64_t N, int dtype, double beta,
                               const vjsd_loss_opts *opts, const float *grad, float *part,
                               double *stats, float *kl, float *rows, float *out, void *stream) {
    int e = check_common(shards, S, N, dtype);
    if (e) return e;
    if (!(beta >= 0.0 && beta <= 1.0)) return VJSD_ERR_BETA;
    LossCfg c;
    if ((e = loss_cfg(opts, &c))) return e;
    if ((e = check_views(shards, S, N, dtype, true, true))) return e;
    if (c.red != VJSD_REDUCE_NONE && !out) return VJSD_ERR_ARG;
    if (N == 0)  // nothing to differentiate; a reduction's out is still written
        return vjsd_loss_forward(shards, S, N, dtype, beta, opts, part, stats, kl, rows, out,
                                 stream);
    if (!part || !stats || !kl || !rows || !grad) return VJSD_ERR_ARG;
    hipStream_t st = (hipStream_t)stream;
    // A token mask runs the two calls: with few tokens kept, the kept rows' whole work in
    // one workgroup each ends the launch on a tail (8192 x 151936 bf16, temperature 2,
    // mean over 3 % of the tokens: 1.06 ms in one launch, 0.92 ms in two calls), where
    // with every token kept one launch gained 3-4 % (2.75-2.78 against 2.86 ms).
    if (S == 1 && mode_of(beta) == vjsd::INTERIOR && c.mask == nullptr) {
        const vjsd::RowOpts ro = row_opts(c);
        vjsd::GradOpts go = grad_opts(c);
        if (c.red == VJSD_REDUCE_MEAN) {  // the kept-row count, before any gradient
            double *cnt = count_of(part, S, N);
            if ((e = hip_status(vjsd::launch_reduce_rows(nullptr, ro, N, false, nullptr, cnt, st))))
                return e;
            go.count = cnt;
        }
        const Shard sh = convert(shards[0], true, true);
        const hipError_t he =
            vjsd::launch_fwd_bwd_fused(dtype, sh, N, beta, grad, stats, kl, rows, st, ro, go);
        if (he == hipSuccess) {
            if (c.red == VJSD_REDUCE_NONE) return VJSD_OK;
            return hip_status(vjsd::launch_reduce_rows(rows, ro, N, c.red == VJSD_REDUCE_MEAN,
                                                       out, nullptr, st));
        }
        if (he != hipErrorNotSupported) return VJSD_ERR_HIP;
    }
    // every other case: the two entry points, which compute the same outputs
    if ((e = vjsd_loss_forward(shards, S, N, dtype, beta, opts, part, stats, kl, rows, out,
                               stream)))
        return e;
    return vjsd_loss_backward(shards, S, N, dtype, beta, opts, stats, kl, grad, part, stream);
}

int vjsd_forward_backward(const vjsd_shard *shards, int S, int64_t N, int dtype, double beta,
                          const float *grad_loss, float *part, double *stats, float *kl,
                          float *loss, void *stream) {
    return vjsd_loss_forward_backward(shards, S, N, dtype, beta, nullptr, grad_loss, part, stats,
                                      kl, loss, nullptr, stream);
}

int vjsd_bwd(const vjsd_shard *shards, int S, int64_t N, int dtype, const double *stats,
             const float *kl, double beta, const float *grad_loss, float *part, void *stream) {
    int e = check_common(shards, S, N, dtype);
    if (e) return e;
    if (!(beta >= 0.0 && beta <= 1.0)) return VJSD_ERR_BETA;
    if ((e = check_views(shards, S, N, dtype, true, true))) return e;
    if (N == 0) return VJSD_OK;
    if (!stats || !kl || !grad_loss || !part) return VJSD_ERR_ARG;
    const int mode = mode_of(beta);
    hipStream_t st = (hipStream_t)stream;
    if ((e = hip_status(vjsd::launch_bwd_prep(mode, N, stats, kl, beta, grad_loss, part, st))))
        return e;
    return bwd_all(shards, S, N, dtype, mode, part, st);
}

int vjsd_bwd_noalloc(const vjsd_shard *shards, int S, int64_t N, int dtype, const double *stats,
                     const float *kl, double beta, const float *grad_loss, void *stream) {
    int e = check_common(shards, S, N, dtype);
    if (e) return e;
    if (!(beta >= 0.0 && beta <= 1.0)) return VJSD_ERR_BETA;
    if ((e = check_views(shards, S, N, dtype, true, true))) return e;
    if (N == 0) return VJSD_OK;
    if (!stats || !kl || !grad_loss) return VJSD_ERR_ARG;
    if (N > VJSD_NOALLOC_MAX_ROWS) return VJSD_ERR_SCRATCH;
    hipStream_t st = (hipStream_t)stream;
    float *rowc = nullptr;
    if ((e = scratch_of(st, &rowc))) return e;
    const int mode = mode_of(beta);
    // k_bwd_prep writes every constant of rows [0, N) that the gradient kernels read
    if ((e = hip_status(vjsd::launch_bwd_prep(mode, N, stats, kl, beta, grad_loss, rowc, st))))
        return e;
    return bwd_all(shards, S, N, dtype, mode, rowc, st);
}

int vkl_fwd(const vjsd_shard *shards, int S, int64_t N, int dtype, int reverse, float *part,
            double *stats, float *kl, float *loss, void *stream) {
    int e = check_common(shards, S, N, dtype);
    if (e) return e;
    if ((e = check_views(shards, S, N, dtype, true, false))) return e;
    if (N == 0) return VJSD_OK;
    if (!part || !stats || !kl || !loss) return VJSD_ERR_ARG;
    hipStream_t st = (hipStream_t)stream;
    for (int k = 0; k < S; ++k) {
        Shard sh = convert(shards[k], true, false);
        if ((e = hip_status(vjsd::launch_kl1(dtype, reverse != 0, sh, N, part_of(part, k, N), st))))
            return e;
    }
    return hip_status(
        vjsd::launch_kl1_merge(reverse != 0, part_of(part, 0, N), S, N, stats, kl, loss, st));
}

int vkl_bwd(const vjsd_shard *shards, int S, int64_t N, int dtype, int reverse,
            const double *stats, const float *kl, const float *grad_loss, float *part,
            void *stream) {
    return vjsd_bwd(shards, S, N, dtype, stats, kl, reverse ? 1.0 : 0.0, grad_loss, part, stream);
}

int ventropy_fwd(const vjsd_shard *shards, int S, int64_t N, int dtype, float *part,
                 double *stats, float *ent, void *stream) {
    int e = check_common(shards, S, N, dtype);
    if (e) return e;
    if ((e = check_views(shards, S, N, dtype, false, false))) return e;
    if (N == 0) return VJSD_OK;
    if (!part || !stats || !ent) return VJSD_ERR_ARG;
    hipStream_t st = (hipStream_t)stream;
    for (int k = 0; k < S; ++k) {
        Shard sh = convert(shards[k], false, false);
        if ((e = hip_status(vjsd::launch_ent1(dtype, sh, N, part_of(part, k, N), st)))) return e;
    }
    return hip_status(vjsd::launch_ent1_merge(part_of(part, 0, N), S, N, stats, ent, st));
}

int ventropy_bwd(const vjsd_shard *shards, int S, int64_t N, int dtype, const double *stats,
                 const float *ent, const float *grad, float *part, void *stream) {
    int e = check_common(shards, S, N, dtype);
    if (e) return e;
    if ((e = check_views(shards, S, N, dtype, false, true))) return e;
    if (N == 0) return VJSD_OK;
    if (!stats || !ent || !grad || !part) return VJSD_ERR_ARG;
    hipStream_t st = (hipStream_t)stream;
    if ((e = hip_status(vjsd::launch_ent_bwd_prep(N, stats, ent, grad, part, st)))) return e;
    for (int k = 0; k < S; ++k) {
        if (!shards[k].gs.p) continue;
        Shard sh = convert(shards[k], false, true);
        if ((e = hip_status(vjsd::launch_ent_bwd(dtype, sh, N, part, st)))) return e;
    }
    return VJSD_OK;
}

static int check_logprobs(const vjsd_shard *shards, int S, int64_t N, int dtype,
                          int64_t vocab_global, const int64_t *ids, int K) {
    int e = check_common(shards, S, N, dtype);
    if (e) return e;
    if (K < 0 || (N > 0 && K > 0 && !ids)) return VJSD_ERR_ARG;
    if (N > 0 && K > 0 && (N * (int64_t)K) / 256 > MAX_ROWS) return VJSD_ERR_ARG;
    for (int k = 0; k < S; ++k)
        if (shards[k].width == 0) return VJSD_ERR_EMPTY_SHARD;
    if (shards[0].vocab_start != 0 ||
        shards[S - 1].vocab_start + shards[S - 1].width != vocab_global)
        return VJSD_ERR_LAYOUT;
    return VJSD_OK;
}

int vlogprobs_fwd(const vjsd_shard *shards, int S, int64_t N, int dtype, int64_t vocab_global,
                  const int64_t *ids, int K, int64_t ignore_index, float *part, double *stats,
                  float *out, int32_t *dev_err, void *stream) {
    int e = check_logprobs(shards, S, N, dtype, vocab_global, ids, K);
    if (e) return e;
    if ((e = check_views(shards, S, N, dtype, false, false))) return e;
    if (N == 0) return VJSD_OK;
    if (!part || !stats || (K > 0 && (!out || !dev_err))) return VJSD_ERR_ARG;
    hipStream_t st = (hipStream_t)stream;
    for (int k = 0; k < S; ++k) {
        Shard sh = convert(shards[k], false, false);
        if ((e = hip_status(vjsd::launch_stats(dtype, 1, sh, N, part_of(part, k, N), st)))) return e;
    }
    if ((e = hip_status(vjsd::launch_merge(part_of(part, 0, N), S, N, 1, stats, st)))) return e;
    if (K == 0) return VJSD_OK;
    for (int k0 = 0; k0 < S; k0 += vjsd::LP_TABLE) {
        vjsd::LpTable tab = lp_table(shards, S, k0);
        if ((e = hip_status(vjsd::launch_lp_gather(dtype, tab, k0 == 0, N, vocab_global, ids, K,
                                                   ignore_index, stats, out, dev_err, st))))
            return e;
    }
    return VJSD_OK;
}

int vlogprobs_bwd(const vjsd_shard *shards, int S, int64_t N, int dtype, int64_t vocab_global,
                  const double *stats, const int64_t *ids, int K, int64_t ignore_index,
                  const float *grad, float *part, void *stream) {
    int e = check_logprobs(shards, S, N, dtype, vocab_global, ids, K);
    if (e) return e;
    if ((e = check_views(shards, S, N, dtype, false, true))) return e;
    if (N == 0) return VJSD_OK;
    if (!stats || !part || (K > 0 && !grad)) return VJSD_ERR_ARG;
    hipStream_t st = (hipStream_t)stream;
    vjsd::LpWeights w;
    w.grad = grad;
    return lp_backward(shards, S, N, dtype, vocab_global, stats, ids, K, ignore_index, w, part, st);
}

int vce_fwd(const vjsd_shard *shards, int S, int64_t N, int dtype, int64_t vocab_global,
            const int64_t *labels, int64_t ignore_index, int reduction, float *part,
            double *stats, float *rows, float *out, int32_t *dev_err, void *stream) {
    int e = check_logprobs(shards, S, N, dtype, vocab_global, labels, 1);
    if (e) return e;
    if ((e = check_views(shards, S, N, dtype, false, false))) return e;
    if (reduction < VJSD_REDUCE_NONE || reduction > VJSD_REDUCE_MEAN) return VJSD_ERR_ARG;
    if (reduction != VJSD_REDUCE_NONE && !out) return VJSD_ERR_ARG;
    hipStream_t st = (hipStream_t)stream;
    if (N == 0) {
        if (reduction != VJSD_REDUCE_NONE)
            return hip_status(
                vjsd::launch_reduce_rows(nullptr, vjsd::RowOpts(), 0, false, out, nullptr, st));
        return VJSD_OK;
    }
    if (!part || !stats || !rows || !dev_err) return VJSD_ERR_ARG;
    vjsd::RowOpts sel;  // rows whose label is ignore_index are never read
    sel.labels = labels;
    sel.ignore = ignore_index;
    for (int k = 0; k < S; ++k) {
        Shard sh = convert(shards[k], false, false);
        if ((e = hip_status(vjsd::launch_stats(dtype, 1, sh, N, part_of(part, k, N), st, sel))))
            return e;
    }
    if ((e = hip_status(vjsd::launch_merge(part_of(part, 0, N), S, N, 1, stats, st)))) return e;
    for (int k0 = 0; k0 < S; k0 += vjsd::LP_TABLE) {
        vjsd::LpTable tab = lp_table(shards, S, k0);
        if ((e = hip_status(vjsd::launch_lp_gather(dtype, tab, k0 == 0, N, vocab_global, labels, 1,
                                                   ignore_index, stats, rows, dev_err, st,
                                                   -1.0f))))
            return e;
    }
    if (reduction == VJSD_REDUCE_NONE) return VJSD_OK;
    return hip_status(vjsd::launch_reduce_rows(rows, sel, N, reduction == VJSD_REDUCE_MEAN, out,
                                               nullptr, st));
}

int vce_bwd(const vjsd_shard *shards, int S, int64_t N, int dtype, int64_t vocab_global,
            const double *stats, const int64_t *labels, int64_t ignore_index, int reduction,
            const float *grad, float *part, void *stream) {
    int e = check_logprobs(shards, S, N, dtype, vocab_global, labels, 1);
    if (e) return e;
    if ((e = check_views(shards, S, N, dtype, false, true))) return e;
    if (reduction < VJSD_REDUCE_NONE || reduction > VJSD_REDUCE_MEAN) return VJSD_ERR_ARG;
    if (N == 0) return VJSD_OK;
    if (!stats || !part || !grad) return VJSD_ERR_ARG;
    hipStream_t st = (hipStream_t)stream;
    vjsd::LpWeights w;
    w.grow = grad;
    w.scalar = reduction != VJSD_REDUCE_NONE;
    if (reduction == VJSD_REDUCE_MEAN) {
        vjsd::RowOpts sel;
        sel.labels = labels;
        sel.ignore = ignore_index;
        double *cnt = count_of(part, S, N);
        if ((e = hip_status(vjsd::launch_reduce_rows(nullptr, sel, N, false, nullptr, cnt, st))))
            return e;
        w.count = cnt;
    }
    return lp_backward(shards, S, N, dtype, vocab_global, stats, labels, 1, ignore_index, w, part,
                       st);
}

int vtopk_kl_fwd(const vjsd_shard *shards, int S, int64_t N, int dtype, int64_t vocab_global,
                 const int64_t *ids, const float *tlogp, int K, int64_t ignore_index, float *part,
                 double *stats, float *kl, int32_t *dev_err, void *stream) {
    int e = check_logprobs(shards, S, N, dtype, vocab_global, ids, K);
    if (e) return e;
    if ((e = check_views(shards, S, N, dtype, false, false))) return e;
    if (N == 0) return VJSD_OK;
    if (!part || !stats || !kl || !dev_err || (K > 0 && !tlogp)) return VJSD_ERR_ARG;
    hipStream_t st = (hipStream_t)stream;
    for (int k = 0; k < S; ++k) {
        Shard sh = convert(shards[k], false, false);
        if ((e = hip_status(vjsd::launch_stats(dtype, 1, sh, N, part_of(part, k, N), st)))) return e;
    }
    if ((e = hip_status(vjsd::launch_merge(part_of(part, 0, N), S, N, 1, stats, st)))) return e;
    for (int k0 = 0; k0 < S; k0 += vjsd::LP_TABLE) {
        vjsd::LpTable tab = lp_table(shards, S, k0);
        if ((e = hip_status(vjsd::launch_topk_kl(dtype, tab, k0 == 0, N, vocab_global, ids, tlogp,
                                                 K, ignore_index, stats, kl, dev_err, st))))
            return e;
    }
    return VJSD_OK;
}

int vtopk_kl_bwd(const vjsd_shard *shards, int S, int64_t N, int dtype, int64_t vocab_global,
                 const double *stats, const int64_t *ids, const float *tlogp, int K,
                 int64_t ignore_index, const float *grad, float *part, void *stream) {
    int e = check_logprobs(shards, S, N, dtype, vocab_global, ids, K);
    if (e) return e;
    if ((e = check_views(shards, S, N, dtype, false, true))) return e;
    if (N == 0) return VJSD_OK;
    if (!stats || !part || !grad || (K > 0 && !tlogp)) return VJSD_ERR_ARG;
    vjsd::LpWeights w;
    w.tlogp = tlogp;
    w.grow = grad;
    return lp_backward(shards, S, N, dtype, vocab_global, stats, ids, K, ignore_index, w, part,
                       (hipStream_t)stream);
}

int vlin_gemm(int64_t M, int64_t N, int64_t K, vlin_operand a, vlin_operand b, void *c,
              int64_t ldc, int out, void *stream) {
    if (M < 0 || N < 0 || K < 0 || !gemm_size_ok(M, N)) return VJSD_ERR_ARG;
    if (out != VLIN_OUT_F32 && out != VLIN_OUT_F32_ACC && out != VLIN_OUT_BF16)
        return VJSD_ERR_ARG;
    int e = check_operand(a, M, K, true);
    if (e) return e;
    if ((e = check_operand(b, N, K, false))) return e;
    if (M == 0 || N == 0) return VJSD_OK;
    const size_t es = out == VLIN_OUT_BF16 ? 2 : 4;
    if (!c || reinterpret_cast<uintptr_t>(c) % es != 0 || ldc < N) return VJSD_ERR_ARG;
    vjsd::GemmArgs g;
    g.M = M;
    g.N = N;
    g.K = K;
    g.a = a.p;
    g.lda = a.ld;
    g.a_f32 = a.dtype == VJSD_F32;
    g.a_kmajor = a.kmajor;
    g.b = b.p;
    g.ldb = b.ld;
    g.b_kmajor = b.kmajor;
    g.c = c;
    g.ldc = ldc;
    g.out = out == VLIN_OUT_F32 ? vjsd::GEMM_F32
                                : (out == VLIN_OUT_F32_ACC ? vjsd::GEMM_F32_ACC : vjsd::GEMM_BF16);
    return hip_status(vjsd::launch_gemm(g, (hipStream_t)stream));
}

size_t vljsd_workspace_bytes(int64_t N, int64_t V, int64_t dim_s, int64_t chunk, int64_t group) {
    if (N < 0 || V < 1 || dim_s < 1 || chunk < 1 || group < 0) return 0;
    return lin_layout(N, V, dim_s, chunk, group).total;
}

int vljsd(const vlin_head *student, const vlin_head *teacher, int64_t N, int64_t V, double beta,
          const vjsd_loss_opts *opts, int64_t chunk, int64_t group, void *workspace, float *out,
          void *grad_h, int64_t ldgh, void *grad_w, int64_t ldgw, void *stream) {
    if (N < 0 || N > MAX_ROWS || V < 1 || chunk < 1 || group < 0 || !out) return VJSD_ERR_ARG;
    if (!(beta >= 0.0 && beta <= 1.0)) return VJSD_ERR_BETA;
    LossCfg c;
    int e = loss_cfg(opts, &c);
    if (e) return e;
    if ((e = check_head(student, N, V)) || (e = check_head(teacher, N, V))) return e;
    const int64_t D = student->dim;
    const bool grads = grad_h != nullptr || grad_w != nullptr;
    if (grads && c.red == VJSD_REDUCE_NONE) return VJSD_ERR_ARG;
    if (grad_h && (ldgh < D || reinterpret_cast<uintptr_t>(grad_h) % 2 != 0)) return VJSD_ERR_ARG;
    if (grad_w && (ldgw < D || reinterpret_cast<uintptr_t>(grad_w) % 2 != 0)) return VJSD_ERR_ARG;
    if (!gemm_size_ok(chunk < N ? chunk : N, V) || !gemm_size_ok(V, D)) return VJSD_ERR_ARG;
    hipStream_t st = (hipStream_t)stream;
    const vjsd::RowOpts ro = row_opts(c);
    if (N == 0) {
        if (grad_w) {  // d out / d w = 0: a product over no tokens
            vjsd::GemmArgs g;
            g.M = V;
            g.N = D;
            g.K = 0;
            g.c = grad_w;
            g.ldc = ldgw;
            g.out = vjsd::GEMM_BF16;
            if ((e = hip_status(vjsd::launch_gemm(g, st)))) return e;
        }
        if (c.red != VJSD_REDUCE_NONE)
            return hip_status(
                vjsd::launch_reduce_rows(nullptr, vjsd::RowOpts(), 0, false, out, nullptr, st));
        return VJSD_OK;
    }
    if (!workspace || reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return VJSD_ERR_ARG;
    const LinLayout L = lin_layout(N, V, D, chunk, group);
    char *ws = static_cast<char *>(workspace);
    float *ls = reinterpret_cast<float *>(ws + L.ls);
    float *lt = reinterpret_cast<float *>(ws + L.lt);
    uint16_t *G = reinterpret_cast<uint16_t *>(ws + L.g);
    uint16_t *Gt = reinterpret_cast<uint16_t *>(ws + L.gt);
    uint16_t *Ht = reinterpret_cast<uint16_t *>(ws + L.ht);
    uint16_t *Wt = reinterpret_cast<uint16_t *>(ws + L.wt);
    float *Hp = reinterpret_cast<float *>(ws + L.hp);
    float *rows = reinterpret_cast<float *>(ws + L.rows);
    double *stats = reinterpret_cast<double *>(ws + L.stats);
    float *kl = reinterpret_cast<float *>(ws + L.kl);
    float *part = reinterpret_cast<float *>(ws + L.part);
    double *count = reinterpret_cast<double *>(ws + L.count);
    float *gw = L.has_gw ? reinterpret_cast<float *>(ws + L.gw) : nullptr;
    const bool mean = c.red == VJSD_REDUCE_MEAN;
    if (grads && mean) {  // the kept-token count over all N, before any block's gradient
        if ((e = hip_status(vjsd::launch_reduce_rows(nullptr, ro, N, false, nullptr, count, st))))
            return e;
    }
    float *rows_out = c.red == VJSD_REDUCE_NONE ? out : rows;
    const int mode = mode_of(beta);
    const int64_t C = L.C, NG = L.NG, ngroups = (N + NG - 1) / NG;
    if (grad_h) {  // w_s^T [D][V], once: the hidden-gradient products read it k-major
        if ((e = hip_status(vjsd::launch_transpose16(static_cast<const uint16_t *>(student->w),
                                                      student->ldw, V, D, Wt, L.ldv, st))))
            return e;
    }
    const uint16_t *hs = static_cast<const uint16_t *>(student->h);
    const uint16_t *ht = static_cast<const uint16_t *>(teacher->h);
    for (int64_t grp = 0; grp < ngroups; ++grp) {
        const int64_t g0 = grp * NG, gn = N - g0 < NG ? N - g0 : NG;
        for (int64_t n0 = g0; n0 < g0 + gn; n0 += C) {
            const int64_t nb = g0 + gn - n0 < C ? g0 + gn - n0 : C;
            // the block's logits, student and teacher
            for (int side = 0; side < 2; ++side) {
                const vlin_head *hd = side == 0 ? student : teacher;
                vjsd::GemmArgs g;
                g.M = nb;
                g.N = V;
                g.K = hd->dim;
                g.a = (side == 0 ? hs : ht) + n0 * hd->ldh;
                g.lda = hd->ldh;
                g.b = hd->w;
                g.ldb = hd->ldw;
                g.c = side == 0 ? ls : lt;
                g.ldc = L.ldl;
                g.out = vjsd::GEMM_F32;
                if ((e = hip_status(vjsd::launch_gemm(g, st)))) return e;
            }
            // the block's per-token loss
            Shard sh;
            sh.start = 0;
            sh.width = V;
            sh.s = {ls, L.ldl, 0, 0};
            sh.t = {lt, L.ldl, 0, 0};
            sh.gs = {G, L.ldl, 0, 0};
            sh.gt = {nullptr, 0, 0, 0};
            vjsd::RowOpts rb = ro;
            rb.mask = ro.mask ? ro.mask + n0 : nullptr;
            // the logit gradient (bf16) for a unit upstream gradient of out[0]
            vjsd::GradOpts go;
            go.ks = ro.ks;
            go.gmul = (c.t2 ? c.T * c.T : 1.0) / c.T;
            go.scalar = true;
            go.mask = rb.mask;
            go.count = mean ? count : nullptr;
            if (grads && mode == vjsd::INTERIOR && !rb.mask) {
                // forward and G in one launch: the block's gradient sweep re-reads what the
                // divergence sweep left in the caches
                if ((e = hip_status(vjsd::launch_fwd_bwd_f32_bf16(sh, nb, beta, stats, kl,
                                                                  rows_out + n0, st, rb, go))))
                    return e;
            } else if (mode != vjsd::INTERIOR) {
                const int rev = mode == vjsd::REV_KL;
                if ((e = hip_status(vjsd::launch_kl1(VJSD_F32, rev, sh, nb, part_of(part, 0, nb),
                                                     st, rb))))
                    return e;
                if ((e = hip_status(vjsd::launch_kl1_merge(rev, part_of(part, 0, nb), 1, nb,
                                                           stats, kl, rows_out + n0, st, rb))))
                    return e;
            } else if ((e = hip_status(vjsd::launch_fwd_fused(VJSD_F32, sh, nb, beta, stats, kl,
                                                               rows_out + n0, st, rb)))) {
                return e;
            }
            if (!grads) continue;
            if (mode != vjsd::INTERIOR || rb.mask) {
                if ((e = hip_status(vjsd::launch_bwd_prep(mode, nb, stats, kl, beta, nullptr,
                                                          part, st, go))))
                    return e;
                if ((e = hip_status(vjsd::launch_bwd_f32_to_bf16(mode, sh, nb, part, st))))
                    return e;
            }
            if (grad_h) {  // G [nb][V] x (w_s^T)^T: both operands k-major
                vjsd::GemmArgs g;
                g.M = nb;
                g.N = D;
                g.K = V;
                g.a = G;
                g.lda = L.ldl;
                g.b = Wt;
                g.ldb = L.ldv;
                uint16_t *dst = static_cast<uint16_t *>(grad_h) + n0 * ldgh;
                const int S = lin_splits(nb, V, D) < L.splits ? lin_splits(nb, V, D) : L.splits;
                if (S > 1) {  // fp32 partials of the K split, then their sum in split order
                    g.ksplit = S;
                    g.split_stride = nb * D;
                    g.c = Hp;
                    g.ldc = D;
                    g.out = vjsd::GEMM_F32;
                    if ((e = hip_status(vjsd::launch_gemm(g, st))) ||
                        (e = hip_status(vjsd::launch_sum_partials(Hp, S, nb * D, nb, D, D, dst,
                                                                  ldgh, st))))
                        return e;
                } else {
                    g.c = dst;
                    g.ldc = ldgh;
                    g.out = vjsd::GEMM_BF16;
                    if ((e = hip_status(vjsd::launch_gemm(g, st)))) return e;
                }
            }
            if (grad_w) {  // the chunk's G and hidden states into the group's transposes
                const int64_t off = n0 - g0;  // a multiple of 8 (lin_layout)
                if ((e = hip_status(vjsd::launch_transpose16(G, L.ldl, nb, V, Gt + off, L.ldt,
                                                              st))) ||
                    (e = hip_status(vjsd::launch_transpose16(hs + n0 * student->ldh,
                                                              student->ldh, nb, D, Ht + off,
                                                              L.ldt, st))))
                    return e;
            }
        }
        if (!grads || !grad_w) continue;
        {  // G^T [V][gn] x h_s [gn][D], summed over the groups in fp32
            vjsd::GemmArgs g;
            g.M = V;
            g.N = D;
            g.K = gn;
            g.a = Gt;
            g.lda = L.ldt;
            g.b = Ht;
            g.ldb = L.ldt;
            if (ngroups == 1 || grp == ngroups - 1) {
                g.c = grad_w;
                g.ldc = ldgw;
                g.out = ngroups == 1 ? vjsd::GEMM_BF16 : vjsd::GEMM_BF16_ACC;
                g.addend = gw;
                g.ldadd = D;
            } else {
                g.c = gw;
                g.ldc = D;
                g.out = grp == 0 ? vjsd::GEMM_F32 : vjsd::GEMM_F32_ACC;
            }
            if ((e = hip_status(vjsd::launch_gemm(g, st)))) return e;
        }
    }
    if (c.red == VJSD_REDUCE_NONE) return VJSD_OK;
    return hip_status(vjsd::launch_reduce_rows(rows, ro, N, mean, out, nullptr, st));
}

int vlin_scale(void *p, int64_t n, int dtype, const float *g, void *stream) {
    if (dtype != VJSD_F32 && dtype != VJSD_F16 && dtype != VJSD_BF16) return VJSD_ERR_DTYPE;
    if (n < 0) return VJSD_ERR_ARG;
    if (n == 0) return VJSD_OK;
    if (!p || !g || reinterpret_cast<uintptr_t>(p) % 16 != 0) return VJSD_ERR_ARG;
    return hip_status(vjsd::launch_scale(dtype, p, n, g, (hipStream_t)stream));
}

}  // extern "C"
