// siblings.hip -- the sibling ops on the same statistics engine: single-pass KL and
// entropy forwards, the entropy backward, and per-id / top-k log-probabilities.
//
// [OPS-PR] DeepSpeed PR #8791 "Add vocabulary-parallel logprobs, entropy and KL ops":
// section What (the three ops, ignore_index positions return 0), section How (MAX and
// SUM of [N] statistics, -inf tokens add nothing, fully -inf rows give NaN and zero
// gradient, closed-form local backward), review thread (empty shards join the merge;
// log-probabilities reject them; the index range check runs every call).
// [JSD-PR] DeepSpeed PR #8958 "[VocabTP] Add vocabulary-parallel generalized JSD with
// Triton kernels", section Scope and limitations: KL's forward is a single input pass.
//
// Single-pass accumulation keeps every running sum relative to the running maxima and
// rebases it when a maximum grows, so no large offset enters a sum.
#include "kernels.hpp"
#include "sweep.hpp"

namespace vjsd {

namespace {

// ---- single-pass KL(p_a || p_b) ---------------------------------------------------
// a is the target side (teacher for forward KL, student for reverse KL).
// A = sum e_a (u_a - u_b) relative to the current reference points (c_a, c_b);
// F = max (u_a - u_b) over raw values: +inf iff some a > -inf meets b = -inf.
struct OpKL1 {
    float ma = NINF, ca = 0.0f, za = 0.0f;
    float mb = NINF, cb = 0.0f, zb = 0.0f;
    float A = 0.0f, F = NINF;
    float ks = L2E;  // log2 e / temperature

    template <int NV, int W>
    __device__ __forceinline__ void run(const float (&xa)[NV][W], const float (&xb)[NV][W],
                                        const int64_t (&)[NV]) {
        constexpr int N = NV * W;
        const float *a = &xa[0][0], *b = &xb[0][0];
        float bma = a[0], bmb = b[0];
#pragma unroll
        for (int i = 1; i < N; ++i) {
            bma = fmaxf(bma, a[i]);
            bmb = fmaxf(bmb, b[i]);
        }
        const float nma = fmaxf(ma, bma), nmb = fmaxf(mb, bmb);
        const float nca = refc(nma, ks), ncb = refc(nmb, ks);
        const float sa = ma == NINF ? 0.0f : ex2(ca - nca);
        const float sb = mb == NINF ? 0.0f : ex2(cb - ncb);
        A = sa * fmaf((ca - nca) - (cb - ncb), za, A);
        float ea[N], eb[N], pa = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const float uar = fmaf(a[i], ks, -nca), ubr = fmaf(b[i], ks, -ncb);
            F = fmaxf(F, uar - ubr);
            const float ua = fmaxf(uar, U_FLOOR), ub = fmaxf(ubr, U_FLOOR);
            ea[i] = ex2(ua);
            eb[i] = ex2(ub);
            pa = fmaf(ea[i], ua - ub, pa);
        }
#pragma unroll
        for (int st = N / 2; st >= 1; st /= 2)
#pragma unroll
            for (int i = 0; i < st; ++i) {
                ea[i] += ea[i + st];
                eb[i] += eb[i + st];
            }
        za = fmaf(za, sa, ea[0]);
        zb = fmaf(zb, sb, eb[0]);
        A += pa;
        ma = nma;
        ca = nca;
        mb = nmb;
        cb = ncb;
    }
};

// Combine two (m_a, z_a, m_b, z_b, A, F) partials, the first argument first.
struct KLPart {
    float ma, za, mb, zb, A, F;
};
__device__ __forceinline__ KLPart kl_combine(KLPart x, KLPart y, float ks) {
    KLPart o;
    o.ma = fmaxf(x.ma, y.ma);
    o.mb = fmaxf(x.mb, y.mb);
    const float ca = refc(o.ma, ks), cb = refc(o.mb, ks);
    o.za = 0.0f;
    o.zb = 0.0f;
    o.A = 0.0f;
    const KLPart *in[2] = {&x, &y};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const KLPart &p = *in[q];
        if (p.mb != NINF) o.zb += p.zb * ex2(refc(p.mb, ks) - cb);
        if (p.ma != NINF) {
            const float da = refc(p.ma, ks) - ca;
            const float db = p.mb == NINF ? 0.0f : refc(p.mb, ks) - cb;
            const float sc = ex2(da);
            o.za += p.za * sc;
            o.A += sc * fmaf(da - db, p.za, p.A);
        }
    }
    o.F = fmaxf(x.F, y.F);
    return o;
}

template <class D, bool REV>
__global__ __launch_bounds__(BLOCK) void k_kl1(RowView sv, RowView tv, int64_t w,
                                               float *__restrict__ part_k, RowOpts ro) {
    using T = typename D::T;
    __shared__ float red[6 * NWAVE];
    const int64_t r = blockIdx.x;
    KLPart p{NINF, 0.0f, NINF, 0.0f, 0.0f, NINF};
    if (w > 0 && !row_dropped(ro, r)) {
        const T *s = row_ptr<T>(sv, r), *t = row_ptr<T>(tv, r);
        const T *a = REV ? s : t, *b = REV ? t : s;
        OpKL1 op;
        op.ks = ro.ks;
        sweep<D, 4, true, BLOCK, true>(a, b, w, head_len<T>(w, a, b), op);
        p = {op.ma, op.za, op.mb, op.zb, op.A, op.F};
        // wave reduction in lane order, then waves in order
        const float ks = ro.ks;
        p = wave_reduce<true>(p, [ks](const KLPart &x, const KLPart &y) { return kl_combine(x, y, ks); });
        const int wave = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) {
            float *d = red + 6 * wave;
            d[0] = p.ma; d[1] = p.za; d[2] = p.mb; d[3] = p.zb; d[4] = p.A; d[5] = p.F;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            p = {red[0], red[1], red[2], red[3], red[4], red[5]};
            for (int q = 1; q < NWAVE; ++q) {
                const float *d = red + 6 * q;
                p = kl_combine(p, KLPart{d[0], d[1], d[2], d[3], d[4], d[5]}, ro.ks);
            }
        }
    }
    if (threadIdx.x == 0) {
        float *o = part_k + r * PART_STRIDE;
        o[0] = p.ma; o[1] = p.za; o[2] = p.mb; o[3] = p.zb; o[4] = p.A; o[5] = p.F;
    }
}

__global__ void k_kl1_merge(int rev, const float *__restrict__ part, int S, int64_t N,
                            double *__restrict__ stats, float *__restrict__ kl,
                            float *__restrict__ loss, RowOpts ro) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= N) return;
    if (row_dropped(ro, r)) {
        double *o = stats + r * 4;
        o[0] = o[1] = o[2] = o[3] = -__builtin_inf();
        masked_row(kl + 2 * r, loss + r);
        return;
    }
    const float ks = ro.ks;
    float ma = NINF, mb = NINF, F = NINF;
    for (int k = 0; k < S; ++k) {
        const float *p = part + ((int64_t)k * N + r) * PART_STRIDE;
        ma = fmaxf(ma, p[0]);
        mb = fmaxf(mb, p[2]);
        F = fmaxf(F, p[5]);
    }
    const double ca = refc(ma, ks), cb = refc(mb, ks);
    double Za = 0.0, Zb = 0.0, A = 0.0;
    for (int k = 0; k < S; ++k) {
        const float *p = part + ((int64_t)k * N + r) * PART_STRIDE;
        if (p[2] != NINF) Zb += (double)p[3] * exp2((double)refc(p[2], ks) - cb);
        if (p[0] != NINF) {
            const double da = (double)refc(p[0], ks) - ca;
            const double db = p[2] == NINF ? 0.0 : (double)refc(p[2], ks) - cb;
            const double sc = exp2(da);
            Za += (double)p[1] * sc;
            A += sc * ((double)p[4] + (da - db) * (double)p[1]);
        }
    }
    const bool undefined = ma == NINF || mb == NINF;
    const double lza = undefined ? 0.0 : log2(Za), lzb = undefined ? 0.0 : log2(Zb);
    double v;
    if (undefined) v = __builtin_nan("");
    else if (F == __builtin_huge_valf()) v = __builtin_inf();
    else v = (A / Za - lza + lzb) * LN2_D;  // sum p_a (lp_a - lp_b), base 2 then nats
    // statistics: a is the teacher for forward KL, the student for reverse KL
    const float ms = rev ? ma : mb, mt = rev ? mb : ma;
    const double Zs = rev ? Za : Zb, Zt = rev ? Zb : Za;
    double *o = stats + r * 4;
    o[0] = ms;
    o[1] = ms == NINF ? -__builtin_inf() : lnz_from_z(ms, Zs, ks);
    o[2] = mt;
    o[3] = mt == NINF ? -__builtin_inf() : lnz_from_z(mt, Zt, ks);
    kl[2 * r] = rev ? 0.0f : (float)v;
    kl[2 * r + 1] = rev ? (float)v : 0.0f;
    if (undefined) kl[2 * r] = kl[2 * r + 1] = __builtin_nanf("");
    loss[r] = (float)(v * (double)ro.lscale);
}

// ---- single-pass entropy ------------------------------------------------------------
// B = sum e u relative to the running reference point; H / ln2 = log2 Z - B / Z.
struct OpEnt1 {
    float m = NINF, c = 0.0f, z = 0.0f, B = 0.0f;

    template <int NV, int W>
    __device__ __forceinline__ void run(const float (&xa)[NV][W], const float (&)[NV][W],
                                        const int64_t (&)[NV]) {
        constexpr int N = NV * W;
        const float *x = &xa[0][0];
        float bm = x[0];
#pragma unroll
        for (int i = 1; i < N; ++i) bm = fmaxf(bm, x[i]);
        const float nm = fmaxf(m, bm), nc = refc(nm);
        const float sc = m == NINF ? 0.0f : ex2(c - nc);
        B = sc * fmaf(c - nc, z, B);
        float e[N], pb = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const float u = fmaxf(fmaf(x[i], L2E, -nc), U_FLOOR);
            e[i] = ex2(u);
            pb = fmaf(e[i], u, pb);
        }
#pragma unroll
        for (int st = N / 2; st >= 1; st /= 2)
#pragma unroll
            for (int i = 0; i < st; ++i) e[i] += e[i + st];
        z = fmaf(z, sc, e[0]);
        B += pb;
        m = nm;
        c = nc;
    }
};

struct EntPart {
    float m, z, B;
};
__device__ __forceinline__ EntPart ent_combine(EntPart x, EntPart y) {
    EntPart o{fmaxf(x.m, y.m), 0.0f, 0.0f};
    const float c = refc(o.m);
    const EntPart *in[2] = {&x, &y};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const EntPart &p = *in[q];
        if (p.m != NINF) {
            const float d = refc(p.m) - c;
            const float sc = ex2(d);
            o.z += p.z * sc;
            o.B += sc * fmaf(d, p.z, p.B);
        }
    }
    return o;
}

template <class D>
__global__ __launch_bounds__(BLOCK) void k_ent1(RowView xv, int64_t w, float *__restrict__ part_k) {
    using T = typename D::T;
    __shared__ float red[3 * NWAVE];
    const int64_t r = blockIdx.x;
    EntPart p{NINF, 0.0f, 0.0f};
    if (w > 0) {
        const T *x = row_ptr<T>(xv, r);
        OpEnt1 op;
        sweep<D, 4, false, BLOCK, true>(x, x, w, head_len<T>(w, x), op);
        p = {op.m, op.z, op.B};
        p = wave_reduce<true>(p, [](const EntPart &x, const EntPart &y) { return ent_combine(x, y); });
        const int wave = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) {
            red[3 * wave] = p.m;
            red[3 * wave + 1] = p.z;
            red[3 * wave + 2] = p.B;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            p = {red[0], red[1], red[2]};
            for (int q = 1; q < NWAVE; ++q)
                p = ent_combine(p, EntPart{red[3 * q], red[3 * q + 1], red[3 * q + 2]});
        }
    }
    if (threadIdx.x == 0) {
        float *o = part_k + r * PART_STRIDE;
        o[0] = p.m; o[1] = p.z; o[2] = p.B;
    }
}

__global__ void k_ent1_merge(const float *__restrict__ part, int S, int64_t N,
                             double *__restrict__ stats, float *__restrict__ ent) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= N) return;
    float m = NINF;
    for (int k = 0; k < S; ++k) m = fmaxf(m, part[((int64_t)k * N + r) * PART_STRIDE]);
    const double c = refc(m);
    double Z = 0.0, B = 0.0;
    for (int k = 0; k < S; ++k) {
        const float *p = part + ((int64_t)k * N + r) * PART_STRIDE;
        if (p[0] != NINF) {
            const double d = (double)refc(p[0]) - c;
            const double sc = exp2(d);
            Z += (double)p[1] * sc;
            B += sc * ((double)p[2] + d * (double)p[1]);
        }
    }
    double *o = stats + r * 4;
    o[0] = m;
    if (m == NINF) {
        o[1] = -__builtin_inf();
        ent[r] = __builtin_nanf("");
    } else {
        o[1] = lnz_from_z(m, Z);
        ent[r] = (float)((log2(Z) - B / Z) * LN2_D);
    }
}

// d/dx = -g p (lp + H) = (-g ln2 / Z) e (u - R),  R = log2 Z - H / ln2
template <class D>
struct OpEntBwd {
    using T = typename D::T;
    T *gx;
    float c, C, R;
    template <int NV, int W>
    __device__ __forceinline__ void run(const float (&x)[NV][W], const float (&)[NV][W],
                                        const int64_t (&col)[NV]) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            float o[W];
#pragma unroll
            for (int i = 0; i < W; ++i) {
                const float u = fmaxf(fmaf(x[j][i], L2E, -c), U_FLOOR);
                o[i] = (C * ex2(u)) * (u - R);
            }
            if constexpr (W == D::VEC) store_vec<D, true>(gx + col[j], o);
            else
#pragma unroll
                for (int i = 0; i < W; ++i) store1<D>(gx + col[j] + i, o[i]);
        }
    }
};

// rowc: c, C, R and the undefined flag
__global__ void k_ent_bwd_prep(int64_t N, const double *__restrict__ stats,
                               const float *__restrict__ ent, const float *__restrict__ grad,
                               float *__restrict__ rowc) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= N) return;
    const float m = (float)stats[r * 4];
    float *o = rowc + r * ROWC;
    o[ROWC_UNDEFINED] = m == NINF ? 1.0f : 0.0f;
    if (m == NINF) return;
    const double Z = z_from_stats(m, stats[r * 4 + 1]);
    o[0] = refc(m);
    o[1] = (float)(-(double)grad[r] * LN2_D / Z);
    o[2] = (float)(log2(Z) - (double)ent[r] * L2E_D);
}

template <class D>
__global__ __launch_bounds__(GRAD_BLOCK) void k_ent_bwd(RowView xv, RowMView gv, int64_t w,
                                                        int64_t cw, int64_t nchunk,
                                                        const float *__restrict__ rowc) {
    using T = typename D::T;
    const int64_t b = blockIdx.x;
    const int64_t r = b / nchunk;
    const T *xrow = row_ptr<T>(xv, r);
    int64_t c0, n;
    chunk_span<false>(xrow, w, cw, b - r * nchunk, c0, n);
    if (n <= 0) return;
    const float *k = rowc + r * ROWC;
    T *gx = row_ptr<T>(gv, r) + c0;
    if (k[ROWC_UNDEFINED] != 0.0f) {
        zero_span<D, GRAD_BLOCK>(gx, n);
        return;
    }
    const T *x = xrow + c0;
    OpEntBwd<D> op;
    op.gx = gx;
    op.c = k[0];
    op.C = k[1];
    op.R = k[2];
    sweep<D, 1, false, GRAD_BLOCK, true>(x, x, n, head_len<T>(n, x, gx), op);
}

// ---- log-probabilities ----------------------------------------------------------------

// One thread per (row, k).  The first launch of a call also resolves ignore_index
// (exactly 0) and out-of-range ids (error flag); every launch gathers the ids its
// table of shards owns: lp = (x - m) - lnZ in fp64.
template <class D>
__global__ void k_lp_gather(LpTable tab, int first, int64_t N, int64_t vocab_global,
                            const int64_t *__restrict__ ids, int K, int64_t ignore,
                            const double *__restrict__ stats, float *__restrict__ out,
                            int32_t *__restrict__ dev_err, float sign) {
    using T = typename D::T;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= N * K) return;
    const int64_t r = i / K;
    const int64_t id = ids[i];
    if (id == ignore) {
        if (first) out[i] = 0.0f;
        return;
    }
    if (id < 0 || id >= vocab_global) {
        if (first) {
            out[i] = __builtin_nanf("");
            *dev_err = 1;
        }
        return;
    }
    for (int q = 0; q < tab.n; ++q) {
        if (id >= tab.start[q] && id < tab.start[q] + tab.width[q]) {
            const double m = stats[r * 4], lz = stats[r * 4 + 1];
            if (m == -__builtin_inf()) {
                out[i] = __builtin_nanf("");
            } else {
                const double x = load1<D>(row_ptr<T>(tab.x[q], r) + (id - tab.start[q]));
                out[i] = (float)((double)sign * ((x - m) - lz));
            }
            return;
        }
    }
}

// Teacher top-k forward KL ([OPS-PR, What]: the teacher top-k forward KL built on the
// log-probabilities of the teacher's top-k ids).  One thread per row sums, in fp64,
// exp(t_k) (t_k - lp_s(id_k)) over the slots whose id this table of shards owns; a slot
// is padding when id_k == ignore or t_k == -inf.  A student logit of -inf under
// teacher mass makes the row +inf; an undefined student row is NaN; an id outside
// [0, vocab_global) raises the error flag (first launch) and makes the row NaN.  The
// first launch of a call writes kl, later launches (more shards) add to it.
template <class D>
__global__ void k_topk_kl(LpTable tab, int first, int64_t N, int64_t vocab_global,
                          const int64_t *__restrict__ ids, const float *__restrict__ tlogp, int K,
                          int64_t ignore, const double *__restrict__ stats,
                          float *__restrict__ kl, int32_t *__restrict__ dev_err) {
    using T = typename D::T;
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= N) return;
    const double m = stats[r * 4], lz = stats[r * 4 + 1];
    const bool undefined = m == -__builtin_inf();
    double acc = 0.0;
    bool bad = false, inf = false;
    for (int k = 0; k < K; ++k) {
        const int64_t id = ids[r * K + k];
        if (id == ignore) continue;
        if (id < 0 || id >= vocab_global) {
            if (first) {
                *dev_err = 1;
                bad = true;
            }
            continue;
        }
        const float t = tlogp[r * K + k];
        if (t == -__builtin_huge_valf()) continue;  // no teacher mass
        if (t != t) bad = true;                     // NaN propagates
        for (int q = 0; q < tab.n; ++q) {
            if (id < tab.start[q] || id >= tab.start[q] + tab.width[q]) continue;
            if (!undefined) {
                const double x = load1<D>(row_ptr<T>(tab.x[q], r) + (id - tab.start[q]));
                if (x == -__builtin_inf()) inf = true;
                else acc += exp((double)t) * ((double)t - ((x - m) - lz));
            }
            break;
        }
    }
    const float part = bad ? __builtin_nanf("") : (inf ? __builtin_huge_valf() : (float)acc);
    if (first) kl[r] = undefined ? __builtin_nanf("") : part;
    else kl[r] += part;
}

// d/dx_j = -G p_j everywhere (G = sum of the valid upstream gradients), then the ids a
// chunk owns are rewritten as (sum of their g) - G p_j, rounded once.
template <class D>
struct OpLpBwd {
    using T = typename D::T;
    T *gx;
    float c, C;
    template <int NV, int W>
    __device__ __forceinline__ void run(const float (&x)[NV][W], const float (&)[NV][W],
                                        const int64_t (&col)[NV]) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            float o[W];
#pragma unroll
            for (int i = 0; i < W; ++i) o[i] = C * ex2(fmaxf(fmaf(x[j][i], L2E, -c), U_FLOOR));
            if constexpr (W == D::VEC) store_vec<D, true>(gx + col[j], o);
            else
#pragma unroll
                for (int i = 0; i < W; ++i) store1<D>(gx + col[j] + i, o[i]);
        }
    }
};

// rowc: c, C = -G / Z, 1 / Z, G and the undefined flag
__global__ void k_lp_bwd_prep(int64_t N, int64_t vocab_global, const double *__restrict__ stats,
                              const int64_t *__restrict__ ids, int K, int64_t ignore,
                              LpWeights wts, float *__restrict__ rowc) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= N) return;
    const float m = (float)stats[r * 4];
    float *o = rowc + r * ROWC;
    double G = 0.0;
    bool any = false;  // a row with no valid slot gets exactly 0 without being read
    for (int k = 0; k < K; ++k) {
        const int64_t id = ids[r * K + k];
        if (id != ignore && id >= 0 && id < vocab_global) {
            G += lp_weight(wts, r, K, k);
            any = true;
        }
    }
    o[ROWC_UNDEFINED] = (m == NINF || !any) ? 1.0f : 0.0f;
    if (m == NINF || !any) return;
    const double Z = z_from_stats(m, stats[r * 4 + 1]);
    o[0] = refc(m);
    o[1] = (float)(-G / Z);
    o[2] = (float)(1.0 / Z);
    o[3] = (float)G;
}

// The value v holds in lane q (q uniform across the wave).
__device__ __forceinline__ int64_t lane_value(int64_t v, int q) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, q);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), q);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

template <class D>
__global__ __launch_bounds__(GRAD_BLOCK) void k_lp_bwd(RowView xv, RowMView gv, int64_t start,
                                                       int64_t w, int64_t cw, int64_t nchunk,
                                                       const int64_t *__restrict__ ids, int K,
                                                       int64_t ignore, LpWeights wts,
                                                       const float *__restrict__ rowc) {
    using T = typename D::T;
    const int64_t b = blockIdx.x;
    const int64_t r = b / nchunk;
    const T *xrow = row_ptr<T>(xv, r);
    int64_t c0, n;
    chunk_span<false>(xrow, w, cw, b - r * nchunk, c0, n);
    if (n <= 0) return;
    const float *k = rowc + r * ROWC;
    T *gx = row_ptr<T>(gv, r) + c0;
    if (k[ROWC_UNDEFINED] != 0.0f) {
        zero_span<D, GRAD_BLOCK>(gx, n);
        return;
    }
    const T *x = xrow + c0;
    // the first GRAD_BLOCK ids are loaded before the sweep, so their latency overlaps
    // the chunk's loads instead of trailing them
    const int64_t *id = ids + r * K;
    const int64_t id0 = (int)threadIdx.x < K ? id[threadIdx.x] : ignore;
    constexpr int VEC = D::VEC;
    if (K <= GRAD_BLOCK && n == (int64_t)GRAD_BLOCK * VEC && head_len<T>(n, x, gx) == 0) {
        // A whole chunk of aligned vectors (every chunk but a row's last): one vector
        // per lane, every id in one lane.  A ballot over the ids finds the few this
        // chunk owns, their values are written into the registers, and the chunk is
        // stored once: no fix-up store has to wait for the streamed one to land.
        const int lane = threadIdx.x;
        const u32x4 raw = ld16<true>(x + lane * VEC);
        const int64_t j0 = id0 - start - c0;
        uint64_t hits = __ballot(lane < K && id0 != ignore && j0 >= 0 && j0 < n);
        float xv[VEC], o[VEC];
        widen<D>(raw, xv);
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = k[1] * ex2(fmaxf(fmaf(xv[e], L2E, -k[0]), U_FLOOR));
        while (hits) {  // uniform: the ids this chunk owns, usually none
            const int q = __builtin_ctzll(hits);
            hits &= hits - 1;
            const int64_t idq = lane_value(id0, q);
            float gsum = 0.0f;  // repeated ids accumulate, in slot order
            for (int q2 = 0; q2 < K; ++q2)
                if (lane_value(id0, q2) == idq) gsum += lp_weight(wts, r, K, q2);
            const int64_t j = idq - start - c0;
            if (lane == (int)(j / VEC)) {
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    if (e == (int)(j % VEC)) {
                        const float p = ex2(fmaxf(fmaf(xv[e], L2E, -k[0]), U_FLOOR)) * k[2];
                        o[e] = gsum - k[3] * p;
                    }
            }
        }
        store_vec<D, true>(gx + lane * VEC, o);
        return;
    }
    OpLpBwd<D> op;
    op.gx = gx;
    op.c = k[0];
    op.C = k[1];
    sweep<D, 1, false, GRAD_BLOCK, true>(x, x, n, head_len<T>(n, x, gx), op);
    __syncthreads();  // this chunk's streamed values land before the id fix-ups
    for (int q = threadIdx.x; q < K; q += GRAD_BLOCK) {
        const int64_t idq = q < GRAD_BLOCK ? id0 : id[q];
        const int64_t j = idq - start - c0;
        if (idq == ignore || j < 0 || j >= n) continue;
        float gsum = 0.0f;
        for (int q2 = 0; q2 < K; ++q2)
            if (id[q2] == idq) gsum += lp_weight(wts, r, K, q2);
        const float p = ex2(fmaxf(fmaf(load1<D>(x + j), L2E, -op.c), U_FLOOR)) * k[2];
        store1<D>(gx + j, gsum - k[3] * p);
    }
}

template <class D>
hipError_t kl1_dt(int rev, const Shard &sh, int64_t N, float *part_k, hipStream_t st,
                  const RowOpts &o) {
    if (rev)
        hipLaunchKernelGGL((k_kl1<D, true>), dim3((unsigned)N), dim3(BLOCK), 0, st, sh.s, sh.t,
                           sh.width, part_k, o);
    else
        hipLaunchKernelGGL((k_kl1<D, false>), dim3((unsigned)N), dim3(BLOCK), 0, st, sh.s, sh.t,
                           sh.width, part_k, o);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kl1(int dtype, int reverse, const Shard &sh, int64_t N, float *part_k,
                      hipStream_t st, const RowOpts &o) {
    switch (dtype) {
        case 0: return kl1_dt<F32>(reverse, sh, N, part_k, st, o);
        case 1: return kl1_dt<F16>(reverse, sh, N, part_k, st, o);
        default: return kl1_dt<BF16>(reverse, sh, N, part_k, st, o);
    }
}

hipError_t launch_kl1_merge(int reverse, const float *part, int S, int64_t N, double *stats,
                            float *kl, float *loss, hipStream_t st, const RowOpts &o) {
    hipLaunchKernelGGL(k_kl1_merge, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, st,
                       reverse, part, S, N, stats, kl, loss, o);
    return hipGetLastError();
}

hipError_t launch_ent1(int dtype, const Shard &sh, int64_t N, float *part_k, hipStream_t st) {
    const dim3 grid((unsigned)N), block(BLOCK);
    switch (dtype) {
        case 0: hipLaunchKernelGGL(k_ent1<F32>, grid, block, 0, st, sh.s, sh.width, part_k); break;
        case 1: hipLaunchKernelGGL(k_ent1<F16>, grid, block, 0, st, sh.s, sh.width, part_k); break;
        default: hipLaunchKernelGGL(k_ent1<BF16>, grid, block, 0, st, sh.s, sh.width, part_k);
    }
    return hipGetLastError();
}

hipError_t launch_ent1_merge(const float *part, int S, int64_t N, double *stats, float *ent,
                             hipStream_t st) {
    hipLaunchKernelGGL(k_ent1_merge, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, st, part, S,
                       N, stats, ent);
    return hipGetLastError();
}

hipError_t launch_ent_bwd_prep(int64_t N, const double *stats, const float *ent,
                               const float *grad, float *rowc, hipStream_t st) {
    hipLaunchKernelGGL(k_ent_bwd_prep, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, st, N,
                       stats, ent, grad, rowc);
    return hipGetLastError();
}

hipError_t launch_ent_bwd(int dtype, const Shard &sh, int64_t N, const float *rowc,
                          hipStream_t st) {
    const Chunks ch = grad_chunks<false>(N, sh.width, dtype == 0 ? 4 : 2);
    if (ch.nchunk == 0) return hipSuccess;
    const dim3 grid((unsigned)(N * ch.nchunk)), block(GRAD_BLOCK);
    switch (dtype) {
        case 0: hipLaunchKernelGGL(k_ent_bwd<F32>, grid, block, 0, st, sh.s, sh.gs, sh.width, ch.cw, ch.nchunk, rowc); break;
        case 1: hipLaunchKernelGGL(k_ent_bwd<F16>, grid, block, 0, st, sh.s, sh.gs, sh.width, ch.cw, ch.nchunk, rowc); break;
        default: hipLaunchKernelGGL(k_ent_bwd<BF16>, grid, block, 0, st, sh.s, sh.gs, sh.width, ch.cw, ch.nchunk, rowc);
    }
    return hipGetLastError();
}

hipError_t launch_lp_gather(int dtype, const LpTable &tab, bool first, int64_t N,
                            int64_t vocab_global, const int64_t *ids, int K, int64_t ignore,
                            const double *stats, float *out, int32_t *dev_err, hipStream_t st,
                            float sign) {
    const int64_t n = N * K;
    const dim3 grid((unsigned)((n + 255) / 256)), block(256);
    const int f = first ? 1 : 0;
    switch (dtype) {
        case 0: hipLaunchKernelGGL(k_lp_gather<F32>, grid, block, 0, st, tab, f, N, vocab_global, ids, K, ignore, stats, out, dev_err, sign); break;
        case 1: hipLaunchKernelGGL(k_lp_gather<F16>, grid, block, 0, st, tab, f, N, vocab_global, ids, K, ignore, stats, out, dev_err, sign); break;
        default: hipLaunchKernelGGL(k_lp_gather<BF16>, grid, block, 0, st, tab, f, N, vocab_global, ids, K, ignore, stats, out, dev_err, sign);
    }
    return hipGetLastError();
}

hipError_t launch_lp_bwd_prep(int64_t N, int64_t vocab_global, const double *stats,
                              const int64_t *ids, int K, int64_t ignore, const LpWeights &w,
                              float *rowc, hipStream_t st) {
    hipLaunchKernelGGL(k_lp_bwd_prep, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, st, N,
                       vocab_global, stats, ids, K, ignore, w, rowc);
    return hipGetLastError();
}

hipError_t launch_lp_bwd(int dtype, const Shard &sh, int64_t N, const int64_t *ids, int K,
                         int64_t ignore, const LpWeights &w, const float *rowc, hipStream_t st) {
    const Chunks ch = grad_chunks<false>(N, sh.width, dtype == 0 ? 4 : 2);
    if (ch.nchunk == 0) return hipSuccess;
    const dim3 grid((unsigned)(N * ch.nchunk)), block(GRAD_BLOCK);
    switch (dtype) {
        case 0: hipLaunchKernelGGL(k_lp_bwd<F32>, grid, block, 0, st, sh.s, sh.gs, sh.start, sh.width, ch.cw, ch.nchunk, ids, K, ignore, w, rowc); break;
        case 1: hipLaunchKernelGGL(k_lp_bwd<F16>, grid, block, 0, st, sh.s, sh.gs, sh.start, sh.width, ch.cw, ch.nchunk, ids, K, ignore, w, rowc); break;
        default: hipLaunchKernelGGL(k_lp_bwd<BF16>, grid, block, 0, st, sh.s, sh.gs, sh.start, sh.width, ch.cw, ch.nchunk, ids, K, ignore, w, rowc);
    }
    return hipGetLastError();
}

hipError_t launch_topk_kl(int dtype, const LpTable &tab, bool first, int64_t N,
                          int64_t vocab_global, const int64_t *ids, const float *tlogp, int K,
                          int64_t ignore, const double *stats, float *kl, int32_t *dev_err,
                          hipStream_t st) {
    const dim3 grid((unsigned)((N + 255) / 256)), block(256);
    const int f = first ? 1 : 0;
    switch (dtype) {
        case 0: hipLaunchKernelGGL(k_topk_kl<F32>, grid, block, 0, st, tab, f, N, vocab_global, ids, tlogp, K, ignore, stats, kl, dev_err); break;
        case 1: hipLaunchKernelGGL(k_topk_kl<F16>, grid, block, 0, st, tab, f, N, vocab_global, ids, tlogp, K, ignore, stats, kl, dev_err); break;
        default: hipLaunchKernelGGL(k_topk_kl<BF16>, grid, block, 0, st, tab, f, N, vocab_global, ids, tlogp, K, ignore, stats, kl, dev_err);
    }
    return hipGetLastError();
}

}  // namespace vjsd
