// sweep.hpp -- the row sweep every streaming kernel is built on.
//
// One workgroup owns one row of one shard.  The row is cut into a scalar head (up
// to the first 16-byte boundary), a body of 16-byte vectors that consecutive lanes
// read from consecutive addresses (a wave touches 1 KiB per load, U loads per input
// in flight per lane) and a scalar tail.  The per-element work is an `Op` whose
//     template <int NV, int W> void run(const float (&a)[NV][W],
//                                       const float (&b)[NV][W],
//                                       const int64_t (&col)[NV])
// receives NV groups of W consecutive elements of the first and second input,
// widened to fp32, starting at the given columns (W is the vector width, or 1 in
// the head and tail).  One-input ops ignore `b`.  STREAM reads the body with the
// nontemporal cache policy (data read once).
#pragma once

#include "device.hpp"

namespace vjsd {

template <class D, int U, bool TWO, int BLK = BLOCK, bool STREAM = false, class Op>
__device__ __forceinline__ void sweep(const typename D::T *__restrict__ s,
                                      const typename D::T *__restrict__ t, int64_t w, int64_t h,
                                      Op &op) {
    using T = typename D::T;
    constexpr int VEC = D::VEC;
    constexpr int BLOCK = BLK;
    const int tid = threadIdx.x;
    for (int64_t i = tid; i < h; i += BLOCK) {
        float a[1][1], b[1][1] = {{0.0f}};
        const int64_t c[1] = {i};
        a[0][0] = load1<D>(s + i);
        if (TWO) b[0][0] = load1<D>(t + i);
        op.template run<1, 1>(a, b, c);
    }
    const int64_t nv = (w - h) / VEC;
    const T *sb = s + h;
    const T *tb = TWO ? t + h : s + h;
    int64_t v = tid;
    for (; v + (int64_t)(U - 1) * BLOCK < nv; v += (int64_t)U * BLOCK) {
        float a[U][VEC], b[U][VEC];
        int64_t c[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t q = (v + (int64_t)u * BLOCK) * VEC;
            c[u] = h + q;
            load_vec<D, STREAM>(sb + q, a[u]);
            if (TWO) load_vec<D, STREAM>(tb + q, b[u]);
        }
        op.template run<U, VEC>(a, b, c);
    }
    if constexpr (U > 1) {
        // the last partial step: a lane's (at most U - 1) vectors are loaded together,
        // then run one by one in the same order (one memory round trip instead of up to
        // U - 1: the several-shard fp32 forward at 4096 x 128256 in four shards, with a
        // partial step per shard and sweep, 1.057 -> 1.034 ms)
        u32x4 ra[U - 1], rb[U - 1];
        bool ok[U - 1];
#pragma unroll
        for (int u = 0; u < U - 1; ++u) {
            const int64_t vu = v + (int64_t)u * BLOCK;
            ok[u] = vu < nv;
            if (ok[u]) {
                ra[u] = ld16<STREAM>(sb + vu * VEC);
                if (TWO) rb[u] = ld16<STREAM>(tb + vu * VEC);
            }
        }
#pragma unroll
        for (int u = 0; u < U - 1; ++u) {
            if (ok[u]) {
                float a[1][VEC], b[1][VEC];
                widen<D>(ra[u], a[0]);
                if (TWO) widen<D>(rb[u], b[0]);
                else
#pragma unroll
                    for (int i = 0; i < VEC; ++i) b[0][i] = 0.0f;
                const int64_t c[1] = {h + (v + (int64_t)u * BLOCK) * VEC};
                op.template run<1, VEC>(a, b, c);
            }
        }
    } else {
        for (; v < nv; v += BLOCK) {
            float a[1][VEC], b[1][VEC];
            const int64_t q = v * VEC;
            const int64_t c[1] = {h + q};
            load_vec<D, STREAM>(sb + q, a[0]);
            if (TWO) load_vec<D, STREAM>(tb + q, b[0]);
            else
#pragma unroll
                for (int i = 0; i < VEC; ++i) b[0][i] = 0.0f;
            op.template run<1, VEC>(a, b, c);
        }
    }
    for (int64_t i = h + nv * VEC + tid; i < w; i += BLOCK) {
        float a[1][1], b[1][1] = {{0.0f}};
        const int64_t c[1] = {i};
        a[0][0] = load1<D>(s + i);
        if (TWO) b[0][0] = load1<D>(t + i);
        op.template run<1, 1>(a, b, c);
    }
}

// The same elements as sweep, in the opposite order: the scalar tail first, then each
// lane's 16-byte vectors from its last down to its first (its top n % U vectors
// together, then groups of U), then the scalar head.  A sweep that follows a forward
// one starts where that one ended.
template <class D, int U, bool TWO, int BLK = BLOCK, bool STREAM = false, class Op>
__device__ __forceinline__ void sweep_rev(const typename D::T *__restrict__ s,
                                          const typename D::T *__restrict__ t, int64_t w,
                                          int64_t h, Op &op) {
    using T = typename D::T;
    constexpr int VEC = D::VEC;
    constexpr int BLOCK = BLK;
    const int tid = threadIdx.x;
    const int64_t nv = (w - h) / VEC;
    for (int64_t i = h + nv * VEC + tid; i < w; i += BLOCK) {
        float a[1][1], b[1][1] = {{0.0f}};
        const int64_t c[1] = {i};
        a[0][0] = load1<D>(s + i);
        if (TWO) b[0][0] = load1<D>(t + i);
        op.template run<1, 1>(a, b, c);
    }
    const T *sb = s + h;
    const T *tb = TWO ? t + h : s + h;
    const int64_t nl = nv > tid ? (nv - tid + BLOCK - 1) / BLOCK : 0;  // this lane's vectors
    const int64_t r = nl % U;
    int64_t j0 = nl - r;  // first of the top r
    if (U > 1 && r > 0) {
        u32x4 ra[U > 1 ? U - 1 : 1], rb[U > 1 ? U - 1 : 1];
#pragma unroll
        for (int u = 0; u < U - 1; ++u) {
            if (u < r) {
                const int64_t v = tid + (j0 + u) * BLOCK;
                ra[u] = ld16<STREAM>(sb + v * VEC);
                if (TWO) rb[u] = ld16<STREAM>(tb + v * VEC);
            }
        }
#pragma unroll
        for (int u = 0; u < U - 1; ++u) {
            if (u < r) {
                float a[1][VEC], b[1][VEC];
                widen<D>(ra[u], a[0]);
                if (TWO) widen<D>(rb[u], b[0]);
                else
#pragma unroll
                    for (int i = 0; i < VEC; ++i) b[0][i] = 0.0f;
                const int64_t c[1] = {h + (tid + (j0 + u) * BLOCK) * VEC};
                op.template run<1, VEC>(a, b, c);
            }
        }
    }
    for (j0 -= U; j0 >= 0; j0 -= U) {
        float a[U][VEC], b[U][VEC];
        int64_t c[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t q = (tid + (j0 + u) * BLOCK) * VEC;
            c[u] = h + q;
            load_vec<D, STREAM>(sb + q, a[u]);
            if (TWO) load_vec<D, STREAM>(tb + q, b[u]);
        }
        op.template run<U, VEC>(a, b, c);
    }
    for (int64_t i = tid; i < h; i += BLOCK) {
        float a[1][1], b[1][1] = {{0.0f}};
        const int64_t c[1] = {i};
        a[0][0] = load1<D>(s + i);
        if (TWO) b[0][0] = load1<D>(t + i);
        op.template run<1, 1>(a, b, c);
    }
}

// Writes n zeros of the storage format (head / 16-byte body / tail), BLK lanes; the
// body with streaming stores.
template <class D, int BLK>
__device__ __forceinline__ void zero_span(typename D::T *p, int64_t n) {
    const int64_t h = head_len<typename D::T>(n, p);
    for (int64_t i = threadIdx.x; i < h; i += BLK) store1<D>(p + i, 0.0f);
    const int64_t nv = (n - h) / D::VEC;
    float z[D::VEC];
#pragma unroll
    for (int i = 0; i < D::VEC; ++i) z[i] = 0.0f;
    for (int64_t v = threadIdx.x; v < nv; v += BLK) store_vec<D, true>(p + h + v * D::VEC, z);
    for (int64_t i = h + nv * D::VEC + threadIdx.x; i < n; i += BLK) store1<D>(p + i, 0.0f);
}

// Online (max, sum of 2^(x*ks - c)) of one input over a batch of n elements: one
// rescale per batch, a tree sum of the batch's exponentials.  With MIN it also keeps
// the smallest element (the range test of the interior divergence's plain form).
template <bool MIN = false>
struct Online {
    float m = NINF, c = 0.0f, z = 0.0f;
    float mn = __builtin_huge_valf();  // MIN only
    float ks = L2E;  // log2 e / temperature

    template <int N>
    __device__ __forceinline__ void add(const float *x) {
        float bm = x[0];
#pragma unroll
        for (int i = 1; i < N; ++i) bm = fmaxf(bm, x[i]);
        if constexpr (MIN) {
            float bn = x[0];
#pragma unroll
            for (int i = 1; i < N; ++i) bn = fminf(bn, x[i]);
            mn = fminf(mn, bn);
        }
        const float nm = fmaxf(m, bm);
        const float nc = refc(nm, ks);
        const float scale = m == NINF ? 0.0f : ex2(c - nc);
        float e[N];
#pragma unroll
        for (int i = 0; i < N; ++i) e[i] = ex2(fmaf(x[i], ks, -nc));
#pragma unroll
        for (int st = N / 2; st >= 1; st /= 2)
#pragma unroll
            for (int i = 0; i < st; ++i) e[i] += e[i + st];
        z = fmaf(z, scale, e[0]);
        m = nm;
        c = nc;
    }
};

// Sweep op of the statistics pass: online (max, sum-exp) of the first input, and of
// the second when WHICH == 3; MIN also tracks each input's smallest element.
template <int WHICH, bool MIN = false>
struct OpStats {
    Online<MIN> a, b;  // first and second swept input
    __device__ explicit OpStats(float ks = L2E) {
        a.ks = ks;
        b.ks = ks;
    }
    template <int NV, int W>
    __device__ __forceinline__ void run(const float (&x)[NV][W], const float (&y)[NV][W],
                                        const int64_t (&)[NV]) {
        a.template add<NV * W>(&x[0][0]);
        if (WHICH == 3) b.template add<NV * W>(&y[0][0]);
    }
};

// (max, sum-exp) over a BLK-lane workgroup, combined in wave order; red holds
// 2 * (BLK / 64) floats.  Every lane returns the result.
template <int BLK = BLOCK>
__device__ __forceinline__ MZ block_mz(MZ v, float *red, float ks = L2E) {
    constexpr int NW = BLK / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_mz(v, ks);
    if (lane == 0) {
        red[2 * wave] = v.m;
        red[2 * wave + 1] = v.z;
    }
    __syncthreads();
    MZ acc{red[0], red[1]};
    for (int k = 1; k < NW; ++k) acc = mz_combine(acc, MZ{red[2 * k], red[2 * k + 1]}, ks);
    __syncthreads();
    return acc;
}

}  // namespace vjsd
