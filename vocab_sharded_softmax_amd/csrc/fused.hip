// fused.hip -- the interior JSD forward in one launch, and the forward and backward in
// one launch.
//
// [JSD-PR] DeepSpeed PR #8958 "[VocabTP] Add vocabulary-parallel generalized JSD with
// Triton kernels", section Scope and limitations: the JSD needs the global normaliser
// before the nonlinear mixture, so statistics and divergence are two passes over the
// input.  With a single shard one workgroup owns a whole row, so both passes can run
// in one workgroup with nothing exchanged between workgroups:
//   k_fwd_row    a row of both inputs fits the workgroup's registers (16-byte aligned
//                rows; 256 lanes x up to 8 16-byte vectors per input, 16384 bf16 / fp16
//                or 8192 fp32 columns, and 512 lanes x up to 10, 40960 / 20480 columns):
//                one HBM read per logit
//   k_fwd_twice  wider rows: the workgroup sweeps its row for the statistics, then
//                sweeps it again for the divergence terms; the merge launch and two
//                kernel boundaries go away, the second read stays
//   k_fwd_shards the same for a row split into up to FUSED_SHARDS logical shards:
//                per-shard statistics merged in the workgroup, then the divergence
//   k_fwdbwd_row / k_fwdbwd_twice   k_fwd_row / k_fwd_twice, then the row's gradients
//                in the same workgroup (below)
// The divergence terms are those of MixTerm (divergence.hpp).  The statistics sweep
// also finds each side's smallest logit: a row whose logits all lie within FAST_RANGE
// of its maximum (no masked token, no underflow) takes the divergence without the
// clamps and the floor that masked tokens need.  Splitting a row over several
// workgroups would need a device-wide exchange per row; on MI355X the cache write-back
// and invalidation that a correct device-scope release/acquire costs exceeds the
// second read it would save.
#include "backward.hpp"
#include "kernels.hpp"
#include "sweep.hpp"

#include <type_traits>

namespace vjsd {

namespace {

// Register-held rows: 256-lane workgroups with 1, 2, 4 or 8 vectors per lane, then
// 512-lane workgroups with 6, 8 or 10 (ROW_WIDE_NVT_MAX).  At 16384 < V <= 40960 bf16 the
// wider workgroup (124 VGPRs at 10 vectors, two workgroups per CU) beat the two sweeps
// by 8-15 % on MI355X (1024 x 37984: 0.063 -> 0.056 ms; 1024 x 32000: 0.061 -> 0.052;
// 8192 x 20000: 0.26 -> 0.24); 1024-lane workgroups spilled at 8 vectors and ran slower
// at 5.  Keeping the statistics' exponentials for the divergence (238 VGPRs at 256 x 8,
// one workgroup per SIMD pair) ran slower too: 0.170 against 0.148 ms at 8192 x 16032.
constexpr int FB = 256;
constexpr int FB_WIDE = 512;
constexpr int ROW_WIDE_NVT_MAX = 10;

// raw 32-bit word of -inf in each storage format (two halves for 16-bit formats)
template <class D>
__device__ __forceinline__ uint32_t ninf_word();
template <>
__device__ __forceinline__ uint32_t ninf_word<F32>() { return 0xff800000u; }
template <>
__device__ __forceinline__ uint32_t ninf_word<F16>() { return 0xfc00fc00u; }
template <>
__device__ __forceinline__ uint32_t ninf_word<BF16>() { return 0xff80ff80u; }

// Empty register barrier: the compiler must assume the packed vectors changed, so it
// re-widens them in each sweep instead of keeping NVT * 2 * VEC floats alive.
__device__ __forceinline__ void opaque(u32x4 &v) {
    asm volatile("" : "+v"(v));
}

// Row maxima (a, b) and minima (na, nb) over the B-lane workgroup; red holds B / 16
// floats.
template <int B>
__device__ __forceinline__ void block_minmax2(float &a, float &b, float &na, float &nb,
                                              float *red) {
    constexpr int FNW = B / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    a = wave_max(a);
    b = wave_max(b);
    na = wave_min(na);
    nb = wave_min(nb);
    if (lane == 0) {
        red[wave] = a;
        red[FNW + wave] = b;
        red[2 * FNW + wave] = na;
        red[3 * FNW + wave] = nb;
    }
    __syncthreads();
    float x = red[0], y = red[FNW], nx = red[2 * FNW], ny = red[3 * FNW];
#pragma unroll
    for (int k = 1; k < FNW; ++k) {
        x = fmaxf(x, red[k]);
        y = fmaxf(y, red[FNW + k]);
        nx = fminf(nx, red[2 * FNW + k]);
        ny = fminf(ny, red[3 * FNW + k]);
    }
    a = x;
    b = y;
    na = nx;
    nb = ny;
    __syncthreads();
}

template <int B>
__device__ __forceinline__ void block_sum2(float &a, float &b, float *red) {
    constexpr int FNW = B / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    a = wave_sum(a);
    b = wave_sum(b);
    if (lane == 0) {
        red[wave] = a;
        red[FNW + wave] = b;
    }
    __syncthreads();
    float x = red[0], y = red[FNW];
#pragma unroll
    for (int k = 1; k < FNW; ++k) {
        x += red[k];
        y += red[FNW + k];
    }
    a = x;
    b = y;
    __syncthreads();
}

// Constants of a row's divergence pass, derived from the row's statistics.
struct RowK {
    MixRow mx;
    int undefined;  // a side has no distribution (all -inf)
    int fast;       // every logit of both sides within FAST_RANGE of its row maximum
};

// Run by one whole wave: the fp64 steps are the costliest part of a row's finish, so
// one wave takes them and the others read the result from LDS.  Lane 0 stores the
// row's statistics and the constants.  (ms, zs), (mt, zt): row maxima and sums of
// 2^(x ks - refc(max)); ns, nt: row minima.
__device__ __forceinline__ void row_constants(float ms, double zs, float mt, double zt, float ns,
                                              float nt, double beta, float ks, double *st,
                                              RowK *out) {
    const bool undefined = ms == NINF || mt == NINF;
    RowK k;
    k.undefined = undefined;
    k.fast = 0;
    k.mx = MixRow{0.0f, 0.0f, 0.0f, 1.0, 1.0, 0.0};
    if (!undefined) {
        k.mx = mix_row(beta, refc(ms, ks), zs, refc(mt, ks), zt);
        k.fast = (ms - ns) * ks <= FAST_RANGE && (mt - nt) * ks <= FAST_RANGE;
    }
    if ((threadIdx.x & 63) == 0) {
        st[0] = ms;
        st[1] = ms == NINF ? -__builtin_inf() : lnz_from_z(ms, zs, ks);
        st[2] = mt;
        st[3] = mt == NINF ? -__builtin_inf() : lnz_from_z(mt, zt, ks);
        *out = k;
    }
}

// The row's per-token values from its two divergence sums (thread 0).
__device__ __forceinline__ void finish_row(const RowK &k, double beta, float at, float as,
                                           float *kl, float *loss, float lscale) {
    double kt2 = 0.0, ks2 = 0.0;
    if (!k.undefined) mix_finish(k.mx, at, as, kt2, ks2);
    finalize_row(INTERIOR, beta, k.undefined, kt2, ks2, NINF, kl, loss, lscale);
}

// Divergence terms of a row held in registers; slots past the row's end (they hold
// -inf) are skipped.
template <class D, int NVT, int B, bool SAFE>
__device__ __forceinline__ void regs_div(const u32x4 (&xs)[NVT], const u32x4 (&xt)[NVT],
                                         int64_t nv, const MixRow &mx, float beta, float ks,
                                         float &at, float &as) {
    constexpr int VEC = D::VEC;
    MixTerm<SAFE> op;
    op.ks = ks;
    op.ct = mx.ct;
    op.cs = mx.cs;
    op.bt = beta;
    op.ksc = mx.ksc;
#pragma unroll
    for (int i = 0; i < NVT; ++i) {
        if (threadIdx.x + (int64_t)i * B < nv) {
            float a[VEC], b[VEC];
            widen<D>(xs[i], a);
            widen<D>(xt[i], b);
#pragma unroll
            for (int e = 0; e < VEC; ++e) op.add(a[e], b[e], at, as);
        }
    }
}

// The forward of one row held in registers by a B-lane workgroup: the body of k_fwd_row
// and k_fwdbwd_row.  Lane l loads vectors l, l + B, ... of each input into xs / xt;
// slots past the row's end hold -inf, which adds exactly nothing to any sum below.
// Thread 0 writes the row's statistics (st), KL pair (klr) and loss; the row stays in
// xs / xt.  nv: the row's 16-byte vectors (the host requires whole vectors).
template <class D, int NVT, int B>
__device__ __forceinline__ void row_forward(const typename D::T *s, const typename D::T *t,
                                            int64_t nv, double beta, double *st, float *klr,
                                            float *lossr, const RowOpts &o, float *red,
                                            RowK &rk, u32x4 (&xs)[NVT], u32x4 (&xt)[NVT]) {
    constexpr int VEC = D::VEC;
#pragma unroll
    for (int i = 0; i < NVT; ++i) {
        const int64_t j = threadIdx.x + (int64_t)i * B;
        if (j < nv) {
            xs[i] = ld16<true>(s + j * VEC);
            xt[i] = ld16<true>(t + j * VEC);
        } else {
            const uint32_t q = ninf_word<D>();
            xs[i] = u32x4{q, q, q, q};
            xt[i] = u32x4{q, q, q, q};
        }
    }
    // ---- statistics: row max and min, then sum of 2^(x ks - c)
    float ms = NINF, mt = NINF, ns = __builtin_huge_valf(), nt = __builtin_huge_valf();
#pragma unroll
    for (int i = 0; i < NVT; ++i) {
        float a[VEC], b[VEC];
        widen<D>(xs[i], a);
        widen<D>(xt[i], b);
        // the minima start from +inf, not the first element: fminf of two widened values
        // makes the compiler quieten both first, three-input minima do not
        float na = __builtin_huge_valf(), nb = __builtin_huge_valf();
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            ms = fmaxf(ms, a[e]);
            mt = fmaxf(mt, b[e]);
            na = fminf(na, a[e]);
            nb = fminf(nb, b[e]);
        }
        // a -inf filled slot past the row's end is left out of the minima (a select, not
        // a branch: a branch here keeps every widened value of the row alive)
        const bool real = threadIdx.x + (int64_t)i * B < nv;
        ns = fminf(ns, real ? na : __builtin_huge_valf());
        nt = fminf(nt, real ? nb : __builtin_huge_valf());
    }
    block_minmax2<B>(ms, mt, ns, nt, red);
#pragma unroll
    for (int i = 0; i < NVT; ++i) {
        opaque(xs[i]);
        opaque(xt[i]);
    }
    const float cs = refc(ms, o.ks), ct = refc(mt, o.ks);
    float zs = 0.0f, zt = 0.0f;
#pragma unroll
    for (int i = 0; i < NVT; ++i) {
        float a[VEC], b[VEC], ea[VEC], eb[VEC];
        widen<D>(xs[i], a);
        widen<D>(xt[i], b);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            ea[e] = ex2(fmaf(a[e], o.ks, -cs));
            eb[e] = ex2(fmaf(b[e], o.ks, -ct));
        }
#pragma unroll
        for (int st = VEC / 2; st >= 1; st /= 2)
#pragma unroll
            for (int e = 0; e < st; ++e) {
                ea[e] += ea[e + st];
                eb[e] += eb[e + st];
            }
        zs += ea[0];
        zt += eb[0];
    }
    block_sum2<B>(zs, zt, red);
    if (threadIdx.x < 64) row_constants(ms, zs, mt, zt, ns, nt, beta, o.ks, st, &rk);
    __syncthreads();
    const RowK k = rk;
    // ---- divergence: terms from registers
    float pt = 0.0f, ps = 0.0f;
    if (!k.undefined) {
#pragma unroll
        for (int i = 0; i < NVT; ++i) {
            opaque(xs[i]);
            opaque(xt[i]);
        }
        if (k.fast) regs_div<D, NVT, B, false>(xs, xt, nv, k.mx, (float)beta, o.ks, pt, ps);
        else regs_div<D, NVT, B, true>(xs, xt, nv, k.mx, (float)beta, o.ks, pt, ps);
    }
    block_sum2<B>(pt, ps, red);
    if (threadIdx.x == 0) finish_row(k, beta, pt, ps, klr, lossr, o.lscale);
}


// One B-lane workgroup per row.
template <class D, int NVT, int B>
__global__ __launch_bounds__(B) void k_fwd_row(RowView sv, RowView tv, int64_t w, double beta,
                                                double *__restrict__ stats,
                                                float *__restrict__ kl,
                                                float *__restrict__ loss, RowOpts o) {
    using T = typename D::T;
    __shared__ float red[4 * (B / 64)];
    __shared__ RowK rk;
    const int64_t r = blockIdx.x;
    if (row_dropped(o, r)) {
        dropped_row(stats + r * 4, kl + 2 * r, loss + r);
        return;
    }
    u32x4 xs[NVT], xt[NVT];
    row_forward<D, NVT, B>(row_ptr<T>(sv, r), row_ptr<T>(tv, r), w / D::VEC, beta, stats + r * 4,
                           kl + 2 * r, loss + r, o, red, rk, xs, xt);
}

// One workgroup per row, any alignment: statistics sweep, then divergence sweep.
// TWICE_BLK lanes, two workgroups per CU (about 512 rows in flight); 256- and
// 1024-lane workgroups measured slower.  The kernel is bound by its reads (with the
// arithmetic close behind), so the last full steps of the statistics sweep (TWICE_BLK x
// TW_U vectors per input each: 16384 16-bit or 8192 fp32 columns) stay on chip, in
// registers and LDS, and open the divergence sweep instead of being read again.  The
// first sweep reads with the default cache policy, the second streams.
constexpr int TWICE_BLK = 512;
constexpr int TW_U = 4;  // 16-byte vectors per lane per input in flight in a sweep step

// Sweep steps held in registers, and in LDS (64 KiB per workgroup each) one more for
// 16-bit inputs and up to two more for fp32.  Measured on MI355X (forward at 8192 x
// 151936 bf16 / 4096 x 151936 fp16 / 4096 x 128256 fp32):
//   bf16  1 step + LDS (125 VGPRs, two workgroups per CU): 1.35 -> 1.25 ms; 2 steps +
//         LDS (247 VGPRs) 1.44 ms; asking the compiler for four waves per SIMD made it
//         spill
//   fp16  1 step (126 VGPRs); with the LDS step it compiled to 167 VGPRs and ran 8 %
//         slower, with 2 steps 1.39 ms; the LDS step with the kernel held to four
//         waves per SIMD (128 VGPRs, a 68-byte spill) runs the forward as fast as
//         without it and the one-launch forward and backward 1.375-1.381 -> 1.323-1.327
//         ms (three alternating runs on one box)
//   fp32  4 steps + LDS (236 VGPRs, one workgroup per CU): 1.18 -> 0.99 ms; an fp32
//         step holds half the columns of a 16-bit one, and holding more beat occupancy
//         here (1 / 2 / 3 steps + LDS: 1.08 / 1.05 / 1.02 ms; 5 steps spilled).  The one
//         workgroup per CU leaves LDS for a second step (128 KiB): forward 1.014-1.023 ->
//         1.006-1.014 ms, forward and backward in one launch 2.265-2.268 -> 2.193-2.198
//         ms (three alternating runs on one box)
template <class D>
constexpr int held_steps() { return sizeof(typename D::T) == 4 ? 4 : 1; }
template <class D>
constexpr int lds_steps() { return sizeof(typename D::T) == 4 ? 2 : 1; }

// The streamed part of k_fwd_twice's divergence sweep, continuing the sums `acc`
// (t, s) of the held steps.  It runs backwards, from the row's end, where the statistics
// sweep stopped, so the gradients' sweep of the one-launch kernel then starts at the
// row's beginning, where this one stops (each sweep opens on the columns read last).
// Measured on MI355X against the forward order, three alternating runs: 4096 x 151936
// fp16 forward and backward in one launch 1.431-1.440 -> 1.398-1.408 ms; bf16 at 8192 x
// 151936 and fp32 at 4096 x 128256 unchanged.
// STREAM: the nontemporal load policy, for a forward whose row is not read again.  The
// one-launch kernel reads the row a third time, for the gradients, and loads this
// sweep with the default policy, which keeps the columns in the caches for that
// sweep: forward and backward in one launch (three alternating runs on one box) at
// 8192 x 151936 bf16 2.771-2.802 -> 2.699-2.724 ms, at 4096 x 151936 fp16 1.340-1.351
// -> 1.279-1.285 ms, at 4096 x 128256 fp32 2.255-2.257 -> 1.975-2.008 ms; the same
// policy in the forward alone made it 3-8 % slower.
template <class D, bool SAFE, bool STREAM = true>
__device__ __forceinline__ void twice_stream(const MixRow &mx, float beta, float ks, bool hold,
                                             const typename D::T *s, const typename D::T *t,
                                             int64_t w, int64_t h, int64_t P, int64_t Q,
                                             float (&acc)[2]) {
    OpMix<SAFE> op;
    op.set(mx, beta, ks);
    op.at[0] = acc[0];
    op.as[0] = acc[1];
    if (hold) {
        sweep_rev<D, TW_U, true, TWICE_BLK, STREAM>(s + Q, t + Q, w - Q, 0, op);
        sweep_rev<D, TW_U, true, TWICE_BLK, STREAM>(s, t, P, h, op);
    } else {
        sweep_rev<D, TW_U, true, TWICE_BLK, STREAM>(s, t, w, h, op);
    }
    acc[0] = op.sum_t();
    acc[1] = op.sum_s();
}

// The held vectors through the statistics op one at a time (one online batch per
// vector), chained like held_div below.
template <class D, class Op>
__device__ __forceinline__ void held_stats(const u32x4 (&hs)[TW_U], const u32x4 (&ht)[TW_U],
                                           Op &op) {
    constexpr int VEC = D::VEC;
#pragma unroll
    for (int u = 0; u < TW_U; ++u) {
        u32x4 xs = hs[u], xt = ht[u];
        if (u > 0) asm volatile("" : "+v"(xs), "+v"(xt), "+v"(op.a.z), "+v"(op.b.z));
        float a[1][VEC], b[1][VEC];
        widen<D>(xs, a[0]);
        widen<D>(xt, b[0]);
        const int64_t c[1] = {0};
        op.template run<1, VEC>(a, b, c);
    }
}

// The held vectors through the divergence op one at a time, vector u into accumulator
// u: the empty asm ties the next vector to the sums of the one before, so only one
// vector's widened values are live at once (all of them at once spill the 16-bit
// kernels out of two workgroups per CU).
template <class D, bool SAFE>
__device__ __forceinline__ void held_div(const u32x4 (&hs)[TW_U], const u32x4 (&ht)[TW_U],
                                         OpMix<SAFE> &op) {
    constexpr int VEC = D::VEC;
#pragma unroll
    for (int u = 0; u < TW_U; ++u) {
        u32x4 xs = hs[u], xt = ht[u];
        if (u > 0) asm volatile("" : "+v"(xs), "+v"(xt), "+v"(op.at[u - 1]), "+v"(op.as[u - 1]));
        float a[VEC], b[VEC];
        widen<D>(xs, a);
        widen<D>(xt, b);
#pragma unroll
        for (int e = 0; e < VEC; ++e) op.add(a[e], b[e], op.at[u], op.as[u]);
    }
}

// The part of a row that the statistics sweep of k_fwd_twice keeps on chip: the last
// HOLD + lh full sweep steps of the row's 16-byte body, elements [P, Q) ([P, PR) in LDS,
// lh <= LHOLD steps, as many as the row has beyond the HOLD register steps; [PR, Q) in
// registers).  Rows whose two inputs sit at different offsets inside 16 bytes (h == w),
// or that are too short for the register steps and one LDS step, hold nothing and are
// swept whole.
struct TwiceSpan {
    int64_t h, P, PR, Q;
    int lh;
    bool hold;
};
template <class D>
__device__ __forceinline__ TwiceSpan twice_span(int64_t w, int64_t h) {
    constexpr int VEC = D::VEC;
    constexpr int64_t STEP = (int64_t)TW_U * TWICE_BLK;  // vectors per input per sweep step
    constexpr int HOLD = held_steps<D>(), LHOLD = lds_steps<D>();
    TwiceSpan sp;
    sp.h = h;
    const int64_t nfull = h < w ? (w - h) / VEC / STEP : 0;
    sp.hold = nfull >= HOLD + (LHOLD > 0 ? 1 : 0);
    // (a constant for one LDS step: the row then holds it whenever it holds at all)
    sp.lh = LHOLD <= 1 ? LHOLD
            : sp.hold  ? (int)(nfull - HOLD < LHOLD ? nfull - HOLD : LHOLD)
                       : 0;
    sp.P = sp.hold ? h + (nfull - HOLD - sp.lh) * STEP * VEC : w;
    sp.PR = sp.P + sp.lh * STEP * VEC;
    sp.Q = sp.hold ? sp.PR + HOLD * STEP * VEC : w;
    return sp;
}
// The held steps: LDS (each lane's own vectors) and registers.
template <class D>
using LdsStep =
    u32x4[lds_steps<D>() ? lds_steps<D>() : 1][2][TW_U][lds_steps<D>() ? TWICE_BLK : 1];
template <class D>
using HeldRegs = u32x4[held_steps<D>()][TW_U];

// The forward of one row by a TWICE_BLK-lane workgroup, the body of k_fwd_twice and
// k_fwdbwd_twice: the statistics sweep, keeping the span sp on chip, the row's
// constants (into rk), then the divergence sweep.  Thread 0 writes the row's
// statistics (st), KL pair (klr) and loss; the held steps stay in lds_step / hs / ht.
// STREAM: the divergence sweep's load policy (twice_stream).
template <class D, bool STREAM = true>
__device__ __forceinline__ void twice_forward(const typename D::T *s, const typename D::T *t,
                                              int64_t w, const TwiceSpan &sp, double beta,
                                              double *st, float *klr, float *lossr,
                                              const RowOpts &o, float *red, RowK &rk,
                                              LdsStep<D> &lds_step, HeldRegs<D> &hs,
                                              HeldRegs<D> &ht) {
    constexpr int VEC = D::VEC;
    constexpr int64_t STEP = (int64_t)TW_U * TWICE_BLK;  // vectors per input per sweep step
    // fp16 rows take the divergence form that admits masked tokens without the range
    // test: tracking the minima costs the fp16 kernel 26 VGPRs and its second workgroup
    // per CU
    constexpr bool RANGE = !std::is_same<D, F16>::value;
    OpStats<3, RANGE> o1(o.ks);
    // A lane reads back from LDS only the vectors it wrote there itself, so the LDS step
    // needs no barrier of its own.
    constexpr int HOLD = held_steps<D>(), LHOLD = lds_steps<D>();
    const int64_t h = sp.h, P = sp.P, PR = sp.PR, Q = sp.Q;
    const bool hold = sp.hold;
    if (hold) {
        sweep<D, TW_U, true, TWICE_BLK>(s, t, P, h, o1);
#pragma unroll
        for (int l = 0; l < LHOLD; ++l) {
            if (LHOLD > 1 && l >= sp.lh) break;
            u32x4 ls[TW_U], lt[TW_U];
#pragma unroll
            for (int u = 0; u < TW_U; ++u) {
                const int64_t q =
                    P + ((int64_t)l * STEP + threadIdx.x + (int64_t)u * TWICE_BLK) * VEC;
                ls[u] = ld16<true>(s + q);
                lt[u] = ld16<true>(t + q);
            }
#pragma unroll
            for (int u = 0; u < TW_U; ++u) {
                lds_step[l][0][u][threadIdx.x] = ls[u];
                lds_step[l][1][u][threadIdx.x] = lt[u];
            }
            held_stats<D>(ls, lt, o1);
        }
#pragma unroll
        for (int k = 0; k < HOLD; ++k) {
#pragma unroll
            for (int u = 0; u < TW_U; ++u) {
                const int64_t q =
                    PR + ((int64_t)k * STEP + threadIdx.x + (int64_t)u * TWICE_BLK) * VEC;
                hs[k][u] = ld16<true>(s + q);
                ht[k][u] = ld16<true>(t + q);
            }
            held_stats<D>(hs[k], ht[k], o1);
        }
        sweep<D, TW_U, true, TWICE_BLK>(s + Q, t + Q, w - Q, 0, o1);
    } else {
        sweep<D, TW_U, true, TWICE_BLK>(s, t, w, h, o1);
    }
    // wave partials, then wave 0 combines them in wave order and derives the constants
    constexpr int NW = TWICE_BLK / 64;
    {
        const MZ ws = wave_mz(MZ{o1.a.m, o1.a.z}, o.ks);
        const MZ wt = wave_mz(MZ{o1.b.m, o1.b.z}, o.ks);
        const float ns = RANGE ? wave_min(o1.a.mn) : NINF;
        const float nt = RANGE ? wave_min(o1.b.mn) : NINF;
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        if (lane == 0) {
            red[2 * wave] = ws.m;
            red[2 * wave + 1] = ws.z;
            red[2 * NW + 2 * wave] = wt.m;
            red[2 * NW + 2 * wave + 1] = wt.z;
            red[4 * NW + 2 * wave] = ns;
            red[4 * NW + 2 * wave + 1] = nt;
        }
        __syncthreads();
        if (wave == 0) {
            MZ ms{red[0], red[1]}, mt{red[2 * NW], red[2 * NW + 1]};
            float mns = red[4 * NW], mnt = red[4 * NW + 1];
            for (int k = 1; k < NW; ++k) {
                ms = mz_combine(ms, MZ{red[2 * k], red[2 * k + 1]}, o.ks);
                mt = mz_combine(mt, MZ{red[2 * NW + 2 * k], red[2 * NW + 2 * k + 1]}, o.ks);
                mns = fminf(mns, red[4 * NW + 2 * k]);
                mnt = fminf(mnt, red[4 * NW + 2 * k + 1]);
            }
            row_constants(ms.m, ms.z, mt.m, mt.z, mns, mnt, beta, o.ks, st, &rk);
        }
        __syncthreads();
    }
    const RowK k = rk;
    float v[2] = {0.0f, 0.0f};
    if (!k.undefined) {
        // the held steps (a small part of the row) always take the form that admits
        // masked tokens: one copy of them keeps the held registers' live range short
        if (hold) {
            OpMix<true> oh;
            oh.set(k.mx, (float)beta, o.ks);
#pragma unroll
            for (int j = 0; j < HOLD; ++j) held_div<D>(hs[j], ht[j], oh);
#pragma unroll
            for (int l = 0; l < LHOLD; ++l) {
                if (LHOLD > 1 && l >= sp.lh) break;
                u32x4 ls[TW_U], lt[TW_U];
#pragma unroll
                for (int u = 0; u < TW_U; ++u) {
                    ls[u] = lds_step[l][0][u][threadIdx.x];
                    lt[u] = lds_step[l][1][u][threadIdx.x];
                }
                held_div<D>(ls, lt, oh);
            }
            v[0] = oh.sum_t();
            v[1] = oh.sum_s();
        }
        if (RANGE && k.fast)
            twice_stream<D, false, STREAM>(k.mx, (float)beta, o.ks, hold, s, t, w, h, P, Q, v);
        else
            twice_stream<D, true, STREAM>(k.mx, (float)beta, o.ks, hold, s, t, w, h, P, Q, v);
    }
    block_sum<2, TWICE_BLK>(v, red);
    if (threadIdx.x == 0) finish_row(k, beta, v[0], v[1], klr, lossr, o.lscale);
}

template <class D>
__global__ __launch_bounds__(TWICE_BLK)
__attribute__((amdgpu_waves_per_eu(sizeof(typename D::T) == 4 ? 2 : 4)))
void k_fwd_twice(RowView sv, RowView tv, int64_t w, double beta, double *__restrict__ stats,
                 float *__restrict__ kl, float *__restrict__ loss, RowOpts o) {
    using T = typename D::T;
    __shared__ float red[6 * (TWICE_BLK / 64)];
    __shared__ RowK rk;
    __shared__ LdsStep<D> lds_step;
    const int64_t r = blockIdx.x;
    if (row_dropped(o, r)) {
        dropped_row(stats + r * 4, kl + 2 * r, loss + r);
        return;
    }
    const T *s = row_ptr<T>(sv, r), *t = row_ptr<T>(tv, r);
    const TwiceSpan sp = twice_span<D>(w, head_len<T>(w, s, t));
    HeldRegs<D> hs, ht;
    twice_forward<D>(s, t, w, sp, beta, stats + r * 4, kl + 2 * r, loss + r, o, red, rk, lds_step,
                     hs, ht);
}

// ---- forward and backward in one launch ---------------------------------------------
//
// [JSD-PR, Changes] The backward needs the forward's statistics and KL pair, which a
// single-shard row's workgroup has just produced: with the upstream gradient known
// before the forward (a per-token weight, or a reduction's scale), the same workgroup
// goes on to the row's gradients.  The register-held row is then read from HBM once for
// both passes; the two-sweep row reuses the steps it holds on chip, and the separate
// backward's constants launch and kernel boundary go away.  Each output is the one the
// forward and backward entry points compute, bit for bit: the forward is the same code,
// and the gradients are element-wise with the same constants (backward.hpp).

// Thread 0, after its row's forward: the backward's constants of row r from the
// statistics and KL pair it has just written to global memory (a thread reads back its
// own writes), as k_bwd_prep derives them.
__device__ __forceinline__ void fused_bwd_constants(const double *stats, const float *kl,
                                                    int64_t r, double beta, const float *grad,
                                                    const GradOpts &go, float *rc) {
    const RowConst k = row_const(stats, r, go.ks);
    bwd_constants(INTERIOR, k, kl + 2 * r, beta, upstream_g(grad, go, r), go.ks, k.undefined, rc);
}

template <class D, int BLK, bool WS, bool WT>
__device__ __forceinline__ void zero_grads(typename D::T *gs, typename D::T *gt, int64_t w) {
    if (WS) zero_span<D, BLK>(gs, w);
    if (WT) zero_span<D, BLK>(gt, w);
}

// Shape of the fused kernels, measured on MI355X against the forward and backward
// launches (kernel time, two calls -> one call):
//   two-sweep rows: waves per SIMD held at 4 for 16-bit inputs (128 VGPRs, two
//     workgroups per CU as the forward alone; bf16 spills 12 bytes, fp16 68), 2 for
//     fp32 (one workgroup per CU, 232 VGPRs); one vector per lane in flight in the
//     gradient sweep (two: 8192 x 151936 bf16 2.82 against 2.75 ms; fp32 ran no faster
//     with two or four, or with the next vector's loads issued before the current
//     one's arithmetic).  8192 x 151936 bf16: 2.83-2.87 -> 2.73-2.75 ms; 4096 x 151936
//     fp16: 1.45-1.46 -> 1.41-1.43 ms (1.32-1.33 ms after the backward divergence
//     sweep and the fp16 LDS step, 1.27-1.28 ms with the default load policy in the
//     divergence sweep); 4096 x 128256 fp32: 2.27-2.29 -> 2.25 ms with two held LDS
//     steps, where the backward part runs at one workgroup per CU (reading the four
//     register steps again instead of keeping them: 2.38-2.44 ms), 1.94-1.95 ms with
//     the default load policy in the divergence sweep
//   512-lane register rows: held to 128 VGPRs, two workgroups per CU (1024 x 37984
//     bf16, student gradient: 0.0916 ms at 134 VGPRs and one workgroup per CU, 0.0815
//     ms with a 20-byte spill; the two calls 0.092-0.096 ms); 8192 x 16032 bf16 (256
//     lanes, 8 vectors): 0.304 -> 0.235 ms; 8192 x 32000: 0.60 -> 0.46-0.49 ms
template <class D>
constexpr int fb_waves() { return sizeof(typename D::T) == 4 ? 2 : 4; }
template <class D>
constexpr int fb_sweep_u() { return 1; }
template <int B>
constexpr int fb_row_waves() { return B == 512 ? 4 : 1; }

// The gradients of a row held in registers (xs, xt) by a B-lane workgroup; CLAMP =
// false for rows the forward found within FAST_RANGE of their maxima (same results,
// two VALU operations fewer per element pair).
template <class D, int NVT, int B, bool WS, bool WT, bool CLAMP>
__device__ __forceinline__ void row_grads(const u32x4 (&xs)[NVT], const u32x4 (&xt)[NVT],
                                          int64_t nv, typename D::T *gs, typename D::T *gt,
                                          const float *rc) {
    constexpr int VEC = D::VEC;
    OpBwd<D, INTERIOR, WS, WT, D, CLAMP> op;
    op.gs = gs;
    op.gt = gt;
    op.set(rc);
#pragma unroll
    for (int i = 0; i < NVT; ++i) {
        const int64_t j = threadIdx.x + (int64_t)i * B;
        if (j < nv) {
            float a[1][VEC], b[1][VEC];
            widen<D>(xs[i], a[0]);
            widen<D>(xt[i], b[0]);
            const int64_t c[1] = {j * VEC};
            op.template run<1, VEC>(a, b, c);
        }
    }
}

// A row held in registers: k_fwd_row's forward, then the gradients from the same
// registers.  The gradient rows start on 16-byte boundaries like the inputs' (the host
// checks).
template <class D, int NVT, int B, bool WS, bool WT>
__global__ __launch_bounds__(B) __attribute__((amdgpu_waves_per_eu(fb_row_waves<B>())))
void k_fwdbwd_row(RowView sv, RowView tv, RowMView gsv,
                                                   RowMView gtv, int64_t w, double beta,
                                                   const float *__restrict__ grad,
                                                   double *stats, float *kl,
                                                   float *__restrict__ loss, RowOpts o,
                                                   GradOpts go) {
    using T = typename D::T;
    constexpr int VEC = D::VEC;
    __shared__ float red[4 * (B / 64)];
    __shared__ RowK rk;
    __shared__ float rc[ROWC];
    const int64_t r = blockIdx.x;
    T *gs = WS ? row_ptr<T>(gsv, r) : nullptr;
    T *gt = WT ? row_ptr<T>(gtv, r) : nullptr;
    if (row_dropped(o, r)) {
        dropped_row(stats + r * 4, kl + 2 * r, loss + r);
        zero_grads<D, B, WS, WT>(gs, gt, w);
        return;
    }
    const int64_t nv = w / VEC;
    u32x4 xs[NVT], xt[NVT];
    row_forward<D, NVT, B>(row_ptr<T>(sv, r), row_ptr<T>(tv, r), nv, beta, stats + r * 4,
                           kl + 2 * r, loss + r, o, red, rk, xs, xt);
    if (threadIdx.x == 0) fused_bwd_constants(stats, kl, r, beta, grad, go, rc);
    __syncthreads();
    if (rc[ROWC_UNDEFINED] != 0.0f) {  // no distribution: exactly zero gradients
        zero_grads<D, B, WS, WT>(gs, gt, w);
        return;
    }
    // The clamp-free gradients for rows within FAST_RANGE, in the 256-lane kernels
    // (8192 x 16032 bf16, A/B on one box: both gradients 0.274-0.277 -> 0.260 ms, the
    // student's 0.214-0.218 -> 0.199-0.206 ms); a second copy of the loop costs the
    // 512-lane kernels 32-40 more bytes of spill, and 1024 x 37984 ran 5 % slower with it.
    if constexpr (B == FB) {
        if (rk.fast) {
            row_grads<D, NVT, B, WS, WT, false>(xs, xt, nv, gs, gt, rc);
            return;
        }
    }
    OpBwd<D, INTERIOR, WS, WT> op;
    op.gs = gs;
    op.gt = gt;
    op.set(rc);
#pragma unroll
    for (int i = 0; i < NVT; ++i) {
        const int64_t j = threadIdx.x + (int64_t)i * B;
        if (j < nv) {
            float a[1][VEC], b[1][VEC];
            widen<D>(xs[i], a[0]);
            widen<D>(xt[i], b[0]);
            const int64_t c[1] = {j * VEC};
            op.template run<1, VEC>(a, b, c);
        }
    }
}

// The two-sweep row: k_fwd_twice's forward, then the gradients, the held steps first
// (registers, then LDS), then the rest of the row read a third time.  Gradient views at
// another offset inside 16 bytes than the inputs' take the whole row from memory.
// Measured on MI355X at 8192 x 151936 bf16, both gradients: 2.73-2.75 ms against
// 2.83-2.87 ms for the forward and backward launches.

// DG: the gradients' storage, the input's or bf16 for fp32 input (the fused-linear
// loss's logit gradient; its rows at the inputs' element offsets).
template <class D, bool WS, bool WT, class DG = D>
__global__ __launch_bounds__(TWICE_BLK)
__attribute__((amdgpu_waves_per_eu(fb_waves<D>(), fb_waves<D>())))
void k_fwdbwd_twice(RowView sv, RowView tv, RowMView gsv, RowMView gtv, int64_t w, double beta,
                    const float *__restrict__ grad, double *stats, float *kl,
                    float *__restrict__ loss, RowOpts o, GradOpts go) {
    using T = typename D::T;
    using TG = typename DG::T;
    constexpr int VEC = D::VEC;
    constexpr int64_t STEP = (int64_t)TW_U * TWICE_BLK;  // vectors per input per sweep step
    constexpr int HOLD = held_steps<D>(), LHOLD = lds_steps<D>();
    constexpr int U = fb_sweep_u<D>();
    __shared__ float red[6 * (TWICE_BLK / 64)];
    __shared__ RowK rk;
    __shared__ LdsStep<D> lds_step;
    __shared__ float rc[ROWC];
    const int64_t r = blockIdx.x;
    TG *gs = WS ? row_ptr<TG>(gsv, r) : nullptr;
    TG *gt = WT ? row_ptr<TG>(gtv, r) : nullptr;
    if (row_dropped(o, r)) {
        dropped_row(stats + r * 4, kl + 2 * r, loss + r);
        zero_grads<DG, TWICE_BLK, WS, WT>(gs, gt, w);
        return;
    }
    const T *s = row_ptr<T>(sv, r), *t = row_ptr<T>(tv, r);
    const TwiceSpan sp = twice_span<D>(w, head_len<T>(w, s, t));
    HeldRegs<D> hs, ht;
    // (the divergence sweep with the default load policy: the gradients read the row again)
    twice_forward<D, false>(s, t, w, sp, beta, stats + r * 4, kl + 2 * r, loss + r, o, red, rk,
                            lds_step, hs, ht);
    if (threadIdx.x == 0) fused_bwd_constants(stats, kl, r, beta, grad, go, rc);
    __syncthreads();
    if (rc[ROWC_UNDEFINED] != 0.0f) {  // no distribution: exactly zero gradients
        zero_grads<DG, TWICE_BLK, WS, WT>(gs, gt, w);
        return;
    }
    OpBwd<D, INTERIOR, WS, WT, DG> op;
    op.gs = gs;
    op.gt = gt;
    op.set(rc);
    // (a bf16 gradient of fp32 input: the inputs alone fix the head, as in k_bwd)
    const int64_t hg = std::is_same<D, DG>::value ? head_len<T>(w, s, t, gs, gt) : sp.h;
    if (!sp.hold || hg != sp.h) {
        sweep<D, U, true, TWICE_BLK, true>(s, t, w, hg, op);
        return;
    }
#pragma unroll
    for (int j = 0; j < HOLD; ++j) {
#pragma unroll
        for (int u = 0; u < TW_U; ++u) {
            // one held vector's widened values live at a time (as held_div)
            u32x4 xs = hs[j][u], xt = ht[j][u];
            if (u > 0) asm volatile("" : "+v"(xs), "+v"(xt));
            float a[1][VEC], b[1][VEC];
            widen<D>(xs, a[0]);
            widen<D>(xt, b[0]);
            const int64_t c[1] = {
                sp.PR + ((int64_t)j * STEP + threadIdx.x + (int64_t)u * TWICE_BLK) * VEC};
            op.template run<1, VEC>(a, b, c);
        }
    }
#pragma unroll
    for (int l = 0; l < LHOLD; ++l) {
        if (LHOLD > 1 && l >= sp.lh) break;
#pragma unroll
        for (int u = 0; u < TW_U; ++u) {
            float a[1][VEC], b[1][VEC];
            widen<D>(lds_step[l][0][u][threadIdx.x], a[0]);
            widen<D>(lds_step[l][1][u][threadIdx.x], b[0]);
            const int64_t c[1] = {
                sp.P + ((int64_t)l * STEP + threadIdx.x + (int64_t)u * TWICE_BLK) * VEC};
            op.template run<1, VEC>(a, b, c);
        }
    }
    sweep<D, U, true, TWICE_BLK, true>(s, t, sp.P, sp.h, op);
    if (WS) op.gs = gs + sp.Q;
    if (WT) op.gt = gt + sp.Q;
    sweep<D, U, true, TWICE_BLK, true>(s + sp.Q, t + sp.Q, w - sp.Q, 0, op);
}

// Orders one wave's LDS writes before that wave's later LDS reads of other lanes'
// values (wavefront-scope release, the wave's barrier, acquire).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Steps of the widest shard's slice that k_fwd_shards holds on chip, as k_fwd_twice
// holds a row's: fp32 four in registers and up to two in LDS (one workgroup per CU, as
// the fp32 two-sweep kernel), 16-bit formats none.  Measured on MI355X (4096 x 128256
// fp32 in shards 60000/0/40000/28256; 8192 x 151936 bf16 in 40000/40000/0/71936): fp32
// 1.16 -> 1.03 ms with four register steps and one LDS step, the merge behind one
// barrier and the sweeps' partial steps loaded at once (one shard: 1.00 ms); a bf16 LDS
// step ran 6 % slower (1.37 -> 1.45 ms), and a register step in the 16-bit kernels, live
// across the loop over shards, costs them their second workgroup per CU.
template <class D>
constexpr int shard_held_steps() { return sizeof(typename D::T) == 4 ? 4 : 0; }
template <class D>
constexpr int shard_lds_steps() { return sizeof(typename D::T) == 4 ? 2 : 0; }

// Several logical shards of a row, one launch: the workgroup sweeps each shard's slice
// for that shard's (max, sum-exp) pair of each input, merges the pairs in shard order
// exactly as the merge launch does (maximum of the maxima, then the rescaled sums in
// fp64; an empty shard adds nothing), then sweeps the slices again for the divergence
// terms.  The pages' cross-rank reductions of [N] statistics become this in-workgroup
// merge when all shards sit on one device [JSD-PR, Changes; OPS-PR, How].  Each wave's
// pairs of every shard are combined after the last shard's sweep, behind one barrier;
// in fp32 the widest shard's last full steps stay on chip for the divergence sweep.

// The divergence sweep of k_fwd_shards over every non-empty shard's slice, last shard
// first (each slice backwards, as twice_stream runs), continuing the sums v of the held
// steps: the held shard qh's slice skips its held columns [P, Q).
template <class D, bool SAFE>
__device__ __forceinline__ void shards_div(const ShardRows &sr, int64_t r, const MixRow &mx,
                                           float beta, float ks, int qh, bool hold, int64_t P,
                                           int64_t Q, float (&v)[2]) {
    using T = typename D::T;
    for (int q = sr.S - 1; q >= 0; --q) {
        const int64_t w = sr.w[q];
        if (w == 0) continue;
        const T *s = row_ptr<T>(sr.s[q], r), *t = row_ptr<T>(sr.t[q], r);
        const int64_t h = head_len<T>(w, s, t);
        twice_stream<D, SAFE>(mx, beta, ks, hold && q == qh, s, t, w, h, P, Q, v);
    }
}

template <class D>
__global__ __launch_bounds__(TWICE_BLK) void k_fwd_shards(ShardRows sr, double beta,
                                                          double *__restrict__ stats,
                                                          float *__restrict__ kl,
                                                          float *__restrict__ loss, RowOpts o) {
    using T = typename D::T;
    constexpr int VEC = D::VEC;
    constexpr int NW = TWICE_BLK / 64;
    constexpr int64_t STEP = (int64_t)TW_U * TWICE_BLK;  // vectors per input per sweep step
    constexpr int HOLD = shard_held_steps<D>(), LHOLD = shard_lds_steps<D>();
    __shared__ float red[6 * NW];
    __shared__ float sp[FUSED_SHARDS][6];  // per shard: (m_s, z_s, m_t, z_t, min_s, min_t)
    __shared__ float wp[FUSED_SHARDS][NW][6];  // the same per shard and wave
    const int64_t r = blockIdx.x;
    if (row_dropped(o, r)) {
        dropped_row(stats + r * 4, kl + 2 * r, loss + r);
        return;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // the widest shard (the first of equals) holds its statistics sweep's last full
    // steps, [P, Q) of its slice ([P, PR) in LDS, lh of them, [PR, Q) in registers),
    // when it has the register steps and one LDS step
    int qh = -1;
    for (int q = 0; q < sr.S; ++q)
        if (sr.w[q] > 0 && (qh < 0 || sr.w[q] > sr.w[qh])) qh = q;
    bool hold = false;
    int lh = 0;
    int64_t P = 0, PR = 0, Q = 0;
    if (qh >= 0 && HOLD + LHOLD > 0) {
        const int64_t w = sr.w[qh];
        const T *s = row_ptr<T>(sr.s[qh], r), *t = row_ptr<T>(sr.t[qh], r);
        const int64_t h = head_len<T>(w, s, t);
        const int64_t nfull = h < w ? (w - h) / VEC / STEP : 0;
        hold = nfull >= HOLD + (LHOLD > 0 ? 1 : 0);
        lh = hold ? (int)(nfull - HOLD < LHOLD ? nfull - HOLD : LHOLD) : 0;
        P = hold ? h + (nfull - HOLD - lh) * STEP * VEC : w;
        PR = P + lh * STEP * VEC;
        Q = hold ? PR + HOLD * STEP * VEC : w;
    }
    // each lane's own vectors
    __shared__ u32x4 lds_step[LHOLD ? LHOLD : 1][2][TW_U][LHOLD ? TWICE_BLK : 1];
    u32x4 hs[HOLD ? HOLD : 1][TW_U], ht[HOLD ? HOLD : 1][TW_U];
    for (int q = 0; q < sr.S; ++q) {
        OpStats<3, true> o1(o.ks);
        const int64_t w = sr.w[q];
        if (w > 0) {
            const T *s = row_ptr<T>(sr.s[q], r), *t = row_ptr<T>(sr.t[q], r);
            const int64_t h = head_len<T>(w, s, t);
            if (hold && q == qh) {
                sweep<D, TW_U, true, TWICE_BLK>(s, t, P, h, o1);
#pragma unroll
                for (int l = 0; l < LHOLD; ++l) {
                    if (l >= lh) break;
                    u32x4 ls[TW_U], lt[TW_U];
#pragma unroll
                    for (int u = 0; u < TW_U; ++u) {
                        const int64_t c =
                            P + ((int64_t)l * STEP + threadIdx.x + (int64_t)u * TWICE_BLK) * VEC;
                        ls[u] = ld16<true>(s + c);
                        lt[u] = ld16<true>(t + c);
                    }
#pragma unroll
                    for (int u = 0; u < TW_U; ++u) {
                        lds_step[l][0][u][threadIdx.x] = ls[u];
                        lds_step[l][1][u][threadIdx.x] = lt[u];
                    }
                    held_stats<D>(ls, lt, o1);
                }
#pragma unroll
                for (int k = 0; k < HOLD; ++k) {
#pragma unroll
                    for (int u = 0; u < TW_U; ++u) {
                        const int64_t c =
                            PR + ((int64_t)k * STEP + threadIdx.x + (int64_t)u * TWICE_BLK) * VEC;
                        hs[k][u] = ld16<true>(s + c);
                        ht[k][u] = ld16<true>(t + c);
                    }
                    held_stats<D>(hs[k], ht[k], o1);
                }
                sweep<D, TW_U, true, TWICE_BLK>(s + Q, t + Q, w - Q, 0, o1);
            } else {
                sweep<D, TW_U, true, TWICE_BLK>(s, t, w, h, o1);
            }
        }
        // this wave's pair for the shard; the waves are combined after the last shard,
        // behind one barrier for all shards
        // (an empty shard's pair is the identity, exactly what its reductions give)
        MZ ws{NINF, 0.0f}, wt{NINF, 0.0f};
        float ns = __builtin_huge_valf(), nt = __builtin_huge_valf();
        if (w > 0) {
            ws = wave_mz(MZ{o1.a.m, o1.a.z}, o.ks);
            wt = wave_mz(MZ{o1.b.m, o1.b.z}, o.ks);
            ns = wave_min(o1.a.mn);
            nt = wave_min(o1.b.mn);
        }
        if (lane == 0) {
            float *d = wp[q][wave];
            d[0] = ws.m;
            d[1] = ws.z;
            d[2] = wt.m;
            d[3] = wt.z;
            d[4] = ns;
            d[5] = nt;
        }
    }
    __syncthreads();
    __shared__ RowK rk;
    if (wave == 0) {
        // lane q combines shard q's wave pairs in wave order (as one shard's workgroup
        // combines them), then the whole wave merges the shards
        if (lane < sr.S) {
            const int q = lane;
            MZ ms{wp[q][0][0], wp[q][0][1]}, mt{wp[q][0][2], wp[q][0][3]};
            float mns = wp[q][0][4], mnt = wp[q][0][5];
            for (int k = 1; k < NW; ++k) {
                ms = mz_combine(ms, MZ{wp[q][k][0], wp[q][k][1]}, o.ks);
                mt = mz_combine(mt, MZ{wp[q][k][2], wp[q][k][3]}, o.ks);
                mns = fminf(mns, wp[q][k][4]);
                mnt = fminf(mnt, wp[q][k][5]);
            }
            sp[q][0] = ms.m;
            sp[q][1] = ms.z;
            sp[q][2] = mt.m;
            sp[q][3] = mt.z;
            sp[q][4] = mns;
            sp[q][5] = mnt;
        }
        // the lanes' LDS writes above come before the reads below
        wave_lds_sync();
        float ms = NINF, mt = NINF, ns = __builtin_huge_valf(), nt = __builtin_huge_valf();
        for (int q = 0; q < sr.S; ++q) {
            ms = fmaxf(ms, sp[q][0]);
            mt = fmaxf(mt, sp[q][2]);
            ns = fminf(ns, sp[q][4]);
            nt = fminf(nt, sp[q][5]);
        }
        const double cs = refc(ms, o.ks), ct = refc(mt, o.ks);
        double zs = 0.0, zt = 0.0;
        for (int q = 0; q < sr.S; ++q) {
            if (sp[q][0] != NINF) zs += (double)sp[q][1] * exp2((double)refc(sp[q][0], o.ks) - cs);
            if (sp[q][2] != NINF) zt += (double)sp[q][3] * exp2((double)refc(sp[q][2], o.ks) - ct);
        }
        row_constants(ms, zs, mt, zt, ns, nt, beta, o.ks, stats + r * 4, &rk);
    }
    __syncthreads();
    const RowK k = rk;
    float v[2] = {0.0f, 0.0f};
    if (!k.undefined) {
        // the held steps first, in the form that admits masked tokens (as k_fwd_twice)
        if (hold) {
            OpMix<true> oh;
            oh.set(k.mx, (float)beta, o.ks);
#pragma unroll
            for (int j = 0; j < HOLD; ++j) held_div<D>(hs[j], ht[j], oh);
#pragma unroll
            for (int l = 0; l < LHOLD; ++l) {
                if (l >= lh) break;
                u32x4 ls[TW_U], lt[TW_U];
#pragma unroll
                for (int u = 0; u < TW_U; ++u) {
                    ls[u] = lds_step[l][0][u][threadIdx.x];
                    lt[u] = lds_step[l][1][u][threadIdx.x];
                }
                held_div<D>(ls, lt, oh);
            }
            v[0] = oh.sum_t();
            v[1] = oh.sum_s();
        }
        if (k.fast) shards_div<D, false>(sr, r, k.mx, (float)beta, o.ks, qh, hold, P, Q, v);
        else shards_div<D, true>(sr, r, k.mx, (float)beta, o.ks, qh, hold, P, Q, v);
    }
    block_sum<2, TWICE_BLK>(v, red);
    if (threadIdx.x == 0) finish_row(k, beta, v[0], v[1], kl + 2 * r, loss + r, o.lscale);
}

// Every row of the view starts on a 16-byte boundary.
template <class V>
bool rows16(const V &v, int64_t N, int esize) {
    if (reinterpret_cast<uintptr_t>(v.p) % 16 != 0) return false;
    if ((v.rs * esize) % 16 != 0 && N > 1) return false;
    if (v.rpb > 0 && (v.bs * esize) % 16 != 0) return false;
    return true;
}

// The register-held row's workgroup shape for rows of nv 16-byte vectors (nv <=
// FB_WIDE * ROW_WIDE_NVT_MAX): 256 lanes with 1, 2, 4 or 8 vectors, then 512 lanes with
// 6, 8 or 10.
enum RowShape { R1, R2, R4, R8, W6, W8, W10 };
RowShape row_shape(int64_t nv) {
    if (nv <= FB) return R1;
    if (nv <= 2 * FB) return R2;
    if (nv <= 4 * FB) return R4;
    if (nv <= 8 * FB) return R8;
    if (nv <= 6 * FB_WIDE) return W6;
    if (nv <= 8 * FB_WIDE) return W8;
    return W10;
}

// Rows of shard sh fit the register-held kernels: whole vectors, at most
// FB_WIDE * ROW_WIDE_NVT_MAX of them, every row of both inputs 16-byte aligned.
template <class D>
bool row_fits(const Shard &sh, int64_t N) {
    constexpr int VEC = D::VEC;
    const int64_t w = sh.width;
    const int esize = (int)sizeof(typename D::T);
    return w > 0 && w % VEC == 0 && w / VEC <= (int64_t)FB_WIDE * ROW_WIDE_NVT_MAX &&
           rows16(sh.s, N, esize) && rows16(sh.t, N, esize);
}

template <class D, int NVT, int B>
hipError_t row_launch(const Shard &sh, int64_t N, double beta, double *stats, float *kl,
                      float *loss, hipStream_t st, const RowOpts &o) {
    hipLaunchKernelGGL((k_fwd_row<D, NVT, B>), dim3((unsigned)N), dim3(B), 0, st, sh.s, sh.t,
                       sh.width, beta, stats, kl, loss, o);
    return hipGetLastError();
}

// Row held in registers when the layout allows it, else the two sweeps.
template <class D>
hipError_t fused_launch(const Shard &sh, int64_t N, double beta, double *stats, float *kl,
                        float *loss, hipStream_t st, const RowOpts &o) {
    if (!row_fits<D>(sh, N)) {
        hipLaunchKernelGGL(k_fwd_twice<D>, dim3((unsigned)N), dim3(TWICE_BLK), 0, st, sh.s,
                           sh.t, sh.width, beta, stats, kl, loss, o);
        return hipGetLastError();
    }
    switch (row_shape(sh.width / D::VEC)) {
        case R1: return row_launch<D, 1, FB>(sh, N, beta, stats, kl, loss, st, o);
        case R2: return row_launch<D, 2, FB>(sh, N, beta, stats, kl, loss, st, o);
        case R4: return row_launch<D, 4, FB>(sh, N, beta, stats, kl, loss, st, o);
        case R8: return row_launch<D, 8, FB>(sh, N, beta, stats, kl, loss, st, o);
        case W6: return row_launch<D, 6, FB_WIDE>(sh, N, beta, stats, kl, loss, st, o);
        case W8: return row_launch<D, 8, FB_WIDE>(sh, N, beta, stats, kl, loss, st, o);
        default: return row_launch<D, ROW_WIDE_NVT_MAX, FB_WIDE>(sh, N, beta, stats, kl, loss, st, o);
    }
}

// Arguments of a forward-and-backward launch.
struct FbArgs {
    double beta;
    const float *grad;
    double *stats;
    float *kl, *loss;
    RowOpts o;
    GradOpts go;
};

template <class D, int NVT, int B, bool WS, bool WT>
hipError_t fb_row_launch(const Shard &sh, int64_t N, const FbArgs &a, hipStream_t st) {
    hipLaunchKernelGGL((k_fwdbwd_row<D, NVT, B, WS, WT>), dim3((unsigned)N), dim3(B), 0, st,
                       sh.s, sh.t, sh.gs, sh.gt, sh.width, a.beta, a.grad, a.stats, a.kl, a.loss,
                       a.o, a.go);
    return hipGetLastError();
}

// The register-held row when the inputs fit it and the wanted gradient views are
// 16-byte aligned too; the two sweeps for rows the register kernels do not take.  Rows
// the forward alone would hold in registers but whose gradient views are not aligned
// are not fused: hipErrorNotSupported, and the caller runs the two entry points.
template <class D, bool WS, bool WT>
hipError_t fb_launch(const Shard &sh, int64_t N, const FbArgs &a, hipStream_t st) {
    const int esize = (int)sizeof(typename D::T);
    if (!row_fits<D>(sh, N)) {
        hipLaunchKernelGGL((k_fwdbwd_twice<D, WS, WT>), dim3((unsigned)N), dim3(TWICE_BLK), 0, st,
                           sh.s, sh.t, sh.gs, sh.gt, sh.width, a.beta, a.grad, a.stats, a.kl,
                           a.loss, a.o, a.go);
        return hipGetLastError();
    }
    if ((WS && !rows16(sh.gs, N, esize)) || (WT && !rows16(sh.gt, N, esize)))
        return hipErrorNotSupported;
    switch (row_shape(sh.width / D::VEC)) {
        case R1: return fb_row_launch<D, 1, FB, WS, WT>(sh, N, a, st);
        case R2: return fb_row_launch<D, 2, FB, WS, WT>(sh, N, a, st);
        case R4: return fb_row_launch<D, 4, FB, WS, WT>(sh, N, a, st);
        case R8: return fb_row_launch<D, 8, FB, WS, WT>(sh, N, a, st);
        case W6: return fb_row_launch<D, 6, FB_WIDE, WS, WT>(sh, N, a, st);
        case W8: return fb_row_launch<D, 8, FB_WIDE, WS, WT>(sh, N, a, st);
        default: return fb_row_launch<D, ROW_WIDE_NVT_MAX, FB_WIDE, WS, WT>(sh, N, a, st);
    }
}

template <class D>
hipError_t fb_want(const Shard &sh, int64_t N, const FbArgs &a, hipStream_t st) {
    const bool ws = sh.gs.p != nullptr, wt = sh.gt.p != nullptr;
    if (ws && wt) return fb_launch<D, true, true>(sh, N, a, st);
    if (ws) return fb_launch<D, true, false>(sh, N, a, st);
    if (wt) return fb_launch<D, false, true>(sh, N, a, st);
    return fused_launch<D>(sh, N, a.beta, a.stats, a.kl, a.loss, st, a.o);
}

}  // namespace

hipError_t launch_fwd_shards(int dtype, const Shard *sh, int S, int64_t N, double beta,
                             double *stats, float *kl, float *loss, hipStream_t st,
                             const RowOpts &o) {
    if (S < 1 || S > FUSED_SHARDS) return hipErrorInvalidValue;
    ShardRows sr{};
    sr.S = S;
    for (int q = 0; q < S; ++q) {
        sr.w[q] = sh[q].width;
        sr.s[q] = sh[q].s;
        sr.t[q] = sh[q].t;
    }
    const dim3 grid((unsigned)N), block(TWICE_BLK);
    switch (dtype) {
        case 0: hipLaunchKernelGGL(k_fwd_shards<F32>, grid, block, 0, st, sr, beta, stats, kl, loss, o); break;
        case 1: hipLaunchKernelGGL(k_fwd_shards<F16>, grid, block, 0, st, sr, beta, stats, kl, loss, o); break;
        default: hipLaunchKernelGGL(k_fwd_shards<BF16>, grid, block, 0, st, sr, beta, stats, kl, loss, o);
    }
    return hipGetLastError();
}

hipError_t launch_fwd_fused(int dtype, const Shard &sh, int64_t N, double beta, double *stats,
                            float *kl, float *loss, hipStream_t st, const RowOpts &o) {
    switch (dtype) {
        case 0: return fused_launch<F32>(sh, N, beta, stats, kl, loss, st, o);
        case 1: return fused_launch<F16>(sh, N, beta, stats, kl, loss, st, o);
        default: return fused_launch<BF16>(sh, N, beta, stats, kl, loss, st, o);
    }
}

hipError_t launch_fwd_bwd_f32_bf16(const Shard &sh, int64_t N, double beta, double *stats,
                                   float *kl, float *loss, hipStream_t st, const RowOpts &o,
                                   const GradOpts &go) {
    if (sh.gs.p == nullptr || sh.gt.p != nullptr) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_fwdbwd_twice<F32, true, false, BF16>), dim3((unsigned)N),
                       dim3(TWICE_BLK), 0, st, sh.s, sh.t, sh.gs, sh.gt, sh.width, beta,
                       (const float *)nullptr, stats, kl, loss, o, go);
    return hipGetLastError();
}

hipError_t launch_fwd_bwd_fused(int dtype, const Shard &sh, int64_t N, double beta,
                                const float *grad, double *stats, float *kl, float *loss,
                                hipStream_t st, const RowOpts &o, const GradOpts &go) {
    const FbArgs a{beta, grad, stats, kl, loss, o, go};
    switch (dtype) {
        case 0: return fb_want<F32>(sh, N, a, st);
        case 1: return fb_want<F16>(sh, N, a, st);
        default: return fb_want<BF16>(sh, N, a, st);
    }
}

}  // namespace vjsd
