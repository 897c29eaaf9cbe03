// fused.hip -- the JSD forward in one HBM pass for rows that fit one workgroup.
//
// [JSD-PR] DeepSpeed PR #8958 "[VocabTP] Add vocabulary-parallel generalized JSD with
// Triton kernels", section Scope and limitations: the JSD needs the global normaliser
// before the nonlinear mixture, so statistics and divergence are two passes over the
// input.  When a whole row of both inputs fits in one workgroup's registers (256 lanes
// x FUSED_NVT_MAX 16-byte vectors per input: up to 16384 bf16 / fp16 or 8192 fp32
// columns), the two passes run over registers and each logit is read from HBM once;
// the row constants are rebuilt from the fp64 statistics exactly as the separate
// passes rebuild them.  Wider rows take the separate statistics, merge and divergence
// launches: splitting a row over several workgroups needs a device-wide exchange per
// row, and on MI355X the cache write-back and invalidation that a correct device-scope
// release/acquire costs exceeds the second read it would save.
#include "kernels.hpp"
#include "sweep.hpp"

namespace vjsd {

namespace {

constexpr int FB = 256;
constexpr int FNW = FB / 64;

// raw 32-bit word of -inf in each storage format (two halves for 16-bit formats)
template <class D>
__device__ __forceinline__ uint32_t ninf_word();
template <>
__device__ __forceinline__ uint32_t ninf_word<F32>() { return 0xff800000u; }
template <>
__device__ __forceinline__ uint32_t ninf_word<F16>() { return 0xfc00fc00u; }
template <>
__device__ __forceinline__ uint32_t ninf_word<BF16>() { return 0xff80ff80u; }

template <class D>
__device__ __forceinline__ void unpack(const uint4 &v, float (&x)[D::VEC]);
template <>
__device__ __forceinline__ void unpack<F32>(const uint4 &v, float (&x)[4]) {
    x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
}
template <>
__device__ __forceinline__ void unpack<BF16>(const uint4 &v, float (&x)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
template <>
__device__ __forceinline__ void unpack<F16>(const uint4 &v, float (&x)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f16x2 h = __builtin_bit_cast(f16x2, w[i]);
        x[2 * i] = (float)h.x;
        x[2 * i + 1] = (float)h.y;
    }
}

// Empty register barrier: the compiler must assume the packed vectors changed, so it
// re-widens them in each sweep instead of keeping NVT * 2 * VEC floats alive.
__device__ __forceinline__ void opaque(uint4 &v) {
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

__device__ __forceinline__ void block_max2(float &a, float &b, float *red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    a = wave_max(a);
    b = wave_max(b);
    if (lane == 0) {
        red[wave] = a;
        red[FNW + wave] = b;
    }
    __syncthreads();
    float x = red[0], y = red[FNW];
#pragma unroll
    for (int k = 1; k < FNW; ++k) {
        x = fmaxf(x, red[k]);
        y = fmaxf(y, red[FNW + k]);
    }
    a = x;
    b = y;
    __syncthreads();
}

__device__ __forceinline__ void block_sum2(float &a, float &b, float *red) {
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

// One workgroup per row.  Lane l holds vectors l, l + FB, ... of each input; slots past
// the row's end hold -inf, which adds exactly nothing to any sum below.
template <class D, int MODE, int NVT>
__global__ __launch_bounds__(FB) void k_fwd_row(RowView sv, RowView tv, int64_t w, double beta,
                                                double *__restrict__ stats,
                                                float *__restrict__ kl,
                                                float *__restrict__ loss) {
    using T = typename D::T;
    constexpr int VEC = D::VEC;
    __shared__ float red[2 * FNW];
    const int64_t r = blockIdx.x;
    const T *s = row_ptr<T>(sv, r), *t = row_ptr<T>(tv, r);
    const int64_t nv = w / VEC;  // whole vectors: the host requires w % VEC == 0
    uint4 xs[NVT], xt[NVT];
#pragma unroll
    for (int i = 0; i < NVT; ++i) {
        const int64_t j = threadIdx.x + (int64_t)i * FB;
        if (j < nv) {
            xs[i] = *reinterpret_cast<const uint4 *>(s + j * VEC);
            xt[i] = *reinterpret_cast<const uint4 *>(t + j * VEC);
        } else {
            const uint32_t q = ninf_word<D>();
            xs[i] = make_uint4(q, q, q, q);
            xt[i] = make_uint4(q, q, q, q);
        }
    }
    // ---- statistics: row max, then sum of 2^(x log2e - c)
    float ms = NINF, mt = NINF;
#pragma unroll
    for (int i = 0; i < NVT; ++i) {
        float a[VEC], b[VEC];
        unpack<D>(xs[i], a);
        unpack<D>(xt[i], b);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            ms = fmaxf(ms, a[e]);
            mt = fmaxf(mt, b[e]);
        }
    }
    block_max2(ms, mt, red);
#pragma unroll
    for (int i = 0; i < NVT; ++i) {
        opaque(xs[i]);
        opaque(xt[i]);
    }
    const float cs = refc(ms), ct = refc(mt);
    float zs = 0.0f, zt = 0.0f;
#pragma unroll
    for (int i = 0; i < NVT; ++i) {
        float a[VEC], b[VEC], ea[VEC], eb[VEC];
        unpack<D>(xs[i], a);
        unpack<D>(xt[i], b);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            ea[e] = ex2(fmaf(a[e], L2E, -cs));
            eb[e] = ex2(fmaf(b[e], L2E, -ct));
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
    block_sum2(zs, zt, red);
    const bool undefined = ms == NINF || mt == NINF;
    const double lzs = ms == NINF ? -__builtin_inf() : lnz_from_z(ms, (double)zs);
    const double lzt = mt == NINF ? -__builtin_inf() : lnz_from_z(mt, (double)zt);
    if (threadIdx.x == 0) {
        double *o = stats + r * 4;
        o[0] = ms;
        o[1] = lzs;
        o[2] = mt;
        o[3] = lzt;
    }
    // ---- divergence: row constants from the stored statistics, terms from registers
    float pt = 0.0f, ps = 0.0f, F = NINF;
    double Zs = 1.0, Zt = 1.0;
    if (!undefined) {
        Zs = z_from_stats(ms, lzs);
        Zt = z_from_stats(mt, lzt);
        OpDivRegs<MODE> op;
        op.cs = cs;
        op.ct = ct;
        op.bf = (float)beta;
        op.gam = (float)((1.0 - beta) * Zt / Zs);
        op.rf = (float)log2(Zs / Zt);
#pragma unroll
        for (int i = 0; i < NVT; ++i) {
            opaque(xs[i]);
            opaque(xt[i]);
        }
#pragma unroll
        for (int i = 0; i < NVT; ++i) {
            float a[VEC], b[VEC];
            unpack<D>(xs[i], a);
            unpack<D>(xt[i], b);
            op.template add<VEC>(a, b);
        }
        pt = op.At;
        ps = op.As;
        F = op.F;
    }
    block_sum2(pt, ps, red);
    float G = NINF;
    block_max2(F, G, red);
    if (threadIdx.x == 0)
        finalize_row(MODE, beta, undefined, pt * (float)(1.0 / Zt), ps * (float)(1.0 / Zs), F,
                     kl + 2 * r, loss + r);
}

template <class D, int MODE, int NVT>
hipError_t row_launch(const Shard &sh, int64_t N, double beta, double *stats, float *kl,
                      float *loss, hipStream_t st) {
    hipLaunchKernelGGL((k_fwd_row<D, MODE, NVT>), dim3((unsigned)N), dim3(FB), 0, st, sh.s, sh.t,
                       sh.width, beta, stats, kl, loss);
    return hipGetLastError();
}

template <class D, int MODE>
hipError_t fused_launch(const Shard &sh, int64_t N, double beta, double *stats, float *kl,
                        float *loss, hipStream_t st, bool *used) {
    constexpr int VEC = D::VEC;
    *used = false;
    const int64_t w = sh.width;
    if (w <= 0 || w % VEC != 0 || N <= 0 || N > 0x7fffffffLL) return hipSuccess;
    const int64_t nv = w / VEC;
    if (nv > (int64_t)FB * FUSED_NVT_MAX) return hipSuccess;
    const int esize = (int)sizeof(typename D::T);
    const RowView *views[2] = {&sh.s, &sh.t};
    for (const RowView *v : views) {  // every row must start on a 16-byte boundary
        if (reinterpret_cast<uintptr_t>(v->p) % 16 != 0) return hipSuccess;
        if ((v->rs * esize) % 16 != 0 && N > 1) return hipSuccess;
        if (v->rpb > 0 && (v->bs * esize) % 16 != 0) return hipSuccess;
    }
    hipError_t e;
    if (nv <= FB) e = row_launch<D, MODE, 1>(sh, N, beta, stats, kl, loss, st);
    else if (nv <= 2 * FB) e = row_launch<D, MODE, 2>(sh, N, beta, stats, kl, loss, st);
    else if (nv <= 4 * FB) e = row_launch<D, MODE, 4>(sh, N, beta, stats, kl, loss, st);
    else e = row_launch<D, MODE, FUSED_NVT_MAX>(sh, N, beta, stats, kl, loss, st);
    if (e == hipSuccess) *used = true;
    return e;
}

template <class D>
hipError_t fused_mode(int mode, const Shard &sh, int64_t N, double beta, double *stats,
                      float *kl, float *loss, hipStream_t st, bool *used) {
    if (mode == INTERIOR) return fused_launch<D, INTERIOR>(sh, N, beta, stats, kl, loss, st, used);
    if (mode == FWD_KL) return fused_launch<D, FWD_KL>(sh, N, beta, stats, kl, loss, st, used);
    return fused_launch<D, REV_KL>(sh, N, beta, stats, kl, loss, st, used);
}

}  // namespace

hipError_t launch_fwd_fused(int dtype, int mode, const Shard &sh, int64_t N, double beta,
                            double *stats, float *kl, float *loss, hipStream_t st, bool *used) {
    switch (dtype) {
        case 0: return fused_mode<F32>(mode, sh, N, beta, stats, kl, loss, st, used);
        case 1: return fused_mode<F16>(mode, sh, N, beta, stats, kl, loss, st, used);
        default: return fused_mode<BF16>(mode, sh, N, beta, stats, kl, loss, st, used);
    }
}

}  // namespace vjsd
