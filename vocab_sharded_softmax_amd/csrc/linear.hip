// linear.hip -- the element-wise helper of the losses that compute their gradients in
// the forward (the fused-linear loss, the distillation loss with its gradients in the
// forward): scaling gradients computed for a unit upstream gradient by the actual one (a
// device scalar), so the caller's backward needs no host synchronisation.
#include "kernels.hpp"

namespace vjsd {
namespace {

constexpr int SCALE_BLOCK = 256;

template <class D>
__global__ __launch_bounds__(SCALE_BLOCK) void k_scale(typename D::T *p, int64_t n,
                                                       const float *__restrict__ g) {
    const float s = g[0];
    if (s == 1.0f) return;  // x * 1 is x in every format: nothing to read or write
    const int64_t nv = n / D::VEC;
    const int64_t stride = (int64_t)gridDim.x * SCALE_BLOCK;
    for (int64_t v = (int64_t)blockIdx.x * SCALE_BLOCK + threadIdx.x; v < nv; v += stride) {
        float x[D::VEC];
        load_vec<D, true>(p + v * D::VEC, x);
#pragma unroll
        for (int i = 0; i < D::VEC; ++i) x[i] *= s;
        store_vec<D, true>(p + v * D::VEC, x);
    }
    for (int64_t i = nv * D::VEC + (int64_t)blockIdx.x * SCALE_BLOCK + threadIdx.x; i < n;
         i += stride)
        store1<D>(p + i, load1<D>(p + i) * s);
}

// dst[c][r] = src[r][c] for 16-bit elements, r < R, c < C: one 128 x 128 tile per
// workgroup through LDS (rows padded by 2 elements), so every row segment read or
// written is 256 bytes.  Interior tiles move 16-byte
// vectors (row strides multiples of 8 elements, bases 16-byte aligned); edge tiles
// move single elements.
constexpr int TT = 128, TT_BLOCK = 256;
constexpr int TT_VEC = TT * TT / 8 / TT_BLOCK;  // 16-byte vectors per thread

__global__ __launch_bounds__(TT_BLOCK) void k_transpose16(const uint16_t *__restrict__ src,
                                                          int64_t lds_, int64_t R, int64_t C,
                                                          uint16_t *__restrict__ dst,
                                                          int64_t ldd, int rows_fast) {
    __shared__ uint16_t tile[TT][TT + 2];
    // consecutive workgroups step along the longer dimension
    const int64_t r0 = (int64_t)(rows_fast ? blockIdx.x : blockIdx.y) * TT;
    const int64_t c0 = (int64_t)(rows_fast ? blockIdx.y : blockIdx.x) * TT;
    const bool full = r0 + TT <= R && c0 + TT <= C;
    const int t = threadIdx.x;
    if (full) {
#pragma unroll
        for (int i = 0; i < TT_VEC; ++i) {  // TT rows x TT / 8 vectors of 8
            const int q = t + TT_BLOCK * i, r = q / (TT / 8), cv = (q % (TT / 8)) * 8;
            const u32x4 v = ld16<false>(src + (r0 + r) * lds_ + c0 + cv);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t w = v[e];
                tile[r][cv + 2 * e] = (uint16_t)(w & 0xffffu);
                tile[r][cv + 2 * e + 1] = (uint16_t)(w >> 16);
            }
        }
    } else {
        for (int q = t; q < TT * TT; q += TT_BLOCK) {
            const int r = q / TT, c = q % TT;
            if (r0 + r < R && c0 + c < C) tile[r][c] = src[(r0 + r) * lds_ + c0 + c];
        }
    }
    __syncthreads();
    if (full) {
#pragma unroll
        for (int i = 0; i < TT_VEC; ++i) {  // TT output rows (source columns) x TT / 8 vectors
            const int q = t + TT_BLOCK * i, c = q / (TT / 8), rv = (q % (TT / 8)) * 8;
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] = (uint32_t)tile[rv + 2 * e][c] | ((uint32_t)tile[rv + 2 * e + 1][c] << 16);
            st16<false>(dst + (c0 + c) * ldd + r0 + rv, u32x4{w[0], w[1], w[2], w[3]});
        }
    } else {
        for (int q = t; q < TT * TT; q += TT_BLOCK) {
            const int c = q / TT, r = q % TT;
            if (r0 + r < R && c0 + c < C) dst[(c0 + c) * ldd + r0 + r] = tile[r][c];
        }
    }
}

__global__ __launch_bounds__(256) void k_sum_partials(const float *__restrict__ part, int S,
                                                     int64_t stride, int64_t M, int64_t N,
                                                     int64_t ldp, uint16_t *__restrict__ out,
                                                     int64_t ldo) {
    const int64_t total = M * N;
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total;
         q += (int64_t)gridDim.x * 256) {
        const int64_t i = q / N, j = q - i * N;
        float v = part[i * ldp + j];
        for (int s = 1; s < S; ++s) v += part[s * stride + i * ldp + j];
        out[i * ldo + j] = (uint16_t)(__builtin_bit_cast(
                                          uint32_t, __builtin_convertvector((f32x2){v, 0.0f},
                                                                            bf16x2)) &
                                      0xffffu);
    }
}

}  // namespace

hipError_t launch_sum_partials(const float *part, int S, int64_t stride, int64_t M, int64_t N,
                               int64_t ldp, uint16_t *out, int64_t ldo, hipStream_t st) {
    if (M == 0 || N == 0) return hipSuccess;
    const int64_t want = (M * N + 255) / 256;
    const unsigned blocks = (unsigned)(want < 16384 ? want : 16384);
    hipLaunchKernelGGL(k_sum_partials, dim3(blocks), dim3(256), 0, st, part, S, stride, M, N, ldp,
                       out, ldo);
    return hipGetLastError();
}

hipError_t launch_transpose16(const uint16_t *src, int64_t lds_, int64_t R, int64_t C,
                              uint16_t *dst, int64_t ldd, hipStream_t st) {
    if (R == 0 || C == 0) return hipSuccess;
    // grid.x runs along the longer dimension; the shorter one (grid.y, at most 65535
    // tiles a launch) is cut into launches
    const int rows_fast = R >= C;
    const int64_t ylen = rows_fast ? C : R, xlen = rows_fast ? R : C;
    constexpr int64_t YMAX = (int64_t)65535 * TT;
    for (int64_t yb = 0; yb < ylen; yb += YMAX) {
        const int64_t yn = ylen - yb < YMAX ? ylen - yb : YMAX;
        const dim3 grid((unsigned)((xlen + TT - 1) / TT), (unsigned)((yn + TT - 1) / TT));
        if (rows_fast)  // columns [yb, yb + yn) of src are rows [yb, yb + yn) of dst
            hipLaunchKernelGGL(k_transpose16, grid, dim3(TT_BLOCK), 0, st, src + yb, lds_, R, yn,
                               dst + yb * ldd, ldd, 1);
        else  // rows [yb, yb + yn) of src are columns of dst
            hipLaunchKernelGGL(k_transpose16, grid, dim3(TT_BLOCK), 0, st, src + yb * lds_, lds_,
                               yn, C, dst + yb, ldd, 0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_scale(int dtype, void *p, int64_t n, const float *g, hipStream_t st) {
    if (n == 0) return hipSuccess;
    const int64_t blocks64 = (n / 8 + SCALE_BLOCK - 1) / SCALE_BLOCK;
    const unsigned blocks = (unsigned)(blocks64 < 8192 ? (blocks64 > 0 ? blocks64 : 1) : 8192);
    if (dtype == 0)
        hipLaunchKernelGGL(k_scale<F32>, dim3(blocks), dim3(SCALE_BLOCK), 0, st,
                           static_cast<float *>(p), n, g);
    else if (dtype == 1)
        hipLaunchKernelGGL(k_scale<F16>, dim3(blocks), dim3(SCALE_BLOCK), 0, st,
                           static_cast<typename F16::T *>(p), n, g);
    else
        hipLaunchKernelGGL(k_scale<BF16>, dim3(blocks), dim3(SCALE_BLOCK), 0, st,
                           static_cast<typename BF16::T *>(p), n, g);
    return hipGetLastError();
}

}  // namespace vjsd
