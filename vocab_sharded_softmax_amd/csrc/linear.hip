// linear.hip -- the element-wise helper of the fused-linear loss: scaling gradients
// computed for a unit upstream gradient by the actual one (a device scalar), so the
// caller's backward needs no host synchronisation.
#include "kernels.hpp"

namespace vjsd {
namespace {

constexpr int SCALE_BLOCK = 256;

template <class D>
__global__ __launch_bounds__(SCALE_BLOCK) void k_scale(typename D::T *p, int64_t n,
                                                       const float *__restrict__ g) {
    const float s = g[0];
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

}  // namespace

hipError_t launch_scale(int dtype, void *p, int64_t n, const float *g, hipStream_t st) {
    if (n == 0) return hipSuccess;
    const int64_t blocks64 = (n / 8 + SCALE_BLOCK - 1) / SCALE_BLOCK;
    const unsigned blocks = (unsigned)(blocks64 < 8192 ? (blocks64 > 0 ? blocks64 : 1) : 8192);
    if (dtype == 0)
        hipLaunchKernelGGL(k_scale<F32>, dim3(blocks), dim3(SCALE_BLOCK), 0, st,
                           static_cast<float *>(p), n, g);
    else
        hipLaunchKernelGGL(k_scale<BF16>, dim3(blocks), dim3(SCALE_BLOCK), 0, st,
                           static_cast<typename BF16::T *>(p), n, g);
    return hipGetLastError();
}

}  // namespace vjsd
