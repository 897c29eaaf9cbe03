// reduce.hip -- the masked token reduction of the distillation loss.
//
// [JSD-PR] DeepSpeed PR #8958 "[VocabTP] Add vocabulary-parallel generalized JSD with
// Triton kernels", section Changes: the per-token ops leave masking and normalisation
// to the caller; DeepSpeedExamples PR #1019 "vocab-parallel KL route for OPSD" keeps
// a token mean over the response tokens.  The sum and the kept-row count are taken
// in fp64 by one workgroup in a fixed order, so the result does not depend on
// timing; an undefined kept row (NaN) reaches the result, a dropped one never does.
#include "kernels.hpp"

namespace vjsd {

namespace {

constexpr int RED_BLOCK = 1024;

__device__ __forceinline__ double wave_sum_d(double v) {
    return wave_reduce<false>(v, [](double a, double b) { return a + b; });
}

// out[0] = sum over kept rows (mean: / kept rows, 0 when none); *count = kept rows.
// A row is kept unless the selector drops it (token mask, or ignored label).
// rows may be null (count only); out and count may each be null.
__global__ __launch_bounds__(RED_BLOCK) void k_reduce_rows(const float *__restrict__ rows,
                                                           RowOpts sel, int64_t N, int mean,
                                                           float *__restrict__ out,
                                                           double *__restrict__ count) {
    constexpr int NW = RED_BLOCK / 64;
    __shared__ double red[2 * NW];
    double sum = 0.0, cnt = 0.0;
    for (int64_t r = threadIdx.x; r < N; r += RED_BLOCK) {
        if (!row_dropped(sel, r)) {
            cnt += 1.0;
            if (rows) sum += (double)rows[r];
        }
    }
    sum = wave_sum_d(sum);
    cnt = wave_sum_d(cnt);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        red[wave] = sum;
        red[NW + wave] = cnt;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double s = 0.0, c = 0.0;
        for (int k = 0; k < NW; ++k) {
            s += red[k];
            c += red[NW + k];
        }
        if (out) out[0] = (float)(mean ? (c > 0.0 ? s / c : 0.0) : s);
        if (count) *count = c;
    }
}

}  // namespace

hipError_t launch_reduce_rows(const float *rows, const RowOpts &sel, int64_t N, bool mean,
                              float *out, double *count, hipStream_t st) {
    hipLaunchKernelGGL(k_reduce_rows, dim3(1), dim3(RED_BLOCK), 0, st, rows, sel, N,
                       mean ? 1 : 0, out, count);
    return hipGetLastError();
}

}  // namespace vjsd
