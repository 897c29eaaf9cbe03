// stats.hip -- input pass 1: per-shard paired softmax statistics, and their merge.
//
// [JSD-PR] DeepSpeed PR #8958 "[VocabTP] Add vocabulary-parallel generalized JSD with
// Triton kernels", section Changes: paired softmax statistics of student and teacher
// computed together.  [OPS-PR] DeepSpeed PR #8791 "Add vocabulary-parallel logprobs,
// entropy and KL ops", section How: the row max and the sum-exp are reduced across
// shards by a MAX then a SUM, and kept apart; review thread: an empty shard joins as
// (-inf, 0).  Here the shards are logical and the merge is one thread per row.
#include "kernels.hpp"
#include "sweep.hpp"

namespace vjsd {

namespace {

// One workgroup per row of the shard.  part_k[r*8 + 0..3] = (m_s, z_s, m_t, z_t) with
// z relative to refc(m, ks); an empty shard or a dropped row writes (-inf, 0).
template <class D, int WHICH>
__global__ __launch_bounds__(BLOCK) void k_stats(RowView sv, RowView tv, int64_t w,
                                                 float *__restrict__ part_k, RowOpts o) {
    using T = typename D::T;
    __shared__ float red[4 * NWAVE];
    const int64_t r = blockIdx.x;
    MZ ms{NINF, 0.0f}, mt{NINF, 0.0f};
    if (w > 0 && !row_dropped(o, r)) {
        if (WHICH == 3) {
            const T *s = row_ptr<T>(sv, r), *t = row_ptr<T>(tv, r);
            OpStats<3> op(o.ks);
            sweep<D, 4, true, BLOCK, true>(s, t, w, head_len<T>(w, s, t), op);
            ms = {op.a.m, op.a.z};
            mt = {op.b.m, op.b.z};
        } else {
            const T *x = row_ptr<T>(WHICH == 1 ? sv : tv, r);
            OpStats<1> op(o.ks);
            sweep<D, 4, false, BLOCK, true>(x, x, w, head_len<T>(w, x), op);
            (WHICH == 1 ? ms : mt) = {op.a.m, op.a.z};
        }
        if (WHICH & 1) ms = block_mz(ms, red, o.ks);
        if (WHICH & 2) mt = block_mz(mt, red, o.ks);
    }
    if (threadIdx.x == 0) {
        float *o = part_k + r * PART_STRIDE;
        if (WHICH & 1) { o[0] = ms.m; o[1] = ms.z; }
        if (WHICH & 2) { o[2] = mt.m; o[3] = mt.z; }
    }
}

__global__ void k_merge(const float *__restrict__ part, int S, int64_t N, int which,
                        double *__restrict__ stats, float ks) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= N) return;
    for (int side = 0; side < 2; ++side) {
        if (!(which & (1 << side))) continue;
        float m = NINF;
        for (int k = 0; k < S; ++k) m = fmaxf(m, part[((int64_t)k * N + r) * PART_STRIDE + 2 * side]);
        double Z = 0.0;
        const double c = refc(m, ks);
        for (int k = 0; k < S; ++k) {
            const float *p = part + ((int64_t)k * N + r) * PART_STRIDE + 2 * side;
            if (p[0] != NINF) Z += (double)p[1] * exp2((double)refc(p[0], ks) - c);
        }
        stats[r * 4 + 2 * side] = m;
        stats[r * 4 + 2 * side + 1] = m == NINF ? -__builtin_inf() : lnz_from_z(m, Z, ks);
    }
}

template <class D>
hipError_t stats_dt(int which, const Shard &sh, int64_t N, float *part_k, const RowOpts &o,
                    hipStream_t st) {
    const dim3 grid((unsigned)N), block(BLOCK);
    if (which == 3)
        hipLaunchKernelGGL((k_stats<D, 3>), grid, block, 0, st, sh.s, sh.t, sh.width, part_k, o);
    else if (which == 1)
        hipLaunchKernelGGL((k_stats<D, 1>), grid, block, 0, st, sh.s, sh.t, sh.width, part_k, o);
    else
        hipLaunchKernelGGL((k_stats<D, 2>), grid, block, 0, st, sh.s, sh.t, sh.width, part_k, o);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_stats(int dtype, int which, const Shard &sh, int64_t N, float *part_k,
                        hipStream_t st, const RowOpts &o) {
    switch (dtype) {
        case 0: return stats_dt<F32>(which, sh, N, part_k, o, st);
        case 1: return stats_dt<F16>(which, sh, N, part_k, o, st);
        default: return stats_dt<BF16>(which, sh, N, part_k, o, st);
    }
}

hipError_t launch_merge(const float *part, int S, int64_t N, int which, double *stats,
                        hipStream_t st, float ks) {
    const int threads = 256;
    const dim3 grid((unsigned)((N + threads - 1) / threads));
    hipLaunchKernelGGL(k_merge, grid, dim3(threads), 0, st, part, S, N, which, stats, ks);
    return hipGetLastError();
}

}  // namespace vjsd
