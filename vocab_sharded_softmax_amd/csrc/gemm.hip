// gemm.hip -- the matrix-core GEMM of the fused-linear loss:
//     C[i][j] (+)= sum_k A(i, k) * B(j, k)
// with bf16 products (an fp32 operand is rounded to bf16, nearest-even, as it is
// staged) accumulated in fp32 by v_mfma_f32_32x32x16_bf16.
//
// [JSD-PR] DeepSpeed PR #8958 "[VocabTP] Add vocabulary-parallel generalized JSD with
// Triton kernels", sections Motivation and Scope and limitations: a fused-linear
// divergence evaluates the loss from tiled LM-head projections instead of stored
// logits.  The three products it needs are the logits (hidden x head^T), the hidden
// gradient (G x head) and the head gradient (G^T x hidden).
//
// Operands: A(i, k) at a[i*lda + k] ("k-major") or a[k*lda + i] ("i-major"), bf16 or
// fp32; B(j, k) at b[j*ldb + k] or b[k*ldb + j], bf16.  Every operand pointer is 16-byte
// aligned and every leading dimension a multiple of 8 elements (4 for fp32), checked
// by the host.
//
// Tiling: a 128 x 128 output tile per workgroup of four waves (2 x 2, 64 x 64 each,
// 2 x 2 MFMA tiles of 32 x 32), k in steps of 64 through double-buffered LDS.  A
// k-major operand is stored k-major in LDS (rows padded to 144 bytes, so the 16-byte
// fragment reads of eight consecutive rows hit disjoint banks); an i/j-major operand
// is stored as loaded (rows of 128 elements padded to 264 bytes) and its fragments
// are gathered element by element.  The workgroup -> tile map gives each of the eight
// XCDs a contiguous range of tiles in i-fastest order, so the tiles that share a
// panel of B run on one XCD, close in time, out of its L2.
#include "kernels.hpp"

namespace vjsd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

constexpr int TM = 128, TN = 128, TK = 64;
constexpr int GTHREADS = 256;
constexpr int LDK = TK + 8;    // k-major LDS row: 72 bf16 = 144 bytes
constexpr int LDI = 128 + 4;   // i/j-major LDS row: 132 bf16 = 264 bytes
constexpr int KM_ELEMS = TM * LDK;  // 9216
constexpr int IM_ELEMS = TK * LDI;  // 8448
constexpr int OP_ELEMS = KM_ELEMS > IM_ELEMS ? KM_ELEMS : IM_ELEMS;

// bf16 bits of an fp32 value, round to nearest even (NaN kept quiet)
__device__ __forceinline__ unsigned short bf16_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (unsigned short)((u >> 16) | 0x40u);
    return (unsigned short)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// One operand's tile: ROWS = 128 rows (i or j) by TK = 64 k, loaded into registers,
// then stored to LDS in bf16.  F32: fp32 storage; KMAJ: k contiguous in memory.
template <bool F32, bool KMAJ>
struct Tile {
    // elements per 16-byte chunk, chunks per thread
    static constexpr int EPC = F32 ? 4 : 8;
    static constexpr int NCH = TM * TK / EPC / GTHREADS;
    u32x4 r[NCH];
    bool full[NCH];

    // chunk q of the tile: (row, k) of its first element (k-major) or (k, row)
    __device__ __forceinline__ static void coords(int q, int &row, int &k) {
        if (KMAJ) {
            constexpr int CPR = TK / EPC;  // chunks per row
            row = q / CPR;
            k = (q % CPR) * EPC;
        } else {
            constexpr int CPR = TM / EPC;
            k = q / CPR;
            row = (q % CPR) * EPC;
        }
    }

    // rows [r0, r0 + 128) (of R) and k [k0, k0 + 64) (of K); zeros outside
    __device__ __forceinline__ void load(const void *p, int64_t ld, int64_t r0, int64_t R,
                                         int64_t k0, int64_t K) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            int row, k;
            coords(threadIdx.x + c * GTHREADS, row, k);
            const int64_t gr = r0 + row, gk = k0 + k;
            // a chunk runs along k (k-major) or along the rows (i/j-major)
            const int64_t lim = KMAJ ? K - gk : R - gr;
            const bool inb = KMAJ ? gr < R : gk < K;
            const int64_t off = KMAJ ? gr * ld + gk : gk * ld + gr;
            full[c] = inb && lim >= EPC;
            if (full[c]) {
                r[c] = F32 ? ld16<false>(static_cast<const float *>(p) + off)
                           : ld16<false>(static_cast<const unsigned short *>(p) + off);
            } else {
                uint32_t w[4] = {0, 0, 0, 0};
                if (inb && lim > 0) {
                    for (int e = 0; e < EPC && e < lim; ++e) {
                        if (F32) {
                            w[e] = __float_as_uint(static_cast<const float *>(p)[off + e]);
                        } else {
                            const uint32_t h = static_cast<const unsigned short *>(p)[off + e];
                            w[e >> 1] |= h << (16 * (e & 1));
                        }
                    }
                }
                r[c] = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
    }

    // bf16 into the LDS tile s (k-major rows of LDK, or k rows of LDI)
    __device__ __forceinline__ void store(unsigned short *s) const {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            int row, k;
            coords(threadIdx.x + c * GTHREADS, row, k);
            unsigned short *d = KMAJ ? s + row * LDK + k : s + k * LDI + row;
            if (F32) {
                u16x4 h;
                h[0] = bf16_bits(__uint_as_float(r[c][0]));
                h[1] = bf16_bits(__uint_as_float(r[c][1]));
                h[2] = bf16_bits(__uint_as_float(r[c][2]));
                h[3] = bf16_bits(__uint_as_float(r[c][3]));
                *reinterpret_cast<u16x4 *>(d) = h;  // 8-byte aligned in both layouts
            } else if (KMAJ) {
                *reinterpret_cast<u32x4 *>(d) = r[c];  // 16-byte aligned
            } else {
                // i/j-major rows are 264 bytes: 8-byte aligned only
                typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                reinterpret_cast<u32x2 *>(d)[0] = u32x2{r[c][0], r[c][1]};
                reinterpret_cast<u32x2 *>(d)[1] = u32x2{r[c][2], r[c][3]};
            }
        }
    }
};

// MFMA operand of rows [base, base + 32), k [kk, kk + 16): lane l holds row
// base + l % 32, k = kk + 8 * (l / 32) + e, e = 0..7.
template <bool KMAJ>
__device__ __forceinline__ bf16x8 frag(const unsigned short *s, int base, int kk) {
    const int l = threadIdx.x & 63;
    const int row = base + (l & 31), k = kk + 8 * (l >> 5);
    if (KMAJ) {
        const u16x8 v = *reinterpret_cast<const u16x8 *>(s + row * LDK + k);
        return __builtin_bit_cast(bf16x8, v);
    } else {
        u16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = s[(k + e) * LDI + row];
        return __builtin_bit_cast(bf16x8, v);
    }
}

template <bool AF32, bool AKM, bool BKM, int OUT>
__global__ __launch_bounds__(GTHREADS) void k_gemm(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) unsigned short lds[2][2][OP_ELEMS];
    // tile of this workgroup: XCD x = blockIdx % 8 owns tiles [x * per, (x + 1) * per)
    const int64_t mt = (g.M + TM - 1) / TM, nt = (g.N + TN - 1) / TN, T = mt * nt;
    const int64_t per = (T + 7) / 8;
    const int64_t t = (int64_t)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (t >= T) return;
    const int64_t m0 = (t % mt) * TM, n0 = (t / mt) * TN;

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    Tile<AF32, AKM> ta;
    Tile<false, BKM> tb;
    const int64_t nk = (g.K + TK - 1) / TK;
    if (nk > 0) {
        ta.load(g.a, g.lda, m0, g.M, 0, g.K);
        tb.load(g.b, g.ldb, n0, g.N, 0, g.K);
        ta.store(lds[0][0]);
        tb.store(lds[0][1]);
    }
    __syncthreads();
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {  // next stage in flight during this stage's products
            ta.load(g.a, g.lda, m0, g.M, (kt + 1) * TK, g.K);
            tb.load(g.b, g.ldb, n0, g.N, (kt + 1) * TK, g.K);
        }
        const unsigned short *sa = lds[cur][0], *sb = lds[cur][1];
#pragma unroll
        for (int kk = 0; kk < TK; kk += 16) {
            bf16x8 fa[2], fb[2];
#pragma unroll
            for (int a = 0; a < 2; ++a) fa[a] = frag<AKM>(sa, wm + 32 * a, kk);
#pragma unroll
            for (int b = 0; b < 2; ++b) fb[b] = frag<BKM>(sb, wn + 32 * b, kk);
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], acc[a][b],
                                                                         0, 0, 0);
        }
        if (more) {
            ta.store(lds[cur ^ 1][0]);
            tb.store(lds[cur ^ 1][1]);
        }
        __syncthreads();
    }

    // result element r of MFMA tile (a, b): row 8 (r / 4) + 4 (lane / 32) + r % 4,
    // column lane % 32
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t i = m0 + wm + 32 * a + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int64_t j = n0 + wn + 32 * b + (lane & 31);
                if (i >= g.M || j >= g.N) continue;
                const float v = acc[a][b][r];
                const int64_t o = i * g.ldc + j;
                if (OUT == GEMM_F32) {
                    static_cast<float *>(g.c)[o] = v;
                } else if (OUT == GEMM_F32_ACC) {
                    static_cast<float *>(g.c)[o] += v;
                } else if (OUT == GEMM_BF16) {
                    static_cast<unsigned short *>(g.c)[o] = bf16_bits(v);
                } else {  // GEMM_BF16_ACC: bf16(addend + v)
                    static_cast<unsigned short *>(g.c)[o] = bf16_bits(g.addend[i * g.ldadd + j] + v);
                }
            }
}

template <bool AF32, bool AKM, bool BKM>
hipError_t gemm_out(const GemmArgs &g, hipStream_t st) {
    const int64_t T = ((g.M + TM - 1) / TM) * ((g.N + TN - 1) / TN);
    const dim3 grid((unsigned)(8 * ((T + 7) / 8)));
    switch (g.out) {
        case GEMM_F32:
            hipLaunchKernelGGL((k_gemm<AF32, AKM, BKM, GEMM_F32>), grid, dim3(GTHREADS), 0, st, g);
            break;
        case GEMM_F32_ACC:
            hipLaunchKernelGGL((k_gemm<AF32, AKM, BKM, GEMM_F32_ACC>), grid, dim3(GTHREADS), 0, st,
                               g);
            break;
        case GEMM_BF16:
            hipLaunchKernelGGL((k_gemm<AF32, AKM, BKM, GEMM_BF16>), grid, dim3(GTHREADS), 0, st, g);
            break;
        default:
            hipLaunchKernelGGL((k_gemm<AF32, AKM, BKM, GEMM_BF16_ACC>), grid, dim3(GTHREADS), 0,
                               st, g);
            break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs &g, hipStream_t st) {
    if (g.M == 0 || g.N == 0) return hipSuccess;
    if (g.a_f32) {
        if (g.a_kmajor) return g.b_kmajor ? gemm_out<true, true, true>(g, st)
                                          : gemm_out<true, true, false>(g, st);
        return g.b_kmajor ? gemm_out<true, false, true>(g, st) : gemm_out<true, false, false>(g, st);
    }
    if (g.a_kmajor) return g.b_kmajor ? gemm_out<false, true, true>(g, st)
                                      : gemm_out<false, true, false>(g, st);
    return g.b_kmajor ? gemm_out<false, false, true>(g, st) : gemm_out<false, false, false>(g, st);
}

}  // namespace vjsd
