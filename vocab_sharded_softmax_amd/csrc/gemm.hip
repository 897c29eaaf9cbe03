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
// aligned, every leading dimension a multiple of 8 elements (4 for fp32), and every
// operand readable over whole rows of ld elements (checked by the host).
//
// Tiling: a 256 x 256 output tile per workgroup, k in steps of 64 through
// double-buffered LDS (one workgroup per CU).  The general kernel (k_gemm) runs four
// waves (2 x 2, 128 x 128 each, 4 x 4 MFMA tiles of 32 x 32, 256 fp32 accumulators per
// lane in AGPRs; 144 KiB of LDS); the direct-to-LDS kernel (k_gemm_dl, below), which
// every product of the loss runs on, eight (4 x 2, 64 x 128 each).  When an operand
// has its rows contiguous (and both are bf16) the global loads run two k-steps ahead
// (two register stages), so a load has two steps of products to arrive in.  Every operand is
// stored k-major in LDS, rows padded to 144 bytes, so each MFMA fragment is one
// 16-byte read and the reads of eight consecutive rows hit disjoint banks.  A k-major
// operand is staged in 16-byte chunks along k; an operand whose rows are contiguous
// (k strided) is staged as 8 (k) x 8 (rows) blocks and transposed in registers into
// 16-byte k-major rows.  Tiles are ordered so that
// consecutive ones share a panel of the larger operand (that panel is then read from
// HBM once), and the workgroup -> tile map gives each of the eight XCDs a contiguous
// range of that order, so the sharing happens inside one XCD's L2.
#include "kernels.hpp"

namespace vjsd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int GTHREADS = 256;
constexpr int LDR = BK + 8;               // LDS row: 72 bf16 = 144 bytes
constexpr int OP_ELEMS = 256 * LDR;       // one operand's stage
constexpr int WTM = 4, WTN = 4;           // MFMA tiles per wave (rows, columns)

// two fp32 values as a bf16 pair (nearest even), the first in the low half
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

__device__ __forceinline__ unsigned short bf16_bits(float f) {
    return (unsigned short)(pack_bf16(f, 0.0f) & 0xffffu);
}

// One operand's 256 (rows) x 64 (k) tile, loaded into registers, then written to LDS
// in bf16, k-major.  Primary template: k contiguous in memory.
template <bool F32, bool KMAJ>
struct Stage {
    static constexpr int EPC = F32 ? 4 : 8;      // elements per 16-byte chunk
    static constexpr int CPR = BK / EPC;         // chunks per row
    static constexpr int NCH = 256 * CPR / GTHREADS;
    u32x4 r[NCH];

    // CHECKED false: the whole 256 x 64 tile is inside the operand.  Chunk c of a
    // thread sits 256 / CPR rows below chunk c - 1: a wave-uniform base plus one
    // per-lane offset.  CHECKED true: a row past the operand reads row R - 1 and a
    // chunk at or past K reads the last chunk of its row (a chunk starts at a multiple
    // of EPC < ld, so it never leaves its row's ld elements); elements outside the
    // operand are then zeroed.
    template <bool CHECKED>
    __device__ __forceinline__ void load(const void *p, int64_t ld, int64_t r0, int64_t R,
                                         int64_t k0, int64_t K) {
        constexpr int ES = F32 ? 4 : 2;
        const int64_t lr = threadIdx.x / CPR, lk = (threadIdx.x % CPR) * EPC;
        if (!CHECKED) {
            const uint32_t lane_off = (uint32_t)((lr * ld + lk) * ES);
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const char *base = static_cast<const char *>(p) +
                                   ((r0 + (int64_t)c * (GTHREADS / CPR)) * ld + k0) * ES;
                r[c] = ld16<false>(base + lane_off);
            }
            return;
        }
        const int64_t klast = (K - 1) / EPC * EPC;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int64_t gr = r0 + lr + (int64_t)c * (GTHREADS / CPR), gk = k0 + lk;
            const int64_t ar = gr < R ? gr : R - 1, ak = gk < klast ? gk : klast;
            u32x4 v = ld16<false>(static_cast<const char *>(p) + (ar * ld + ak) * ES);
            const bool rok = gr < R;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (F32) {
                    if (!(rok && gk + i < K)) v[i] = 0u;
                } else {
                    const uint32_t m = ((rok && gk + 2 * i < K) ? 0x0000ffffu : 0u) |
                                       ((rok && gk + 2 * i + 1 < K) ? 0xffff0000u : 0u);
                    v[i] &= m;
                }
            }
            r[c] = v;
        }
    }

    __device__ __forceinline__ void store(unsigned short *s) const {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int q = threadIdx.x + c * GTHREADS;
            unsigned short *d = s + (q / CPR) * LDR + (q % CPR) * EPC;
            if (F32) {
                typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                *reinterpret_cast<u32x2 *>(d) =
                    u32x2{pack_bf16(__uint_as_float(r[c][0]), __uint_as_float(r[c][1])),
                          pack_bf16(__uint_as_float(r[c][2]), __uint_as_float(r[c][3]))};
            } else {
                *reinterpret_cast<u32x4 *>(d) = r[c];
            }
        }
    }
};

// Rows contiguous in memory, k strided: thread t owns the block k in
// [8 (t % 8), + 8) x rows [8 (t / 8), + 8) of the tile.
template <bool F32>
struct Stage<F32, false> {
    static constexpr int EPC = F32 ? 4 : 8;
    static constexpr int W = 8 / EPC;  // 16-byte loads per k-row of the block
    static_assert((BK / 8) * (256 / 8) == GTHREADS, "one block per thread");
    u32x4 r[8][W];

    // CHECKED as for the k-major stage, with the roles of rows and k swapped: a k-row
    // at or past K reads k-row K - 1, a chunk at or past R the last chunk of its k-row.
    template <bool CHECKED>
    __device__ __forceinline__ void load(const void *p, int64_t ld, int64_t r0, int64_t R,
                                         int64_t k0, int64_t K) {
        const int kb = threadIdx.x & 7, rb = threadIdx.x >> 3;
        constexpr int ES = F32 ? 4 : 2;
        if (!CHECKED) {  // wave-uniform base per load plus one per-lane offset
            const uint32_t lane_off = (uint32_t)((8 * kb * ld + 8 * rb) * ES);
#pragma unroll
            for (int kr = 0; kr < 8; ++kr)
#pragma unroll
                for (int w = 0; w < W; ++w) {
                    const char *base = static_cast<const char *>(p) +
                                       ((k0 + kr) * ld + r0 + w * EPC) * ES;
                    r[kr][w] = ld16<false>(base + lane_off);
                }
            return;
        }
        const int64_t rlast = (R - 1) / EPC * EPC;
#pragma unroll
        for (int kr = 0; kr < 8; ++kr) {
            const int64_t gk = k0 + 8 * kb + kr;
            const int64_t ak = gk < K ? gk : K - 1;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const int64_t gr = r0 + 8 * rb + w * EPC;
                const int64_t ar = gr < rlast ? gr : rlast;
                u32x4 v = ld16<false>(static_cast<const char *>(p) + (ak * ld + ar) * ES);
                const bool kok = gk < K;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (F32) {
                        if (!(kok && gr + i < R)) v[i] = 0u;
                    } else {
                        const uint32_t m = ((kok && gr + 2 * i < R) ? 0x0000ffffu : 0u) |
                                           ((kok && gr + 2 * i + 1 < R) ? 0xffff0000u : 0u);
                        v[i] &= m;
                    }
                }
                r[kr][w] = v;
            }
        }
    }

    // element (k = kr, row = j) of the block as fp32 / bf16 bits
    __device__ __forceinline__ float f32_at(int kr, int j) const {
        const uint32_t u = r[kr][j / 4][j % 4];
        return __uint_as_float(u);
    }
    __device__ __forceinline__ uint32_t half_at(int kr, int j) const {
        const uint32_t u = r[kr][0][j / 2];
        return (j & 1) ? (u >> 16) : (u & 0xffffu);
    }

    __device__ __forceinline__ void store(unsigned short *s) const {
        const int kb = threadIdx.x & 7, rb = threadIdx.x >> 3;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (F32) o[q] = pack_bf16(f32_at(2 * q, j), f32_at(2 * q + 1, j));
                else o[q] = half_at(2 * q, j) | (half_at(2 * q + 1, j) << 16);
            }
            *reinterpret_cast<u32x4 *>(s + (8 * rb + j) * LDR + 8 * kb) =
                u32x4{o[0], o[1], o[2], o[3]};
        }
    }
};

// MFMA operand of rows [base, base + 32), k [kk, kk + 16): lane l holds row
// base + l % 32, k = kk + 8 * (l / 32) + e, e = 0..7.
__device__ __forceinline__ bf16x8 frag(const unsigned short *s, int base, int kk) {
    const int l = threadIdx.x & 63;
    const u32x4 v = *reinterpret_cast<const u32x4 *>(s + (base + (l & 31)) * LDR + kk + 8 * (l >> 5));
    return __builtin_bit_cast(bf16x8, v);
}

// Tile (m0, n0) at position t of the order.  The larger operand's panels are taken
// GL at a time (the outer group), and within that group the other operand's panels GS
// at a time, so the 32 tiles an XCD runs at once form a GS x GL block: each of its
// panels is fetched once for the block, and each of the larger operand's panels once
// from HBM for all of the other operand.
__device__ __forceinline__ void tile_of(int64_t t, int64_t mt, int64_t nt, int a_larger,
                                        int64_t &m0, int64_t &n0) {
    constexpr int64_t GL = 8, GS = 4;
    const int64_t nl = a_larger ? mt : nt, ns = a_larger ? nt : mt;  // larger / smaller
    const int64_t gi = t / (ns * GL), lb = gi * GL;
    const int64_t gl = nl - lb < GL ? nl - lb : GL;
    const int64_t u = t - gi * ns * GL;
    const int64_t si = u / (GS * gl), sb = si * GS;
    const int64_t gs = ns - sb < GS ? ns - sb : GS;
    const int64_t v = u - si * GS * gl;
    const int64_t is = sb + v % gs, il = lb + v / gs;
    m0 = (a_larger ? il : is) * BM;
    n0 = (a_larger ? is : il) * BN;
}

// The accumulators to C: result element r of MFMA tile (a, b) is row
// 8 (r / 4) + 4 (lane / 32) + r % 4, column lane % 32; one row pointer per output row.
// The accumulating outputs read the addends of one row block of MFMA tiles (64 per lane)
// together, then store that block: an add per element made each load wait behind the
// store before it (an fp32 accumulate of a 151936 x 3584 head gradient over 2048 tokens
// took 5.8 ms against 2.6 ms stored), and all 256 at once would not fit the registers.
template <int OUT, int TM = WTM, int TN = WTN>
__device__ __forceinline__ void store_tile(const GemmArgs &g, const f32x16 (&acc)[TM][TN],
                                           int64_t m0, int64_t n0, int wm, int wn, int lane) {
    const bool rows_in = m0 + BM <= g.M && n0 + BN <= g.N;
    const int64_t jl = n0 + wn + (lane & 31);
    constexpr bool ACC = OUT == GEMM_F32_ACC || OUT == GEMM_BF16_ACC;
    const float *src = OUT == GEMM_F32_ACC ? static_cast<const float *>(g.c) : g.addend;
    const int64_t lds_ = OUT == GEMM_F32_ACC ? g.ldc : g.ldadd;
#pragma unroll
    for (int a = 0; a < TM; ++a) {
        float add[TN][16];
        if constexpr (ACC) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t i = m0 + wm + 32 * a + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
#pragma unroll
                for (int b = 0; b < TN; ++b) {
                    const int64_t j = jl + 32 * b;
                    add[b][r] = (rows_in || (i < g.M && j < g.N)) ? src[i * lds_ + j] : 0.0f;
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t i = m0 + wm + 32 * a + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (!rows_in && i >= g.M) continue;
            const int64_t row = i * g.ldc;
#pragma unroll
            for (int b = 0; b < TN; ++b) {
                const int64_t j = jl + 32 * b;
                if (!rows_in && j >= g.N) continue;
                const float v = acc[a][b][r];
                const int64_t o = row + j;
                // results are written with the streaming policy: they are read much
                // later, and through the L2 they would evict the operand panels the
                // tiles running beside this one still share
                if (OUT == GEMM_F32)
                    __builtin_nontemporal_store(v, static_cast<float *>(g.c) + o);
                else if (OUT == GEMM_F32_ACC)
                    __builtin_nontemporal_store(add[b][r] + v, static_cast<float *>(g.c) + o);
                else if (OUT == GEMM_BF16)
                    __builtin_nontemporal_store(bf16_bits(v), static_cast<unsigned short *>(g.c) + o);
                else  // GEMM_BF16_ACC: bf16(addend + v)
                    __builtin_nontemporal_store(bf16_bits(add[b][r] + v),
                                                static_cast<unsigned short *>(g.c) + o);
            }
        }
        // the next block's loads stay behind this block's stores
        if constexpr (ACC) asm volatile("" ::: "memory");
    }
}

template <bool AF32, bool AKM, bool BKM, int OUT>
__global__ __launch_bounds__(GTHREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) unsigned short lds[2][2][OP_ELEMS];
    // tile of this workgroup: XCD x = blockIdx % 8 owns tiles [x * per, (x + 1) * per)
    // of an order in which consecutive tiles share a panel of the larger operand
    const int64_t mt = (g.M + BM - 1) / BM, nt = (g.N + BN - 1) / BN, T = mt * nt;
    const int64_t per = (T + 7) / 8;
    const int64_t t = (int64_t)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (t >= T) return;
    int64_t m0, n0;
    tile_of(t, mt, nt, g.n_fastest, m0, n0);

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = (wave >> 1) * (32 * WTM), wn = (wave & 1) * (32 * WTN);
    f32x16 acc[WTM][WTN];
#pragma unroll
    for (int a = 0; a < WTM; ++a)
#pragma unroll
        for (int b = 0; b < WTN; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    const int64_t nk = (g.K + BK - 1) / BK;
    const bool rows_in = m0 + BM <= g.M && n0 + BN <= g.N;
    // a stage with every element inside both operands is loaded without tests
    auto load_stage = [&](auto &sa, auto &sb, int64_t k0) {
        if (rows_in && k0 + BK <= g.K) {
            sa.template load<false>(g.a, g.lda, m0, g.M, k0, g.K);
            sb.template load<false>(g.b, g.ldb, n0, g.N, k0, g.K);
        } else {
            sa.template load<true>(g.a, g.lda, m0, g.M, k0, g.K);
            sb.template load<true>(g.b, g.ldb, n0, g.N, k0, g.K);
        }
    };
    bf16x8 fa[2][WTM], fb[2][WTN];
    auto read_frags = [&](int buf, const unsigned short *la, const unsigned short *lb, int kk) {
#pragma unroll
        for (int a = 0; a < WTM; ++a) fa[buf][a] = frag(la, wm + 32 * a, kk);
#pragma unroll
        for (int b = 0; b < WTN; ++b) fb[buf][b] = frag(lb, wn + 32 * b, kk);
    };
    // the products of one LDS stage; sub-step 0's fragments are already in fa/fb[0]
    auto products = [&](const unsigned short *la, const unsigned short *lb) {
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            // the next sub-step's fragments are read while this one's products run
            if (s + 1 < BK / 16) read_frags((s + 1) & 1, la, lb, 16 * (s + 1));
#pragma unroll
            for (int a = 0; a < WTM; ++a)
#pragma unroll
                for (int b = 0; b < WTN; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s & 1][a], fb[s & 1][b],
                                                                         acc[a][b], 0, 0, 0);
        }
    };
    // one register stage when an operand is fp32 or both are k-major (their staging
    // registers leave no room for a second); two otherwise
    if constexpr (AF32 || (AKM && BKM)) {
        Stage<AF32, AKM> sa;
        Stage<false, BKM> sb;
        if (nk > 0) {
            load_stage(sa, sb, 0);
            sa.store(lds[0][0]);
            sb.store(lds[0][1]);
        }
        __syncthreads();
        if (nk > 0) read_frags(0, lds[0][0], lds[0][1], 0);
        for (int64_t kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            const bool more = kt + 1 < nk;
            if (more) load_stage(sa, sb, (kt + 1) * BK);  // in flight during the products
            products(lds[cur][0], lds[cur][1]);
            if (more) {
                sa.store(lds[cur ^ 1][0]);
                sb.store(lds[cur ^ 1][1]);
            }
            __syncthreads();
            if (more) read_frags(0, lds[cur ^ 1][0], lds[cur ^ 1][1], 0);
        }
    } else {  // two register stages: stage s is loaded two steps before its products
        Stage<false, AKM> sa0, sa1;
        Stage<false, BKM> sb0, sb1;
        if (nk > 0) load_stage(sa0, sb0, 0);
        if (nk > 1) load_stage(sa1, sb1, BK);
        if (nk > 0) {
            sa0.store(lds[0][0]);
            sb0.store(lds[0][1]);
        }
        __syncthreads();
        if (nk > 0) read_frags(0, lds[0][0], lds[0][1], 0);
        // step kt: its data is in lds[P]; register set P (free since its store) takes
        // stage kt + 2; set 1 - P (stage kt + 1) goes to lds[1 - P]
        auto step = [&](auto &sa_p, auto &sb_p, auto &sa_q, auto &sb_q, int P, int64_t kt) {
            if (kt + 2 < nk) load_stage(sa_p, sb_p, (kt + 2) * BK);
            products(lds[P][0], lds[P][1]);
            if (kt + 1 < nk) {
                sa_q.store(lds[P ^ 1][0]);
                sb_q.store(lds[P ^ 1][1]);
            }
            __syncthreads();
            if (kt + 1 < nk) read_frags(0, lds[P ^ 1][0], lds[P ^ 1][1], 0);
        };
        int64_t kt = 0;
        for (; kt + 1 < nk; kt += 2) {
            step(sa0, sb0, sa1, sb1, 0, kt);
            step(sa1, sb1, sa0, sb0, 1, kt + 1);
        }
        if (kt < nk) step(sa0, sb0, sa1, sb1, 0, kt);
    }

    store_tile<OUT>(g, acc, m0, n0, wm, wn, lane);
}

// ---- both operands bf16 and k-major, K a multiple of 64: global loads straight into LDS
//
// gfx950's global_load_lds_dwordx4 writes each lane's 16 bytes at consecutive LDS
// addresses (no staging registers).  A stage is k = 64, so each LDS row is one full
// 128-byte line of its operand row: the eight lanes of a row load the whole line
// (loads of half lines fetch every line twice from L2, and that bound the earlier
// stage of k = 32).  Two stages of 64 KiB: the loads of stage kt + 1 run during stage
// kt's products.  The chunk c of row r sits at slot c ^ dswz(r): sixteen consecutive
// rows' 16-byte reads of one chunk fall on distinct banks whether the LDS serves eight
// or sixteen lanes a cycle.  A row past the edge loads row M - 1 (N - 1): it feeds only
// outputs that are not stored.
constexpr int DBK = 64, DST = 2;
// eight waves of 64 x 128 each (2 x 4 MFMA tiles, 128 accumulators), two per SIMD: one
// wave's products run while the other waits on its fragment reads or loads.  Measured
// on MI355X against four waves of 128 x 128: logits of 1024 tokens (1024 x 151936 x
// 3584, fp32 out) 1.25 -> 1.10 ms, of 4096 tokens 4.75 -> 4.40 ms, the head gradient
// over 8192 tokens 8.8-9.0 -> 8.0 ms; sixteen waves of 64 x 64 ran as eight; loading
// through registers instead of straight into LDS ran as eight.
constexpr int DL_WAVES = 8, DL_TM = 2, DL_TN = 4;
constexpr int DSTAGE = 2 * 256 * DBK;  // bf16 elements of one stage (A rows, then B rows)

__device__ __forceinline__ int dswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm() {
    __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() {
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

__device__ __forceinline__ bf16x8 dfrag(const unsigned short *s, int base, int chunk) {
    const int l = threadIdx.x & 63;
    const int row = base + (l & 31), c = chunk + (l >> 5);
    const u32x4 v = *reinterpret_cast<const u32x4 *>(s + row * DBK + 8 * (c ^ dswz(row)));
    return __builtin_bit_cast(bf16x8, v);
}

template <int OUT, int NWV, int TM, int TN>
__global__ __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(NWV / 4, NWV / 4)))
void k_gemm_dl(GemmArgs g) {
    static_assert((BM / (32 * TM)) * (BN / (32 * TN)) == NWV, "waves tile the workgroup tile");
    constexpr int WGN = BN / (32 * TN);  // waves along N
    constexpr int RPW = 256 / NWV;       // operand rows each wave loads per stage
    __shared__ __attribute__((aligned(1024))) unsigned short lds[DST][DSTAGE];
    const int64_t mt = (g.M + BM - 1) / BM, nt = (g.N + BN - 1) / BN, T = mt * nt;
    // work items: ksplit per tile, split-major (each split runs the whole tile order)
    const int64_t items = T * g.ksplit;
    const int64_t per = (items + 7) / 8;
    const int64_t it = (int64_t)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (it >= items) return;
    const int64_t split = it / T, t = it - split * T;
    int64_t m0, n0;
    tile_of(t, mt, nt, g.n_fastest, m0, n0);
    // this item's stages of k = 64
    const int64_t nk_all = g.K / DBK, nk_per = (nk_all + g.ksplit - 1) / g.ksplit;
    const int64_t kb = split * nk_per;
    const int64_t nk = nk_all - kb < nk_per ? (nk_all - kb > 0 ? nk_all - kb : 0) : nk_per;

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = (wave / WGN) * (32 * TM), wn = (wave % WGN) * (32 * TN);
    f32x16 acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    // this wave loads rows [RPW wave, + RPW) of A and of B: instructions of 8 rows each;
    // lane i of an instruction covers row + i / 8, slot i % 8
    constexpr int NI = RPW / 8;  // load instructions per operand per wave and stage
    const int64_t rl = lane >> 3;
    const int cl = lane & 7;
    const uint16_t *pa = static_cast<const uint16_t *>(g.a);
    const uint16_t *pb = static_cast<const uint16_t *>(g.b);
    typedef __attribute__((address_space(3))) void lds_void;
    auto issue = [&](int64_t s) {
        unsigned short *st = lds[s % DST];
        const int64_t k0 = (kb + s) * DBK;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int r = RPW * wave + 8 * j + (int)rl;
            const int c = cl ^ dswz(r);
            const int64_t ra = m0 + r < g.M ? m0 + r : g.M - 1;
            const int64_t rb = n0 + r < g.N ? n0 + r : g.N - 1;
            const int row0 = RPW * wave + 8 * j;
            __builtin_amdgcn_global_load_lds(pa + ra * g.lda + k0 + 8 * c,
                                             (lds_void *)(st + row0 * DBK), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(pb + rb * g.ldb + k0 + 8 * c,
                                             (lds_void *)(st + 256 * DBK + row0 * DBK), 16, 0, 0);
        }
    };

    // Software pipeline over the four MFMA sub-steps F0..F3 of a stage: F(i + 1)'s
    // fragments are read while F(i)'s products run; after F2, the wait and barrier for
    // the next stage, whose loads then go into the buffer this stage leaves, and whose
    // F0 is read while F3's products run.
    bf16x8 fa[2][TM], fb[2][TN];
    auto read = [&](int buf, int64_t s, int sub) {
        const unsigned short *la = lds[s % DST], *lb = la + 256 * DBK;
#pragma unroll
        for (int a = 0; a < TM; ++a) fa[buf][a] = dfrag(la, wm + 32 * a, 2 * sub);
#pragma unroll
        for (int b = 0; b < TN; ++b) fb[buf][b] = dfrag(lb, wn + 32 * b, 2 * sub);
    };
    auto mma = [&](int buf) {
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int b = 0; b < TN; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][a], fb[buf][b],
                                                                     acc[a][b], 0, 0, 0);
    };
    if (nk > 0) {
        issue(0);
        if (nk > 1) {
            issue(1);
            wait_vm<2 * NI>();  // stage 0 landed; stage 1 may be in flight
        } else {
            wait_vm<0>();
        }
        // plain barriers: the waits cover this wave's loads, and __syncthreads()'s fence
        // would also wait for the stage still in flight
        __builtin_amdgcn_s_barrier();
        read(0, 0, 0);
    }
    // (the last stage is peeled off, so that no branch separates the next stage's
    // fragment reads from the products they overlap)
    // The scheduler otherwise moves the fragment reads next to the products that use
    // them; ordered groups keep each sub-step's products interleaved one for one with the
    // next sub-step's reads (mask 0x008: MFMA, 0x100: LDS read).  The fused-linear loss
    // at N=8192, V=151936, D=3584, A/B on one box: 40.27-40.54 -> 38.85-39.29 ms with the
    // three sub-steps before the barrier interleaved, and on another 38.06-38.19 ->
    // 37.83-37.86 ms with the one after it and the last stage's too; all six reads
    // first and then the products, or the reads first in each pair or two to a
    // product, ran 39.8-41.0 ms.
    auto interleave = [&]() {
#pragma unroll
        for (int i = 0; i < TM + TN; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - (TM + TN), 0);
    };
    for (int64_t kt = 0; kt + 1 < nk; ++kt) {
        read(1, kt, 1);
        mma(0);
        interleave();
        read(0, kt, 2);
        mma(1);
        interleave();
        read(1, kt, 3);
        mma(0);
        interleave();
        // every wave's reads of stage kt are complete before the barrier (F3 is waited
        // for here), and stage kt + 1 has landed for this wave; after the barrier the
        // next issue may overwrite stage kt's buffer
        wait_lgkm0();
        wait_vm<0>();
        __builtin_amdgcn_s_barrier();
        if (kt + 2 < nk) issue(kt + 2);
        read(0, kt + 1, 0);
        mma(1);
        interleave();
    }
    if (nk > 0) {
        read(1, nk - 1, 1);
        mma(0);
        interleave();
        read(0, nk - 1, 2);
        mma(1);
        interleave();
        read(1, nk - 1, 3);
        mma(0);
        interleave();
        mma(1);
    }
    if (g.ksplit > 1) {  // this split's partial product, fp32
        GemmArgs gp = g;
        gp.c = static_cast<float *>(g.c) + split * g.split_stride;
        store_tile<GEMM_F32, TM, TN>(gp, acc, m0, n0, wm, wn, lane);
        return;
    }
    store_tile<OUT, TM, TN>(g, acc, m0, n0, wm, wn, lane);
}

template <bool AF32, bool AKM, bool BKM>
hipError_t gemm_out(const GemmArgs &g, hipStream_t st) {
    const int64_t T = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
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

hipError_t launch_gemm(const GemmArgs &gin, hipStream_t st) {
    if (gin.M == 0 || gin.N == 0) return hipSuccess;
    // a K split needs the direct-to-LDS kernel (both operands bf16, k-major, K % 64 == 0)
    if (gin.ksplit > 1 && (gin.a_f32 || !gin.a_kmajor || !gin.b_kmajor || gin.K % DBK != 0 ||
                           gin.K == 0))
        return hipErrorInvalidValue;
    GemmArgs g = gin;
    // consecutive tiles share a panel of the operand with more bytes
    g.n_fastest = (double)g.M * (g.a_f32 ? 4 : 2) > (double)g.N * 2;
    if (!g.a_f32 && g.a_kmajor && g.b_kmajor && g.K > 0 && g.K % DBK == 0) {
        const int64_t T = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN) * g.ksplit;
        const dim3 grid((unsigned)(8 * ((T + 7) / 8)));
        const dim3 block(64 * DL_WAVES);
        switch (g.out) {
            case GEMM_F32:
                hipLaunchKernelGGL((k_gemm_dl<GEMM_F32, DL_WAVES, DL_TM, DL_TN>), grid, block, 0, st, g);
                break;
            case GEMM_F32_ACC:
                hipLaunchKernelGGL((k_gemm_dl<GEMM_F32_ACC, DL_WAVES, DL_TM, DL_TN>), grid, block, 0, st, g);
                break;
            case GEMM_BF16:
                hipLaunchKernelGGL((k_gemm_dl<GEMM_BF16, DL_WAVES, DL_TM, DL_TN>), grid, block, 0, st, g);
                break;
            default:
                hipLaunchKernelGGL((k_gemm_dl<GEMM_BF16_ACC, DL_WAVES, DL_TM, DL_TN>), grid, block, 0, st, g);
                break;
        }
        return hipGetLastError();
    }
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
