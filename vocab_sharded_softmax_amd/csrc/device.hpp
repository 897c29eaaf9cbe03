// device.hpp -- device-side building blocks of libvjsd (gfx950, wave64).
//
// Page keys: [JSD-PR] DeepSpeed PR #8958 "[VocabTP] Add vocabulary-parallel
// generalized JSD with Triton kernels"; [OPS-PR] DeepSpeed PR #8791 "Add
// vocabulary-parallel logprobs, entropy and KL ops".
//
// Arithmetic model.  Every kernel works in base 2: a logit x of a row with max m
// becomes u = x*L2E - c with c = fl32(m*L2E), evaluated by one fused multiply-add,
// whose exact product keeps a large common offset out of the rounding (the
// offset-robust statistics of [OPS-PR, How]).  exp and log are the hardware
// v_exp_f32 (2^x) and v_log_f32 (log2 x).  A row's sum of 2^u is kept relative to
// c; statistics handed between calls are (m, ln sum exp(x - m)) in fp64 and each
// kernel rebuilds its fp32 row constants from them in fp64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vjsd {

constexpr int BLOCK = 256;  // 4 waves of 64 lanes per row-workgroup
constexpr int NWAVE = BLOCK / 64;
constexpr float L2E = 1.44269504088896340736f;  // log2(e), fp32
constexpr double L2E_D = 1.44269504088896340736;
constexpr double LN2_D = 0.69314718055994530942;
constexpr float LN2F = 0.69314718055994530942f;
constexpr float NINF = -__builtin_huge_valf();
// Lower clamp of u: 2^-512 is exactly 0 in fp32, and a clamped u keeps e * u finite
// (0 * -inf would be NaN) for masked tokens.
constexpr float U_FLOOR = -512.0f;
// Added inside the mixture so log2 never sees 0 (both sides underflowed or masked);
// 2^-126 is far below any mass that can move an fp32 result.
constexpr float W_FLOOR = 1.17549435e-38f;
// Workspace layout: per-row constants (ROWC floats per row) for the streaming
// backward kernels, then per-(shard, row) partials (PART_STRIDE floats each).
constexpr int ROWC = 16;
constexpr int PART_STRIDE = 8;
constexpr int ROWC_KS = 10;         // slot holding the exponent scale log2 e / T
constexpr int ROWC_UNDEFINED = 15;  // slot holding 1.0f for a row with no distribution
// Streaming gradient kernels: one wave per workgroup, each lane one 16-byte vector of
// a row chunk, consecutive workgroups on consecutive chunks of a row.
constexpr int GRAD_BLOCK = 64;

// ---- storage formats -------------------------------------------------------------

struct F32 {
    using T = float;
    static constexpr int VEC = 4;  // elements per 16-byte access
};
struct F16 {
    using T = uint16_t;
    static constexpr int VEC = 8;
};
struct BF16 {
    using T = uint16_t;
    static constexpr int VEC = 8;
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <class D>
__device__ __forceinline__ float load1(const typename D::T *p);
template <>
__device__ __forceinline__ float load1<F32>(const float *p) { return *p; }
template <>
__device__ __forceinline__ float load1<F16>(const uint16_t *p) {
    return (float)__builtin_bit_cast(_Float16, *p);
}
template <>
__device__ __forceinline__ float load1<BF16>(const uint16_t *p) {
    return __uint_as_float((uint32_t)*p << 16);
}

// Raw 16-byte accesses.  STREAM selects the nontemporal cache policy, for data that
// is read or written once.  On MI355X it lifts a read-only pass over two inputs from
// about 6.2 to 6.9 TB/s, and a pass that reads two inputs and writes two outputs from
// about 5.4 to 6.2 TB/s (streaming only one side of the latter gains little).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <bool STREAM>
__device__ __forceinline__ u32x4 ld16(const void *p) {
    if constexpr (STREAM) return __builtin_nontemporal_load(static_cast<const u32x4 *>(p));
    else return *static_cast<const u32x4 *>(p);
}
template <bool STREAM>
__device__ __forceinline__ void st16(void *p, u32x4 v) {
    if constexpr (STREAM) __builtin_nontemporal_store(v, static_cast<u32x4 *>(p));
    else *static_cast<u32x4 *>(p) = v;
}

// 16 raw bytes of the storage format widened to fp32, and fp32 values narrowed
// (round to nearest even) to 16 raw bytes.
template <class D>
__device__ __forceinline__ void widen(u32x4 v, float (&x)[D::VEC]);
template <>
__device__ __forceinline__ void widen<F32>(u32x4 v, float (&x)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(v[i]);
}
template <>
__device__ __forceinline__ void widen<BF16>(u32x4 v, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(v[i] << 16);
        x[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
}
template <>
__device__ __forceinline__ void widen<F16>(u32x4 v, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // through a scalar: hipcc bit-casts a vector element expression from element 0
        const uint32_t wi = v[i];
        const f16x2 h = __builtin_bit_cast(f16x2, wi);
        x[2 * i] = (float)h.x;
        x[2 * i + 1] = (float)h.y;
    }
}

template <class D>
__device__ __forceinline__ u32x4 narrow(const float (&x)[D::VEC]);
template <>
__device__ __forceinline__ u32x4 narrow<F32>(const float (&x)[4]) {
    return u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                 __float_as_uint(x[3])};
}
template <>
__device__ __forceinline__ u32x4 narrow<BF16>(const float (&x)[8]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = __builtin_bit_cast(uint32_t,
                                  __builtin_convertvector((f32x2){x[2 * i], x[2 * i + 1]}, bf16x2));
    return w;
}
template <>
__device__ __forceinline__ u32x4 narrow<F16>(const float (&x)[8]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = __builtin_bit_cast(uint32_t,
                                  __builtin_convertvector((f32x2){x[2 * i], x[2 * i + 1]}, f16x2));
    return w;
}

// 16-byte load widened to fp32; 16-byte store of fp32 values in the storage format.
template <class D, bool STREAM = false>
__device__ __forceinline__ void load_vec(const typename D::T *p, float (&x)[D::VEC]) {
    widen<D>(ld16<STREAM>(p), x);
}
template <class D, bool STREAM = false>
__device__ __forceinline__ void store_vec(typename D::T *p, const float (&x)[D::VEC]) {
    st16<STREAM>(p, narrow<D>(x));
}

// four fp32 values as four bf16 (nearest even) in 8 bytes; p 8-byte aligned
__device__ __forceinline__ void st_bf16x4(uint16_t *p, const float (&x)[4]) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x[0], x[1]}, bf16x2));
    const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x[2], x[3]}, bf16x2));
    *reinterpret_cast<u32x2 *>(p) = u32x2{lo, hi};
}

// Round-to-nearest-even stores of fp32 results in the storage format.
template <class D>
__device__ __forceinline__ void store1(typename D::T *p, float v);
template <>
__device__ __forceinline__ void store1<F32>(float *p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store1<F16>(uint16_t *p, float v) {
    *p = __builtin_bit_cast(uint16_t, (_Float16)v);
}
template <>
__device__ __forceinline__ void store1<BF16>(uint16_t *p, float v) {
    *p = __builtin_bit_cast(uint16_t, (__bf16)v);
}

// ---- views and rows --------------------------------------------------------------

// Row view as passed to kernels (mirrors the ABI's view; strides in elements).
struct RowView {
    const void *p;
    int64_t rs, rpb, bs;
};
struct RowMView {
    void *p;
    int64_t rs, rpb, bs;
};

__device__ __forceinline__ int64_t row_offset(int64_t r, int64_t rs, int64_t rpb, int64_t bs) {
    return rpb > 0 ? (r / rpb) * bs + (r % rpb) * rs : r * rs;
}
template <class T>
__device__ __forceinline__ const T *row_ptr(const RowView &v, int64_t r) {
    return static_cast<const T *>(v.p) + row_offset(r, v.rs, v.rpb, v.bs);
}
template <class T>
__device__ __forceinline__ T *row_ptr(const RowMView &v, int64_t r) {
    return v.p ? static_cast<T *>(v.p) + row_offset(r, v.rs, v.rpb, v.bs) : nullptr;
}

// Elements before the first 16-byte boundary of a row whose views all share the same
// offset inside 16 bytes; if they do not, the whole row goes through the scalar path.
template <class T>
__device__ __forceinline__ int64_t head_len(int64_t w, const void *a, const void *b = nullptr,
                                            const void *c = nullptr, const void *d = nullptr) {
    const uintptr_t off = reinterpret_cast<uintptr_t>(a) & 15;
    bool same = true;
    if (b) same &= (reinterpret_cast<uintptr_t>(b) & 15) == off;
    if (c) same &= (reinterpret_cast<uintptr_t>(c) & 15) == off;
    if (d) same &= (reinterpret_cast<uintptr_t>(d) & 15) == off;
    if (!same) return w;
    const int64_t h = (int64_t)(((16 - off) & 15) / sizeof(T));
    return h < w ? h : w;
}

// Chunk q of a row of w elements: columns [c0, c0 + n); n <= 0 past the row's end.
// ALIGNED puts chunk boundaries at multiples of cw elements of the address space of
// `row` (the first chunk runs from the row start to the first boundary), so that no
// wave's 1 KiB request straddles two 1 KiB blocks where a row's size is not a multiple
// of 1 KiB (a 151936-wide bf16 row is 296.75 KiB).  On MI355X that made the two-read,
// two-write JSD backward 2-4 % faster and the one-read, one-write backwards 2-3 %
// slower, so each kernel chooses.  cw is a power of two (a mask, not a 64-bit
// division, finds the row's offset inside a chunk).
template <bool ALIGNED, class T>
__device__ __forceinline__ void chunk_span(const T *row, int64_t w, int64_t cw, int64_t q,
                                           int64_t &c0, int64_t &n) {
    const int64_t lead =
        ALIGNED ? (int64_t)((reinterpret_cast<uintptr_t>(row) / sizeof(T)) & (uint64_t)(cw - 1)) : 0;
    const int64_t a = q * cw - lead;
    c0 = a > 0 ? a : 0;
    n = (a + cw < w ? a + cw : w) - c0;
}

// ---- hardware exp2 / log2 and the base-2 reference point ---------------------------

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

// Scale of the base-2 exponent.  Logits x at temperature T enter every kernel as
// u = x * ks - c with ks = fl32(log2 e / T): the division by T is folded into the
// scale the exponent needs anyway (T = 1 gives ks = L2E).  Statistics keep the raw
// row max m, and lnZ = ln sum exp((x - m) / T) of the tempered logits.

// Reference point c = fl32(m * ks) of a row max m (0 for an empty / masked row).
__device__ __forceinline__ float refc(float m, float ks = L2E) { return m == NINF ? 0.0f : m * ks; }

// Row normaliser rebuilt from stored statistics: Z = sum 2^(x*ks - c) = 2^(lnZ*log2e + res)
// with res = m*ks - c exact in fp64.
__device__ __forceinline__ double z_from_stats(float m, double lnZ, float ks = L2E) {
    const double res = (double)m * (double)ks - (double)refc(m, ks);
    return exp2(lnZ * L2E_D + res);
}
// Inverse: ln sum exp((x - m) / T) from Z relative to c.
__device__ __forceinline__ double lnz_from_z(float m, double Z, float ks = L2E) {
    const double res = (double)m * (double)ks - (double)refc(m, ks);
    return (log2(Z) - res) * LN2_D;
}

// Per-call options of the distillation-loss form of the forward passes (kernel
// argument, by value): the exponent scale, the loss multiplier and the row mask.
struct RowOpts {
    float ks = L2E;                   // log2 e / temperature
    float lscale = 1.0f;              // T^2 when the loss is temperature-scaled, else 1
    const uint8_t *mask = nullptr;    // [N]; a zero entry drops the row; null keeps all
    const int64_t *labels = nullptr;  // [N]; a label equal to `ignore` drops the row
    int64_t ignore = 0;
};
// A dropped row is never read: its outputs are zeros.
__device__ __forceinline__ bool row_dropped(const RowOpts &o, int64_t r) {
    return (o.mask != nullptr && o.mask[r] == 0) ||
           (o.labels != nullptr && o.labels[r] == o.ignore);
}

// Upstream-gradient options of the distillation-loss form of the backward: the row
// r's gradient scale is g_r * gmul, g_r = grad[r] (per-row) or grad[0] (reduced;
// divided by max(*count, 1) for a mean), and 0 for a row the mask drops.  A NULL
// grad stands for a unit upstream gradient.
struct GradOpts {
    float ks = L2E;                  // log2 e / temperature
    double gmul = 1.0;               // T^2 (if scaled) * (1/T): chain rule through x / T
    bool scalar = false;             // grad is one value for all rows
    const uint8_t *mask = nullptr;   // [N]; zero drops the row
    const double *count = nullptr;   // device: kept rows, for a mean (null: no division)
};

// ---- wave reductions (fixed order: deterministic results) ---------------------------
//
// A butterfly over the 64 lanes of a wave that never touches LDS.  The first four
// steps read the partner lane through a DPP modifier of the combining instruction:
// quad permutations [1,0,3,2] and [2,3,0,1] for lane bits 0 and 1, the half-row mirror
// (lane j of an 8-lane group reads lane 7 - j) for bit 2, and the rotation of each
// 16-lane row by 8 for bit 3.  The last two steps use gfx950's v_permlane16_swap and
// v_permlane32_swap with both operands equal, which leave in every lane the value of
// the lower and of the upper row (half) of the pair it belongs to.  After the step
// across bit k every aligned group of 2^(k+1) lanes holds the same value, which is
// what makes the mirror a valid bit-2 partner.  ORDERED combines pass the lower lane's
// operand first, so every lane computes the bit-identical result; unordered ones
// (commutative combines: sum, max) let the DPP read fold into the combining
// instruction.  All 64 lanes must be active.

template <class T>
struct Words {
    static_assert(sizeof(T) % 4 == 0, "wave reductions move 32-bit words");
    uint32_t w[sizeof(T) / 4];
};

// v read from the DPP partner given by CTRL (row and bank masks full).
template <int CTRL, class T>
__device__ __forceinline__ T dpp_read(const T &v) {
    Words<T> a = __builtin_bit_cast(Words<T>, v);
#pragma unroll
    for (unsigned i = 0; i < sizeof(T) / 4; ++i)
        a.w[i] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a.w[i], CTRL, 0xF, 0xF, true);
    return __builtin_bit_cast(T, a);
}

template <int BIT, int CTRL, bool ORDERED, class T, class F>
__device__ __forceinline__ T bfly_dpp(const T &v, F &&f) {
    const T p = dpp_read<CTRL>(v);
    if constexpr (!ORDERED) {
        return f(v, p);
    } else {
        const bool upper = (threadIdx.x & BIT) != 0;
        return upper ? f(p, v) : f(v, p);
    }
}

// Step across lane bit 4 (ROW32 false) or 5 (true): f(lower value, upper value).
template <bool ROW32, class T, class F>
__device__ __forceinline__ T bfly_swap(const T &v, F &&f) {
    const Words<T> a = __builtin_bit_cast(Words<T>, v);
    Words<T> lo, hi;
#pragma unroll
    for (unsigned i = 0; i < sizeof(T) / 4; ++i) {
        uint32_t r0, r1;
        if constexpr (ROW32) {
            const auto r = __builtin_amdgcn_permlane32_swap(a.w[i], a.w[i], false, false);
            r0 = r[0];  // through scalars: a bit-cast vector element reads element 0
            r1 = r[1];
        } else {
            const auto r = __builtin_amdgcn_permlane16_swap(a.w[i], a.w[i], false, false);
            r0 = r[0];
            r1 = r[1];
        }
        lo.w[i] = r0;
        hi.w[i] = r1;
    }
    return f(__builtin_bit_cast(T, lo), __builtin_bit_cast(T, hi));
}

template <bool ORDERED, class T, class F>
__device__ __forceinline__ T wave_reduce(T v, F &&f) {
    v = bfly_dpp<1, 0xB1, ORDERED>(v, f);   // quad_perm [1,0,3,2]
    v = bfly_dpp<2, 0x4E, ORDERED>(v, f);   // quad_perm [2,3,0,1]
    v = bfly_dpp<4, 0x141, ORDERED>(v, f);  // row_half_mirror
    v = bfly_dpp<8, 0x128, ORDERED>(v, f);  // row_ror:8
    v = bfly_swap<false>(v, f);
    return bfly_swap<true>(v, f);
}

__device__ __forceinline__ float wave_sum(float v) {
    return wave_reduce<false>(v, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ float wave_max(float v) {
    return wave_reduce<false>(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_min(float v) {
    return wave_reduce<false>(v, [](float a, float b) { return fminf(a, b); });
}

// Online (max, sum of 2^(x*ks - refc(max))) pair.
struct MZ {
    float m, z;
};
__device__ __forceinline__ MZ mz_combine(MZ a, MZ b, float ks = L2E) {
    const float m = fmaxf(a.m, b.m);
    const float c = refc(m, ks);
    const float za = a.m == NINF ? 0.0f : a.z * ex2(refc(a.m, ks) - c);
    const float zb = b.m == NINF ? 0.0f : b.z * ex2(refc(b.m, ks) - c);
    return {m, za + zb};
}
__device__ __forceinline__ MZ wave_mz(MZ v, float ks = L2E) {
    return wave_reduce<true>(v, [ks](MZ a, MZ b) { return mz_combine(a, b, ks); });
}

// ---- workgroup reductions: waves as above, then the wave results in wave order ------

// Sum of NV floats over a BLK-lane workgroup; result valid in thread 0.  `red` is LDS
// of NV * (BLK / 64) floats.
template <int NV, int BLK = BLOCK>
__device__ __forceinline__ void block_sum(float (&v)[NV], float *red) {
    constexpr int NW = BLK / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = wave_sum(v[i]);
    if (lane == 0)
#pragma unroll
        for (int i = 0; i < NV; ++i) red[i * NW + wave] = v[i];
    __syncthreads();
    if (threadIdx.x == 0)
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            float a = red[i * NW];
#pragma unroll
            for (int k = 1; k < NW; ++k) a += red[i * NW + k];
            v[i] = a;
        }
}

}  // namespace vjsd
