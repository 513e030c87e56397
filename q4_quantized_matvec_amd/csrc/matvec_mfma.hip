// Batched Q4_0 / Q8_0 dequant-matvec (1 <= B <= 32 activation rows) on the
// gfx950 matrix cores.
//
// Definition ("Research record" page, "Native Metal diagnostic: buffer
// ownership": 18-byte Q4_0 blocks, weight = (quant - 8) * scale; "Verified
// model facts": the Q8_0 token table):
//   y[b][n] = sum_k d[n][k/32] * c[n][k] * op(x)[b][k]   (+ residual[b][n]),
// c = q - 8 (Q4_0) or the int8 code q (Q8_0).
//
// With eight activation rows every weight feeds eight products, more than the
// vector ALUs sustain at HBM speed; v_mfma_f32_16x16x32_f16 takes them, one
// block (32 k) per instruction, so the block scale is applied once per 16 x 16
// result tile:
//   D[i][n] = sum_{k in block} X[i][k] * c[n][k] ,   acc += d[n][block] * D .
// Both operands are exact in binary16.  c is an integer of at most 8 bits
// (built as 1024 + q with one mask-or, then one packed subtract).  The
// activations of each step of 256 k are scaled by a power of two s per batch
// row, chosen so that the largest |s x| lies in [2^11, 2^12), and carried as
// two halves, hi = fp16(s x) and lo = fp16(s x - hi), 22 significant bits: the
// 16 MFMA rows are 8 batch rows x {hi, lo}, every product is exact, and 1/s is
// applied exactly to the step's partial sums.
//
// One kernel.  A workgroup (4 wavefronts) owns 64 output rows and a range of
// K steps; per step of 8 blocks:
//  * operand build: each wavefront converts 2 of the 8 blocks for all batch
//    rows (applying the input transform: gain multiply for RMSNorm, SiLU(x)*u
//    for SwiGLU), the step's per-row maxima meet in LDS, and the halves are
//    written to LDS in MFMA operand order;
//  * weights: lane (n, g) = (lane % 16, lane / 16) of a wavefront holds 2
//    consecutive blocks of row n (36 or 68 contiguous bytes, loaded one step
//    ahead); permlane32/16 swaps transpose the 4 x 4 lane groups so that for
//    every block lane group g holds its share of the codes (Q4_0: payload
//    bytes 4g..4g+3, i.e. elements 4g..4g+3 as low nibbles and 4g+16..4g+19 as
//    high nibbles, the latter kept x16 and paired with activations / 16;
//    Q8_0: payload bytes 8g..8g+7); 8 MFMAs per wavefront.
// RMSNorm's 1/rms factor is common to a whole row, so it is applied to the
// finished sums; the sums of squares are gathered from the same operand
// build.  K is split over S workgroups when the row count alone cannot fill
// the chip; the partial sums are added in split order by whichever workgroup
// of the row range finishes last, so results are bitwise reproducible.
//
// More than 8 activation rows are taken in groups of 8 (at most 4 groups):
// each workgroup computes one group, and the workgroups of one row range and
// its groups are dispatched one after another to the same XCD, so the
// weights come from HBM once and the later groups read them from that XCD's
// L2.
#include <mutex>
#include <type_traits>

#include "common.hpp"

namespace {
using namespace q4dev;

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_al4_t __attribute__((ext_vector_type(4), aligned(4)));
typedef float f32x4_al16_t __attribute__((ext_vector_type(4), aligned(16)));

constexpr int kWG = 256;            // 4 wavefronts
constexpr int kSeg = 8;             // blocks per step (one MFMA each per wavefront)
constexpr int kMaxB = 8;             // activation rows per group (one MFMA operand)
constexpr int kMaxGroups = 4;
constexpr int kMaxBatch = kMaxB * kMaxGroups;
constexpr int kMinWGs = 512;        // below this, the shared-step kernel
constexpr int kTargetWGs = 1024;    // shared-step kernel: split K toward this many workgroups
constexpr int kMaxS = 32;           // K splits at most (the final writer holds them in registers)
constexpr int kCounters = 4096;     // split tickets: row ranges of a K-split launch
constexpr int kCounterStride = 32;  // one ticket per 128-byte line: atomics on one line serialise
constexpr size_t kCounterBytes = static_cast<size_t>(kCounters) * kCounterStride * sizeof(int);

template <int FMT>
struct BF;
template <>
struct BF<0> {
    static constexpr int kBytes = 18;
    static constexpr int kLaneDw = 9;  // two blocks: 36 bytes
};
template <>
struct BF<1> {
    static constexpr int kBytes = 34;
    static constexpr int kLaneDw = 17;  // two blocks: 68 bytes
};

// act(g) * u with act = SiLU or (GELU) the tanh form of GELU; a template
// parameter so that the GELU code is only in the kernels that use it (larger
// kernels start measurably slower when launched back to back with others).
template <bool GELU>
__device__ __forceinline__ float act_mul(float g, float u) {
    if constexpr (GELU) return 0.5f * g * (1.0f + tanhf(0.7978845608028654f * (g + 0.044715f * g * g * g))) * u;
    else return g / (1.0f + expf(-g)) * u;
}

// Offset inside a block of element e (0..7) of lane group g.
template <int FMT>
__device__ __forceinline__ int elem_of(int g, int e) {
    if constexpr (FMT == 0) return e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4);
    else return 8 * g + e;
}

// Power-of-two exponent that puts m (the largest magnitude of a step) in
// [2^11, 2^12); 0 for zero, infinite or NaN maxima (values pass unscaled).
__device__ __forceinline__ int step_shift(float m) {
    if (!(m > 0.f) || !(m <= 3.4e38f)) return 0;
    int e;
    (void)frexpf(m, &e);
    return min(max(12 - e, -120), 120);
}

__device__ __forceinline__ float max4(f32x4_t v) { return fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)); }

// Row range rx and batch group gi of this workgroup.  With one group the
// grid is (row ranges, K splits).  With NG > 1 groups, workgroups go to the
// 8 XCDs in turn (id mod 8), so id = 8 (NG r + gi) + x for row range
// 8 r + x puts the NG groups of a row range on one XCD, consecutively; the
// grid is padded to whole octets and ids past the last row range idle.
struct GroupView {
    int rx, gi, Bg;  // row range, group, activation rows of the group
    bool live;
};
__device__ __forceinline__ GroupView group_view(int rg, int NG, int B) {
    if (NG == 1) return {static_cast<int>(blockIdx.x), 0, B, static_cast<int>(blockIdx.x) < rg};
    const int L = blockIdx.x, j = L >> 3;
    const int gi = j % NG, rx = (j / NG) * 8 + (L & 7);
    return {rx, gi, min(kMaxB, B - kMaxB * gi), rx < rg};
}

// A copy the compiler cannot see through.  When both results of one
// permlane swap are reinterpreted as floating point, this compiler has been
// seen to merge the two reinterpretations into one (computing a[0] + a[0]
// for a[0] + a[1]); every second result that is used as a float or half is
// therefore passed through this copy first.
__device__ __forceinline__ uint32_t opaque_copy(uint32_t v) {
    uint32_t r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
    return r;
}

// Maximum over the 4 lanes l, l^16, l^32, l^48; every one of them receives it.
__device__ __forceinline__ float rows_max(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float m = fmaxf(__builtin_bit_cast(float, a[0]), __builtin_bit_cast(float, opaque_copy(a[1])));
    const uint32_t um = __builtin_bit_cast(uint32_t, m);
    auto b = __builtin_amdgcn_permlane16_swap(um, um, false, false);
    return fmaxf(__builtin_bit_cast(float, b[0]), __builtin_bit_cast(float, opaque_copy(b[1])));
}
// Sum over the 4 lanes l, l^16, l^32, l^48; every one of them receives the
// same bits (both steps add commutatively).
__device__ __forceinline__ float rows_sum(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float m = __builtin_bit_cast(float, a[0]) + __builtin_bit_cast(float, opaque_copy(a[1]));
    const uint32_t um = __builtin_bit_cast(uint32_t, m);
    auto b = __builtin_amdgcn_permlane16_swap(um, um, false, false);
    return __builtin_bit_cast(float, b[0]) + __builtin_bit_cast(float, opaque_copy(b[1]));
}

// Eight per-lane values v[b] (one per batch row) reduced over the 64 lanes at
// once; on return lane l holds the result for b = l / 8.  Each exchange round
// halves what a lane carries: lanes l and l ^ 32 (permlane32 swap) keep b < 4
// in the low half and b >= 4 in the high half, lanes l and l ^ 16
// (permlane16 swap) split those again, lanes l and l ^ 8 (row rotation by 8)
// once more, and three DPP rounds finish over the 8 lanes of each half-row.
// About 20 instructions, where eight separate wavefront reductions take
// about 120 and their DPP hazards.
template <bool MAX>
__device__ __forceinline__ float red_op(float a, float b) {
    return MAX ? fmaxf(a, b) : a + b;
}
template <bool MAX>
__device__ __forceinline__ float reduce8_by_lane(const float (&v)[kMaxB]) {
    float r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // lanes 0..31: b = j; lanes 32..63: b = j + 4
        auto s = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v[j]),
                                                  __builtin_bit_cast(uint32_t, v[j + 4]), false, false);
        r[j] = red_op<MAX>(__builtin_bit_cast(float, s[0]), __builtin_bit_cast(float, opaque_copy(s[1])));
    }
    float t[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {  // 16-lane row q: b = j + 2 (q % 2) + 4 (q / 2)
        auto s = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, r[j]),
                                                  __builtin_bit_cast(uint32_t, r[j + 2]), false, false);
        t[j] = red_op<MAX>(__builtin_bit_cast(float, s[0]), __builtin_bit_cast(float, opaque_copy(s[1])));
    }
    const bool up = (threadIdx.x & 8) != 0;  // lanes with bit 3 set keep b odd
    const float keep = up ? t[1] : t[0], send = up ? t[0] : t[1];
    float w = red_op<MAX>(keep, dpp_keep<0x128>(send));  // row_ror:8 = lane ^ 8 within the row
    w = red_op<MAX>(w, dpp_keep<0xB1>(w));                // quad_perm [1,0,3,2]
    w = red_op<MAX>(w, dpp_keep<0x4E>(w));                // quad_perm [2,3,0,1]
    return red_op<MAX>(w, dpp_keep<0x141>(w));            // row_half_mirror: the two quads
}

// Lane groups 0..3 hold v_t for t = 0..3; afterwards v_s at lane group g is
// the old v_g of lane group s (a 4 x 4 transpose across the 16-lane rows).
__device__ __forceinline__ void transpose4(uint32_t &v0, uint32_t &v1, uint32_t &v2, uint32_t &v3) {
    auto a = __builtin_amdgcn_permlane32_swap(v0, v2, false, false);
    auto b = __builtin_amdgcn_permlane32_swap(v1, v3, false, false);
    auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    v0 = c[0];
    v1 = c[1];
    v2 = d[0];
    v3 = d[1];
}

__device__ __forceinline__ half8_t make_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    u32x4_t v = {a, b, c, d};
    return __builtin_bit_cast(half8_t, v);
}

// Eight Q4_0 codes of one lane (payload bytes b0..b3) as exact halves:
// low nibbles q - 8, high nibbles 16 (q - 8).  One byte permute places two
// code bytes under the exponent byte 0x64 (the halves 1024 + byte); a mask
// keeps one nibble of each (1024 + q or 1024 + 16 q), and a packed subtract
// removes the offset.
__device__ __forceinline__ half8_t q4_codes(uint32_t w) {
    const uint32_t p01 = __builtin_amdgcn_perm(0x64646464u, w, 0x04010400u);
    const uint32_t p23 = __builtin_amdgcn_perm(0x64646464u, w, 0x04030402u);
    const half2_t lo_off = {static_cast<_Float16>(-1032.0f), static_cast<_Float16>(-1032.0f)};
    const half2_t hi_off = {static_cast<_Float16>(-1152.0f), static_cast<_Float16>(-1152.0f)};
    const half2_t h0 = __builtin_bit_cast(half2_t, p01 & 0xFF0FFF0Fu) + lo_off;
    const half2_t h1 = __builtin_bit_cast(half2_t, p23 & 0xFF0FFF0Fu) + lo_off;
    const half2_t h2 = __builtin_bit_cast(half2_t, p01 & 0xFFF0FFF0u) + hi_off;
    const half2_t h3 = __builtin_bit_cast(half2_t, p23 & 0xFFF0FFF0u) + hi_off;
    return make_half8(__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1),
                      __builtin_bit_cast(uint32_t, h2), __builtin_bit_cast(uint32_t, h3));
}

// Eight Q8_0 codes (two words of int8) as exact halves: byte ^ 0x80 is the
// code + 128, placed in the mantissa of 1024.
__device__ __forceinline__ half8_t q8_codes(uint32_t w0, uint32_t w1) {
    const half2_t off = {static_cast<_Float16>(-1152.0f), static_cast<_Float16>(-1152.0f)};
    const half2_t h0 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(w0, w0, 0x0C010C00u) ^ 0x64806480u) + off;
    const half2_t h1 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(w0, w0, 0x0C030C02u) ^ 0x64806480u) + off;
    const half2_t h2 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(w1, w1, 0x0C010C00u) ^ 0x64806480u) + off;
    const half2_t h3 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(w1, w1, 0x0C030C02u) ^ 0x64806480u) + off;
    return make_half8(__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1),
                      __builtin_bit_cast(uint32_t, h2), __builtin_bit_cast(uint32_t, h3));
}

// One lane's window of two blocks: 16-byte loads plus a tail word, 4-byte aligned.
template <int DW>
__device__ __forceinline__ void load_seg(const uint8_t *p, uint32_t (&dw)[DW]) {
#pragma unroll
    for (int q = 0; q < (DW - 1) / 4; ++q) {
        const u32x4_al4_t v = *reinterpret_cast<const u32x4_al4_t *>(p + 16 * q);
        dw[4 * q] = v.x;
        dw[4 * q + 1] = v.y;
        dw[4 * q + 2] = v.z;
        dw[4 * q + 3] = v.w;
    }
    dw[DW - 1] = *reinterpret_cast<const uint32_t *>(p + 4 * (DW - 1));
}

// The 8 weight operands of one step from a lane's two-block window.
template <int FMT>
__device__ __forceinline__ void weight_operands(const uint32_t (&dw)[BF<FMT>::kLaneDw], half8_t (&wf)[kSeg]) {
    if constexpr (FMT == 0) {
        // even block: payload at byte 2 of the window; odd block: at byte 20
        uint32_t e0 = __builtin_amdgcn_alignbyte(dw[1], dw[0], 2);
        uint32_t e1 = __builtin_amdgcn_alignbyte(dw[2], dw[1], 2);
        uint32_t e2 = __builtin_amdgcn_alignbyte(dw[3], dw[2], 2);
        uint32_t e3 = __builtin_amdgcn_alignbyte(dw[4], dw[3], 2);
        uint32_t o0 = dw[5], o1 = dw[6], o2 = dw[7], o3 = dw[8];
        transpose4(e0, e1, e2, e3);
        transpose4(o0, o1, o2, o3);
        wf[0] = q4_codes(e0); wf[1] = q4_codes(o0);
        wf[2] = q4_codes(e1); wf[3] = q4_codes(o1);
        wf[4] = q4_codes(e2); wf[5] = q4_codes(o2);
        wf[6] = q4_codes(e3); wf[7] = q4_codes(o3);
    } else {
        uint32_t e[8], o[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            e[t] = __builtin_amdgcn_alignbyte(dw[t + 1], dw[t], 2);
            o[t] = dw[9 + t];
        }
        transpose4(e[0], e[2], e[4], e[6]);
        transpose4(e[1], e[3], e[5], e[7]);
        transpose4(o[0], o[2], o[4], o[6]);
        transpose4(o[1], o[3], o[5], o[7]);
        wf[0] = q8_codes(e[0], e[1]); wf[1] = q8_codes(o[0], o[1]);
        wf[2] = q8_codes(e[2], e[3]); wf[3] = q8_codes(o[2], o[3]);
        wf[4] = q8_codes(e[4], e[5]); wf[5] = q8_codes(o[4], o[5]);
        wf[6] = q8_codes(e[6], e[7]); wf[7] = q8_codes(o[6], o[7]);
    }
}

// Output of a workgroup whose wavefront w < T holds, per lane (col, g), the
// sums ya (batch row 2g) and yb (2g + 1) of output row n of its tile, and
// whose ssq_w holds the four wavefronts' sums of squares per batch row (RMSNorm).
// Without a K split the workgroup writes y (residual, 1/rms or SiLU(g)*u
// applied); with one, it stores its partials, takes a ticket, and the last
// split of the row range adds the S partials in split order.
struct FinishArgs {
    int N, K, B, S, glu, rx;  // B: rows of the group; glu: a gated output; rx: the row range
    float eps;
    float *y;
    const float *res;
    int *counters;
    float *ssq_part;
    float *part;
};

template <int KIND, int T, bool GELU>
__device__ __forceinline__ void finish(const FinishArgs &fa_, float ya, float yb, int n, bool rvalid, int pl,
                                       int pu, float (&ssq_w)[4][kMaxB]) {
    constexpr int kRows = 16 * T, kPairs = 8 * T;
    constexpr int kHalf = T > 1 ? T / 2 : 1;
    __shared__ float upx[kPairs][kMaxB];  // SwiGLU output: up-row sums of the pairs
    __shared__ int ticket;
    const int N = fa_.N, K = fa_.K, B = fa_.B, S = fa_.S, glu = fa_.glu, rx = fa_.rx;
    const float eps = fa_.eps;
    float *y = fa_.y;
    const float *res = fa_.res;
    int *counters = fa_.counters;
    float *ssq_part = fa_.ssq_part, *part = fa_.part;
    const int P = N >> 1;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int g = lane >> 4;
    auto range_ssq = [&](int b) { return ((ssq_w[0][b] + ssq_w[1][b]) + ssq_w[2][b]) + ssq_w[3][b]; };
    const int ba = 2 * g, bb = 2 * g + 1;
    const int64_t ln = N;
    if (S == 1) {
        float ia = 1.f, ib = 1.f;
        if constexpr (KIND == 1) {
            ia = 1.0f / sqrtf(range_ssq(ba) / static_cast<float>(K) + eps);
            ib = 1.0f / sqrtf(range_ssq(bb) / static_cast<float>(K) + eps);
        }
        if (glu) {
            if (wv >= kHalf && wv < T) {
                upx[pl][ba] = ya * ia;
                upx[pl][bb] = yb * ib;
            }
            __syncthreads();
            if (wv < kHalf && rvalid) {
                const int64_t lp = P;
                if (ba < B) y[ba * lp + pu] = act_mul<GELU>(ya * ia, upx[pl][ba]);
                if (bb < B) y[bb * lp + pu] = act_mul<GELU>(yb * ib, upx[pl][bb]);
            }
            return;
        }
        if (rvalid) {
            if (ba < B) y[ba * ln + n] = res ? ya * ia + res[ba * ln + n] : ya * ia;
            if (bb < B) y[bb * ln + n] = res ? yb * ib + res[bb * ln + n] : yb * ib;
        }
        return;
    }
    // Split K: partial sums go to the workspace with device-scope stores
    // (written through the compute die's L2), the workgroup takes a ticket,
    // and the last one adds the S partials in split order with device-scope
    // loads.  Device-scope fences are avoided on purpose: on this part they
    // write back and invalidate the whole L2 of the die.
    if (rvalid) {
        float *pp = part + static_cast<int64_t>(blockIdx.y) * B * ln;
        if (ba < B) __hip_atomic_store(pp + ba * ln + n, ya, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (bb < B) __hip_atomic_store(pp + bb * ln + n, yb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if constexpr (KIND == 1) {
        if (threadIdx.x < B)
            __hip_atomic_store(ssq_part + (static_cast<int64_t>(rx) * S + blockIdx.y) * kMaxB +
                                   threadIdx.x,
                               range_ssq(threadIdx.x), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);  // every store of this wavefront has completed
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (threadIdx.x == 0)
        ticket = __hip_atomic_fetch_add(&counters[rx * kCounterStride], 1, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (ticket != S - 1) return;
    // Final writer: every partial it needs is requested before any is added
    // (device-scope loads miss the die's L2, so each round trip is long), and
    // the S partials of a row are added in split order.
    const int64_t step = static_cast<int64_t>(B) * ln;
    __shared__ float inv_s[kMaxB];
    if constexpr (KIND == 1) {
        if (threadIdx.x < B) {
            const float *sq = ssq_part + static_cast<int64_t>(rx) * S * kMaxB + threadIdx.x;
            float t[kMaxS];
#pragma unroll
            for (int q = 0; q < kMaxS; ++q)
                t[q] = __hip_atomic_load(sq + (q < S ? q : 0) * kMaxB, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            float tot = 0.f;
#pragma unroll
            for (int q = 0; q < kMaxS; ++q)
                if (q < S) tot += t[q];
            inv_s[threadIdx.x] = 1.0f / sqrtf(tot / static_cast<float>(K) + eps);
        }
    }
    // up to two rows per thread: outputs tid and tid + 256, or the gate and up
    // rows of SwiGLU output tid
    const int outs = glu ? kPairs : kRows;
    int row[2], ob[2];
    bool act[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int o = glu ? static_cast<int>(threadIdx.x) : static_cast<int>(threadIdx.x) + r * kWG;
        ob[r] = o / outs;
        const int nn = rx * outs + (o % outs);
        act[r] = o < outs * B && nn < (glu ? P : N);
        row[r] = glu ? (r == 0 ? nn : P + nn) : nn;
    }
    float pv[2][kMaxS];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const float *pb = part + static_cast<int64_t>(act[r] ? ob[r] : 0) * ln + (act[r] ? row[r] : 0);
#pragma unroll
        for (int q = 0; q < kMaxS; ++q)
            pv[r][q] = __hip_atomic_load(pb + (q < S ? q : 0) * step, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    float sum[2] = {0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int q = 0; q < kMaxS; ++q)
            if (q < S) sum[r] += pv[r][q];
    if constexpr (KIND == 1) __syncthreads();
    if (glu) {
        if (act[0]) {
            const float inv = KIND == 1 ? inv_s[ob[0]] : 1.f;
            y[ob[0] * static_cast<int64_t>(P) + (row[0])] = act_mul<GELU>(sum[0] * inv, sum[1] * inv);
        }
    } else {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            if (!act[r]) continue;
            const float v = sum[r] * (KIND == 1 ? inv_s[ob[r]] : 1.f);
            y[ob[r] * ln + row[r]] = res ? v + res[ob[r] * ln + row[r]] : v;
        }
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(&counters[rx * kCounterStride], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int FMT, int KIND, bool GELU>
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(3))) void mv_mfma_step_kernel(
    const uint8_t *__restrict__ W, int N, int K, int B, const float *__restrict__ x,
    const float *__restrict__ u, const float *__restrict__ nw, int64_t ld, float eps, float *y,
    const float *res, int *__restrict__ counters, float *__restrict__ ssq_part,
    float *__restrict__ part, int S, int cps, int glu, int rg, int NG) {
    constexpr int kBytes = BF<FMT>::kBytes;
    constexpr int kDw = BF<FMT>::kLaneDw;
    __shared__ u32x4_t frag[2][kSeg][64];    // activation operands of a step
    __shared__ f32x4_t stepmax[2][kMaxB];    // per batch row: the 4 wavefronts' maxima
    __shared__ float ssq_w[4][kMaxB];
    const GroupView gv_ = group_view(rg, NG, B);
    if (!gv_.live) return;  // padding of the last octet (workgroup-uniform)
    const int rx = gv_.rx;
    {
        // this group's activation rows, outputs and workspace regions
        const int64_t g8 = static_cast<int64_t>(kMaxB) * gv_.gi;
        const int64_t outw = glu ? (N >> 1) : N;
        x += g8 * ld;
        if (u) u += g8 * ld;
        y += g8 * outw;
        if (res) res += g8 * N;
        part += static_cast<int64_t>(gv_.gi) * S * kMaxB * N;
        ssq_part += static_cast<int64_t>(gv_.gi) * rg * S * kMaxB;
        counters += gv_.gi * rg * kCounterStride;
        B = gv_.Bg;
    }

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int col = lane & 15, g = lane >> 4;
    // Rows of this lane: 64 consecutive rows per workgroup, or with a SwiGLU
    // output 32 gate rows (wavefronts 0, 1) and their 32 up rows (2, 3).
    const int P = N >> 1;
    const int pu = rx * 32 + 16 * (wv & 1) + col;  // pair (SwiGLU output)
    const int n = glu ? (wv < 2 ? pu : P + pu) : rx * 64 + wv * 16 + col;
    const bool rvalid = glu ? pu < P : n < N;
    const int nl = rvalid ? n : N - 1;
    const int nb = K / 32, kc = nb / kSeg;
    const int c0 = blockIdx.y * cps;
    const int c1 = min(kc, c0 + cps);
    const uint8_t *wrow = W + static_cast<int64_t>(nl) * nb * kBytes + g * 2 * kBytes;
    const int64_t seg = kSeg * kBytes;
    // operand-build role of this lane: MFMA row 2 * batch + {hi, lo}
    const int xb = (lane & 15) >> 1, xp = lane & 1;
    const bool xlive = xb < B;
    const float *xr = x + static_cast<int64_t>(xlive ? xb : 0) * ld;
    const float *ur = KIND == 2 ? u + static_cast<int64_t>(xlive ? xb : 0) * ld : nullptr;

    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
    const f32x4_t one = {1.f, 1.f, 1.f, 1.f};
    float ssq = 0.f;
    uint32_t dw[kDw], nx[kDw];
    load_seg<kDw>(wrow + c0 * seg, dw);
    for (int c = c0; c < c1; ++c) {
        const int buf = c & 1;
        // ---- activations of this step, blocks 2wv and 2wv+1 (loaded before
        // the next step's weights, so waiting for them never waits for those)
        f32x4_t xv[2][2], tv[2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int kb = 32 * (kSeg * c + 2 * wv + h);
            const int k0 = kb + elem_of<FMT>(g, 0), k1 = kb + elem_of<FMT>(g, 4);
            xv[h][0] = xlive ? *reinterpret_cast<const f32x4_al16_t *>(xr + k0) : zero;
            xv[h][1] = xlive ? *reinterpret_cast<const f32x4_al16_t *>(xr + k1) : zero;
            if constexpr (KIND == 1) {
                tv[h][0] = (xlive && nw) ? *reinterpret_cast<const f32x4_al16_t *>(nw + k0) : one;
                tv[h][1] = (xlive && nw) ? *reinterpret_cast<const f32x4_al16_t *>(nw + k1) : one;
            } else if constexpr (KIND == 2) {
                tv[h][0] = xlive ? *reinterpret_cast<const f32x4_al16_t *>(ur + k0) : zero;
                tv[h][1] = xlive ? *reinterpret_cast<const f32x4_al16_t *>(ur + k1) : zero;
            }
        }
        load_seg<kDw>(wrow + min(c + 1, c1 - 1) * seg, nx);

        float v[2][8];
        float lm = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float a = xv[h][e >> 2][e & 3];
                float t = a;
                if constexpr (KIND == 1) {
                    ssq = fmaf(a, a, ssq);
                    t = a * tv[h][e >> 2][e & 3];
                } else if constexpr (KIND == 2) {
                    t = act_mul<GELU>(a, tv[h][e >> 2][e & 3]);
                }
                v[h][e] = t;
                lm = fmaxf(lm, fabsf(t));
            }
        }
        lm = rows_max(lm);
        if (g == 0 && xp == 0) stepmax[buf][xb][wv] = lm;
        __syncthreads();
        const float s = ldexpf(1.0f, step_shift(max4(stepmax[buf][xb])));
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            half8_t hv;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float t = v[h][e] * s;
                if (FMT == 0 && e >= 4) t *= 0.0625f;
                const _Float16 hi = static_cast<_Float16>(t);
                hv[e] = xp == 0 ? hi : static_cast<_Float16>(t - static_cast<float>(hi));
            }
            frag[buf][2 * wv + h][lane] = __builtin_bit_cast(u32x4_t, hv);
        }
        // 1/s of the two batch rows whose sums this lane accumulates
        const float fa = ldexpf(1.0f, -step_shift(max4(stepmax[buf][2 * g])));
        const float fb = ldexpf(1.0f, -step_shift(max4(stepmax[buf][2 * g + 1])));
        __syncthreads();

        // ---- weights: the block scales of this lane's two blocks, then every
        // lane group's, then the codes
        const uint32_t dp = __builtin_amdgcn_perm(dw[(kDw - 1) / 2], dw[0], 0x07060100u);
        uint32_t dps[4];
        {
            auto r = __builtin_amdgcn_permlane32_swap(dp, dp, false, false);
            auto s01 = __builtin_amdgcn_permlane16_swap(r[0], r[0], false, false);
            auto s23 = __builtin_amdgcn_permlane16_swap(r[1], r[1], false, false);
            dps[0] = s01[0];
            dps[1] = opaque_copy(s01[1]);
            dps[2] = s23[0];
            dps[3] = opaque_copy(s23[1]);
        }
        half8_t wf[kSeg];
        weight_operands<FMT>(dw, wf);
        f32x4_t st = zero;
#pragma unroll
        for (int jj = 0; jj < kSeg; ++jj) {
            const f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                __builtin_bit_cast(half8_t, frag[buf][jj][lane]), wf[jj], zero, 0, 0, 0);
            const uint32_t sc = dps[jj >> 1];
            if (jj & 1) {
                st[0] = fma_hi(sc, d[0], st[0]);
                st[1] = fma_hi(sc, d[1], st[1]);
                st[2] = fma_hi(sc, d[2], st[2]);
                st[3] = fma_hi(sc, d[3], st[3]);
            } else {
                st[0] = fma_lo(sc, d[0], st[0]);
                st[1] = fma_lo(sc, d[1], st[1]);
                st[2] = fma_lo(sc, d[2], st[2]);
                st[3] = fma_lo(sc, d[3], st[3]);
            }
        }
        // result rows 4g..4g+3 are (batch 2g: hi, lo), (batch 2g+1: hi, lo)
        acc[0] = fmaf(fa, st[0], acc[0]);
        acc[1] = fmaf(fa, st[1], acc[1]);
        acc[2] = fmaf(fb, st[2], acc[2]);
        acc[3] = fmaf(fb, st[3], acc[3]);
#pragma unroll
        for (int t = 0; t < kDw; ++t) dw[t] = nx[t];
    }

    // RMSNorm: sums of squares of this K range per batch row, in a fixed order
    // (lanes with xp == 1 hold the same elements and are not counted).
    if constexpr (KIND == 1) {
        const float t = rows_sum(xp == 0 ? ssq : 0.f);
        if (g == 0 && xp == 0) ssq_w[wv][xb] = t;
        __syncthreads();
    }
    const int pl = 16 * (wv & 1) + col;
    const float ya = acc[0] + acc[1];
    const float yb = acc[2] + acc[3];
    const FinishArgs fa_{N, K, B, S, glu, rx, eps, y, res, counters, ssq_part, part};
    finish<KIND, 4, GELU>(fa_, ya, yb, n, rvalid, pl, pu, ssq_w);
}

template <int FMT, int KIND, int T, bool GELU>
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(3))) void mv_mfma_tile_kernel(
    const uint8_t *__restrict__ W, int N, int K, int B, const float *__restrict__ x,
    const float *__restrict__ u, const float *__restrict__ nw, int64_t ld, float eps, float *y,
    const float *res, int *__restrict__ counters, float *__restrict__ ssq_part,
    float *__restrict__ part, int S, int spw, int glu, int rg, int NG) {
    constexpr int kBytes = BF<FMT>::kBytes;
    constexpr int kDw = BF<FMT>::kLaneDw;
    __shared__ u32x4_t opnd[4][kSeg][64];               // per wavefront: its step's activation operands
    __shared__ f32x4_t red[4][T][64];                   // per-wavefront partial tiles
    __shared__ float ssq_w[4][kMaxB];
    constexpr int kRows = 16 * T, kPairs = 8 * T;       // output rows (pairs) of a workgroup
    const GroupView gv_ = group_view(rg, NG, B);
    if (!gv_.live) return;  // padding of the last octet (workgroup-uniform)
    const int rx = gv_.rx;
    {
        // this group's activation rows, outputs and workspace regions
        const int64_t g8 = static_cast<int64_t>(kMaxB) * gv_.gi;
        const int64_t outw = glu ? (N >> 1) : N;
        x += g8 * ld;
        if (u) u += g8 * ld;
        y += g8 * outw;
        if (res) res += g8 * N;
        part += static_cast<int64_t>(gv_.gi) * S * kMaxB * N;
        ssq_part += static_cast<int64_t>(gv_.gi) * rg * S * kMaxB;
        counters += gv_.gi * rg * kCounterStride;
        B = gv_.Bg;
    }

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int col = lane & 15, g = lane >> 4;
    const int P = N >> 1;
    // Row tile t of the workgroup: 16 consecutive rows, or with a SwiGLU
    // output the gate rows of 16 pairs (t < T/2) and their up rows.
    constexpr int kHalf = T > 1 ? T / 2 : 1;                       // gate tiles (SwiGLU output)
    auto tile_pair = [&](int t) { return 16 * (t % kHalf) + col; };  // pair within the workgroup
    auto tile_row = [&](int t, bool &valid) {
        if (glu) {
            const int pr = rx * kPairs + tile_pair(t);
            valid = pr < P;
            return t < kHalf ? pr : P + pr;
        }
        const int r = rx * kRows + 16 * t + col;
        valid = r < N;
        return r;
    };
    const int nb = K / 32, kc = nb / kSeg;
    const int64_t seg = kSeg * kBytes;
    const uint8_t *wrow[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        bool v;
        const int r = tile_row(t, v);
        wrow[t] = W + static_cast<int64_t>(v ? r : N - 1) * nb * kBytes + g * 2 * kBytes;
    }
    // Staging role of this lane: 4 consecutive activations (k = 4 lane ..) of
    // its wavefront's step, for every batch row.  They land in block
    // jl = lane / 8 at operand lane group gl, halves el .. el + 3.
    const int jl = lane >> 3, q8 = lane & 7;
    const int gl = FMT == 0 ? (q8 & 3) : (q8 >> 1);
    const int el = FMT == 0 ? (q8 >= 4 ? 4 : 0) : 4 * (q8 & 1);
    const float hscale = (FMT == 0 && q8 >= 4) ? 0.0625f : 1.0f;  // high nibbles: codes x16, x / 16

    f32x4_t acc[T];
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = zero;
    float ssq[kMaxB];
#pragma unroll
    for (int b = 0; b < kMaxB; ++b) ssq[b] = 0.f;

    const int c_base = blockIdx.y * 4 * spw;
    for (int r = 0; r < spw; ++r) {
        const int c = c_base + 4 * r + wv;  // this wavefront's step
        if (c >= kc) break;                 // wave-uniform; steps only grow with r
        // ---- activations first (loads return in order), then the weights
        const int64_t kx = static_cast<int64_t>(c) * (32 * kSeg) + 4 * lane;
        // (every load is unconditional, rows past B re-read the last one,
        // whose sums are computed and never stored, so the compiler can wait
        // for these loads alone and not for the weights behind them)
        f32x4_t xv[kMaxB], tv[kMaxB];
        f32x4_t gv = {1.f, 1.f, 1.f, 1.f};
        if constexpr (KIND == 1) {
            const f32x4_t gl4 = *reinterpret_cast<const f32x4_al16_t *>((nw ? nw : x) + kx);
            if (nw) gv = gl4;
        }
#pragma unroll
        for (int b = 0; b < kMaxB; ++b) {
            const int64_t bo = static_cast<int64_t>(min(b, B - 1)) * ld + kx;
            xv[b] = *reinterpret_cast<const f32x4_al16_t *>(x + bo);
            if constexpr (KIND == 2) tv[b] = *reinterpret_cast<const f32x4_al16_t *>(u + bo);
        }
        uint32_t dw[T][kDw];
#pragma unroll
        for (int t = 0; t < T; ++t) load_seg<kDw>(wrow[t] + c * seg, dw[t]);

        // ---- transform, per-batch-row step maximum, exact halves into LDS
        float mx[kMaxB];
#pragma unroll
        for (int b = 0; b < kMaxB; ++b) {
            f32x4_t t = xv[b];
            if constexpr (KIND == 1) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ssq[b] = fmaf(xv[b][e], xv[b][e], ssq[b]);
                    t[e] = xv[b][e] * gv[e];
                }
            } else if constexpr (KIND == 2) {
#pragma unroll
                for (int e = 0; e < 4; ++e) t[e] = act_mul<GELU>(xv[b][e], tv[b][e]);
            }
            xv[b] = t;
            mx[b] = fmaxf(fmaxf(fabsf(t[0]), fabsf(t[1])), fmaxf(fabsf(t[2]), fabsf(t[3])));
        }
        const int shl = step_shift(reduce8_by_lane<true>(mx));  // batch row lane / 8
        int sh[kMaxB];
#pragma unroll
        for (int b = 0; b < kMaxB; ++b) sh[b] = __builtin_amdgcn_readlane(shl, 8 * b);
        uint8_t *obase = reinterpret_cast<uint8_t *>(&opnd[wv][jl][16 * gl]) + 2 * el;
#pragma unroll
        for (int b = 0; b < kMaxB; ++b) {
            const float sc = ldexpf(hscale, sh[b]);
            half2_t h01, h23, l01, l23;
            float v0 = xv[b][0] * sc, v1 = xv[b][1] * sc, v2 = xv[b][2] * sc, v3 = xv[b][3] * sc;
            h01.x = static_cast<_Float16>(v0);
            h01.y = static_cast<_Float16>(v1);
            h23.x = static_cast<_Float16>(v2);
            h23.y = static_cast<_Float16>(v3);
            l01.x = static_cast<_Float16>(v0 - static_cast<float>(h01.x));
            l01.y = static_cast<_Float16>(v1 - static_cast<float>(h01.y));
            l23.x = static_cast<_Float16>(v2 - static_cast<float>(h23.x));
            l23.y = static_cast<_Float16>(v3 - static_cast<float>(h23.y));
            uint2 hv, lv;
            hv.x = __builtin_bit_cast(uint32_t, h01);
            hv.y = __builtin_bit_cast(uint32_t, h23);
            lv.x = __builtin_bit_cast(uint32_t, l01);
            lv.y = __builtin_bit_cast(uint32_t, l23);
            *reinterpret_cast<uint2 *>(obase + 16 * (2 * b)) = hv;      // MFMA row 2b: hi
            *reinterpret_cast<uint2 *>(obase + 16 * (2 * b + 1)) = lv;  // MFMA row 2b + 1: lo
        }
        // the wavefront reads back what its own lanes wrote (LDS operations
        // of one wavefront complete in order)
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
        half8_t af[kSeg];
#pragma unroll
        for (int jj = 0; jj < kSeg; ++jj) af[jj] = __builtin_bit_cast(half8_t, opnd[wv][jj][lane]);
        // 1/s of the two batch rows whose sums this lane accumulates
        int sa = sh[0], sb = sh[1];
#pragma unroll
        for (int q = 1; q < 4; ++q)
            if (g == q) {
                sa = sh[2 * q];
                sb = sh[2 * q + 1];
            }
        const float fa = ldexpf(1.0f, -sa);
        const float fb = ldexpf(1.0f, -sb);

#pragma unroll
        for (int t = 0; t < T; ++t) {
            // block scales of this lane's two blocks, then every lane group's
            const uint32_t dp = __builtin_amdgcn_perm(dw[t][(kDw - 1) / 2], dw[t][0], 0x07060100u);
            uint32_t dps[4];
            {
                auto rr = __builtin_amdgcn_permlane32_swap(dp, dp, false, false);
                auto s01 = __builtin_amdgcn_permlane16_swap(rr[0], rr[0], false, false);
                auto s23 = __builtin_amdgcn_permlane16_swap(rr[1], rr[1], false, false);
                dps[0] = s01[0];
                dps[1] = opaque_copy(s01[1]);
                dps[2] = s23[0];
                dps[3] = opaque_copy(s23[1]);
            }
            half8_t wf[kSeg];
            weight_operands<FMT>(dw[t], wf);
            f32x4_t st = zero;
#pragma unroll
            for (int jj = 0; jj < kSeg; ++jj) {
                const f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[jj], wf[jj], zero, 0, 0, 0);
                const uint32_t scw = dps[jj >> 1];
                if (jj & 1) {
                    st[0] = fma_hi(scw, d[0], st[0]);
                    st[1] = fma_hi(scw, d[1], st[1]);
                    st[2] = fma_hi(scw, d[2], st[2]);
                    st[3] = fma_hi(scw, d[3], st[3]);
                } else {
                    st[0] = fma_lo(scw, d[0], st[0]);
                    st[1] = fma_lo(scw, d[1], st[1]);
                    st[2] = fma_lo(scw, d[2], st[2]);
                    st[3] = fma_lo(scw, d[3], st[3]);
                }
            }
            // result rows 4g..4g+3 are (batch 2g: hi, lo), (batch 2g+1: hi, lo)
            acc[t][0] = fmaf(fa, st[0], acc[t][0]);
            acc[t][1] = fmaf(fa, st[1], acc[t][1]);
            acc[t][2] = fmaf(fb, st[2], acc[t][2]);
            acc[t][3] = fmaf(fb, st[3], acc[t][3]);
        }
        __builtin_amdgcn_wave_barrier();  // operand reads done before the next round's writes
    }

    // ---- the four wavefronts' partial tiles meet in LDS; wavefront w < T
    // adds tile w's partials in wavefront order
#pragma unroll
    for (int t = 0; t < T; ++t) red[wv][t][lane] = acc[t];
    if constexpr (KIND == 1) {
        // sums of squares of this workgroup's K range per batch row
        const float t = reduce8_by_lane<false>(ssq);
        if ((lane & 7) == 0) ssq_w[wv][lane >> 3] = t;
    }
    __syncthreads();
    const int tw = wv < T ? wv : T - 1;  // this wavefront's tile (wavefronts >= T have none)
    f32x4_t tot = red[0][tw][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
        const f32x4_t p4 = red[w][tw][lane];
        tot[0] += p4[0];
        tot[1] += p4[1];
        tot[2] += p4[2];
        tot[3] += p4[3];
    }
    bool rvalid;
    const int n = tile_row(tw, rvalid);
    rvalid = rvalid && wv < T;
    const int pl = tile_pair(tw);                     // pair within the workgroup (SwiGLU output)
    const int pu = rx * kPairs + pl;
    const float ya = tot[0] + tot[1];
    const float yb = tot[2] + tot[3];
    const FinishArgs fa_{N, K, B, S, glu, rx, eps, y, res, counters, ssq_part, part};
    finish<KIND, T, GELU>(fa_, ya, yb, n, rvalid, pl, pu, ssq_w);
}

// ------------------------------------------ K-stationary streaming kernel
// A workgroup of WV wavefronts owns a K range of WV steps (one per
// wavefront) and a run of up to TMAX row tiles of 16 rows.  Each wavefront
// converts its step's activations into exact halves once, keeps them in
// registers for the whole kernel, and streams the row tiles' weights past
// them (PF tiles in flight), writing each tile's partial sums to LDS.  At the
// end the wavefronts' partials are added in wavefront order.  When the
// workgroup covers the whole K (S = 1) it writes y itself; otherwise it
// stores its K range's partials and mv_splitk_reduce_kernel, launched next,
// adds the S ranges in order (no tickets or device-scope synchronisation: on
// this part those cost three memory round trips at the end of every row
// range).  With a SwiGLU output the first half of the workgroup's tiles are
// gate tiles and the second half the matching up tiles.
template <int FMT, int KIND, int TMAX, bool GELU, int WV>
__global__ __launch_bounds__(64 * WV) __attribute__((amdgpu_waves_per_eu(3))) void mv_mfma_kstat_kernel(
    const uint8_t *__restrict__ W, int N, int K, int B, const float *__restrict__ x,
    const float *__restrict__ u, const float *__restrict__ nw, int64_t ld, float eps, float *y,
    const float *res, int *__restrict__ counters, float *__restrict__ ssq_part,
    float *__restrict__ part, int S, int tpw, int glu, int rg, int NG) {
    constexpr int kBytes = BF<FMT>::kBytes;
    constexpr int kDw = BF<FMT>::kLaneDw;
#ifndef Q4_KS_PF
#define Q4_KS_PF 3
#endif
    constexpr int PF = FMT == 1 ? 2 : Q4_KS_PF;  // row tiles in flight ahead of the one multiplied
    // operand transposition (per wavefront, at the start) and the partials of
    // every tile (at the end) share one LDS region; a barrier separates them
    constexpr size_t kOpndBytes = sizeof(u32x4_t) * WV * kSeg * 64;
    constexpr size_t kRedBytes = sizeof(float2) * WV * TMAX * 64;
    __shared__ __attribute__((aligned(16))) uint8_t smem[kOpndBytes > kRedBytes ? kOpndBytes : kRedBytes];
    auto opnd = reinterpret_cast<u32x4_t(*)[kSeg][64]>(smem);
    auto red = reinterpret_cast<float2(*)[TMAX][64]>(smem);
    __shared__ float ssq_w[WV][kMaxB];
    __shared__ float inv_s[kMaxB];
    const GroupView gv_ = group_view(rg, NG, B);
    if (!gv_.live) return;  // padding of the last octet (workgroup-uniform)
    const int rx = gv_.rx;
    {
        const int64_t g8 = static_cast<int64_t>(kMaxB) * gv_.gi;
        const int64_t outw = glu ? (N >> 1) : N;
        x += g8 * ld;
        if (u) u += g8 * ld;
        y += g8 * outw;
        if (res) res += g8 * N;
        part += static_cast<int64_t>(gv_.gi) * S * kMaxB * N;
        ssq_part += static_cast<int64_t>(gv_.gi) * S * kMaxB;
        B = gv_.Bg;
    }
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, g = lane >> 4;
    const int nb = K / 32, kc = nb / kSeg;
    const int c = blockIdx.y * WV + wv;  // this wavefront's step
    const bool active = c < kc;         // wave-uniform
    const int P = N >> 1;
    // tiles of this workgroup: t < nt; row of tile t for this lane
    const int half = tpw >> 1;
    const int units = glu ? (P + 15) / 16 : (N + 15) / 16;  // gate tiles (SwiGLU output) or tiles
    const int per = glu ? half : tpw;
    const int u0 = rx * per;
    const int nu = max(0, min(per, units - u0));
    const int nt = glu ? 2 * nu : nu;
    auto tile_row = [&](int t, bool &valid) {
        if (glu) {
            const int pr = 16 * (u0 + (t < half ? t : t - half)) + col;
            valid = pr < P;
            return t < half ? pr : P + pr;
        }
        const int r = 16 * (u0 + t) + col;
        valid = r < N;
        return r;
    };
    auto tile_of = [&](int t) { return glu ? (t < nu ? t : t - nu + half) : t; };  // slot of the t-th live tile
    const int64_t seg = kSeg * kBytes;
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};

    // ---- loads first: this wavefront's step of the activations, then the
    // first PF row tiles.  Loads return in order, so the conversion below
    // waits for the activations only, while the weights are on their way.  A
    // wavefront past the last step skips the stream and adds zeros; in
    // workgroups of 8 or 12 wavefronts it skips the conversion too.  (The
    // branch around the conversion costs about 26 VGPRs: with 4 wavefronts
    // that measured slower than converting the last step again, and with 16,
    // at most 128 VGPRs, it spills.)
    const int cs = min(c, kc - 1);
    constexpr int NBUF = PF + 1;
    const uint8_t *wbase = W + g * 2 * kBytes + static_cast<int64_t>(cs) * seg;
    const int ntc = max(nt, 1);
    auto fetch = [&](int i, uint32_t (&dst)[kDw]) {  // i-th live tile, clamped to the last
        bool v;
        const int r = tile_row(tile_of(min(i, ntc - 1)), v);
        load_seg<kDw>(wbase + static_cast<int64_t>(v ? r : N - 1) * nb * kBytes, dst);
    };
    // ring of NBUF tiles: tile i lives in ring[i % NBUF]; every load is
    // unconditional (clamped), so the outstanding-load count stays exact
    uint32_t ring[NBUF][kDw];

    // ---- this wavefront's step: activations -> exact halves (MFMA operand order)
    half8_t af[kSeg];
    float fa = 0.f, fb = 0.f;
    float sqa = 0.f;  // RMSNorm: lane l holds batch row l / 8's sum of squares over the step
    constexpr bool kSkipIdleConversion = WV == 8 || WV == 12;
    if (!kSkipIdleConversion || active) {
        const int jl = lane >> 3, q8 = lane & 7;
        const int gl = FMT == 0 ? (q8 & 3) : (q8 >> 1);
        const int el = FMT == 0 ? (q8 >= 4 ? 4 : 0) : 4 * (q8 & 1);
        const float hscale = (FMT == 0 && q8 >= 4) ? 0.0625f : 1.0f;
        const int64_t kx = static_cast<int64_t>(cs) * (32 * kSeg) + 4 * lane;
        f32x4_t xv[kMaxB], tv[kMaxB];
        f32x4_t gvv = {1.f, 1.f, 1.f, 1.f};
        if constexpr (KIND == 1) {
            if (nw) gvv = *reinterpret_cast<const f32x4_al16_t *>(nw + kx);
        }
#pragma unroll
        for (int b = 0; b < kMaxB; ++b) {
            const int64_t bo = static_cast<int64_t>(min(b, B - 1)) * ld + kx;
            xv[b] = *reinterpret_cast<const f32x4_al16_t *>(x + bo);
            if constexpr (KIND == 2) tv[b] = *reinterpret_cast<const f32x4_al16_t *>(u + bo);
        }
#pragma unroll
        for (int p = 0; p < PF; ++p) fetch(p, ring[p]);
        float ssq[kMaxB], mx[kMaxB];
        // rows past B repeat row B - 1: their sums are computed and never stored
#pragma unroll
        for (int b = 0; b < kMaxB; ++b) {
            f32x4_t t = xv[b];
            ssq[b] = 0.f;
            if constexpr (KIND == 1) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ssq[b] = fmaf(xv[b][e], xv[b][e], ssq[b]);
                    t[e] = xv[b][e] * gvv[e];
                }
            } else if constexpr (KIND == 2) {
#pragma unroll
                for (int e = 0; e < 4; ++e) t[e] = act_mul<GELU>(xv[b][e], tv[b][e]);
            }
            xv[b] = t;
            mx[b] = fmaxf(fmaxf(fabsf(t[0]), fabsf(t[1])), fmaxf(fabsf(t[2]), fabsf(t[3])));
        }
        const int shl = step_shift(reduce8_by_lane<true>(mx));  // batch row lane / 8
        int sh[kMaxB];
#pragma unroll
        for (int b = 0; b < kMaxB; ++b) sh[b] = __builtin_amdgcn_readlane(shl, 8 * b);
        uint8_t *obase = reinterpret_cast<uint8_t *>(&opnd[wv][jl][16 * gl]) + 2 * el;
#pragma unroll
        for (int b = 0; b < kMaxB; ++b) {
            const float sc = ldexpf(hscale, sh[b]);
            half2_t h01, h23, l01, l23;
            const float v0 = xv[b][0] * sc, v1 = xv[b][1] * sc, v2 = xv[b][2] * sc, v3 = xv[b][3] * sc;
            h01.x = static_cast<_Float16>(v0);
            h01.y = static_cast<_Float16>(v1);
            h23.x = static_cast<_Float16>(v2);
            h23.y = static_cast<_Float16>(v3);
            l01.x = static_cast<_Float16>(v0 - static_cast<float>(h01.x));
            l01.y = static_cast<_Float16>(v1 - static_cast<float>(h01.y));
            l23.x = static_cast<_Float16>(v2 - static_cast<float>(h23.x));
            l23.y = static_cast<_Float16>(v3 - static_cast<float>(h23.y));
            uint2 hv, lv;
            hv.x = __builtin_bit_cast(uint32_t, h01);
            hv.y = __builtin_bit_cast(uint32_t, h23);
            lv.x = __builtin_bit_cast(uint32_t, l01);
            lv.y = __builtin_bit_cast(uint32_t, l23);
            *reinterpret_cast<uint2 *>(obase + 16 * (2 * b)) = hv;      // MFMA row 2b: hi
            *reinterpret_cast<uint2 *>(obase + 16 * (2 * b + 1)) = lv;  // MFMA row 2b + 1: lo
        }
        if constexpr (KIND == 1) sqa = reduce8_by_lane<false>(ssq);  // batch row lane / 8
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wavefront reads back its own writes
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int jj = 0; jj < kSeg; ++jj) af[jj] = __builtin_bit_cast(half8_t, opnd[wv][jj][lane]);
        int sa = sh[0], sb = sh[1];
#pragma unroll
        for (int q = 1; q < 4; ++q)
            if (g == q) {
                sa = sh[2 * q];
                sb = sh[2 * q + 1];
            }
        fa = ldexpf(1.0f, -sa);
        fb = ldexpf(1.0f, -sb);
    }
    __syncthreads();  // every wavefront holds its operands: the LDS region is free

    // ---- stream the row tiles past the step's operands; each tile's partial
    // sums go to its LDS slot at once (live tile i -> slot tile_of(i): gate
    // tiles first, up tiles from slot tpw / 2; only live slots are read back)
    // A wavefront past the last step writes zeros to its slots.
    if (nt > 0 && !active) {
        for (int i = 0; i < nt; ++i) red[wv][tile_of(i)][lane] = make_float2(0.f, 0.f);
    } else if (nt > 0) {  // workgroup-uniform
        auto process = [&](int i, const uint32_t (&cur)[kDw]) {
            const uint32_t dp = __builtin_amdgcn_perm(cur[(kDw - 1) / 2], cur[0], 0x07060100u);
            uint32_t dps[4];
            {
                auto rr = __builtin_amdgcn_permlane32_swap(dp, dp, false, false);
                auto s01 = __builtin_amdgcn_permlane16_swap(rr[0], rr[0], false, false);
                auto s23 = __builtin_amdgcn_permlane16_swap(rr[1], rr[1], false, false);
                dps[0] = s01[0];
                dps[1] = opaque_copy(s01[1]);
                dps[2] = s23[0];
                dps[3] = opaque_copy(s23[1]);
            }
            half8_t wf[kSeg];
            weight_operands<FMT>(cur, wf);
            f32x4_t st = zero;
#pragma unroll
            for (int jj = 0; jj < kSeg; ++jj) {
                const f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[jj], wf[jj], zero, 0, 0, 0);
                const uint32_t scw = dps[jj >> 1];
                if (jj & 1) {
                    st[0] = fma_hi(scw, d[0], st[0]);
                    st[1] = fma_hi(scw, d[1], st[1]);
                    st[2] = fma_hi(scw, d[2], st[2]);
                    st[3] = fma_hi(scw, d[3], st[3]);
                } else {
                    st[0] = fma_lo(scw, d[0], st[0]);
                    st[1] = fma_lo(scw, d[1], st[1]);
                    st[2] = fma_lo(scw, d[2], st[2]);
                    st[3] = fma_lo(scw, d[3], st[3]);
                }
            }
            // result rows 4g..4g+3 are (batch 2g: hi, lo), (batch 2g+1: hi, lo)
            red[wv][tile_of(i)][lane] = make_float2(fa * (st[0] + st[1]), fb * (st[2] + st[3]));
        };
        int i0 = 0;
        for (; i0 + NBUF <= nt; i0 += NBUF) {
#pragma unroll
            for (int q = 0; q < NBUF; ++q) {
                fetch(i0 + q + PF, ring[(q + PF) % NBUF]);
                process(i0 + q, ring[q]);
            }
        }
#pragma unroll
        for (int q = 0; q < NBUF; ++q)
            if (i0 + q < nt) process(i0 + q, ring[q]);
    }

    if constexpr (KIND == 1) {
        if ((lane & 7) == 0) ssq_w[wv][lane >> 3] = active ? sqa : 0.f;
    }
    __syncthreads();
    // outputs of the workgroup: (live tile i, batch row b, row col) -> thread o
    // (tid + 256 k); with a SwiGLU output only the gate tiles are walked and
    // each output also reads its up tile
    constexpr int kNT = 64 * WV;
    constexpr int kOut = (TMAX * 16 * kMaxB + kNT - 1) / kNT;  // outputs per thread at most
    const int nout = (glu ? nu : nt) * 16 * kMaxB;
    float vg[kOut], vu[kOut];
#pragma unroll
    for (int k = 0; k < kOut; ++k) {
        const int o = threadIdx.x + kNT * k;
        vg[k] = vu[k] = 0.f;
        if (o < nout) {
            const int i = o / (16 * kMaxB), b = (o / 16) % kMaxB, r = o % 16;
            const int ln = r + 16 * (b >> 1);
            const int sg = tile_of(i), su = glu ? tile_of(i + nu) : 0;
            float a = 0.f, a2 = 0.f;
#pragma unroll
            for (int w = 0; w < WV; ++w) {
                const float2 q = red[w][sg][ln];
                a += (b & 1) ? q.y : q.x;
                if (glu) {
                    const float2 q2 = red[w][su][ln];
                    a2 += (b & 1) ? q2.y : q2.x;
                }
            }
            vg[k] = a;
            vu[k] = a2;
        }
    }
    auto out_index = [&](int o, int &b, int &n, bool &ok) {
        const int i = o / (16 * kMaxB), r = o % 16;
        b = (o / 16) % kMaxB;
        n = 16 * (u0 + i) + r;  // row (or pair) index of the gate / plain tile
        ok = o < nout && b < B && n < (glu ? P : N);
    };
    const int64_t ln = N;
    if (S == 1) {
        if constexpr (KIND == 1) {
            if (threadIdx.x < kMaxB) {
                const int b = threadIdx.x;
                float tot = 0.f;
                for (int w = 0; w < WV; ++w) tot += ssq_w[w][b];
                inv_s[b] = 1.0f / sqrtf(tot / static_cast<float>(K) + eps);
            }
            __syncthreads();
        }
#pragma unroll
        for (int k = 0; k < kOut; ++k) {
            int b, n;
            bool ok;
            out_index(threadIdx.x + kNT * k, b, n, ok);
            if (!ok) continue;
            const float inv = KIND == 1 ? inv_s[b] : 1.f;
            if (glu) y[b * static_cast<int64_t>(P) + n] = act_mul<GELU>(vg[k] * inv, vu[k] * inv);
            else y[b * ln + n] = res ? vg[k] * inv + res[b * ln + n] : vg[k] * inv;
        }
        return;
    }
    // K split over S workgroups: plain stores of this K range's partials (and,
    // once per K range, its sums of squares); mv_splitk_reduce_kernel, the
    // next launch, adds the S partials in split order.
    {
        float *pp = part + static_cast<int64_t>(blockIdx.y) * B * ln;
#pragma unroll
        for (int k = 0; k < kOut; ++k) {
            int b, n;
            bool ok;
            out_index(threadIdx.x + kNT * k, b, n, ok);
            if (!ok) continue;
            pp[b * ln + n] = vg[k];
            if (glu) pp[b * ln + P + n] = vu[k];
        }
    }
    if constexpr (KIND == 1) {
        if (rx == 0 && threadIdx.x < B) {
            const int b = threadIdx.x;
            float tot = 0.f;
            for (int w = 0; w < WV; ++w) tot += ssq_w[w][b];
            ssq_part[static_cast<int64_t>(blockIdx.y) * kMaxB + b] = tot;
        }
    }
}

// Adds the S partials of a K-split launch in split order and applies the
// epilogue: 1/rms (sums of squares of the S K ranges), residual, or the
// SwiGLU / GeGLU of the gate and up sums.  One thread per output.
template <int KIND, bool GELU>
__global__ __launch_bounds__(kWG) void mv_splitk_reduce_kernel(int N, int K, int B, int S, int glu,
                                                              float eps, const float *__restrict__ part,
                                                              const float *__restrict__ ssq_part,
                                                              float *y, const float *res) {
    const int P = N >> 1;
    const int outw = glu ? P : N;
    const int64_t o = static_cast<int64_t>(blockIdx.x) * kWG + threadIdx.x;
    if (o >= static_cast<int64_t>(B) * outw) return;
    const int b = static_cast<int>(o / outw), n = static_cast<int>(o % outw);
    const int gi = b / kMaxB, bl = b % kMaxB;
    const int Bg = min(kMaxB, B - kMaxB * gi);
    const int64_t ln = N;
    const float *pg = part + static_cast<int64_t>(gi) * S * kMaxB * ln + bl * ln + n;
    const int64_t step = static_cast<int64_t>(Bg) * ln;
    float inv = 1.f;
    if constexpr (KIND == 1) {
        const float *sq = ssq_part + static_cast<int64_t>(gi) * S * kMaxB + bl;
        float tot = 0.f;
        for (int q = 0; q < S; ++q) tot += sq[q * kMaxB];
        inv = 1.0f / sqrtf(tot / static_cast<float>(K) + eps);
    }
    float sg = 0.f, su = 0.f;
    for (int q = 0; q < S; ++q) {
        sg += pg[q * step];
        if (glu) su += pg[q * step + P];
    }
    if (glu) y[static_cast<int64_t>(b) * P + n] = act_mul<GELU>(sg * inv, su * inv);
    else y[b * ln + n] = res ? sg * inv + res[b * ln + n] : sg * inv;
}

// ---------------------------------------------------------------- host side
struct Plan {
    bool tiles;  // the tile kernel, else the shared-step kernel
    bool kstat;  // the K-stationary streaming kernel (T = row tiles per workgroup)
    int wv;      // its wavefronts per workgroup
    int T, rg, kc, S, spw;
    int NG, gx;  // batch groups; grid width (row ranges, padded to octets when NG > 1)
    size_t off_ssq, off_part, bytes;
};

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

#ifndef Q4_MFMA_KSTAT
#define Q4_MFMA_KSTAT 1  // 0: the tile / shared-step kernels only
#endif
#ifndef Q4_KS_WHOLE_MAX
#define Q4_KS_WHOLE_MAX 16  // longest K (in steps) one K-stationary workgroup covers whole
#endif
#ifndef Q4_KS_MIN_UNITS
#define Q4_KS_MIN_UNITS 512  // fewest row tiles for the K-split K-stationary kernel
#endif
constexpr int kKsTmaxQ4 = 12;  // row tiles per workgroup of the K-stationary kernel
#ifndef Q4_KS_TARGET_WGS
#define Q4_KS_TARGET_WGS 768
#endif
constexpr int kKsTargetWGs = Q4_KS_TARGET_WGS;

// The K-stationary kernel where it measured faster (see the plan below);
// otherwise the tile kernel (each wavefront converts its own step's
// activations and feeds four row tiles, two for Q8_0) when it yields kMinWGs
// workgroups, else the shared-step kernel (64 rows per workgroup, the four
// wavefronts share one step's operands), whose finer K split fills the chip
// on small matrices.  K is split over at most kMaxS workgroups, and not at
// all when the row ranges outnumber the tickets.
Plan make_plan(int64_t N, int64_t K, int64_t B, int fmt, bool glu = false) {
    Plan p;
    p.NG = static_cast<int>((B + kMaxB - 1) / kMaxB);
    p.kc = static_cast<int>(K / (32 * kSeg));
    const int rounds = (p.kc + 3) / 4;
    // K-stationary kernel, where it measured faster than the tile kernels
    // (Q4_0 only; 5376 x 21504 and the Qwen3-4B projections at B = 8):
    //  * K of at most 16 steps: one workgroup of WV = 4 ceil(steps / 4)
    //    wavefronts covers the whole K (no split), when that still gives
    //    at least 128 workgroups; with 16 wavefronts (1,024 threads, one
    //    workgroup per CU) only for 144..384 of them and B <= 16: with 128
    //    (a gated output of 4,096 rows) and at B = 32 the other kernels
    //    measured faster;
    //  * longer K: workgroups of 4 wavefronts over K ranges of 4 steps, the
    //    ranges' partials added in order by a second launch, for matrices of
    //    at least 512 row tiles.
    // Elsewhere (few rows, Q8_0 tables) the tile / shared-step kernels below.
    auto kstat_plan = [&](int wv) {
        p.wv = wv;
        p.S = (p.kc + wv - 1) / wv;
        p.spw = 1;
        p.tiles = true;
        const int tmax = kKsTmaxQ4;
        const int64_t units = glu ? (N / 2 + 15) / 16 : (N + 15) / 16;
        const int permax = glu ? tmax / 2 : tmax;
        const int64_t target = std::max<int64_t>(64, static_cast<int64_t>(kKsTargetWGs) * 4 / wv);
        int per = static_cast<int>((units * p.S * p.NG + target - 1) / target);
        per = std::max(1, std::min(per, permax));
        p.rg = static_cast<int>((units + per - 1) / per);
        p.T = glu ? 2 * per : per;
        return units;
    };
    p.kstat = false;
    if (Q4_MFMA_KSTAT && fmt == 0) {
        if (p.kc <= Q4_KS_WHOLE_MAX) {
            kstat_plan((p.kc + 3) / 4 * 4);
            const int64_t wgs = static_cast<int64_t>(p.rg) * p.NG;
            p.kstat = p.wv <= 12 ? wgs >= 128 : (wgs >= 144 && wgs <= 384 && p.NG <= 2);
        }
        if (!p.kstat && p.kc > 12 && p.kc <= 4 * kMaxS) p.kstat = kstat_plan(4) >= Q4_KS_MIN_UNITS;
    }
    if (!p.kstat) {
        p.tiles = true;
        p.T = fmt == 1 ? 2 : 4;
        p.rg = static_cast<int>((N + 16 * p.T - 1) / (16 * p.T));
        p.spw = static_cast<int64_t>(p.rg) * p.NG > kCounters ? rounds : (rounds + kMaxS - 1) / kMaxS;
        p.S = (rounds + p.spw - 1) / p.spw;
        if (static_cast<int64_t>(p.rg) * p.S * p.NG < kMinWGs) {
            p.tiles = false;
            p.T = 4;
            p.rg = static_cast<int>((N + 63) / 64);
            const int wgs = (kTargetWGs + p.NG - 1) / p.NG;
            int want = std::max(1, std::min(std::min(p.kc, kMaxS), (wgs + p.rg - 1) / p.rg));
            if (static_cast<int64_t>(p.rg) * p.NG > kCounters) want = 1;
            p.spw = (p.kc + want - 1) / want;
            p.S = (p.kc + p.spw - 1) / p.spw;
        }
    }
#ifndef Q4_MFMA_XCD_PAD
#define Q4_MFMA_XCD_PAD 1
#endif
    // Workgroups go to the 8 XCDs in turn (linear id mod 8).  With a grid
    // width that is a multiple of 8, the K splits of a row range (same x,
    // different y) run on one XCD and share its L2 for the cache lines their
    // K ranges have in common; the padding workgroups exit at once.
    p.gx = p.NG == 1 ? ((Q4_MFMA_XCD_PAD && p.S > 1) ? (p.rg + 7) / 8 * 8 : p.rg) : (p.rg + 7) / 8 * 8 * p.NG;
    // per group: S partial rows of its (up to 8) activation rows, and the
    // sums of squares of each row range and split
    const int64_t gB = p.NG == 1 ? B : kMaxB;
    p.off_ssq = kCounterBytes;
    const size_t ssq =
        p.S > 1 ? align256(static_cast<size_t>(p.NG) * p.rg * p.S * kMaxB * sizeof(float)) : 0;
    p.off_part = p.off_ssq + ssq;
    p.bytes = p.off_part +
              (p.S > 1 ? align256(static_cast<size_t>(p.NG) * p.S * gB * N * sizeof(float)) : 0);
    return p;
}

template <int FMT, int KIND, bool GELU>
void launch_act(const uint8_t *W, int N, int K, int B, const float *x, const float *u, const float *nw,
                int64_t ld, float eps, float *y, const float *res, void *ws, const Plan &p, int glu,
                hipStream_t s) {
    // (no workspace when K is not split: the kernels touch it only for S > 1)
    uint8_t *w8 = static_cast<uint8_t *>(ws);
    int *ctr = w8 ? reinterpret_cast<int *>(w8) : nullptr;
    float *ssq = w8 ? reinterpret_cast<float *>(w8 + p.off_ssq) : nullptr;
    float *part = w8 ? reinterpret_cast<float *>(w8 + p.off_part) : nullptr;
    const dim3 grid(p.gx, p.S);
    if constexpr (FMT == 0) {  // (the plan takes it for Q4_0 only)
    if (p.kstat) {
        constexpr int TM = kKsTmaxQ4;
        switch (p.wv) {
#define Q4_KS_CASE(WVN)                                                                                        \
    case WVN:                                                                                                  \
        hipLaunchKernelGGL((mv_mfma_kstat_kernel<FMT, KIND, TM, GELU, WVN>), grid, dim3(64 * WVN), 0, s, W, N, K, \
                           B, x, u, nw, ld, eps, y, res, ctr, ssq, part, p.S, p.T, glu, p.rg, p.NG);            \
        break;
            Q4_KS_CASE(4)
            Q4_KS_CASE(8)
            Q4_KS_CASE(12)
            Q4_KS_CASE(16)
#undef Q4_KS_CASE
        }
        if (p.S > 1) {
            const int64_t outs = static_cast<int64_t>(B) * (glu ? N / 2 : N);
            hipLaunchKernelGGL((mv_splitk_reduce_kernel<KIND, GELU>), dim3(static_cast<unsigned>((outs + kWG - 1) / kWG)),
                               dim3(kWG), 0, s, N, K, B, p.S, glu, eps, part, ssq, y, res);
        }
        return;
    }
    }
    if (!p.tiles) {
        hipLaunchKernelGGL((mv_mfma_step_kernel<FMT, KIND, GELU>), grid, dim3(kWG), 0, s, W, N, K, B, x, u,
                           nw, ld, eps, y, res, ctr, ssq, part, p.S, p.spw, glu, p.rg, p.NG);
        return;
    }
    constexpr int T = FMT == 1 ? 2 : 4;
    hipLaunchKernelGGL((mv_mfma_tile_kernel<FMT, KIND, T, GELU>), grid, dim3(kWG), 0, s, W, N, K, B, x, u,
                       nw, ld, eps, y, res, ctr, ssq, part, p.S, p.spw, glu, p.rg, p.NG);
}

// GeGLU kernels exist for Q4_0 only (the gated projections).
template <int FMT, int KIND>
void launch(const uint8_t *W, int N, int K, int B, const float *x, const float *u, const float *nw,
            int64_t ld, float eps, float *y, const float *res, void *ws, const Plan &p, int glu, bool gelu,
            hipStream_t s) {
    if constexpr (FMT == 0) {
        if (gelu) {
            launch_act<FMT, KIND, true>(W, N, K, B, x, u, nw, ld, eps, y, res, ws, p, glu, s);
            return;
        }
    }
    launch_act<FMT, KIND, false>(W, N, K, B, x, u, nw, ld, eps, y, res, ws, p, glu, s);
}

bool overlaps(const void *a, size_t an, const void *b, size_t bn) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + bn && y < x + an;
}

constexpr size_t kStaticScratchBytes = Q4_NOALLOC_SCRATCH_BYTES;  // allocation-free variant's scratch
q4_status static_scratch(hipStream_t s, void **out);

// use_static: the allocation-free variant; ws / ws_bytes are ignored and the
// per-device static scratch is used once every argument has been checked.
template <int FMT>
q4_status batched_entry(const char *name, const void *Wv, int64_t N, int64_t K, const float *x,
                        const float *x2, int64_t ldx, int64_t B, int op_kind, int out_op,
                        const float *norm_w, float eps, float *y, const float *res, void *ws,
                        size_t ws_bytes, void *stream, bool use_static = false) {
    q4::clear_error();
    Q4_CHECK(out_op == Q4_OUT_PLAIN || out_op == Q4_OUT_SWIGLU || out_op == Q4_OUT_GEGLU,
             Q4_ERR_INVALID_ARG, "%s: unknown output transform %d", name, out_op);
    Q4_CHECK(out_op == Q4_OUT_PLAIN || (N % 2 == 0 && !res), Q4_ERR_INVALID_ARG,
             "%s: a gated (SwiGLU / GeGLU) output needs an even N and no residual", name);
    Q4_CHECK(Wv && x && y, Q4_ERR_INVALID_ARG, "%s: W, x and y must not be NULL", name);
    Q4_CHECK(N >= 1 && K >= 1 && B >= 1, Q4_ERR_INVALID_ARG, "%s: N=%lld K=%lld B=%lld must be >= 1",
             name, (long long)N, (long long)K, (long long)B);
    Q4_CHECK(op_kind >= Q4_IN_PLAIN && op_kind <= Q4_IN_GEGLU, Q4_ERR_INVALID_ARG,
             "%s: unknown input transform %d", name, op_kind);
    Q4_CHECK((op_kind != Q4_IN_SWIGLU && op_kind != Q4_IN_GEGLU) || x2, Q4_ERR_INVALID_ARG,
             "%s: a gated input needs x2", name);
    Q4_CHECK(!((op_kind == Q4_IN_SWIGLU || op_kind == Q4_IN_GEGLU) && out_op != Q4_OUT_PLAIN) ||
                 (op_kind == Q4_IN_GEGLU) == (out_op == Q4_OUT_GEGLU),
             Q4_ERR_UNSUPPORTED, "%s: a gated input and a gated output must use the same activation", name);
    Q4_CHECK(FMT == 0 || (op_kind != Q4_IN_GEGLU && out_op != Q4_OUT_GEGLU), Q4_ERR_UNSUPPORTED,
             "%s: GeGLU transforms are provided for Q4_0 weights", name);
    Q4_CHECK(op_kind != Q4_IN_RMSNORM || eps >= 0.f, Q4_ERR_INVALID_ARG, "%s: eps must be >= 0", name);
    Q4_CHECK(ldx >= K, Q4_ERR_SHAPE, "%s: ld_x=%lld < K=%lld", name, (long long)ldx, (long long)K);
    Q4_CHECK(K % 256 == 0, Q4_ERR_UNSUPPORTED, "%s: K=%lld is not a multiple of 256", name,
             (long long)K);
    Q4_CHECK(B <= kMaxBatch, Q4_ERR_UNSUPPORTED, "%s: B=%lld > 32", name, (long long)B);
    Q4_CHECK(N <= (1 << 30) && K <= (1 << 24) && ldx <= (1 << 26), Q4_ERR_UNSUPPORTED,
             "%s: N or K too large", name);
    Q4_CHECK(q4::aligned(Wv, 16), Q4_ERR_ALIGNMENT, "%s: W must be 16-byte aligned", name);
    Q4_CHECK(q4::aligned(x, 16) && (!x2 || q4::aligned(x2, 16)) && ldx % 4 == 0 &&
                 (!norm_w || q4::aligned(norm_w, 16)),
             Q4_ERR_ALIGNMENT, "%s: x, x2 and norm_w must be 16-byte aligned with ld_x a multiple of 4",
             name);
    Q4_CHECK(q4::aligned(y, 4) && (!res || q4::aligned(res, 4)), Q4_ERR_ALIGNMENT,
             "%s: y and residual must be 4-byte aligned", name);
    const size_t xbytes = static_cast<size_t>((B - 1) * ldx + K) * sizeof(float);
    const size_t ybytes = static_cast<size_t>(B * (out_op != Q4_OUT_PLAIN ? N / 2 : N)) * sizeof(float);
    Q4_CHECK(!overlaps(y, ybytes, x, xbytes) && (!x2 || !overlaps(y, ybytes, x2, xbytes)),
             Q4_ERR_INVALID_ARG, "%s: y must not overlap x or x2", name);
    const Plan p = make_plan(N, K, B, FMT, out_op != Q4_OUT_PLAIN);
    hipStream_t s = q4::as_stream(stream);
    if (use_static) {
        Q4_CHECK(p.bytes <= kStaticScratchBytes, Q4_ERR_UNSUPPORTED,
                 "%s: N=%lld K=%lld B=%lld needs %zu bytes of scratch, more than the %zu held per device",
                 name, (long long)N, (long long)K, (long long)B, p.bytes, kStaticScratchBytes);
        q4_status st = static_scratch(s, &ws);
        if (st != Q4_OK) return st;
        ws_bytes = kStaticScratchBytes;
    }
    Q4_CHECK(ws && q4::aligned(ws, 256), Q4_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned",
             name);
    Q4_CHECK(ws_bytes >= p.bytes, Q4_ERR_WORKSPACE, "%s: workspace of %zu bytes < %zu needed", name,
             ws_bytes, p.bytes);
    const uint8_t *W = static_cast<const uint8_t *>(Wv);
    const int n = static_cast<int>(N), k = static_cast<int>(K), b = static_cast<int>(B);
    const int glu = out_op == Q4_OUT_PLAIN ? 0 : 1;
    const bool gelu = op_kind == Q4_IN_GEGLU || out_op == Q4_OUT_GEGLU;
    if (op_kind == Q4_IN_RMSNORM)
        launch<FMT, 1>(W, n, k, b, x, nullptr, norm_w, ldx, eps, y, res, ws, p, glu, gelu, s);
    else if (op_kind == Q4_IN_SWIGLU || op_kind == Q4_IN_GEGLU)
        launch<FMT, 2>(W, n, k, b, x, x2, nullptr, ldx, eps, y, res, ws, p, glu, gelu, s);
    else
        launch<FMT, 0>(W, n, k, b, x, nullptr, nullptr, ldx, eps, y, res, ws, p, glu, gelu, s);
    return q4::launch_status(name);
}

}  // namespace

namespace q4 {

void matvec_mfma_whole_k(int fmt, const void *Wv, int N, int K, const float *x, const float *x2,
                         const float *norm_w, int64_t ldx, int B, int op_kind, int out_op, float eps,
                         float *y, const float *res, hipStream_t s) {
    Plan p{};
    p.NG = 1;
    p.kc = K / (32 * kSeg);
    p.kstat = false;
    p.tiles = true;
    p.wv = 4;
    p.T = fmt == 1 ? 2 : 4;
    p.rg = (N + 16 * p.T - 1) / (16 * p.T);
    p.spw = (p.kc + 3) / 4;  // every round of 4 steps in one workgroup
    p.S = 1;
    p.gx = p.rg;
    const uint8_t *W = static_cast<const uint8_t *>(Wv);
    const int glu = out_op == Q4_OUT_PLAIN ? 0 : 1;
    const bool gelu = op_kind == Q4_IN_GEGLU || out_op == Q4_OUT_GEGLU;
    const bool gated_in = op_kind == Q4_IN_SWIGLU || op_kind == Q4_IN_GEGLU;
    auto go = [&](auto fmt_tag) {
        constexpr int F = decltype(fmt_tag)::value;
        if (op_kind == Q4_IN_RMSNORM)
            launch<F, 1>(W, N, K, B, x, nullptr, norm_w, ldx, eps, y, res, nullptr, p, glu, gelu, s);
        else if (gated_in)
            launch<F, 2>(W, N, K, B, x, x2, nullptr, ldx, eps, y, res, nullptr, p, glu, gelu, s);
        else
            launch<F, 0>(W, N, K, B, x, nullptr, nullptr, ldx, eps, y, res, nullptr, p, glu, gelu, s);
    };
    if (fmt == 0) go(std::integral_constant<int, 0>{});
    else go(std::integral_constant<int, 1>{});
}

}  // namespace q4

extern "C" size_t matvec_batched_workspace(int64_t N, int64_t K, int64_t B) {
    if (N < 1 || K < 256 || K % 256 != 0 || B < 1 || B > kMaxBatch) return 0;
    size_t m = 0;
    for (int fmt = 0; fmt < 2; ++fmt)
        for (int glu = 0; glu < 2; ++glu) m = std::max(m, make_plan(N, K, B, fmt, glu != 0).bytes);
    return m;
}

extern "C" q4_status q4_0_matvec_batched(const void *W, int64_t N, int64_t K, const float *x,
                                         const float *x2, int64_t ld_x, int64_t B,
                                         q4_input_op op, q4_output_op out_op, const float *norm_w,
                                         float eps, float *y, const float *residual, void *ws,
                                         size_t ws_bytes, void *stream) {
    return batched_entry<0>("q4_0_matvec_batched", W, N, K, x, x2, ld_x, B, op, out_op, norm_w,
                            eps, y, residual, ws, ws_bytes, stream);
}

extern "C" q4_status q8_0_matvec_batched(const void *W, int64_t N, int64_t K, const float *x,
                                         const float *x2, int64_t ld_x, int64_t B,
                                         q4_input_op op, q4_output_op out_op, const float *norm_w,
                                         float eps, float *y, const float *residual, void *ws,
                                         size_t ws_bytes, void *stream) {
    return batched_entry<1>("q8_0_matvec_batched", W, N, K, x, x2, ld_x, B, op, out_op, norm_w,
                            eps, y, residual, ws, ws_bytes, stream);
}

// ------------------------------------------------ allocation-free variant
namespace {

// Scratch of q4_0_matvec_batched_noalloc: the split tickets, sums of squares
// and split-K partials live in this array, one copy per device, held until
// the process ends.  In host code its name is only a stand-in; the device
// address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

__global__ void zero_words_kernel(uint32_t *p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// Device address of the current device's scratch.  On the first call on a
// device the tickets are cleared by a fill kernel on `s`, ordered before the
// caller's kernel (a memset node would not be safe inside a captured graph).
q4_status static_scratch(hipStream_t s, void **out) {
    int dev = -1;
    Q4_HIP_CHECK(hipGetDevice(&dev));
    Q4_CHECK(dev >= 0 && dev < kMaxDevices, Q4_ERR_UNSUPPORTED,
             "q4_0_matvec_batched_noalloc: device %d beyond the %d supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        Q4_HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        Q4_CHECK(p && q4::aligned(p, 256), Q4_ERR_HIP,
                 "q4_0_matvec_batched_noalloc: the scratch symbol has no usable device address");
        const int words = static_cast<int>(kCounterBytes / sizeof(uint32_t));
        hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, s,
                           static_cast<uint32_t *>(p), words);
        q4_status st = q4::launch_status("q4_0_matvec_batched_noalloc (scratch clear)");
        if (st != Q4_OK) return st;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return Q4_OK;
}

}  // namespace

extern "C" q4_status q4_0_matvec_batched_noalloc(const void *W, int64_t N, int64_t K,
                                                 const float *x, const float *x2, int64_t ld_x,
                                                 int64_t B, q4_input_op op, q4_output_op out_op,
                                                 const float *norm_w, float eps, float *y,
                                                 const float *residual, void *stream) {
    return batched_entry<0>("q4_0_matvec_batched_noalloc", W, N, K, x, x2, ld_x, B, op, out_op,
                            norm_w, eps, y, residual, nullptr, 0, stream, true);
}
