// Batched Q4_0 / Q8_0 dequant-matvec (1 <= B <= 8 activation rows) on the
// gfx950 matrix cores.
//
// Definition ("Research record" page, "Native Metal diagnostic: buffer
// ownership": 18-byte Q4_0 blocks, weight = (quant - 8) * scale; "Verified
// model facts": the Q8_0 token table):
//   y[b][n] = sum_k d[n][k/32] * c[n][k] * x[b][k]   (+ residual[b][n]),
// c = q - 8 (Q4_0) or the int8 code q (Q8_0).
//
// With eight activation rows every weight feeds eight products, which is more
// than the vector ALUs can keep up with at HBM speed; v_mfma_f32_16x16x32_f16
// takes them instead, one Q4_0 block (32 k) per instruction, so the block
// scale is applied once per 16x16 result tile:
//   D[i][n] = sum_{k in block} X[i][k] * c[n][k] ,  y += d[n][block] * D .
// Operands are exact in binary16: c is an integer of at most 8 bits, and the
// activations are carried as two halves, X = hi + lo with
// hi = fp16(s_b x), lo = fp16(s_b x - hi) (22 significant bits), so the 16
// MFMA rows are 8 batch rows x {hi, lo} and every product is exact.  s_b is a
// power of two per batch row that puts max |s_b x| in [2^12, 2^13): binary16
// can neither overflow nor lose the small elements, and dividing by s_b at
// the end is exact.
//
// Two launches:
//  * prep (one workgroup per batch slot): applies the input transform (plain,
//    RMSNorm, SwiGLU), finds s_b and writes the activations in MFMA operand
//    order, XF[block][lane] = 8 halves; it also clears the split counters.
//  * main: a wavefront owns 16 output rows and walks K in steps of 8 blocks.
//    Lane (n, g) = (lane % 16, lane / 16) loads 2 consecutive blocks of row n
//    (36 or 68 contiguous bytes, 4-byte aligned); permlane16/32 swaps
//    transpose the 4 x 4 lane groups so that for every block lane group g
//    holds its part of the codes (Q4_0: payload bytes 4g..4g+3, i.e. elements
//    4g..4g+3 in low nibbles and 4g+16..4g+19 in high nibbles, the high ones
//    kept x16 and paired with activations / 16; Q8_0: payload bytes
//    8g..8g+7).  Codes become halves with one mask-or (1024 + q) and one
//    packed subtract.  K is split over S workgroups when the row count alone
//    cannot fill the chip; their partial sums are added in a fixed order by
//    whichever workgroup finishes last, so results are bitwise reproducible.
#include "common.hpp"

namespace {
using namespace q4dev;

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_al4_t __attribute__((ext_vector_type(4), aligned(4)));
typedef float f32x4_al16_t __attribute__((ext_vector_type(4), aligned(16)));

constexpr int kWG = 256;          // 4 wavefronts
constexpr int kRowsWG = 64;       // 16 rows per wavefront
constexpr int kSeg = 8;           // blocks per wavefront step (one MFMA each)
constexpr int kTargetWGs = 1024;  // about 4 workgroups per compute unit
constexpr int kPrepThreads = 256;  // one workgroup converts 64 blocks of one row
constexpr int kMaxB = 8;

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

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Offset of element e (0..7) of lane group g inside a block, and its
// activation factor (high Q4_0 nibbles are kept x16 in the weight operand).
template <int FMT>
__device__ __forceinline__ int elem_of(int g, int e) {
    if constexpr (FMT == 0) return e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4);
    else return 8 * g + e;
}

// ---------------------------------------------------------------- prep kernel
template <int FMT, int KIND>
__global__ __launch_bounds__(kPrepThreads) void mfma_prep_kernel(
    const float *__restrict__ x, const float *__restrict__ u, const float *__restrict__ nw,
    float eps, int64_t ld, int K, int B, u32x4_t *__restrict__ xf, float *__restrict__ sinv,
    int *__restrict__ counters, int n_counters) {
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int nb = K / 32;
    if (b == 0 && blockIdx.y == 0)
        for (int i = tid; i < n_counters; i += kPrepThreads) counters[i] = 0;
    const bool live = b < B;
    float s = 0.f, inv = 1.f;
    if (live) {
        const float *xr = x + static_cast<int64_t>(b) * ld;
        const float *ur = KIND == 2 ? u + static_cast<int64_t>(b) * ld : nullptr;
        float ss = 0.f, mx = 0.f;
        for (int k = tid; k < K; k += kPrepThreads) {
            float v = xr[k];
            if constexpr (KIND == 1) {
                ss = fmaf(v, v, ss);
                v = v * (nw ? nw[k] : 1.0f);
            } else if constexpr (KIND == 2) {
                v = silu_mul(v, ur[k]);
            }
            mx = fmaxf(mx, fabsf(v));
        }
        __shared__ float red_s[kPrepThreads / 64], red_m[kPrepThreads / 64];
        const float ws = wave_sum(ss), wm = wave_max(mx);
        if ((tid & 63) == 0) {
            red_s[tid >> 6] = ws;
            red_m[tid >> 6] = wm;
        }
        __syncthreads();
        float tss = 0.f, tmx = 0.f;
        for (int w = 0; w < kPrepThreads / 64; ++w) {
            tss += red_s[w];
            tmx = fmaxf(tmx, red_m[w]);
        }
        if constexpr (KIND == 1) {
            inv = 1.0f / sqrtf(tss / static_cast<float>(K) + eps);
            tmx = tmx * inv;
        }
        int e = 0;
        if (tmx > 0.f && tmx <= 3.4e38f) (void)frexpf(tmx, &e);
        const int sh = min(max(13 - e, -120), 120);
        s = (tmx <= 3.4e38f) ? ldexpf(1.0f, sh) : 1.0f;  // inf / nan rows keep scale 1
        if (tid == 0 && blockIdx.y == 0) sinv[b] = (tmx <= 3.4e38f) ? ldexpf(1.0f, -sh) : 1.0f;
    } else if (tid == 0 && blockIdx.y == 0) {
        sinv[b] = 0.f;
    }
    const float *xr = x + static_cast<int64_t>(live ? b : 0) * ld;
    const float *ur = KIND == 2 ? u + static_cast<int64_t>(live ? b : 0) * ld : nullptr;
    const int it = blockIdx.y * kPrepThreads + tid;  // (block, lane group) item
    if (it < nb * 4) {
        const int j = it >> 2, g = it & 3;
        half8_t hi, lo;
        if (live) {
            // Two runs of 4 contiguous elements (x and u are 16-byte aligned).
            const int k0 = 32 * j + elem_of<FMT>(g, 0);
            const int k1 = 32 * j + elem_of<FMT>(g, 4);
            float v[8];
            const f32x4_al16_t a0 = *reinterpret_cast<const f32x4_al16_t *>(xr + k0);
            const f32x4_al16_t a1 = *reinterpret_cast<const f32x4_al16_t *>(xr + k1);
            v[0] = a0.x; v[1] = a0.y; v[2] = a0.z; v[3] = a0.w;
            v[4] = a1.x; v[5] = a1.y; v[6] = a1.z; v[7] = a1.w;
            if constexpr (KIND == 2) {
                const f32x4_al16_t b0 = *reinterpret_cast<const f32x4_al16_t *>(ur + k0);
                const f32x4_al16_t b1 = *reinterpret_cast<const f32x4_al16_t *>(ur + k1);
                v[0] = silu_mul(v[0], b0.x); v[1] = silu_mul(v[1], b0.y);
                v[2] = silu_mul(v[2], b0.z); v[3] = silu_mul(v[3], b0.w);
                v[4] = silu_mul(v[4], b1.x); v[5] = silu_mul(v[5], b1.y);
                v[6] = silu_mul(v[6], b1.z); v[7] = silu_mul(v[7], b1.w);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float t = v[e];
                if constexpr (KIND == 1) {
                    const int k = (e < 4 ? k0 + e : k1 + e - 4);
                    t = t * inv * (nw ? nw[k] : 1.0f);
                }
                t *= s;
                if (FMT == 0 && e >= 4) t *= 0.0625f;
                const _Float16 h = static_cast<_Float16>(t);
                hi[e] = h;
                lo[e] = static_cast<_Float16>(t - static_cast<float>(h));
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                hi[e] = static_cast<_Float16>(0.0f);
                lo[e] = static_cast<_Float16>(0.0f);
            }
        }
        u32x4_t *dst = xf + static_cast<int64_t>(j) * 64 + 16 * g + 2 * b;
        dst[0] = __builtin_bit_cast(u32x4_t, hi);
        dst[1] = __builtin_bit_cast(u32x4_t, lo);
    }
}

// ---------------------------------------------------------------- main kernel
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
// low nibbles q - 8, high nibbles 16 (q - 8).
__device__ __forceinline__ half8_t q4_codes(uint32_t w) {
    const uint32_t p01 = __builtin_amdgcn_perm(w, w, 0x0C010C00u);
    const uint32_t p23 = __builtin_amdgcn_perm(w, w, 0x0C030C02u);
    const half2_t lo_off = {static_cast<_Float16>(-1032.0f), static_cast<_Float16>(-1032.0f)};
    const half2_t hi_off = {static_cast<_Float16>(-1152.0f), static_cast<_Float16>(-1152.0f)};
    const half2_t h0 = __builtin_bit_cast(half2_t, (p01 & 0x000F000Fu) | 0x64006400u) + lo_off;
    const half2_t h1 = __builtin_bit_cast(half2_t, (p23 & 0x000F000Fu) | 0x64006400u) + lo_off;
    const half2_t h2 = __builtin_bit_cast(half2_t, (p01 & 0x00F000F0u) | 0x64006400u) + hi_off;
    const half2_t h3 = __builtin_bit_cast(half2_t, (p23 & 0x00F000F0u) | 0x64006400u) + hi_off;
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

template <int FMT>
__global__ __launch_bounds__(kWG) void mv_mfma_kernel(
    const uint8_t *__restrict__ W, int N, int K, int B, const u32x4_t *__restrict__ xf,
    const float *__restrict__ sinv, float *y, const float *res, float *__restrict__ part,
    int *__restrict__ counters, int S, int cps) {
    constexpr int kBytes = BF<FMT>::kBytes;
    constexpr int kDw = BF<FMT>::kLaneDw;
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int col = lane & 15, g = lane >> 4;
    const int n = blockIdx.x * kRowsWG + wv * 16 + col;
    const int nl = min(n, N - 1);
    const int nb = K / 32, kc = nb / kSeg;
    const int c0 = blockIdx.y * cps;
    const int c1 = min(kc, c0 + cps);
    const uint8_t *wrow = W + static_cast<int64_t>(nl) * nb * kBytes + g * 2 * kBytes;

    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
    const int64_t seg = kSeg * kBytes;
    uint32_t dw[kDw], nx[kDw];
    load_seg<kDw>(wrow + c0 * seg, dw);
    for (int c = c0; c < c1; ++c) {
        // activations of this step first, then the next step's weights, so
        // waiting for the former never waits for the latter
        u32x4_t xa[kSeg];
        const u32x4_t *xp = xf + static_cast<int64_t>(c) * kSeg * 64 + lane;
#pragma unroll
        for (int jj = 0; jj < kSeg; ++jj) xa[jj] = xp[jj * 64];
        load_seg<kDw>(wrow + min(c + 1, c1 - 1) * seg, nx);

        // Block scales of this lane's two blocks, then every lane group's.
        uint32_t dp = __builtin_amdgcn_perm(dw[(kDw - 1) / 2], dw[0], 0x07060100u);
        uint32_t dps[4];
        {
            auto r = __builtin_amdgcn_permlane32_swap(dp, dp, false, false);
            auto s01 = __builtin_amdgcn_permlane16_swap(r[0], r[0], false, false);
            auto s23 = __builtin_amdgcn_permlane16_swap(r[1], r[1], false, false);
            dps[0] = s01[0];
            dps[1] = s01[1];
            dps[2] = s23[0];
            dps[3] = s23[1];
        }
        half8_t wf[kSeg];
        if constexpr (FMT == 0) {
            // even block: payload at byte 2 of the lane's window; odd block: at byte 20
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
#pragma unroll
        for (int jj = 0; jj < kSeg; ++jj) {
            const f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                __builtin_bit_cast(half8_t, xa[jj]), wf[jj], zero, 0, 0, 0);
            const uint32_t sc = dps[jj >> 1];
            if (jj & 1) {
                acc[0] = fma_hi(sc, d[0], acc[0]);
                acc[1] = fma_hi(sc, d[1], acc[1]);
                acc[2] = fma_hi(sc, d[2], acc[2]);
                acc[3] = fma_hi(sc, d[3], acc[3]);
            } else {
                acc[0] = fma_lo(sc, d[0], acc[0]);
                acc[1] = fma_lo(sc, d[1], acc[1]);
                acc[2] = fma_lo(sc, d[2], acc[2]);
                acc[3] = fma_lo(sc, d[3], acc[3]);
            }
        }
#pragma unroll
        for (int t = 0; t < kDw; ++t) dw[t] = nx[t];
    }
    // Result rows 4g..4g+3 are (batch 2g: hi, lo), (batch 2g+1: hi, lo).
    const int ba = 2 * g, bb = 2 * g + 1;
    const float ya = (acc[0] + acc[1]) * sinv[ba];
    const float yb = (acc[2] + acc[3]) * sinv[bb];
    const int64_t ln = N;
    if (S == 1) {
        if (n < N) {
            if (ba < B) y[ba * ln + n] = res ? ya + res[ba * ln + n] : ya;
            if (bb < B) y[bb * ln + n] = res ? yb + res[bb * ln + n] : yb;
        }
        return;
    }
    // Split K: partial sums go to the workspace with device-scope stores
    // (written through the compute die's L2), the workgroup takes a ticket,
    // and the last one adds the S partials in split order with device-scope
    // loads.  Device-scope fences are avoided on purpose: on this part they
    // write back and invalidate the whole L2 of the die.
    if (n < N) {
        float *pp = part + static_cast<int64_t>(blockIdx.y) * B * ln;
        if (ba < B) __hip_atomic_store(pp + ba * ln + n, ya, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (bb < B) __hip_atomic_store(pp + bb * ln + n, yb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);  // every store of this wavefront has completed
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    __shared__ int ticket;
    if (threadIdx.x == 0)
        ticket = __hip_atomic_fetch_add(&counters[blockIdx.x], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (ticket != S - 1) return;
    for (int o = threadIdx.x; o < kRowsWG * B; o += kWG) {
        const int b = o / kRowsWG;
        const int nn = blockIdx.x * kRowsWG + (o % kRowsWG);
        if (nn >= N) continue;
        const float *pb = part + static_cast<int64_t>(b) * ln + nn;
        const int64_t step = static_cast<int64_t>(B) * ln;
        float v = 0.f;
        int sp = 0;
        for (; sp + 8 <= S; sp += 8) {  // eight loads in flight, added in split order
            float t[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                t[u] = __hip_atomic_load(pb + (sp + u) * step, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int u = 0; u < 8; ++u) v += t[u];
        }
        for (; sp < S; ++sp) v += __hip_atomic_load(pb + sp * step, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        y[b * ln + nn] = res ? v + res[b * ln + nn] : v;
    }
    if (threadIdx.x == 0) __hip_atomic_store(&counters[blockIdx.x], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- host side
struct Plan {
    int rg, kc, S, cps;
    size_t off_sinv, off_xf, off_part, bytes;
};

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

Plan make_plan(int64_t N, int64_t K, int64_t B) {
    Plan p;
    p.rg = static_cast<int>((N + kRowsWG - 1) / kRowsWG);
    p.kc = static_cast<int>(K / (32 * kSeg));
    const int want = std::max(1, std::min(p.kc, (kTargetWGs + p.rg - 1) / p.rg));
    p.cps = (p.kc + want - 1) / want;
    p.S = (p.kc + p.cps - 1) / p.cps;
    p.off_sinv = align256(static_cast<size_t>(p.rg) * sizeof(int));
    p.off_xf = p.off_sinv + 256;
    p.off_part = p.off_xf + static_cast<size_t>(K / 32) * 64 * 16;
    p.bytes = p.off_part + (p.S > 1 ? align256(static_cast<size_t>(p.S) * B * N * sizeof(float)) : 0);
    return p;
}

template <int FMT, int KIND>
void launch_prep(const float *x, const float *u, const float *nw, float eps, int64_t ld, int K,
                 int B, void *ws, const Plan &p, hipStream_t s) {
    uint8_t *w8 = static_cast<uint8_t *>(ws);
    const int parts = (K / 32 * 4 + kPrepThreads - 1) / kPrepThreads;
    hipLaunchKernelGGL((mfma_prep_kernel<FMT, KIND>), dim3(kMaxB, parts), dim3(kPrepThreads), 0, s, x, u,
                       nw, eps, ld, K, B, reinterpret_cast<u32x4_t *>(w8 + p.off_xf),
                       reinterpret_cast<float *>(w8 + p.off_sinv), reinterpret_cast<int *>(w8), p.rg);
}

template <int FMT>
q4_status batched_entry(const char *name, const void *Wv, int64_t N, int64_t K, const float *x,
                        const float *x2, int64_t ldx, int64_t B, int op_kind, const float *norm_w,
                        float eps, float *y, const float *res, void *ws, size_t ws_bytes,
                        void *stream) {
    q4::clear_error();
    Q4_CHECK(Wv && x && y, Q4_ERR_INVALID_ARG, "%s: W, x and y must not be NULL", name);
    Q4_CHECK(N >= 1 && K >= 1 && B >= 1, Q4_ERR_INVALID_ARG, "%s: N=%lld K=%lld B=%lld must be >= 1",
             name, (long long)N, (long long)K, (long long)B);
    Q4_CHECK(op_kind >= Q4_IN_PLAIN && op_kind <= Q4_IN_SWIGLU, Q4_ERR_INVALID_ARG,
             "%s: unknown input transform %d", name, op_kind);
    Q4_CHECK(op_kind != Q4_IN_SWIGLU || x2, Q4_ERR_INVALID_ARG, "%s: SwiGLU needs x2", name);
    Q4_CHECK(op_kind != Q4_IN_RMSNORM || eps >= 0.f, Q4_ERR_INVALID_ARG, "%s: eps must be >= 0", name);
    Q4_CHECK(ldx >= K, Q4_ERR_SHAPE, "%s: ld_x=%lld < K=%lld", name, (long long)ldx, (long long)K);
    Q4_CHECK(K % 256 == 0, Q4_ERR_UNSUPPORTED, "%s: K=%lld is not a multiple of 256", name,
             (long long)K);
    Q4_CHECK(B <= kMaxB, Q4_ERR_UNSUPPORTED, "%s: B=%lld > 8", name, (long long)B);
    Q4_CHECK(N <= (1 << 30) && K <= (1 << 24) && ldx <= (1 << 26), Q4_ERR_UNSUPPORTED,
             "%s: N or K too large", name);
    Q4_CHECK(q4::aligned(Wv, 16), Q4_ERR_ALIGNMENT, "%s: W must be 16-byte aligned", name);
    Q4_CHECK(q4::aligned(x, 16) && (!x2 || q4::aligned(x2, 16)) && ldx % 4 == 0, Q4_ERR_ALIGNMENT,
             "%s: x and x2 must be 16-byte aligned with ld_x a multiple of 4", name);
    Q4_CHECK(q4::aligned(y, 4) && (!res || q4::aligned(res, 4)) && (!norm_w || q4::aligned(norm_w, 4)),
             Q4_ERR_ALIGNMENT, "%s: y, residual and norm_w must be 4-byte aligned", name);
    const Plan p = make_plan(N, K, B);
    Q4_CHECK(ws && q4::aligned(ws, 256), Q4_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned",
             name);
    Q4_CHECK(ws_bytes >= p.bytes, Q4_ERR_WORKSPACE, "%s: workspace of %zu bytes < %zu needed", name,
             ws_bytes, p.bytes);
    hipStream_t s = q4::as_stream(stream);
    const int k = static_cast<int>(K), b = static_cast<int>(B);
    if (op_kind == Q4_IN_RMSNORM) launch_prep<FMT, 1>(x, nullptr, norm_w, eps, ldx, k, b, ws, p, s);
    else if (op_kind == Q4_IN_SWIGLU) launch_prep<FMT, 2>(x, x2, nullptr, eps, ldx, k, b, ws, p, s);
    else launch_prep<FMT, 0>(x, nullptr, nullptr, eps, ldx, k, b, ws, p, s);
    uint8_t *w8 = static_cast<uint8_t *>(ws);
    hipLaunchKernelGGL((mv_mfma_kernel<FMT>), dim3(p.rg, p.S), dim3(kWG), 0, s,
                       static_cast<const uint8_t *>(Wv), static_cast<int>(N), k, b,
                       reinterpret_cast<const u32x4_t *>(w8 + p.off_xf),
                       reinterpret_cast<const float *>(w8 + p.off_sinv), y, res,
                       reinterpret_cast<float *>(w8 + p.off_part), reinterpret_cast<int *>(w8), p.S,
                       p.cps);
    return q4::launch_status(name);
}

}  // namespace

extern "C" size_t matvec_batched_workspace(int64_t N, int64_t K, int64_t B) {
    if (N < 1 || K < 256 || K % 256 != 0 || B < 1 || B > kMaxB) return 0;
    return make_plan(N, K, B).bytes;
}

extern "C" q4_status q4_0_matvec_batched(const void *W, int64_t N, int64_t K, const float *x,
                                         const float *x2, int64_t ld_x, int64_t B,
                                         q4_input_op op, const float *norm_w, float eps, float *y,
                                         const float *residual, void *ws, size_t ws_bytes,
                                         void *stream) {
    return batched_entry<0>("q4_0_matvec_batched", W, N, K, x, x2, ld_x, B, op, norm_w, eps, y,
                            residual, ws, ws_bytes, stream);
}

extern "C" q4_status q8_0_matvec_batched(const void *W, int64_t N, int64_t K, const float *x,
                                         const float *x2, int64_t ld_x, int64_t B,
                                         q4_input_op op, const float *norm_w, float eps, float *y,
                                         const float *residual, void *ws, size_t ws_bytes,
                                         void *stream) {
    return batched_entry<1>("q8_0_matvec_batched", W, N, K, x, x2, ld_x, B, op, norm_w, eps, y,
                            residual, ws, ws_bytes, stream);
}
