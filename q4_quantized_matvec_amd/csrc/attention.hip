// Split-K grouped-query decode attention over an fp32 or binary16 KV cache,
// gfx950.
//
// Definition ("GELO LLM" page, 05 "Components": cached GQA attention where a
// decode step's single query row attends every cached position plus the new
// one; 02 "Definitions & glossary": several query heads share one K/V head; a
// sliding-window layer attends only the last W tokens):
//   o_h = sum_j softmax_j(scale * q_h . k_j) v_j ,  j in [lo, n),
//   lo = max(0, n - W) (W = 0: lo = 0), kv head of query head h = h / G.
//
// Pass 1 (one workgroup per (split, kv head, sequence); a split is one
// 64-position chunk, or at long context several in a row): the G query heads
// that share the kv head are held in VGPRs (pre-scaled), the keys are read
// once for all of them, an exact softmax (running over the split's chunks)
// gives (m, l) and the un-normalised sum_j e^(s_j - m) v_j is formed with the
// same weights for every query head.  Pass 2 merges the splits of each query
// head: o = sum_c e^(m_c - M) o_c / sum_c e^(m_c - M) l_c over the non-empty
// splits, M = max m_c, taken in a fixed order, so the result does not depend
// on scheduling.
#include "common.hpp"

namespace {
using namespace q4dev;

constexpr int kWG = 256;
constexpr int kChunk = 64;  // positions per chunk (one per lane in the softmax pass)

// Up to kSplitFrom chunks over all (sequence, kv head) pairs, every chunk is
// a workgroup of its own: that keeps the most loads in flight.  Beyond it,
// consecutive chunks are grouped into splits (one workgroup and one partial
// each) so that about kSplitTarget workgroups remain: fewer partials for the
// merge and fewer per-workgroup query loads, with enough waves left to keep
// HBM busy.
#ifndef Q4_ATTN_SPLIT_TARGET
#define Q4_ATTN_SPLIT_TARGET 1024
#endif
constexpr int kSplitTarget = Q4_ATTN_SPLIT_TARGET;

// Score products on the matrix cores for binary16 caches (see
// attn_split_kernel).
#ifndef Q4_ATTN_MFMA
#define Q4_ATTN_MFMA 1
#endif
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Power-of-two exponent that puts m (the largest magnitude of a query row) in
// [2^11, 2^12); 0 for zero, infinite or NaN maxima.
__device__ __forceinline__ int row_shift(float m) {
    if (!(m > 0.f) || !(m <= 3.4e38f)) return 0;
    int e;
    (void)frexpf(m, &e);
    return min(max(12 - e, -120), 120);
}
constexpr int kSplitFrom = 4 * kSplitTarget;

struct AttnGeom {
    int G;    // query heads per kv head
    int nch;  // chunks per (sequence, kv head)
    int cps;  // chunks per split
    int ns;   // splits per (sequence, kv head)
};

// Chunking depends only on the layout and window (never on n), so the
// workspace size and the captured launch stay valid as n grows.
AttnGeom attn_geom(const q4_kv_layout &kv, int64_t n_q_heads, int64_t window) {
    AttnGeom g;
    g.G = static_cast<int>(n_q_heads / kv.n_kv_heads);
    const int64_t maxvis = window > 0 ? std::min<int64_t>(window, kv.cap) : kv.cap;
    g.nch = static_cast<int>((maxvis + kChunk - 1) / kChunk);
    const int64_t total = static_cast<int64_t>(g.nch) * kv.n_kv_heads * kv.batch;
    g.cps = total < kSplitFrom ? 1 : static_cast<int>(total / kSplitTarget);
    g.ns = (g.nch + g.cps - 1) / g.cps;
    return g;
}

// A copy the compiler cannot see through.  When both results of one
// permlane swap are reinterpreted as floats, this compiler has been seen to
// merge the two reinterpretations (computing a[0] + a[0] for a[0] + a[1]), so
// every second result used as a float goes through this copy first.
__device__ __forceinline__ uint32_t opaque_copy(uint32_t v) {
    uint32_t r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
    return r;
}

// Sum over aligned groups of L lanes (L = 8, 16, 32 or 64); every lane of a
// group receives the same bits.  Within a 16-lane row: DPP; across rows:
// permlane swaps (no LDS traffic).
template <int L>
__device__ __forceinline__ float group_sum(float v) {
    v += dpp<0xB1>(v);   // xor 1
    v += dpp<0x4E>(v);   // xor 2
    v += dpp<0x141>(v);  // half-row mirror: groups of 8
    if constexpr (L >= 16) v += dpp<0x140>(v);  // row mirror: groups of 16
    if constexpr (L >= 32) {  // rows (0,1) and (2,3)
        const uint32_t u = __builtin_bit_cast(uint32_t, v);
        auto s = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        v = __builtin_bit_cast(float, s[0]) + __builtin_bit_cast(float, opaque_copy(s[1]));
    }
    if constexpr (L >= 64) {  // the two halves of the wavefront
        const uint32_t u = __builtin_bit_cast(uint32_t, v);
        auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        v = __builtin_bit_cast(float, s[0]) + __builtin_bit_cast(float, opaque_copy(s[1]));
    }
    return v;
}

// One workgroup per (split, kv head, sequence).  A split is cps consecutive
// 64-position chunks, taken in order with a running softmax: per chunk the
// new maximum rescales the running denominator and weighted value sums by
// exp(m_old - m_new) (exact softmax over the split, one partial per split).
// Loads are issued in batches ahead of their use so the wavefronts keep many
// rows in flight.
// Fused query/key preparation (gqa_decode_attn_rope): q and the new key are
// read raw from the merged projection row, RMS-normalised per head with their
// gains and rotated (NeoX pairs i, i + hd/2); the new key and value rows are
// appended to the caches by the workgroup whose chunk holds the position.
struct RopeArgs {
    const float *kraw, *vraw;  // raw key / value rows of kv head 0 (vraw NULL: V from K)
    int64_t ldkv;              // row stride of kraw / vraw
    const float *qn, *kn;      // per-head gains [hd]
    double rstep;              // theta^(-2/hd), computed on the host
    float eps;
    void *kcw, *vcw;           // the caches (element type of the layout), written at slot pos % cap
};

// Cache elements: fp32, or binary16 read into fp32 exactly and written with
// round-to-nearest-even.  Four consecutive elements per access.
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
template <typename KT>
__device__ __forceinline__ float4 load4(const KT *p) {
    if constexpr (sizeof(KT) == 4) {
        const f32x4_ev v = ld_kv(reinterpret_cast<const f32x4_ev *>(p));
        return make_float4(v.x, v.y, v.z, v.w);
    } else {
        const half4_t h = __builtin_bit_cast(half4_t, ld_kv(reinterpret_cast<const u32x2_ev *>(p)));
        return make_float4(static_cast<float>(h.x), static_cast<float>(h.y), static_cast<float>(h.z),
                           static_cast<float>(h.w));
    }
}
template <typename KT>
__device__ __forceinline__ void store4(KT *p, float a, float b, float c, float d) {
    if constexpr (sizeof(KT) == 4) {
        *reinterpret_cast<float4 *>(p) = make_float4(a, b, c, d);
    } else {
        half4_t h;
        h.x = static_cast<_Float16>(a);
        h.y = static_cast<_Float16>(b);
        h.z = static_cast<_Float16>(c);
        h.w = static_cast<_Float16>(d);
        *reinterpret_cast<uint2 *>(p) = __builtin_bit_cast(uint2, h);
    }
}

// cos / sin of pos * theta^(-2i/hd): frequency by binary powers of
// theta^(-2/hd) in fp64, angle reduced by 2 pi in fp64, then single-precision
// sincos of the reduced angle (i < 256).
__device__ __forceinline__ void rope_cs(int64_t pos, double r, int i, float &cs, float &sn) {
    double f = 1.0, rp = r;  // r = theta^(-2/hd)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        f = ((i >> k) & 1) ? f * rp : f;
        rp = rp * rp;
    }
    const double ang = static_cast<double>(pos) * f;
    const double two_pi = 6.283185307179586;
    const double red = __builtin_fma(-two_pi, rint(ang * (1.0 / two_pi)), ang);
    sincosf(static_cast<float>(red), &sn, &cs);
}

template <int HD, int GM, bool ROPE, bool MULTI, typename KT>
__global__ __launch_bounds__(kWG) void attn_split_kernel(
    const float *__restrict__ q, int64_t ldq, int G, const KT *kc, const KT *vc, int64_t cap,
    int64_t sb, int64_t sh, int64_t st, const int64_t *__restrict__ n_dev, int64_t window,
    float scale, int ns, int cps, float *__restrict__ part, RopeArgs ra) {
    constexpr int LPK = HD / 8;              // score pass: lanes per key, 8 elements per lane
    constexpr int KPW = 64 / LPK;            // keys per wavefront per step
    constexpr int SIT = kChunk / (4 * KPW);  // score steps per wavefront
    constexpr int TPK = HD / 4;              // value pass: threads per key (float4 each)
    constexpr int KG = kWG / TPK;            // value pass: key groups
    constexpr int VIT = kChunk / KG;         // value pass: keys per thread
    __shared__ __align__(16) float sc[kChunk * GM];  // scores, then weights: [pos][g]
    __shared__ __align__(16) float4 red[KG > 1 ? (KG - 1) * GM * TPK : 1];
    __shared__ float alpha_s[GM];  // rescale of the running sums at this chunk

    const int sp = blockIdx.x, g0 = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // fused preparation: n_dev holds the new token's position, n = pos + 1
    const int64_t n = ROPE ? *n_dev + 1 : *n_dev;
    int64_t lo = window > 0 ? n - window : 0;
    lo = max(lo, n - cap);
    lo = max(lo, int64_t(0));
    const int64_t s0 = lo + static_cast<int64_t>(sp) * cps * kChunk;  // first position of the split
    const int64_t span = min(static_cast<int64_t>(cps) * kChunk, n - s0);

    const size_t unit = ((static_cast<size_t>(b) * gridDim.y + g0) * ns + sp) * GM;
    float *po = part + unit * HD;  // [GM][HD]
    float *pml = part + static_cast<size_t>(gridDim.z) * gridDim.y * ns * GM * HD + unit * 2;
    if (span <= 0) {
        if (threadIdx.x < G) {
            pml[2 * threadIdx.x] = -INFINITY;
            pml[2 * threadIdx.x + 1] = 0.f;
        }
        return;
    }
    const KT *kb = kc + b * sb + g0 * sh;
    const KT *vb = vc + b * sb + g0 * sh;
    // slot of position j of the current chunk (positions past the chunk end
    // re-read its first row): one 64-bit remainder per chunk, then 32-bit
    // wrap-around
    const int cap32 = static_cast<int>(cap);
    int sbase = 0, cnt = 0;
    auto slot = [&](int j) {
        int sl = sbase + (j < cnt ? j : 0);
        if (sl >= cap32) sl -= cap32;
        if (sl >= cap32) sl %= cap32;  // only for caches shorter than a chunk
        return static_cast<int64_t>(sl) * st;
    };

    // ---- scores, SG keys per wavefront at a time (bounds the registers held)
    constexpr int SG = SIT < 8 ? SIT : 8;
    const int sub = lane % LPK, kgl = lane / LPK;
    // lane sub holds elements [4 sub, 4 sub + 4) and HD/2 + [4 sub, 4 sub + 4),
    // i.e. four whole RoPE pairs
    auto load8 = [&](const float *p, float (&v)[8]) {
        const float4 a = *reinterpret_cast<const float4 *>(p + sub * 4);
        const float4 bq = *reinterpret_cast<const float4 *>(p + HD / 2 + sub * 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = bq.x; v[5] = bq.y; v[6] = bq.z; v[7] = bq.w;
    };
    float rc[4], rs[4];   // RoPE cos / sin of this lane's pairs
    float gq[8], gk[8];   // gains of this lane's elements
    auto norm_rope = [&](float (&v)[8], const float (&gain)[8]) {  // in place
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(v[e], v[e], ss);
        ss = group_sum<LPK>(ss);
        const float inv = 1.0f / sqrtf(ss / static_cast<float>(HD) + ra.eps);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x0 = v[e] * inv * gain[e], x1 = v[e + 4] * inv * gain[e + 4];
            v[e] = x0 * rc[e] - x1 * rs[e];
            v[e + 4] = x1 * rc[e] + x0 * rs[e];
        }
        return inv;
    };
    if constexpr (ROPE) {
        const int64_t pos = n - 1;
        const double r = ra.rstep;
#pragma unroll
        for (int e = 0; e < 4; ++e) rope_cs(pos, r, 4 * sub + e, rc[e], rs[e]);
        load8(ra.qn, gq);
        load8(ra.kn, gk);
        if (pos >= s0 && pos < s0 + span) {
            // this split holds the new position: append its key and value rows
            float kv8[8], vv8[8];
            const float *kr = ra.kraw + b * ra.ldkv + static_cast<int64_t>(g0) * HD;
            load8(kr, kv8);
            float raw[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) raw[e] = kv8[e];
            const float kinv = norm_rope(kv8, gk);
            if (ra.vraw) load8(ra.vraw + b * ra.ldkv + static_cast<int64_t>(g0) * HD, vv8);
            else {
#pragma unroll
                for (int e = 0; e < 8; ++e) vv8[e] = raw[e] * kinv;  // unit-gain RMSNorm of the raw key
            }
            if (wave == 0 && kgl == 0) {
                const int64_t off = b * sb + static_cast<int64_t>(g0) * sh + (pos % cap) * st;
                KT *kd = static_cast<KT *>(ra.kcw) + off, *vd = static_cast<KT *>(ra.vcw) + off;
                store4(kd + sub * 4, kv8[0], kv8[1], kv8[2], kv8[3]);
                store4(kd + HD / 2 + sub * 4, kv8[4], kv8[5], kv8[6], kv8[7]);
                store4(vd + sub * 4, vv8[0], vv8[1], vv8[2], vv8[3]);
                store4(vd + HD / 2 + sub * 4, vv8[4], vv8[5], vv8[6], vv8[7]);
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_waitcnt(0);  // the rows are written before any wavefront reads them
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __syncthreads();
        }
    }
    float qv[GM][8];
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        load8(q + b * ldq + static_cast<int64_t>(g0 * G + min(g, G - 1)) * HD, qv[g]);
        if constexpr (ROPE) (void)norm_rope(qv[g], gq);
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[g][e] *= scale;
    }
    // Matrix-core scores (binary16 keys): the scaled query rows go through
    // LDS (the value-reduction buffer, unused until the end) into
    // v_mfma_f32_16x16x32_f16 A operands.  A row 2h + t holds head h's part t
    // of q_h * 2^e_h = hi + lo (hi = binary16 of the scaled row, lo = binary16
    // of the remainder; e_h puts the row's largest magnitude in [2^11, 2^12)),
    // so hi + lo carries about 22 bits of every element and each product with
    // a binary16 key is exact in the fp32 accumulation; rows of heads >= GM
    // are zero.  Lane (i, g) holds A[i][8g .. 8g + 7] of each of the HD / 32
    // steps of 32 dimensions; the key operand of lane (n, g) is the 16
    // contiguous bytes of key n at the same dimensions.
    // Taken at hd 512 with 8 heads, where the vector ALUs bound the layer.
    // At hd 128 and 256 (2 or 4 heads) it measured slower or level (the
    // operands' registers cost occupancy and most MFMA rows are zero), and at
    // hd 512 with fewer heads the operands would cost the same occupancy.
    constexpr bool kMfma = Q4_ATTN_MFMA && sizeof(KT) == 2 && HD == 512 && GM == 8;
    constexpr int kQs = kMfma ? HD / 32 : 1;
    [[maybe_unused]] half8_t qa[kQs];
    __shared__ float qscale_s[8];
    if constexpr (kMfma) {
        float *qs = reinterpret_cast<float *>(red);  // [GM][HD]
        static_assert(sizeof(red) >= sizeof(float) * GM * HD, "query staging");
        if (wave == 0) {
#pragma unroll
            for (int g = 0; g < GM; ++g) {
                float *d = qs + g * HD;
                *reinterpret_cast<float4 *>(d + 4 * sub) = make_float4(qv[g][0], qv[g][1], qv[g][2], qv[g][3]);
                *reinterpret_cast<float4 *>(d + HD / 2 + 4 * sub) = make_float4(qv[g][4], qv[g][5], qv[g][6], qv[g][7]);
            }
        }
        __syncthreads();
        const int arow = lane & 15, ag = lane >> 4, ah = arow >> 1;
        const bool live = ah < GM;  // rows of heads past GM stay zero
        const float *qh = qs + min(ah, GM - 1) * HD + 8 * ag;
        float m = 0.f;
#pragma unroll
        for (int st_ = 0; st_ < kQs; ++st_) {
            const float4 a = *reinterpret_cast<const float4 *>(qh + 32 * st_);
            const float4 c = *reinterpret_cast<const float4 *>(qh + 32 * st_ + 4);
            m = fmaxf(m, fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))));
            m = fmaxf(m, fmaxf(fmaxf(fabsf(c.x), fabsf(c.y)), fmaxf(fabsf(c.z), fabsf(c.w))));
        }
        // the four lane groups of a row hold the row's four quarters
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        const int sh = row_shift(m);
        const float sc4 = ldexpf(1.0f, sh);
        if (wave == 0 && ag == 0 && (arow & 1) == 0) qscale_s[ah] = ldexpf(1.0f, -sh);
#pragma unroll
        for (int st_ = 0; st_ < kQs; ++st_) {
            half8_t v;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xv = qh[32 * st_ + e] * sc4;
                const _Float16 hi = static_cast<_Float16>(xv);
                v[e] = (arow & 1) ? static_cast<_Float16>(xv - static_cast<float>(hi)) : hi;
            }
            qa[st_] = live ? v : half8_t{};
        }
        __syncthreads();  // qscale_s written; every wavefront has its operands
    }
    // ---- value-pass roles and running state
    const int kg = threadIdx.x / TPK, d4 = threadIdx.x % TPK;
    constexpr int VG = VIT < 16 ? VIT : 16;  // keys per thread at a time
    constexpr int HPW = (GM + 3) / 4;        // softmax: heads per wavefront
    float4 acc[GM];
#pragma unroll
    for (int g = 0; g < GM; ++g) acc[g] = make_float4(0.f, 0.f, 0.f, 0.f);
    float m_run[HPW], l_run[HPW];
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
        m_run[i] = -INFINITY;
        l_run[i] = 0.f;
    }
    // one chunk per split unless MULTI (then the value sums stay live across
    // the score pass, which costs registers)
    const int nck = MULTI ? static_cast<int>((span + kChunk - 1) / kChunk) : 1;
#pragma unroll 1
    for (int ci = 0; ci < nck; ++ci) {
    const int64_t p0 = s0 + static_cast<int64_t>(ci) * kChunk;
    cnt = static_cast<int>(min(int64_t(kChunk), n - p0));
    sbase = static_cast<int>(p0 % cap);
    if constexpr (kMfma) {
        // wavefront w scores keys 16w .. 16w + 15 of the chunk: HD / 32 steps
        // of 32 dimensions, up to 8 key loads of 16 bytes in flight per lane
        constexpr int KB = kQs < 8 ? kQs : 8;
        const int key = 16 * wave + (lane & 15);
        const KT *kp = kb + slot(key) + 8 * (lane >> 4);
        f32x4_t dacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s0 = 0; s0 < kQs; s0 += KB) {
            f32x4_ev kw[KB];
#pragma unroll
            for (int t = 0; t < KB; ++t) kw[t] = ld_kv(reinterpret_cast<const f32x4_ev *>(kp + 32 * (s0 + t)));
#pragma unroll
            for (int t = 0; t < KB; ++t)
                dacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[s0 + t], __builtin_bit_cast(half8_t, kw[t]), dacc,
                                                              0, 0, 0);
        }
        // result rows 4g .. 4g + 3: (head 2g: hi, lo), (head 2g + 1: hi, lo);
        // heads past G (hence past GM) are not read
        const int h0 = 2 * (lane >> 4);
        const float s_a = (dacc[0] + dacc[1]) * qscale_s[h0];
        const float s_b = (dacc[2] + dacc[3]) * qscale_s[h0 + 1];
        if (h0 < G) sc[key * GM + h0] = key < cnt ? s_a : -INFINITY;
        if (h0 + 1 < G) sc[key * GM + h0 + 1] = key < cnt ? s_b : -INFINITY;
    } else {
#pragma unroll 1
    for (int i0 = 0; i0 < SIT; i0 += SG) {
        float kr[SG][8];
#pragma unroll
        for (int it = 0; it < SG; ++it) {
            const int jj = (i0 + it) * 4 * KPW + wave * KPW + kgl;
            // each load instruction covers contiguous bytes of the key row
            const KT *kp = kb + slot(jj);
            const float4 a = load4(kp + sub * 4), c = load4(kp + HD / 2 + sub * 4);
            kr[it][0] = a.x; kr[it][1] = a.y; kr[it][2] = a.z; kr[it][3] = a.w;
            kr[it][4] = c.x; kr[it][5] = c.y; kr[it][6] = c.z; kr[it][7] = c.w;
        }
#pragma unroll
        for (int it = 0; it < SG; ++it) {
            const int jj = (i0 + it) * 4 * KPW + wave * KPW + kgl;
#pragma unroll
            for (int g = 0; g < GM; ++g) {
                float s = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) s = __builtin_fmaf(qv[g][e], kr[it][e], s);
                s = group_sum<LPK>(s);
                if (sub == 0 && g < G) sc[jj * GM + g] = jj < cnt ? s : -INFINITY;
            }
        }
    }
    }
    __syncthreads();

    // ---- softmax over the chunk against the running maximum: one wavefront
    // per query head, one lane per position
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
        const int g = wave + 4 * i;
        if (g < G) {
            const float s = sc[lane * GM + g];
            const float m_new = fmaxf(m_run[i], wave_max(s));
            const float e = lane < cnt ? __expf(s - m_new) : 0.f;
            const float a = __expf(m_run[i] - m_new);  // 0 at the first chunk
            l_run[i] = __builtin_fmaf(l_run[i], a, wave_sum(e));
            m_run[i] = m_new;
            sc[lane * GM + g] = e;
            if (lane == 0) alpha_s[g] = a;
        }
    }
    __syncthreads();

    // ---- weighted values: TPK threads per key (4 dims each), KG key groups
    if (MULTI && ci > 0) {  // nothing to rescale at the first chunk
#pragma unroll
        for (int g = 0; g < GM; ++g) {
            const float a = g < G ? alpha_s[g] : 0.f;
            acc[g].x *= a; acc[g].y *= a; acc[g].z *= a; acc[g].w *= a;
        }
    }
#pragma unroll 1
    for (int i0 = 0; i0 < VIT; i0 += VG) {
        float4 vv[VG];
#pragma unroll
        for (int it = 0; it < VG; ++it)
            vv[it] = load4(vb + slot(kg + (i0 + it) * KG) + 4 * d4);
#pragma unroll
        for (int it = 0; it < VG; ++it) {
            const int j = kg + (i0 + it) * KG;  // weights of positions past cnt are 0
#pragma unroll
            for (int g = 0; g < GM; ++g) {
                const float w = sc[j * GM + g];
                acc[g].x = __builtin_fmaf(w, vv[it].x, acc[g].x);
                acc[g].y = __builtin_fmaf(w, vv[it].y, acc[g].y);
                acc[g].z = __builtin_fmaf(w, vv[it].z, acc[g].z);
                acc[g].w = __builtin_fmaf(w, vv[it].w, acc[g].w);
            }
        }
    }
    if (MULTI) __syncthreads();  // sc and alpha_s are rewritten by the next chunk
    }  // chunks
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
        const int g = wave + 4 * i;
        if (g < G && lane == 0) {
            pml[2 * g] = m_run[i];
            pml[2 * g + 1] = l_run[i];
        }
    }
    if constexpr (KG > 1) {
        if (kg > 0) {
#pragma unroll
            for (int g = 0; g < GM; ++g) red[((kg - 1) * GM + g) * TPK + d4] = acc[g];
        }
        __syncthreads();
        if (kg == 0) {
#pragma unroll
            for (int g = 0; g < GM; ++g) {
                float4 s4 = acc[g];
                for (int k = 1; k < KG; ++k) {  // fixed order
                    const float4 r = red[((k - 1) * GM + g) * TPK + d4];
                    s4.x += r.x; s4.y += r.y; s4.z += r.z; s4.w += r.w;
                }
                if (g < G) reinterpret_cast<float4 *>(po + g * HD)[d4] = s4;
            }
        }
    } else {
#pragma unroll
        for (int g = 0; g < GM; ++g)
            if (g < G) reinterpret_cast<float4 *>(po + g * HD)[d4] = acc[g];
    }
}

// Merge: one workgroup per (query head, sequence, 64-dimension slice); four
// groups take interleaved split partials (np of them, in ascending order
// within a group), each with a running maximum: the maxima, sums and
// partial vectors are requested together (one memory round trip), every
// batch of kU partials rescales what came before by exp(m_old - m_new), and
// the four groups are combined in a fixed order, rescaled to the largest
// maximum.  So the result does not depend on scheduling.
__global__ __launch_bounds__(kWG) void attn_merge_kernel(const float *__restrict__ part, int G,
                                                         int Hkv, int np, int GM, int hd,
                                                         float *__restrict__ out, int64_t ldo,
                                                         int B) {
    __shared__ float rm[3][64], rn[3][64], rd[3][64];
    const int h = blockIdx.x, b = blockIdx.y;
    const int g0 = h / G, g = h % G;
    const int cg = threadIdx.x >> 6, dl = threadIdx.x & 63;
    const int d = blockIdx.z * 64 + dl;
    const size_t units_total = static_cast<size_t>(B) * Hkv * np * GM;
    const float *pml = part + units_total * hd;
    const size_t u0 = (static_cast<size_t>(b) * Hkv + g0) * np * GM + g;
    float M = -INFINITY, num = 0.f, den = 0.f;
    constexpr int kU = 8;  // partials in flight per thread, added in ascending order
    for (int c0 = cg; c0 < np; c0 += 4 * kU) {
        float lv[kU], mv[kU], pv[kU];
#pragma unroll
        for (int r = 0; r < kU; ++r) {
            const int c = min(c0 + 4 * r, np - 1);
            const size_t u = u0 + static_cast<size_t>(c) * GM;
            lv[r] = pml[2 * u + 1];
            mv[r] = pml[2 * u];
            pv[r] = d < hd ? part[u * hd + d] : 0.f;
        }
        float mb = M;
#pragma unroll
        for (int r = 0; r < kU; ++r)
            if (c0 + 4 * r < np && lv[r] > 0.f) mb = fmaxf(mb, mv[r]);
        if (mb > M) {  // rescale what the earlier batches added (nothing before the first)
            const float a = __expf(M - mb);
            num *= a;
            den *= a;
            M = mb;
        }
#pragma unroll
        for (int r = 0; r < kU; ++r) {
            if (c0 + 4 * r < np && lv[r] > 0.f) {
                const float w = __expf(mv[r] - M);
                num = __builtin_fmaf(w, pv[r], num);
                den = __builtin_fmaf(w, lv[r], den);
            }
        }
    }
    if (cg > 0) {
        rm[cg - 1][dl] = M;
        rn[cg - 1][dl] = num;
        rd[cg - 1][dl] = den;
    }
    __syncthreads();
    if (cg == 0 && d < hd) {
        float Mx = M;
        for (int k = 0; k < 3; ++k) Mx = fmaxf(Mx, rm[k][dl]);
        if (Mx == -INFINITY) {  // no key at all
            out[b * ldo + static_cast<int64_t>(h) * hd + d] = 0.f;
            return;
        }
        const float a0 = __expf(M - Mx);  // 0 for a group without partials
        num *= a0;
        den *= a0;
        for (int k = 0; k < 3; ++k) {
            const float a = __expf(rm[k][dl] - Mx);
            num = __builtin_fmaf(a, rn[k][dl], num);
            den = __builtin_fmaf(a, rd[k][dl], den);
        }
        out[b * ldo + static_cast<int64_t>(h) * hd + d] = den > 0.f ? num / den : 0.f;
    }
}

template <int HD, bool ROPE, bool MULTI, typename KT>
void launch_split_hd(int GM, dim3 grid, hipStream_t s, const float *q, int64_t ldq, int G,
                     const KT *kc, const KT *vc, const q4_kv_layout &kv,
                     const int64_t *n_dev, int64_t window, float scale, int ns, int cps, float *part,
                     const RopeArgs &ra) {
#define Q4_ATTN_CASE(GG)                                                                          \
    case GG:                                                                                      \
        hipLaunchKernelGGL((attn_split_kernel<HD, GG, ROPE, MULTI, KT>), grid, dim3(kWG), 0, s, q, ldq, G, kc, \
                           vc, kv.cap, kv.stride_b, kv.stride_h, kv.stride_t, n_dev, window, scale, \
                           ns, cps, part, ra);                                                    \
        break;
    switch (GM) { Q4_ATTN_CASE(1) Q4_ATTN_CASE(2) Q4_ATTN_CASE(4) Q4_ATTN_CASE(8) Q4_ATTN_CASE(16) }
#undef Q4_ATTN_CASE
}

int round_group(int G) {
    int gm = 1;
    while (gm < G) gm *= 2;
    return gm;
}

}  // namespace

extern "C" size_t gqa_decode_attn_workspace(const q4_kv_layout *kv, int64_t n_q_heads,
                                            int64_t window) {
    if (!kv || kv->n_kv_heads < 1 || n_q_heads < 1 || n_q_heads % kv->n_kv_heads || kv->cap < 1 ||
        kv->batch < 1 || kv->head_dim < 1 || window < 0)
        return 0;
    AttnGeom g = attn_geom(*kv, n_q_heads, window);
    q4_kv_layout k2 = *kv;
    // partial rows are stored padded to the kernel's group size
    const int gm = round_group(g.G);
    const size_t units = static_cast<size_t>(k2.batch) * k2.n_kv_heads * g.ns * gm;
    return units * (static_cast<size_t>(k2.head_dim) + 2) * sizeof(float);
}

namespace {
// The split kernel for head_dim hd, cache element type KT, with or without the
// fused preparation, one or several chunks per split.
template <typename KT>
void launch_split(int64_t hd, int gm, dim3 grid, hipStream_t s, const float *q, int64_t ldq, int G,
                  const void *k_cache, const void *v_cache, const q4_kv_layout &kv,
                  const int64_t *n_dev, int64_t window, float scale, const AttnGeom &g, float *part,
                  const RopeArgs *ra) {
    const KT *kc = static_cast<const KT *>(k_cache), *vc = static_cast<const KT *>(v_cache);
    const RopeArgs none{};
#define Q4_ATTN_HD(H)                                                                             \
    case H:                                                                                       \
        if (ra && g.cps > 1)                                                                      \
            launch_split_hd<H, true, true, KT>(gm, grid, s, q, ldq, G, kc, vc, kv, n_dev, window,  \
                                               scale, g.ns, g.cps, part, *ra);                    \
        else if (ra)                                                                              \
            launch_split_hd<H, true, false, KT>(gm, grid, s, q, ldq, G, kc, vc, kv, n_dev, window, \
                                                scale, g.ns, g.cps, part, *ra);                   \
        else if (g.cps > 1)                                                                       \
            launch_split_hd<H, false, true, KT>(gm, grid, s, q, ldq, G, kc, vc, kv, n_dev, window, \
                                                scale, g.ns, g.cps, part, none);                  \
        else                                                                                      \
            launch_split_hd<H, false, false, KT>(gm, grid, s, q, ldq, G, kc, vc, kv, n_dev,       \
                                                 window, scale, g.ns, g.cps, part, none);         \
        break;
    switch (hd) { Q4_ATTN_HD(64) Q4_ATTN_HD(128) Q4_ATTN_HD(256) Q4_ATTN_HD(512) }
#undef Q4_ATTN_HD
}

// Validation and launch shared by gqa_decode_attn and gqa_decode_attn_rope.
q4_status attn_entry(const char *name, const float *q, int64_t ldq, int64_t n_q_heads,
                     const void *k_cache, const void *v_cache, const q4_kv_layout *kv,
                     const int64_t *n_dev, int64_t window, float scale, float *out, int64_t ldo,
                     void *ws, size_t ws_bytes, void *stream, const RopeArgs *ra) {
    q4_status st = q4::check_kv_layout(name, kv);
    if (st != Q4_OK) return st;
    Q4_CHECK(q && k_cache && v_cache && n_dev && out, Q4_ERR_INVALID_ARG,
             "%s: q, caches, the position / count and out must not be NULL", name);
    Q4_CHECK(window >= 0, Q4_ERR_INVALID_ARG, "%s: window must be >= 0", name);
    Q4_CHECK(n_q_heads >= 1 && n_q_heads % kv->n_kv_heads == 0, Q4_ERR_SHAPE,
             "%s: n_q_heads %lld is not a multiple of n_kv_heads %lld", name, (long long)n_q_heads,
             (long long)kv->n_kv_heads);
    const int64_t hd = kv->head_dim;
    Q4_CHECK(hd == 64 || hd == 128 || hd == 256 || hd == 512, Q4_ERR_UNSUPPORTED,
             "%s: head_dim %lld not in {64, 128, 256, 512}", name, (long long)hd);
    const int G = static_cast<int>(n_q_heads / kv->n_kv_heads);
    Q4_CHECK(G <= 16, Q4_ERR_UNSUPPORTED, "%s: %d query heads per kv head > 16", name, G);
    Q4_CHECK(ldq >= n_q_heads * hd && ldo >= n_q_heads * hd, Q4_ERR_SHAPE,
             "%s: row strides smaller than the rows", name);
    Q4_CHECK(kv->stride_t % 4 == 0 && kv->stride_h % 4 == 0 && kv->stride_b % 4 == 0 && ldq % 4 == 0,
             Q4_ERR_ALIGNMENT, "%s: cache strides and row strides must be multiples of 4", name);
    Q4_CHECK(q4::aligned(q, 16) && q4::aligned(k_cache, 16) && q4::aligned(v_cache, 16) &&
                 q4::aligned(out, 4) && q4::aligned(n_dev, 8),
             Q4_ERR_ALIGNMENT, "%s: q and caches must be 16-byte aligned", name);
    const size_t need = gqa_decode_attn_workspace(kv, n_q_heads, window);
    Q4_CHECK(ws && ws_bytes >= need && q4::aligned(ws, 256), Q4_ERR_WORKSPACE,
             "%s: workspace of %zu bytes (256-byte aligned) needed, got %zu", name, need, ws_bytes);
    AttnGeom g = attn_geom(*kv, n_q_heads, window);
    const int gm = round_group(G);
    hipStream_t s = q4::as_stream(stream);
    float *part = static_cast<float *>(ws);
    dim3 grid(g.ns, static_cast<unsigned>(kv->n_kv_heads), static_cast<unsigned>(kv->batch));
    if (kv->dtype == Q4_KV_F16)
        launch_split<_Float16>(hd, gm, grid, s, q, ldq, G, k_cache, v_cache, *kv, n_dev, window, scale,
                               g, part, ra);
    else
        launch_split<float>(hd, gm, grid, s, q, ldq, G, k_cache, v_cache, *kv, n_dev, window, scale, g,
                            part, ra);
    q4_status ls = q4::launch_status(name);
    if (ls != Q4_OK) return ls;
    hipLaunchKernelGGL(attn_merge_kernel,
                       dim3(static_cast<unsigned>(n_q_heads), static_cast<unsigned>(kv->batch),
                            static_cast<unsigned>((hd + 63) / 64)),
                       dim3(kWG), 0, s, part, G, static_cast<int>(kv->n_kv_heads), g.ns, gm,
                       static_cast<int>(hd), out, ldo, static_cast<int>(kv->batch));
    return q4::launch_status(name);
}
}  // namespace

extern "C" q4_status gqa_decode_attn(const float *q, int64_t ldq, int64_t n_q_heads,
                                     const void *k_cache, const void *v_cache,
                                     const q4_kv_layout *kv, const int64_t *n_dev, int64_t window,
                                     float scale, float *out, int64_t ldo, void *ws,
                                     size_t ws_bytes, void *stream) {
    q4::clear_error();
    return attn_entry("gqa_decode_attn", q, ldq, n_q_heads, k_cache, v_cache, kv, n_dev, window,
                      scale, out, ldo, ws, ws_bytes, stream, nullptr);
}

extern "C" q4_status gqa_decode_attn_rope(const float *qkv, int64_t ld, int64_t n_q_heads,
                                          const float *q_norm, const float *k_norm,
                                          const q4_kv_layout *kv, const int64_t *pos_dev,
                                          double theta, float eps, int v_from_k, void *k_cache,
                                          void *v_cache, int64_t window, float scale, float *out,
                                          int64_t ldo, void *ws, size_t ws_bytes, void *stream) {
    q4::clear_error();
    const char *name = "gqa_decode_attn_rope";
    Q4_CHECK(kv && qkv && q_norm && k_norm, Q4_ERR_INVALID_ARG,
             "%s: qkv, q_norm, k_norm and kv must not be NULL", name);
    Q4_CHECK(theta > 0.0 && eps >= 0.f, Q4_ERR_INVALID_ARG, "%s: theta > 0, eps >= 0", name);
    const int64_t nq = n_q_heads * kv->head_dim, nk = kv->n_kv_heads * kv->head_dim;
    Q4_CHECK(ld >= nq + nk + (v_from_k ? 0 : nk), Q4_ERR_SHAPE, "%s: ld smaller than q | k | v", name);
    Q4_CHECK(q4::aligned(q_norm, 16) && q4::aligned(k_norm, 16) && ld % 4 == 0, Q4_ERR_ALIGNMENT,
             "%s: gains must be 16-byte aligned and ld a multiple of 4", name);
    RopeArgs ra;
    ra.kraw = qkv + nq;
    ra.vraw = v_from_k ? nullptr : qkv + nq + nk;
    ra.ldkv = ld;
    ra.qn = q_norm;
    ra.kn = k_norm;
    ra.rstep = std::pow(theta, -2.0 / static_cast<double>(kv->head_dim));
    ra.eps = eps;
    ra.kcw = k_cache;
    ra.vcw = v_cache;
    return attn_entry(name, qkv, ld, n_q_heads, k_cache, v_cache, kv, pos_dev, window, scale, out,
                      ldo, ws, ws_bytes, stream, &ra);
}
