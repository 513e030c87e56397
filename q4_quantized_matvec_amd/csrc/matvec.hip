// Q4_0 / Q8_0 dequant-matvec and the Q8_0 embedding gather for gfx950.
//
// Block formats (Research record, "Native Metal diagnostic: buffer ownership":
// 18-byte Q4_0 blocks = binary16 scale + 16 payload bytes, weight =
// (quant - 8) * scale; "Verified model facts": Q8_0 token table):
//   Q4_0: [d:f16][16 code bytes]; byte j = element j (low) | element j+16 (high)
//   Q8_0: [d:f16][32 int8 codes]
//
// Fast path (B = 1, K % 256 == 0): one wavefront walks a contiguous range of
// output rows.  Lane l owns block columns l, l+64, ... of its K range and keeps
// their 32 activations in VGPRs for the whole kernel, so activations are read
// from memory once per wavefront and the weight bytes are the only stream.
// Per row every lane issues one 16-byte load of its block's codes (the 2-byte
// alignment is served by the hardware as a single dwordx4) plus the 2-byte
// scale, one row ahead of the arithmetic.  Adjacent lanes read adjacent
// blocks, so a wavefront's loads of one row cover 1152 contiguous bytes.
//
// Q4_0 arithmetic: each 4-bit code is moved into the low bits of a 16-bit lane
// with a mask, which makes it the binary16 subnormal q * 2^-24.  v_fma_mix_f32
// widens that half exactly and multiplies it with the fp32 activation, so
// every product q * x is formed exactly in one FMA and no convert is needed:
//   s = sum_j q_j x_j * 2^-24 ;  y += d * (s * 2^24 - 8 * sum_j x_j)
// (the per-block sum of activations is computed once, at load time).
//
// Large K is split over the four wavefronts of a workgroup (2 or 4 parts)
// whose partial sums meet in LDS and are added in a fixed order.
#include "common.hpp"

namespace {
using namespace q4dev;

constexpr int kWG = 256;

template <int FMT>
struct Fmt;
template <>
struct Fmt<0> {  // Q4_0
    static constexpr int kBytes = 18;
    static constexpr int kDwords = 4;
};
template <>
struct Fmt<1> {  // Q8_0
    static constexpr int kBytes = 34;
    static constexpr int kDwords = 8;
};

// One row's raw words per owned column: the 4-byte-aligned window holding
// the block (kDwords + 1 words) and the row's residual.
// Transform applied to the activation rows as they are read (fuses the
// producer of the matvec input into its prologue):
//   kind 0: x
//   kind 1: rmsnorm(x) = w * x / sqrt(mean(x^2) + eps)   (w NULL: unit gain)
//   kind 2: act(x) * u, act = silu (x / (1 + exp(-x))) or gelu (tanh form)
//   post-norm (the kernels' POST parameter, with kind 1): x is the residual
//   stream h and u a block output z; the input is rmsnorm(h') with
//   h' = h + pw * z / sqrt(mean(z^2) + eps), and workgroup 0 of each row
//   writes h' to hout
struct InOp {
    int kind;
    const float *u;  // kind 2: second operand; post-norm: z; same row stride as x
    const float *w;  // kind 1: gain
    float eps;
    int64_t ld;      // row stride of x (and u, hout) in elements
    int glu;         // 1 / 2: y[p] = act(z[p]) * z[p + N/2] for the N/2 pairs, act = silu / gelu
                     // (whole K per wavefront)
    int act;         // kind 2: 0 silu, 1 gelu
    const float *pw; // post-norm gain
    float *hout;     // post-norm: h'
};

// act(g) * u with act = SiLU or (GELU) the tanh form of GELU.  A template
// parameter, not a runtime flag: the GELU code would otherwise sit in every
// instantiation, and kernels that start with cold instruction caches (one
// after another in a decode step) are measurably slower when larger.
template <bool GELU>
__device__ __forceinline__ float act_mul(float g, float u) {
    if constexpr (GELU) return 0.5f * g * (1.0f + tanhf(0.7978845608028654f * (g + 0.044715f * g * g * g))) * u;
    else return g / (1.0f + expf(-g)) * u;
}
// The runtime form, for the generic (slow-path) kernel.
__device__ __forceinline__ float glu_mul(int a, float g, float u) {
    return a ? act_mul<true>(g, u) : act_mul<false>(g, u);
}

// Sum of the staged float4 t over the 8 consecutive lanes that hold one
// 32-element block (lanes 8m .. 8m+7); every lane of the group gets it.  The
// adds run in a fixed order, so the sums are reproducible.  All lanes must be
// active.
__device__ __forceinline__ float block_sum8(float4 t) {
    float p = (t.x + t.y) + (t.z + t.w);
    p += dpp<0xB1>(p);   // quad_perm [1,0,3,2]
    p += dpp<0x4E>(p);   // quad_perm [2,3,0,1]
    p += dpp<0x141>(p);  // row_half_mirror: the other quad of the 8
    return p;
}

template <int FMT, int JX>
struct RowRegs {
    uint32_t w[JX][Fmt<FMT>::kDwords + 1];
    float res;  // residual of the row (read from a valid dummy address when there is none)
};

// Loads one row's blocks for the lane's columns.  Every load is issued
// unconditionally (columns past the end are clamped to a real block and their
// activations are zero), so the compiler can count outstanding loads exactly
// and never has to drain the queue with vmcnt(0).
//
// A block starts at byte 18c (34c for Q8_0), i.e. at 0 or 2 mod 4.  Loads are
// issued from the 4-byte-aligned address at or below the block start (2-byte
// aligned 16-byte loads stream far slower than 4-byte aligned ones); the
// words are re-aligned in registers by selectors that depend only on the
// parity of the column, which is fixed per lane.
template <int FMT, int JX>
__device__ __forceinline__ void load_row(const uint8_t *wrow, const int (&col)[JX],
                                         const float *resp, RowRegs<FMT, JX> &r) {
    r.res = *resp;
#pragma unroll
    for (int j = 0; j < JX; ++j) {
        const uint8_t *b = wrow + ((static_cast<size_t>(col[j]) * Fmt<FMT>::kBytes) & ~size_t(3));
#pragma unroll
        for (int h = 0; h < Fmt<FMT>::kDwords / 4; ++h) {
            const u32x4_a4 v = *reinterpret_cast<const u32x4_a4 *>(b + 16 * h);
            r.w[j][4 * h + 0] = v.x;
            r.w[j][4 * h + 1] = v.y;
            r.w[j][4 * h + 2] = v.z;
            r.w[j][4 * h + 3] = v.w;
        }
        r.w[j][Fmt<FMT>::kDwords] = *reinterpret_cast<const uint32_t *>(b + 4 * Fmt<FMT>::kDwords);
    }
}

// Blocks per K part when KS wavefronts split a row: rounded up to a multiple
// of 8 so every part starts on an even column.
__host__ __device__ inline int ks_part_blocks(int nb, int ks) { return ((nb + ks - 1) / ks + 7) / 8 * 8; }

// Tunables of the B = 1 path (compile-time).
#ifndef Q4_MV_PREFETCH
#define Q4_MV_PREFETCH 2  // rows of loads in flight ahead of the row being reduced
#endif
#ifndef Q4_MV_PREFETCH_JX1
#define Q4_MV_PREFETCH_JX1 4  // K <= 2048 (one block column per lane): 5.45 -> 4.98 us at 2048 x 6144
#endif
#ifndef Q4_MV_PREFETCH_Q8
#define Q4_MV_PREFETCH_Q8 1
#endif
#ifndef Q4_MV_X_LDS
#define Q4_MV_X_LDS 1     // stage the activations through LDS once per workgroup
#endif
#ifndef Q4_MV_WG_PER_CU
#define Q4_MV_WG_PER_CU 0 // 0: chosen from the register footprint
#endif
#ifndef Q4_MV_KS_MIN
#define Q4_MV_KS_MIN 1    // smallest K split (wavefronts per row) considered
#endif
#ifndef Q4_MV_KS_PER_CU
#define Q4_MV_KS_PER_CU 1 // workgroups per CU when K is split over wavefronts
#endif
#ifndef Q4_MV_MIN_ROWS
#define Q4_MV_MIN_ROWS 7  // rows per wavefront that amortise a workgroup's staging of x
#endif
#ifndef Q4_MV_MIN_ROWS_JX1
#define Q4_MV_MIN_ROWS_JX1 7
#endif
#ifndef Q4_MV_MAX_JX
#define Q4_MV_MAX_JX 4    // most block columns per lane before K is split over wavefronts
#endif
#ifndef Q4_MV_MIN_WAVES
#define Q4_MV_MIN_WAVES 1 // occupancy hint (waves per SIMD) for the register allocator
#endif

constexpr int kXLdsFloats = 8192;  // LDS staging of x when the whole K fits

// B = 1 fast path.  KS wavefronts of a workgroup split K; 4 / KS row groups;
// PF rows of loads in flight per wavefront.
// With three Q4_0 block columns per lane (K up to 6144) the kernel fits three
// wavefronts per SIMD only at <= 168 VGPRs; the launch bound holds it there.
template <int FMT, int JX, int KS, int PF, bool GLU, bool GELU, bool POST>
__global__ __launch_bounds__(kWG, FMT == 0 && JX == 3 && KS == 1 ? 3 : Q4_MV_MIN_WAVES) void mv_b1_kernel(const uint8_t *__restrict__ W,
                                                    const float *x, float *y, const float *res,
                                                    int N, int K, InOp op) {
    constexpr int RG = 4 / KS;
    constexpr int NBUF = PF + 1;
    // batch row of this workgroup (each batch row streams the matrix itself;
    // repeated passes are mostly served by the last-level cache)
    {
        const int64_t b = blockIdx.y;
        x += b * op.ld;
        if (op.u) op.u += b * op.ld;
        if (POST) op.hout += b * op.ld;
        y += b * static_cast<int64_t>(GLU ? N / 2 : N);
        if (res) res += b * static_cast<int64_t>(N);
    }
    constexpr bool kXLds = Q4_MV_X_LDS && KS == 1;
    __shared__ float red[4];
    constexpr int kFlush = 32;  // split-K rows reduced per barrier pair
    __shared__ float kpart[KS > 1 ? 4 * kFlush : 1];
    __shared__ float kres[KS > 1 ? 4 * kFlush : 1];
    __shared__ float xs[kXLds ? kXLdsFloats : 1];
    __shared__ float xsum[kXLds ? kXLdsFloats / 32 : 1];  // per-block sums of the staged activations
    const int lane = threadIdx.x & 63;
    // wave-uniform: keeps row addressing in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ks = wave % KS;
    const int rg = wave / KS;
    const int nb = K >> 5;
    const int nbw = ks_part_blocks(nb, KS);
    const int c0 = ks * nbw;
    const int c1 = min(nb, c0 + nbw);
    const size_t row_bytes = static_cast<size_t>(nb) * Fmt<FMT>::kBytes;

    // Contiguous row range of this row group (sizes differ by at most one).
    // Output units: rows, or (gate row p, up row p + N/2) pairs with a SwiGLU
    // output, processed as two consecutive iterations.
    const int G = gridDim.x * RG;
    const int g = blockIdx.x * RG + rg;
    const int units = GLU ? N / 2 : N;
    const int per = GLU ? 2 : 1;
    const int q = units / G, r = units % G;
    const int cnt = per * (q + (g < r ? 1 : 0));
    const int row0 = g * q + min(g, r);
    const int iters = per * (q + (r > 0 ? 1 : 0));  // same for every wavefront of the grid

    bool valid[JX];
    int col[JX];
#pragma unroll
    for (int j = 0; j < JX; ++j) {
        const int c = c0 + lane + 64 * j;
        valid[j] = c < c1;
        col[j] = min(c, nb - 1);
    }
    // Byte offset of the block inside its aligned window: 0 for even columns,
    // 2 for odd ones (c0 is a multiple of 8 and the clamp target nb - 1 is odd,
    // so the parity of every owned column is the lane's parity).  v_perm_b32
    // selectors: code word i = window bytes [off+2+4i, off+6+4i) out of the
    // pair (w[i+1]:w[i]); scale = window bytes [off, off+2) zero-extended.
    const bool odd = lane & 1;
    const uint32_t sel_q = odd ? 0x07060504u : 0x05040302u;
    const uint32_t sel_d = odd ? 0x0C0C0302u : 0x0C0C0100u;
    // Q4_0: code bytes 4i, 4i+2 (sel_e) or 4i+1, 4i+3 (sel_o) of word i, each
    // zero-extended into a 16-bit lane.
    const uint32_t sel_e = odd ? 0x0C060C04u : 0x0C040C02u;
    const uint32_t sel_o = odd ? 0x0C070C05u : 0x0C050C03u;

    // Without a residual the residual slot reads x[0] and is ignored.
    const bool has_res = res != nullptr;
    // Iterations past the group's range re-read its last row (already in this
    // CU's caches) instead of the next group's first rows.
    const int ulast = min(row0 + max(cnt / per, 1) - 1, units - 1);
    auto fetch = [&](int it, RowRegs<FMT, JX> &r) {
        const int un = min(row0 + (GLU ? (it >> 1) : it), ulast);
        const int row = (GLU && (it & 1)) ? un + units : un;
        load_row<FMT, JX>(W + static_cast<size_t>(row) * row_bytes, col, has_res ? res + row : x, r);
    };
    RowRegs<FMT, JX> buf[NBUF];
    // The activation loads go out before the first rows: loads return in
    // order, so activations requested after the rows would wait for them.
    // Without LDS staging the rows go first.
    if constexpr (!kXLds) {
#pragma unroll
        for (int p = 0; p < PF; ++p) fetch(p, buf[p]);
    }

    // Activations of the lane's block columns stay in registers.  With the
    // whole K in one wavefront the workgroup stages x through LDS once; the
    // input transform is applied on the way (sum of squares reduced in LDS).
    float inv = 1.f;
    if constexpr (POST) {
        static_assert(kXLds, "the post-norm input is staged through LDS");
        // Post-norm: h' = h + pw * z / rms(z), then RMSNorm of h' as for kind
        // 1.  Every operand of the row is requested before the first weight
        // rows (loads return in order); z's sum of squares is reduced first.
        // K <= 2048 JX here, so 2 JX float4 per thread cover the row.
        constexpr int kXV = 2 * JX;
        static_assert(kXV * 4 * kWG <= kXLdsFloats, "row staging");
        const int nv = K >> 2;
        const float4 *hg = reinterpret_cast<const float4 *>(x);
        const float4 *zg = reinterpret_cast<const float4 *>(op.u);
        const float4 *pg = reinterpret_cast<const float4 *>(op.pw);
        const float4 *gg = reinterpret_cast<const float4 *>(op.w);
        float4 *xl = reinterpret_cast<float4 *>(xs);
        float4 *ho = reinterpret_cast<float4 *>(op.hout);
        float4 zv[kXV], hv[kXV], pv[kXV], gv[kXV];
#pragma unroll
        for (int r = 0; r < kXV; ++r) {
            const int i = min(static_cast<int>(threadIdx.x) + r * kWG, nv - 1);
            zv[r] = zg[i];
            hv[r] = hg[i];
            pv[r] = pg[i];
            gv[r] = gg ? gg[i] : make_float4(1.f, 1.f, 1.f, 1.f);
        }
#pragma unroll
        for (int p = 0; p < PF; ++p) fetch(p, buf[p]);
        float sz = 0.f;
#pragma unroll
        for (int r = 0; r < kXV; ++r)
            if (static_cast<int>(threadIdx.x) + r * kWG < nv)
                sz = __builtin_fmaf(zv[r].x, zv[r].x, __builtin_fmaf(zv[r].y, zv[r].y,
                     __builtin_fmaf(zv[r].z, zv[r].z, __builtin_fmaf(zv[r].w, zv[r].w, sz))));
        sz = wave_sum(sz);
        if (lane == 0) red[wave] = sz;
        __syncthreads();
        const float rz = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / static_cast<float>(K) + op.eps);
        __syncthreads();  // red[] is reused for h'
        const bool writer = blockIdx.x == 0;
        float ss = 0.f;
#pragma unroll
        for (int r = 0; r < kXV; ++r) {
            const int i = threadIdx.x + r * kWG;
            float4 t;
            t.x = __builtin_fmaf(pv[r].x, zv[r].x * rz, hv[r].x);
            t.y = __builtin_fmaf(pv[r].y, zv[r].y * rz, hv[r].y);
            t.z = __builtin_fmaf(pv[r].z, zv[r].z * rz, hv[r].z);
            t.w = __builtin_fmaf(pv[r].w, zv[r].w * rz, hv[r].w);
            if (i < nv) {
                if (writer) ho[i] = t;
                ss = __builtin_fmaf(t.x, t.x, __builtin_fmaf(t.y, t.y, __builtin_fmaf(t.z, t.z, __builtin_fmaf(t.w, t.w, ss))));
            }
            t.x *= gv[r].x;
            t.y *= gv[r].y;
            t.z *= gv[r].z;
            t.w *= gv[r].w;
            const float bs = block_sum8(t);  // K is a multiple of 256: no group straddles nv
            if (i < nv) {
                xl[i] = t;
                if ((i & 7) == 0) xsum[i >> 3] = bs;
            }
        }
        ss = wave_sum(ss);
        if (lane == 0) red[wave] = ss;
        __syncthreads();
        inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / static_cast<float>(K) + op.eps);
        __syncthreads();
    } else if constexpr (kXLds) {
        const float4 *xg = reinterpret_cast<const float4 *>(x);
        const float4 *ug = reinterpret_cast<const float4 *>(op.u);
        float4 *xl = reinterpret_cast<float4 *>(xs);
        float ss = 0.f;
        // every load of the row first (one memory round trip), then the
        // transform and the LDS stores; indices past the row re-read its last
        // element and are not stored
        // (RMSNorm: the gain is applied here and 1/rms once the sum of
        // squares is known; SwiGLU: u is loaded alongside)
        constexpr int kXV = kXLdsFloats / 4 / kWG;
        const int nv = K >> 2;
        const float4 *sg = op.kind == 2 ? ug : reinterpret_cast<const float4 *>(op.w);
        float4 v[kXV], u[kXV];
#pragma unroll
        for (int r = 0; r < kXV; ++r) v[r] = xg[min(static_cast<int>(threadIdx.x) + r * kWG, nv - 1)];
        if (sg) {
#pragma unroll
            for (int r = 0; r < kXV; ++r) u[r] = sg[min(static_cast<int>(threadIdx.x) + r * kWG, nv - 1)];
        }
#pragma unroll
        for (int p = 0; p < PF; ++p) fetch(p, buf[p]);
#pragma unroll
        for (int r = 0; r < kXV; ++r) {
            const int i = threadIdx.x + r * kWG;
            float4 t = v[r];
            if (op.kind == 2) {
                t.x = act_mul<GELU>(t.x, u[r].x);
                t.y = act_mul<GELU>(t.y, u[r].y);
                t.z = act_mul<GELU>(t.z, u[r].z);
                t.w = act_mul<GELU>(t.w, u[r].w);
            }
            if (i < nv)
                ss = __builtin_fmaf(t.x, t.x, __builtin_fmaf(t.y, t.y, __builtin_fmaf(t.z, t.z, __builtin_fmaf(t.w, t.w, ss))));
            if (op.kind == 1 && sg) {
                t.x *= u[r].x;
                t.y *= u[r].y;
                t.z *= u[r].z;
                t.w *= u[r].w;
            }
            const float bs = block_sum8(t);  // K is a multiple of 256: no group straddles nv
            if (i < nv) {
                xl[i] = t;
                if ((i & 7) == 0) xsum[i >> 3] = bs;
            }
        }
        if (op.kind == 1) {
            ss = wave_sum(ss);
            if (lane == 0) red[wave] = ss;
        }
        __syncthreads();
        if (op.kind == 1) {
            inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / static_cast<float>(K) + op.eps);
            __syncthreads();  // red[] is reused by the row reductions of split-K shapes
        }
    } else if (op.kind == 1) {
        // every wavefront reduces the whole row itself, 8 loads in flight per lane
        float ss = 0.f;
        const float4 *xg = reinterpret_cast<const float4 *>(x);
        const int nv = K >> 2;
        for (int i0 = 0; i0 < nv; i0 += 8 * 64) {
            float4 v[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) v[r] = xg[min(i0 + lane + 64 * r, nv - 1)];
#pragma unroll
            for (int r = 0; r < 8; ++r)
                if (i0 + lane + 64 * r < nv)
                    ss = __builtin_fmaf(v[r].x, v[r].x, __builtin_fmaf(v[r].y, v[r].y,
                         __builtin_fmaf(v[r].z, v[r].z, __builtin_fmaf(v[r].w, v[r].w, ss))));
        }
        inv = 1.0f / sqrtf(wave_sum(ss) / static_cast<float>(K) + op.eps);
    }
    // 1/rms is the same for the whole workgroup: keep it in a scalar register
    inv = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, inv)));
    float xr[JX][32];
    float xc[JX];
#pragma unroll
    for (int j = 0; j < JX; ++j) {
        const int c = c0 + lane + 64 * j;
        float s = 0.f;
        if (valid[j]) {
            const float4 *xp = kXLds ? reinterpret_cast<const float4 *>(xs + c * 32)
                                     : reinterpret_cast<const float4 *>(x + static_cast<size_t>(c) * 32);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float4 v = xp[i];
                if (!kXLds && op.kind == 2) {
                    const float4 u = reinterpret_cast<const float4 *>(op.u + static_cast<size_t>(c) * 32)[i];
                    v.x = act_mul<GELU>(v.x, u.x);
                    v.y = act_mul<GELU>(v.y, u.y);
                    v.z = act_mul<GELU>(v.z, u.z);
                    v.w = act_mul<GELU>(v.w, u.w);
                }
                xr[j][4 * i + 0] = v.x;
                xr[j][4 * i + 1] = v.y;
                xr[j][4 * i + 2] = v.z;
                xr[j][4 * i + 3] = v.w;
            }
            if (op.kind == 1 && !kXLds && op.w) {  // staged values already carry the gain
                const float4 *wg = reinterpret_cast<const float4 *>(op.w + static_cast<size_t>(c) * 32);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float4 g4 = wg[i];
                    xr[j][4 * i + 0] *= g4.x;
                    xr[j][4 * i + 1] *= g4.y;
                    xr[j][4 * i + 2] *= g4.z;
                    xr[j][4 * i + 3] *= g4.w;
                }
            }
            if constexpr (kXLds) {
                s = xsum[c];
            } else {
#pragma unroll
                for (int i = 0; i < 32; ++i) s += xr[j][i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 32; ++i) xr[j][i] = 0.f;
        }
        xc[j] = -8.f * s;
    }


    float gate = 0.f;  // SwiGLU output: the gate row's sum, kept for its pair
    auto process = [&](int it, const RowRegs<FMT, JX> &cur) {
        const bool act = it < cnt;
        float acc = 0.f;
        if (act) {
            // 2*JX independent FMA chains (blocks interleaved, low/high code
            // halves apart) so dependent-issue latency stays hidden.
            float sa[JX], sb[JX];
#pragma unroll
            for (int j = 0; j < JX; ++j) sa[j] = sb[j] = 0.f;
            if constexpr (FMT == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
#pragma unroll
                    for (int j = 0; j < JX; ++j) {
                        // e = code bytes (4i, 4i+2), o = (4i+1, 4i+3), one per 16-bit
                        // lane.  Low nibbles -> binary16 subnormals q * 2^-24; high
                        // nibbles stay in bits 4..7 (16 q * 2^-24) and are summed
                        // apart, the sum scaled by 1/16 once (exact).
                        const uint32_t e = __builtin_amdgcn_perm(cur.w[j][i + 1], cur.w[j][i], sel_e);
                        const uint32_t o = __builtin_amdgcn_perm(cur.w[j][i + 1], cur.w[j][i], sel_o);
                        const uint32_t le = e & 0x000F000Fu, he = e & 0x00F000F0u;
                        const uint32_t lo = o & 0x000F000Fu, ho = o & 0x00F000F0u;
                        sa[j] = fma_lo(le, xr[j][4 * i + 0], sa[j]);
                        sb[j] = fma_lo(he, xr[j][16 + 4 * i + 0], sb[j]);
                        sa[j] = fma_lo(lo, xr[j][4 * i + 1], sa[j]);
                        sb[j] = fma_lo(ho, xr[j][16 + 4 * i + 1], sb[j]);
                        sa[j] = fma_hi(le, xr[j][4 * i + 2], sa[j]);
                        sb[j] = fma_hi(he, xr[j][16 + 4 * i + 2], sb[j]);
                        sa[j] = fma_hi(lo, xr[j][4 * i + 3], sa[j]);
                        sb[j] = fma_hi(ho, xr[j][16 + 4 * i + 3], sb[j]);
                    }
                }
#pragma unroll
                for (int j = 0; j < JX; ++j) {
                    const float d = half_bits_to_float(__builtin_amdgcn_perm(0u, cur.w[j][0], sel_d));
                    // high nibbles were taken x16: sb / 16 (exact)
                    const float t = __builtin_fmaf(d, __builtin_fmaf(__builtin_fmaf(sb[j], 0.0625f, sa[j]), 16777216.f, xc[j]), acc);
                    acc = valid[j] ? t : acc;
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
#pragma unroll
                    for (int j = 0; j < JX; ++j) {
                        const uint32_t w = __builtin_amdgcn_perm(cur.w[j][i + 1], cur.w[j][i], sel_q);
                        sa[j] = __builtin_fmaf(static_cast<float>(static_cast<int8_t>(w)), xr[j][4 * i + 0], sa[j]);
                        sb[j] = __builtin_fmaf(static_cast<float>(static_cast<int8_t>(w >> 8)), xr[j][4 * i + 1], sb[j]);
                        sa[j] = __builtin_fmaf(static_cast<float>(static_cast<int8_t>(w >> 16)), xr[j][4 * i + 2], sa[j]);
                        sb[j] = __builtin_fmaf(static_cast<float>(static_cast<int8_t>(w >> 24)), xr[j][4 * i + 3], sb[j]);
                    }
                }
#pragma unroll
                for (int j = 0; j < JX; ++j) {
                    const float d = half_bits_to_float(__builtin_amdgcn_perm(0u, cur.w[j][0], sel_d));
                    const float t = __builtin_fmaf(d, sa[j] + sb[j], acc);
                    acc = valid[j] ? t : acc;
                }
            }
        }
        acc = wave_sum(acc) * inv;  // RMSNorm: 1/rms of the row, once per output
        const int row = row0 + it;
        if constexpr (KS == 1) {
            if constexpr (GLU) {
                if ((it & 1) == 0) gate = acc;
                else if (act && lane == 0) y[row0 + (it >> 1)] = act_mul<GELU>(gate, acc);
            } else if (act && lane == 0) {
                y[row] = has_res ? acc + cur.res : acc;
            }
        } else {
            // split K: park the partial (and the residual) in LDS; rows are
            // reduced in batches of kFlush with two barriers per batch
            const int slot = it % kFlush;
            if (lane == 0) {
                kpart[(rg * KS + ks) * kFlush + slot] = acc;
                if (ks == 0) kres[rg * kFlush + slot] = cur.res;
            }
            if (slot == kFlush - 1 || it + 1 == iters) {
                __syncthreads();
                if (ks == 0 && lane <= slot) {
                    const int r = it - slot + lane;
                    if (r < cnt) {
                        float v = kpart[(rg * KS) * kFlush + lane];
#pragma unroll
                        for (int k = 1; k < KS; ++k) v += kpart[(rg * KS + k) * kFlush + lane];  // fixed order
                        y[row0 + r] = has_res ? v + kres[rg * kFlush + lane] : v;
                    }
                }
                __syncthreads();
            }
        }
    };

    // Ring of NBUF register sets: row it lives in buf[it % NBUF]; the loads of
    // row it + PF are issued before row it is reduced.  The unrolled body keeps
    // every buffer index a compile-time constant and has no branch around a
    // load; the tail issues no loads.
    int it0 = 0;
    for (; it0 + NBUF <= iters; it0 += NBUF) {
#pragma unroll
        for (int u = 0; u < NBUF; ++u) {
            fetch(it0 + u + PF, buf[(u + PF) % NBUF]);
            process(it0 + u, buf[u]);
        }
    }
#pragma unroll
    for (int u = 0; u < NBUF; ++u)
        if (it0 + u < iters) process(it0 + u, buf[u]);
}

// Generic path: any K % 32 == 0, 1 <= B <= 8, scale/codes read as 16-bit words.
template <int FMT, int B, int KIND>
__global__ __launch_bounds__(kWG) void mv_generic_kernel(const uint8_t *__restrict__ W,
                                                         const float *__restrict__ x, float *y,
                                                         const float *res, int N, int K, InOp op) {
    const int lane = threadIdx.x & 63;
    const int nb = K >> 5;
    const size_t row_bytes = static_cast<size_t>(nb) * Fmt<FMT>::kBytes;
    const int waves = gridDim.x * (kWG / 64);
    float inv[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
        inv[b] = 1.f;
        if constexpr (KIND == 1) {
            float ss = 0.f;
            for (int i = lane; i < K; i += 64) ss = __builtin_fmaf(x[b * op.ld + i], x[b * op.ld + i], ss);
            inv[b] = 1.0f / sqrtf(wave_sum(ss) / static_cast<float>(K) + op.eps);
        }
    }
    for (int row = blockIdx.x * (kWG / 64) + (threadIdx.x >> 6); row < N; row += waves) {
        float acc[B];
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] = 0.f;
        for (int c = lane; c < nb; c += 64) {
            const uint16_t *h = reinterpret_cast<const uint16_t *>(W + row * row_bytes +
                                                                   static_cast<size_t>(c) * Fmt<FMT>::kBytes);
            const float d = half_bits_to_float(h[0]);
            float w[32];
            if constexpr (FMT == 0) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t v = h[1 + j];  // code bytes 2j (low 8 bits) and 2j+1
                    w[2 * j] = static_cast<float>(static_cast<int>(v & 15u) - 8);
                    w[2 * j + 16] = static_cast<float>(static_cast<int>((v >> 4) & 15u) - 8);
                    w[2 * j + 1] = static_cast<float>(static_cast<int>((v >> 8) & 15u) - 8);
                    w[2 * j + 17] = static_cast<float>(static_cast<int>((v >> 12) & 15u) - 8);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const uint32_t v = h[1 + j];
                    w[2 * j] = static_cast<float>(static_cast<int8_t>(v & 0xFFu));
                    w[2 * j + 1] = static_cast<float>(static_cast<int8_t>(v >> 8));
                }
            }
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const size_t off = static_cast<size_t>(b) * op.ld + static_cast<size_t>(c) * 32;
                const float *xb = x + off;
                float s = 0.f;
#pragma unroll
                for (int i = 0; i < 32; ++i) {
                    float xv = xb[i];
                    if constexpr (KIND == 1) xv = xv * inv[b] * (op.w ? op.w[c * 32 + i] : 1.0f);
                    else if constexpr (KIND == 2) xv = glu_mul(op.act, xv, op.u[off + i]);
                    s = __builtin_fmaf(w[i], xv, s);
                }
                acc[b] = __builtin_fmaf(d, s, acc[b]);
            }
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const float t = wave_sum(acc[b]);
            if (lane == 0) {
                const size_t o = static_cast<size_t>(b) * N + row;
                y[o] = t + (res ? res[o] : 0.f);
            }
        }
    }
}

// x[b][:] = dequantised row tokens[b] of a Q8_0 table; one thread per block.
__global__ __launch_bounds__(kWG) void q8_gather_kernel(const uint8_t *__restrict__ E,
                                                        const int32_t *__restrict__ tok,
                                                        float *__restrict__ x, int V, int K,
                                                        int B, float scale) {
    const int nb = K >> 5;
    const int t = blockIdx.x * kWG + threadIdx.x;
    if (t >= B * nb) return;
    const int b = t / nb, c = t % nb;
    const int id = tok[b];
    float *out = x + static_cast<size_t>(b) * K + static_cast<size_t>(c) * 32;
    if (id < 0 || id >= V) {
        for (int i = 0; i < 32; ++i) out[i] = __builtin_nanf("");
        return;
    }
    const uint8_t *blk = E + (static_cast<size_t>(id) * nb + c) * 34;
    const float d = half_bits_to_float(*reinterpret_cast<const uint16_t *>(blk));
    // scaled rows: (d * q) * scale, the product of the dequantised value and the scale
    const uint16_t *h = reinterpret_cast<const uint16_t *>(blk + 2);
    for (int j = 0; j < 16; ++j) {
        const uint32_t v = h[j];
        out[2 * j] = d * static_cast<float>(static_cast<int8_t>(v & 0xFFu)) * scale;
        out[2 * j + 1] = d * static_cast<float>(static_cast<int8_t>(v >> 8)) * scale;
    }
}

template <int FMT, int JX, int KS>
void launch_b1(const uint8_t *W, const float *x, float *y, const float *res, int N, int K,
               int B, const InOp &op, hipStream_t s) {
    constexpr int PF = FMT == 0 ? (JX == 1 ? Q4_MV_PREFETCH_JX1 : Q4_MV_PREFETCH) : Q4_MV_PREFETCH_Q8;
    constexpr int RG = 4 / KS;
    const int want = (N + RG - 1) / RG;
    // Workgroups per CU: every workgroup stages the whole activation row once,
    // so a workgroup should own enough rows to amortise that (measured on
    // the 31B projections: about 7 rows per wavefront with the whole K in
    // one wavefront; one workgroup per CU when K is split over wavefronts).
    int per_cu = KS > 1 ? Q4_MV_KS_PER_CU
                        : std::max(1, std::min(3, N / (q4::device_cus() * RG * (JX == 1 ? Q4_MV_MIN_ROWS_JX1 : Q4_MV_MIN_ROWS))));
    if (Q4_MV_WG_PER_CU) per_cu = Q4_MV_WG_PER_CU;
    const int nwg = std::max(1, std::min(want, per_cu * q4::device_cus()));
    // GeGLU kernels exist for Q4_0 only (the gated projections)
    const bool gelu = (op.kind == 2 && op.act) || op.glu == 2;
    if constexpr (FMT == 0 && KS == 1) {
        if (op.pw) {  // post-norm input (q4_0_matvec_post_norm)
            if (op.glu && gelu)
                hipLaunchKernelGGL((mv_b1_kernel<FMT, JX, KS, PF, true, true, true>), dim3(nwg, B), dim3(kWG), 0,
                                   s, W, x, y, res, N, K, op);
            else if (op.glu)
                hipLaunchKernelGGL((mv_b1_kernel<FMT, JX, KS, PF, true, false, true>), dim3(nwg, B), dim3(kWG), 0,
                                   s, W, x, y, res, N, K, op);
            else
                hipLaunchKernelGGL((mv_b1_kernel<FMT, JX, KS, PF, false, false, true>), dim3(nwg, B), dim3(kWG),
                                   0, s, W, x, y, res, N, K, op);
            return;
        }
    }
    if constexpr (KS == 1) {
        if (op.glu) {
            if constexpr (FMT == 0) {
                if (gelu) {
                    hipLaunchKernelGGL((mv_b1_kernel<FMT, JX, KS, PF, true, true, false>), dim3(nwg, B), dim3(kWG),
                                       0, s, W, x, y, res, N, K, op);
                    return;
                }
            }
            hipLaunchKernelGGL((mv_b1_kernel<FMT, JX, KS, PF, true, false, false>), dim3(nwg, B), dim3(kWG), 0, s,
                               W, x, y, res, N, K, op);
            return;
        }
    }
    if constexpr (FMT == 0) {
        if (gelu) {
            hipLaunchKernelGGL((mv_b1_kernel<FMT, JX, KS, PF, false, true, false>), dim3(nwg, B), dim3(kWG), 0, s,
                               W, x, y, res, N, K, op);
            return;
        }
    }
    hipLaunchKernelGGL((mv_b1_kernel<FMT, JX, KS, PF, false, false, false>), dim3(nwg, B), dim3(kWG), 0, s, W, x,
                       y, res, N, K, op);
}

template <int FMT, int KS>
void launch_b1_jx(int jx, const uint8_t *W, const float *x, float *y, const float *res, int N,
                  int K, int B, const InOp &op, hipStream_t s) {
    switch (jx) {
        case 1: launch_b1<FMT, 1, KS>(W, x, y, res, N, K, B, op, s); break;
        case 2: launch_b1<FMT, 2, KS>(W, x, y, res, N, K, B, op, s); break;
        case 3: launch_b1<FMT, 3, KS>(W, x, y, res, N, K, B, op, s); break;
        default: launch_b1<FMT, 4, KS>(W, x, y, res, N, K, B, op, s); break;
    }
}

template <int FMT>
void launch_generic(int B, const uint8_t *W, const float *x, float *y, const float *res, int N,
                    int K, const InOp &op, hipStream_t s) {
    const int nwg = std::max(1, std::min((N + 3) / 4, 4 * q4::device_cus()));
#define Q4_CASE(BB, KK) \
    case BB: hipLaunchKernelGGL((mv_generic_kernel<FMT, BB, KK>), dim3(nwg), dim3(kWG), 0, s, W, x, y, res, N, K, op); break;
#define Q4_SWITCH(KK) \
    switch (B) { Q4_CASE(1, KK) Q4_CASE(2, KK) Q4_CASE(3, KK) Q4_CASE(4, KK) Q4_CASE(5, KK) Q4_CASE(6, KK) Q4_CASE(7, KK) Q4_CASE(8, KK) }
    if (op.kind == 1) { Q4_SWITCH(1) }
    else if (op.kind == 2) { Q4_SWITCH(2) }
    else { Q4_SWITCH(0) }
#undef Q4_SWITCH
#undef Q4_CASE
}

bool ranges_overlap(const void *a, size_t an, const void *b, size_t bn) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + bn && y < x + an;
}

template <int FMT>
q4_status matvec_entry(const char *name, const void *Wv, int64_t N, int64_t K, const float *x,
                       const float *x2, int64_t ldx, int64_t B, int op_kind, int out_op,
                       const float *norm_w, float eps, float *y, const float *res, void *stream) {
    q4::clear_error();
    Q4_CHECK(out_op == Q4_OUT_PLAIN || out_op == Q4_OUT_SWIGLU || out_op == Q4_OUT_GEGLU,
             Q4_ERR_INVALID_ARG, "%s: unknown output transform %d", name, out_op);
    const bool glu_out = out_op != Q4_OUT_PLAIN;
    Q4_CHECK(!glu_out || (N % 2 == 0 && !res), Q4_ERR_INVALID_ARG,
             "%s: a gated (SwiGLU / GeGLU) output needs an even N and no residual", name);
    Q4_CHECK(Wv && x && y, Q4_ERR_INVALID_ARG, "%s: W, x and y must not be NULL", name);
    Q4_CHECK(N >= 1 && K >= 1 && B >= 1, Q4_ERR_INVALID_ARG, "%s: N=%lld K=%lld B=%lld must be >= 1",
             name, (long long)N, (long long)K, (long long)B);
    Q4_CHECK(op_kind >= Q4_IN_PLAIN && op_kind <= Q4_IN_GEGLU, Q4_ERR_INVALID_ARG,
             "%s: unknown input transform %d", name, op_kind);
    const bool gated_in = op_kind == Q4_IN_SWIGLU || op_kind == Q4_IN_GEGLU;
    Q4_CHECK(!gated_in || x2, Q4_ERR_INVALID_ARG, "%s: a gated input needs x2", name);
    Q4_CHECK(!(gated_in && glu_out) || (op_kind == Q4_IN_GEGLU) == (out_op == Q4_OUT_GEGLU),
             Q4_ERR_UNSUPPORTED, "%s: a gated input and a gated output must use the same activation",
             name);
    Q4_CHECK(FMT == 0 || (op_kind != Q4_IN_GEGLU && out_op != Q4_OUT_GEGLU), Q4_ERR_UNSUPPORTED,
             "%s: GeGLU transforms are provided for Q4_0 weights", name);
    Q4_CHECK(op_kind != Q4_IN_RMSNORM || eps >= 0.f, Q4_ERR_INVALID_ARG, "%s: eps must be >= 0", name);
    Q4_CHECK(ldx >= K, Q4_ERR_SHAPE, "%s: ld_x=%lld < K=%lld", name, (long long)ldx, (long long)K);
    Q4_CHECK(K % 32 == 0, Q4_ERR_SHAPE, "%s: K=%lld is not a multiple of 32", name, (long long)K);
    Q4_CHECK(B <= 8, Q4_ERR_UNSUPPORTED, "%s: B=%lld > 8", name, (long long)B);
    Q4_CHECK(N <= (1 << 30) && K <= (1 << 24) && ldx <= (1 << 26), Q4_ERR_UNSUPPORTED,
             "%s: N or K too large", name);
    Q4_CHECK(q4::aligned(Wv, 2), Q4_ERR_ALIGNMENT, "%s: W must be 2-byte aligned", name);
    Q4_CHECK(q4::aligned(x, 4) && q4::aligned(y, 4) && (!res || q4::aligned(res, 4)) &&
                 (!x2 || q4::aligned(x2, 4)) && (!norm_w || q4::aligned(norm_w, 4)),
             Q4_ERR_ALIGNMENT, "%s: x, x2, norm_w, y and residual must be 4-byte aligned", name);
    const uint8_t *W = static_cast<const uint8_t *>(Wv);
    hipStream_t s = q4::as_stream(stream);
    const int n = static_cast<int>(N), k = static_cast<int>(K);
    const int nb = k / 32;
    InOp op{gated_in ? 2 : op_kind, gated_in ? x2 : nullptr, op_kind == Q4_IN_RMSNORM ? norm_w : nullptr,
            eps, ldx, out_op == Q4_OUT_SWIGLU ? 1 : out_op == Q4_OUT_GEGLU ? 2 : 0,
            op_kind == Q4_IN_GEGLU ? 1 : 0};
    const bool x16 = K % 256 == 0 && q4::aligned(x, 16) && (!op.u || q4::aligned(op.u, 16)) &&
                     (!op.w || q4::aligned(op.w, 16)) && ldx % 4 == 0;
    int ks = 0;
    if (x16) {
        for (int cand : {1, 2, 4})
            if (cand >= Q4_MV_KS_MIN && ks_part_blocks(nb, cand) <= 64 * (cand == 4 ? 4 : Q4_MV_MAX_JX)) {
                ks = cand;
                break;
            }
    }
    Q4_CHECK(!glu_out || ks == 1, Q4_ERR_UNSUPPORTED,
             "%s: a gated output needs K %% 256 == 0, K <= 8192, 16-byte aligned x", name);
    // 3 <= B <= 8 rows: the matrix-core tile kernel without a K split reads W
    // once per call and needs no workspace.  It is faster than the vector
    // kernel once per row where the rows give it enough workgroups (measured:
    // 21504 x 5376 at B = 3, 4, 8 in 28.5, 28.6, 29.0 us against 34.4, 43.9,
    // 80.8 us; 6144 x 2560 at B = 8 10.8 against 17.7 us; 2560 x 9728 slower
    // at every B, 27.0 against 11.3-32.0 us).
    const size_t xbytes = static_cast<size_t>((B - 1) * ldx + K) * sizeof(float);
    const size_t ybytes = static_cast<size_t>(B * (glu_out ? N / 2 : N)) * sizeof(float);
    if (x16 && q4::aligned(Wv, 16) && B >= 3 && (N >= 16384 || (B >= 6 && N >= 4096)) &&
        !ranges_overlap(y, ybytes, x, xbytes) && (!op.u || !ranges_overlap(y, ybytes, op.u, xbytes))) {
        q4::matvec_mfma_whole_k(FMT, Wv, n, k, x, op.u, op.w, ldx, static_cast<int>(B), op_kind, out_op, eps,
                                y, res, s);
        return q4::launch_status(name);
    }
    if (ks) {
        const int jx = (ks_part_blocks(nb, ks) + 63) / 64;
        const int b = static_cast<int>(B);
        if (ks == 1) launch_b1_jx<FMT, 1>(jx, W, x, y, res, n, k, b, op, s);
        else if (ks == 2) launch_b1_jx<FMT, 2>(jx, W, x, y, res, n, k, b, op, s);
        else launch_b1_jx<FMT, 4>(jx, W, x, y, res, n, k, b, op, s);
    } else {
        launch_generic<FMT>(static_cast<int>(B), W, x, y, res, n, k, op, s);
    }
    return q4::launch_status(name);
}

}  // namespace

extern "C" q4_status q4_0_matvec(const void *W, int64_t N, int64_t K, const float *x, int64_t B,
                                 float *y, const float *residual, void *stream) {
    return matvec_entry<0>("q4_0_matvec", W, N, K, x, nullptr, K, B, Q4_IN_PLAIN, Q4_OUT_PLAIN,
                           nullptr, 0.f, y, residual, stream);
}

extern "C" q4_status q8_0_matvec(const void *W, int64_t N, int64_t K, const float *x, int64_t B,
                                 float *y, const float *residual, void *stream) {
    return matvec_entry<1>("q8_0_matvec", W, N, K, x, nullptr, K, B, Q4_IN_PLAIN, Q4_OUT_PLAIN,
                           nullptr, 0.f, y, residual, stream);
}

namespace {
bool spans_overlap(const void *a, size_t an, const void *b, size_t bn) {
    const uintptr_t p = reinterpret_cast<uintptr_t>(a), q = reinterpret_cast<uintptr_t>(b);
    return p < q + bn && q < p + an;
}
}  // namespace

extern "C" q4_status q4_0_matvec_post_norm(const void *W, int64_t N, int64_t K, const float *h,
                                           const float *z, int64_t ld, int64_t B,
                                           const float *post_w, const float *pre_w, float eps,
                                           float *h_out, q4_output_op out_op, float *y,
                                           void *stream) {
    q4::clear_error();
    const char *name = "q4_0_matvec_post_norm";
    Q4_CHECK(W && h && z && post_w && h_out && y, Q4_ERR_INVALID_ARG,
             "%s: W, h, z, post_w, h_out and y must not be NULL", name);
    Q4_CHECK(out_op == Q4_OUT_PLAIN || out_op == Q4_OUT_SWIGLU || out_op == Q4_OUT_GEGLU,
             Q4_ERR_INVALID_ARG, "%s: unknown output transform %d", name, out_op);
    Q4_CHECK(N >= 1 && K >= 1 && B >= 1, Q4_ERR_INVALID_ARG, "%s: N=%lld K=%lld B=%lld must be >= 1",
             name, (long long)N, (long long)K, (long long)B);
    Q4_CHECK(out_op == Q4_OUT_PLAIN || N % 2 == 0, Q4_ERR_INVALID_ARG,
             "%s: a gated (SwiGLU / GeGLU) output needs an even N", name);
    Q4_CHECK(eps >= 0.f, Q4_ERR_INVALID_ARG, "%s: eps must be >= 0", name);
    Q4_CHECK(B <= 8, Q4_ERR_UNSUPPORTED, "%s: B=%lld > 8", name, (long long)B);
    Q4_CHECK(K % 256 == 0 && K <= kXLdsFloats, Q4_ERR_UNSUPPORTED,
             "%s: K=%lld must be a multiple of 256 and at most %d", name, (long long)K, kXLdsFloats);
    Q4_CHECK(ld >= K, Q4_ERR_SHAPE, "%s: ld=%lld < K=%lld", name, (long long)ld, (long long)K);
    Q4_CHECK(N <= (1 << 30) && ld <= (1 << 26), Q4_ERR_UNSUPPORTED, "%s: N or ld too large", name);
    Q4_CHECK(q4::aligned(W, 2), Q4_ERR_ALIGNMENT, "%s: W must be 2-byte aligned", name);
    Q4_CHECK(q4::aligned(h, 16) && q4::aligned(z, 16) && q4::aligned(h_out, 16) &&
                 q4::aligned(post_w, 16) && (!pre_w || q4::aligned(pre_w, 16)) && ld % 4 == 0,
             Q4_ERR_ALIGNMENT,
             "%s: h, z, h_out and the gains must be 16-byte aligned with ld a multiple of 4", name);
    Q4_CHECK(q4::aligned(y, 4), Q4_ERR_ALIGNMENT, "%s: y must be 4-byte aligned", name);
    const size_t rows = static_cast<size_t>((B - 1) * ld + K) * sizeof(float);
    const size_t ybytes = static_cast<size_t>(B * (out_op != Q4_OUT_PLAIN ? N / 2 : N)) * sizeof(float);
    Q4_CHECK(!spans_overlap(h_out, rows, h, rows) && !spans_overlap(h_out, rows, z, rows),
             Q4_ERR_INVALID_ARG, "%s: h_out must not overlap h or z", name);
    Q4_CHECK(!spans_overlap(y, ybytes, h, rows) && !spans_overlap(y, ybytes, z, rows) &&
                 !spans_overlap(y, ybytes, h_out, rows),
             Q4_ERR_INVALID_ARG, "%s: y must not overlap h, z or h_out", name);
    const int glu = out_op == Q4_OUT_SWIGLU ? 1 : out_op == Q4_OUT_GEGLU ? 2 : 0;
    InOp op{1, z, pre_w, eps, ld, glu, 0, post_w, h_out};
    const int nb = static_cast<int>(K / 32);
    launch_b1_jx<0, 1>((ks_part_blocks(nb, 1) + 63) / 64, static_cast<const uint8_t *>(W), h, y, nullptr,
                       static_cast<int>(N), static_cast<int>(K), static_cast<int>(B), op,
                       q4::as_stream(stream));
    return q4::launch_status(name);
}

extern "C" q4_status q4_0_matvec_fused(const void *W, int64_t N, int64_t K, const float *x,
                                       const float *x2, int64_t ld_x, int64_t B, q4_input_op op,
                                       q4_output_op out_op, const float *norm_w, float eps,
                                       float *y, const float *residual, void *stream) {
    return matvec_entry<0>("q4_0_matvec_fused", W, N, K, x, x2, ld_x, B, op, out_op, norm_w, eps,
                           y, residual, stream);
}

extern "C" q4_status q8_0_matvec_fused(const void *W, int64_t N, int64_t K, const float *x,
                                       const float *x2, int64_t ld_x, int64_t B, q4_input_op op,
                                       q4_output_op out_op, const float *norm_w, float eps,
                                       float *y, const float *residual, void *stream) {
    return matvec_entry<1>("q8_0_matvec_fused", W, N, K, x, x2, ld_x, B, op, out_op, norm_w, eps,
                           y, residual, stream);
}

extern "C" q4_status q8_0_gather_scaled(const void *E, int64_t V, int64_t K,
                                        const int32_t *tokens, int64_t B, float scale, float *x,
                                        void *stream) {
    q4::clear_error();
    Q4_CHECK(E && tokens && x, Q4_ERR_INVALID_ARG, "q8_0_gather: E, tokens and x must not be NULL");
    Q4_CHECK(V >= 1 && K >= 1 && B >= 1, Q4_ERR_INVALID_ARG, "q8_0_gather: V, K, B must be >= 1");
    Q4_CHECK(K % 32 == 0, Q4_ERR_SHAPE, "q8_0_gather: K=%lld is not a multiple of 32", (long long)K);
    Q4_CHECK(V <= (1 << 30) && K <= (1 << 24) && B <= (1 << 20), Q4_ERR_UNSUPPORTED,
             "q8_0_gather: sizes too large");
    Q4_CHECK(q4::aligned(E, 2) && q4::aligned(tokens, 4) && q4::aligned(x, 4), Q4_ERR_ALIGNMENT,
             "q8_0_gather: E must be 2-byte, tokens and x 4-byte aligned");
    const int total = static_cast<int>(B) * static_cast<int>(K / 32);
    hipLaunchKernelGGL(q8_gather_kernel, dim3((total + kWG - 1) / kWG), dim3(kWG), 0,
                       q4::as_stream(stream), static_cast<const uint8_t *>(E), tokens, x,
                       static_cast<int>(V), static_cast<int>(K), static_cast<int>(B), scale);
    return q4::launch_status("q8_0_gather");
}

extern "C" q4_status q8_0_gather(const void *E, int64_t V, int64_t K, const int32_t *tokens,
                                 int64_t B, float *x, void *stream) {
    return q8_0_gather_scaled(E, V, K, tokens, B, 1.0f, x, stream);
}
