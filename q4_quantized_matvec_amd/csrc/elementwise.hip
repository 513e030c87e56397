// RMSNorm, SwiGLU, per-head QK-norm + NeoX RoPE with KV-cache append, and the
// greedy argmax, for gfx950.
//
// Definitions ("GELO LLM" page, 02 "Definitions & glossary" and 05
// "Components"; "Research record" page, "Native Metal diagnostic"):
//   rmsnorm  y = w * x / sqrt(mean(x^2) + eps)
//   QK-norm  the same RMSNorm per head_dim slice with one shared gain, before RoPE
//   RoPE     NeoX pairing (i, i + hd/2), angle pos * theta^(-2i/hd)
//   SwiGLU   silu(g) * u;  GeGLU  gelu(g) * u with gelu in its tanh form
//   post-norm x += w * y / sqrt(mean(y^2) + eps)  (sandwich norm before the residual add)
//   softcap  l = c * tanh(l / c)
//   argmax   greedy choice, lowest token id on equal logits
#include "common.hpp"

namespace {
using namespace q4dev;

constexpr int kWG = 256;

// One workgroup of 1024 threads per row.  ADD: y[i] += the normalised x[i]
// (a post-norm joining the residual stream y) instead of y[i] = it.  Rows of
// up to 8192 elements are loaded once, all loads of a thread in flight
// together; longer rows are read twice.
constexpr int kNormWG = 1024, kNormU = 8;
template <bool ADD>
__global__ __launch_bounds__(kNormWG) void rmsnorm_kernel(const float *x, const float *__restrict__ w,
                                                          float *y, int dim, float eps) {
    __shared__ float red[kNormWG / 64];
    const float *xr = x + static_cast<size_t>(blockIdx.x) * dim;
    float *yr = y + static_cast<size_t>(blockIdx.x) * dim;
    const int tid = threadIdx.x;
    float v[kNormU], g[kNormU], d[kNormU];  // input, gain, (ADD) the accumulated row
    float ss = 0.f;
    const bool held = dim <= kNormWG * kNormU;
    if (held) {
        // every load of the thread goes out before the reduction: one round trip
#pragma unroll
        for (int u = 0; u < kNormU; ++u) {
            const int i = tid + u * kNormWG;
            const int ic = i < dim ? i : dim - 1;
            v[u] = xr[ic];
            g[u] = w ? w[ic] : 1.0f;
            if constexpr (ADD) d[u] = yr[ic];
        }
#pragma unroll
        for (int u = 0; u < kNormU; ++u) {
            if (tid + u * kNormWG >= dim) v[u] = 0.f;
            ss = __builtin_fmaf(v[u], v[u], ss);
        }
    } else {
        for (int i0 = 0; i0 < dim; i0 += kNormWG * kNormU) {
#pragma unroll
            for (int u = 0; u < kNormU; ++u) {
                const int i = i0 + tid + u * kNormWG;
                v[u] = i < dim ? xr[i] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < kNormU; ++u) ss = __builtin_fmaf(v[u], v[u], ss);
        }
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int k = 0; k < kNormWG / 64; ++k) tot += red[k];  // fixed order
    const float inv = 1.0f / sqrtf(tot / static_cast<float>(dim) + eps);
    if (held) {
#pragma unroll
        for (int u = 0; u < kNormU; ++u) {
            const int i = tid + u * kNormWG;
            if (i < dim) {
                const float t = v[u] * inv * g[u];
                if constexpr (ADD) yr[i] = d[u] + t;
                else yr[i] = t;
            }
        }
        return;
    }
    for (int i0 = 0; i0 < dim; i0 += kNormWG * kNormU) {
#pragma unroll
        for (int u = 0; u < kNormU; ++u) {
            const int i = i0 + tid + u * kNormWG;
            if (i < dim) {
                const float t = xr[i] * inv * (w ? w[i] : 1.0f);
                if constexpr (ADD) yr[i] += t;
                else yr[i] = t;
            }
        }
    }
}

// act(g) * u, act = SiLU (a == 0) or the tanh form of GELU (a == 1).
__global__ __launch_bounds__(kWG) void glu_kernel(const float *g, const float *u, float *h,
                                                  int64_t rows, int64_t n, int64_t ld, int a) {
    const int64_t total = rows * n;
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * kWG + threadIdx.x; t < total;
         t += static_cast<int64_t>(gridDim.x) * kWG) {
        const int64_t r = t / n, i = t % n;
        const float gv = g[r * ld + i];
        const float act = a ? 0.5f * gv * (1.0f + tanhf(0.7978845608028654f * (gv + 0.044715f * gv * gv * gv)))
                            : gv / (1.0f + expf(-gv));
        h[t] = act * u[r * ld + i];
    }
}

__global__ __launch_bounds__(kWG) void softcap_kernel(float *v, int64_t n, float c, float inv_c) {
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * kWG + threadIdx.x; t < n;
         t += static_cast<int64_t>(gridDim.x) * kWG)
        v[t] = c * tanhf(v[t] * inv_c);
}

// One wavefront per (sequence, head).  Heads [0, Hq) are query heads (written
// back in place); heads [Hq, Hq + Hkv) are key heads whose rotated row (and the
// value row) are appended to the caches at slot pos % cap.
constexpr int kMaxPairsPerLane = 4;  // head_dim <= 512
constexpr int kMaxPassPerLane = 8;   // unrotated elements (p-RoPE), head_dim <= 512

// KT: the caches' element type (fp32, or binary16 written with round to
// nearest even).
template <typename KT>
__global__ __launch_bounds__(64) void qk_norm_rope_kernel(
    float *q, int64_t ldq, const float *k, const float *v, int64_t ldkv,
    const float *__restrict__ qn, const float *__restrict__ kn, int Hq, int hd,
    const int64_t *__restrict__ pos_dev, double r, float eps, int v_from_k,
    KT *kc, KT *vc, int64_t cap, int64_t sb, int64_t sh, int64_t st, int rot) {
    // p-RoPE: elements [0, rot) rotate as a NeoX rotation of a rot-dimensional
    // vector (pairs i, i + rot/2, angle pos * theta^(-2i/rot)); elements
    // [rot, hd) are only normalised.  rot == hd is the full rotation.
    const int b = blockIdx.y;
    const int head = blockIdx.x;
    const int lane = threadIdx.x;
    const int half = rot >> 1;
    const bool is_q = head < Hq;
    const int g = head - Hq;
    const float *src = is_q ? q + b * ldq + static_cast<int64_t>(head) * hd
                            : k + b * ldkv + static_cast<int64_t>(g) * hd;
    const float *gain = is_q ? qn : kn;

    // Every load (values and gains) goes out before the reduction, with
    // clamped addresses (zeroed afterwards), so all return in one round trip.
    float a[kMaxPairsPerLane], c[kMaxPairsPerLane], ga[kMaxPairsPerLane], gc[kMaxPairsPerLane];
#pragma unroll
    for (int p = 0; p < kMaxPairsPerLane; ++p) {
        const int i = min(lane + 64 * p, half - 1);
        a[p] = src[i];
        c[p] = src[i + half];
        ga[p] = gain[i];
        gc[p] = gain[i + half];
    }
    float t[kMaxPassPerLane], gt[kMaxPassPerLane];
#pragma unroll
    for (int p = 0; p < kMaxPassPerLane; ++p) {
        const int i = min(rot + lane + 64 * p, hd - 1);
        t[p] = src[i];
        gt[p] = gain[i];
    }
    float ss = 0.f;
#pragma unroll
    for (int p = 0; p < kMaxPairsPerLane; ++p) {
        if (lane + 64 * p >= half) a[p] = c[p] = 0.f;
        ss = __builtin_fmaf(a[p], a[p], __builtin_fmaf(c[p], c[p], ss));
    }
#pragma unroll
    for (int p = 0; p < kMaxPassPerLane; ++p) {
        if (rot + lane + 64 * p >= hd) t[p] = 0.f;
        ss = __builtin_fmaf(t[p], t[p], ss);
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / static_cast<float>(hd) + eps);
    const int64_t pos = *pos_dev;
    // Frequencies theta^(-2i/rot) = r^i with r = theta^(-2/rot) (computed once
    // on the host), by binary powers in fp64 (a relative error of a few
    // 1e-16, far below what the angle needs); the angle pos * r^i is reduced
    // by 2 pi in fp64 and the reduced angle (|a| <= pi) goes to
    // single-precision sincos.
    double rp[9];  // r^(2^k), k = 0..8 (pairs i < 256)
    rp[0] = r;
#pragma unroll
    for (int k = 1; k < 9; ++k) rp[k] = rp[k - 1] * rp[k - 1];

    float *dst = nullptr;  // the query row, in place
    KT *kdst = nullptr, *vdst = nullptr;
    if (is_q) {
        dst = q + b * ldq + static_cast<int64_t>(head) * hd;
    } else if (pos >= 0) {
        const int64_t base = b * sb + g * sh + (pos % cap) * st;
        kdst = kc + base;
        vdst = vc + base;
    }
#pragma unroll
    for (int p = 0; p < kMaxPairsPerLane; ++p) {
        const int i = lane + 64 * p;
        if (i < half) {
            double inv_freq = 1.0;
#pragma unroll
            for (int k = 0; k < 9; ++k) inv_freq = ((i >> k) & 1) ? inv_freq * rp[k] : inv_freq;
            const double ang = static_cast<double>(pos) * inv_freq;
            const double two_pi = 6.283185307179586;
            const double red = __builtin_fma(-two_pi, rint(ang * (1.0 / two_pi)), ang);
            float sn, cs;
            sincosf(static_cast<float>(red), &sn, &cs);
            const float x0 = a[p] * inv * ga[p];
            const float x1 = c[p] * inv * gc[p];
            if (dst) {
                dst[i] = x0 * cs - x1 * sn;
                dst[i + half] = x1 * cs + x0 * sn;
            }
            if (kdst) {
                kdst[i] = static_cast<KT>(x0 * cs - x1 * sn);
                kdst[i + half] = static_cast<KT>(x1 * cs + x0 * sn);
            }
            if (vdst) {
                if (v_from_k) {
                    vdst[i] = static_cast<KT>(a[p] * inv);
                    vdst[i + half] = static_cast<KT>(c[p] * inv);
                } else {
                    const float *vs = v + b * ldkv + static_cast<int64_t>(g) * hd;
                    vdst[i] = static_cast<KT>(vs[i]);
                    vdst[i + half] = static_cast<KT>(vs[i + half]);
                }
            }
        }
    }
#pragma unroll
    for (int p = 0; p < kMaxPassPerLane; ++p) {
        const int i = rot + lane + 64 * p;
        if (i < hd) {
            const float x0 = t[p] * inv * gt[p];
            if (dst) dst[i] = x0;
            if (kdst) kdst[i] = static_cast<KT>(x0);
            if (vdst) {
                if (v_from_k) vdst[i] = static_cast<KT>(t[p] * inv);
                else vdst[i] = static_cast<KT>(v[b * ldkv + static_cast<int64_t>(g) * hd + i]);
            }
        }
    }
}

// (value, index) order of the greedy choice: larger value, then lower index;
// NaN never compares greater, so it never wins.
__device__ __forceinline__ bool arg_better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

// Two-pass argmax.  Pass 1: kArgParts workgroups per row, each reducing a
// contiguous slice (8 loads in flight per thread) to (value, index).
constexpr int kArgParts = 64;
__global__ __launch_bounds__(256) void argmax_part_kernel(const float *__restrict__ logits, int64_t V,
                                                          float *__restrict__ pv, int *__restrict__ pi) {
    __shared__ float sv[4];
    __shared__ int si[4];
    const int part = blockIdx.x, b = blockIdx.y;
    const int64_t per = (V + kArgParts - 1) / kArgParts;
    const int64_t s = static_cast<int64_t>(part) * per;
    const int64_t e = min(V, s + per);
    const float *row = logits + static_cast<int64_t>(b) * V;
    float best = -INFINITY;
    int bi = 0x7fffffff;
    constexpr int kU = 8;
    for (int64_t i0 = s + threadIdx.x; i0 < e; i0 += 256 * kU) {
        float v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) v[u] = row[min(i0 + u * 256, e - 1)];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t i = i0 + u * 256;
            if (i < e && arg_better(v[u], static_cast<int>(i), best, bi)) {
                best = v[u];
                bi = static_cast<int>(i);
            }
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(best, off);
        const int oi = __shfl_xor(bi, off);
        if (arg_better(ov, oi, best, bi)) {
            best = ov;
            bi = oi;
        }
    }
    if ((threadIdx.x & 63) == 0) {
        sv[threadIdx.x >> 6] = best;
        si[threadIdx.x >> 6] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < 4; ++w)
            if (arg_better(sv[w], si[w], best, bi)) {
                best = sv[w];
                bi = si[w];
            }
        pv[b * kArgParts + part] = best;
        pi[b * kArgParts + part] = bi;
    }
}

// Pass 2: one wavefront per row, lane l holding slice l.
__global__ __launch_bounds__(64) void argmax_final_kernel(const float *__restrict__ pv,
                                                          const int *__restrict__ pi, int32_t *out) {
    const int b = blockIdx.x, l = threadIdx.x;
    float best = pv[b * kArgParts + l];
    int bi = pi[b * kArgParts + l];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(best, off);
        const int oi = __shfl_xor(bi, off);
        if (arg_better(ov, oi, best, bi)) {
            best = ov;
            bi = oi;
        }
    }
    if (l == 0) out[b] = bi == 0x7fffffff ? 0 : bi;
}

// One workgroup per row; (value, index) with the lowest index among equal
// maxima.  NaN never compares greater, so it never wins.
__global__ __launch_bounds__(1024) void argmax_kernel(const float *__restrict__ logits,
                                                      int32_t *out, int64_t V) {
    __shared__ float sv[1024];
    __shared__ int si[1024];
    const float *row = logits + static_cast<int64_t>(blockIdx.x) * V;
    float best = -INFINITY;
    int bi = 0x7fffffff;
    auto consider = [&](float v, int i) {
        if (v > best || (v == best && i < bi)) {  // a NaN never wins
            best = v;
            bi = i;
        }
    };
    constexpr int kU = 8;  // loads in flight per thread
    if ((reinterpret_cast<uintptr_t>(row) & 15) == 0) {
        const int nv = static_cast<int>(V >> 2);
        const float4 *r4 = reinterpret_cast<const float4 *>(row);
        for (int base = threadIdx.x; base < nv; base += 1024 * kU) {
            float4 v[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) v[u] = r4[min(base + u * 1024, nv - 1)];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int i = base + u * 1024;
                if (i < nv) {
                    consider(v[u].x, 4 * i);
                    consider(v[u].y, 4 * i + 1);
                    consider(v[u].z, 4 * i + 2);
                    consider(v[u].w, 4 * i + 3);
                }
            }
        }
        for (int64_t i = 4 * static_cast<int64_t>(nv) + threadIdx.x; i < V; i += 1024)
            consider(row[i], static_cast<int>(i));
    } else {
        for (int base = threadIdx.x; base < V; base += 1024 * kU) {
            float v[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) v[u] = row[min(static_cast<int64_t>(base + u * 1024), V - 1)];
#pragma unroll
            for (int u = 0; u < kU; ++u)
                if (base + u * 1024 < V) consider(v[u], base + u * 1024);
        }
    }
    sv[threadIdx.x] = best;
    si[threadIdx.x] = bi;
    __syncthreads();
    for (int s = 512; s > 0; s >>= 1) {
        if (threadIdx.x < s) {
            const float ov = sv[threadIdx.x + s];
            const int oi = si[threadIdx.x + s];
            if (ov > sv[threadIdx.x] || (ov == sv[threadIdx.x] && oi < si[threadIdx.x])) {
                sv[threadIdx.x] = ov;
                si[threadIdx.x] = oi;
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) out[blockIdx.x] = si[0] == 0x7fffffff ? 0 : si[0];
}

}  // namespace

extern "C" q4_status rmsnorm(const float *x, const float *w, int64_t rows, int64_t dim, float eps,
                             float *y, void *stream) {
    q4::clear_error();
    Q4_CHECK(x && y, Q4_ERR_INVALID_ARG, "rmsnorm: x and y must not be NULL");
    Q4_CHECK(rows >= 1 && dim >= 1 && eps >= 0.f, Q4_ERR_INVALID_ARG,
             "rmsnorm: rows, dim must be >= 1 and eps >= 0");
    Q4_CHECK(rows <= (1 << 30) && dim <= (1 << 26), Q4_ERR_UNSUPPORTED, "rmsnorm: sizes too large");
    Q4_CHECK(q4::aligned(x, 4) && q4::aligned(y, 4) && (!w || q4::aligned(w, 4)), Q4_ERR_ALIGNMENT,
             "rmsnorm: x, w, y must be 4-byte aligned");
    hipLaunchKernelGGL(rmsnorm_kernel<false>, dim3(static_cast<unsigned>(rows)), dim3(kNormWG), 0,
                       q4::as_stream(stream), x, w, y, static_cast<int>(dim), eps);
    return q4::launch_status("rmsnorm");
}

extern "C" q4_status rmsnorm_add(const float *y, const float *w, int64_t rows, int64_t dim,
                                 float eps, float *x, void *stream) {
    q4::clear_error();
    Q4_CHECK(x && y, Q4_ERR_INVALID_ARG, "rmsnorm_add: y and x must not be NULL");
    Q4_CHECK(rows >= 1 && dim >= 1 && eps >= 0.f, Q4_ERR_INVALID_ARG,
             "rmsnorm_add: rows, dim must be >= 1 and eps >= 0");
    Q4_CHECK(rows <= (1 << 30) && dim <= (1 << 26), Q4_ERR_UNSUPPORTED, "rmsnorm_add: sizes too large");
    Q4_CHECK(q4::aligned(x, 4) && q4::aligned(y, 4) && (!w || q4::aligned(w, 4)), Q4_ERR_ALIGNMENT,
             "rmsnorm_add: y, w, x must be 4-byte aligned");
    const size_t bytes = static_cast<size_t>(rows * dim) * sizeof(float);
    const uintptr_t a = reinterpret_cast<uintptr_t>(x), b = reinterpret_cast<uintptr_t>(y);
    Q4_CHECK(a + bytes <= b || b + bytes <= a, Q4_ERR_INVALID_ARG, "rmsnorm_add: y must not overlap x");
    hipLaunchKernelGGL(rmsnorm_kernel<true>, dim3(static_cast<unsigned>(rows)), dim3(kNormWG), 0,
                       q4::as_stream(stream), y, w, x, static_cast<int>(dim), eps);
    return q4::launch_status("rmsnorm_add");
}

namespace {
q4_status glu_entry(const char *name, const float *g, const float *u, int64_t rows, int64_t n,
                    int64_t ld, float *h, void *stream, int a) {
    q4::clear_error();
    Q4_CHECK(g && u && h, Q4_ERR_INVALID_ARG, "%s: g, u and h must not be NULL", name);
    Q4_CHECK(rows >= 1 && n >= 1 && ld >= n, Q4_ERR_INVALID_ARG,
             "%s: rows, n must be >= 1 and ld >= n", name);
    Q4_CHECK(q4::aligned(g, 4) && q4::aligned(u, 4) && q4::aligned(h, 4), Q4_ERR_ALIGNMENT,
             "%s: g, u, h must be 4-byte aligned", name);
    const int64_t total = rows * n;
    const int64_t want = (total + kWG - 1) / kWG;
    const unsigned grid = static_cast<unsigned>(std::min<int64_t>(want, 4096));
    hipLaunchKernelGGL(glu_kernel, dim3(grid), dim3(kWG), 0, q4::as_stream(stream), g, u, h, rows, n,
                       ld, a);
    return q4::launch_status(name);
}
}  // namespace

extern "C" q4_status swiglu(const float *g, const float *u, int64_t rows, int64_t n, int64_t ld,
                            float *h, void *stream) {
    return glu_entry("swiglu", g, u, rows, n, ld, h, stream, 0);
}

extern "C" q4_status geglu(const float *g, const float *u, int64_t rows, int64_t n, int64_t ld,
                           float *h, void *stream) {
    return glu_entry("geglu", g, u, rows, n, ld, h, stream, 1);
}

extern "C" q4_status softcap(float *v, int64_t n, float cap, void *stream) {
    q4::clear_error();
    Q4_CHECK(v && n >= 1, Q4_ERR_INVALID_ARG, "softcap: v must not be NULL and n >= 1");
    Q4_CHECK(cap > 0.f && cap <= 3.0e38f, Q4_ERR_INVALID_ARG, "softcap: cap must be > 0 and finite");
    Q4_CHECK(q4::aligned(v, 4), Q4_ERR_ALIGNMENT, "softcap: v must be 4-byte aligned");
    const int64_t want = (n + kWG - 1) / kWG;
    const unsigned grid = static_cast<unsigned>(std::min<int64_t>(want, 4096));
    hipLaunchKernelGGL(softcap_kernel, dim3(grid), dim3(kWG), 0, q4::as_stream(stream), v, n, cap,
                       1.0f / cap);
    return q4::launch_status("softcap");
}

namespace q4 {
q4_status check_kv_layout(const char *name, const q4_kv_layout *kv) {
    Q4_CHECK(kv, Q4_ERR_INVALID_ARG, "%s: kv layout must not be NULL", name);
    Q4_CHECK(kv->batch >= 1 && kv->n_kv_heads >= 1 && kv->head_dim >= 2 && kv->cap >= 1,
             Q4_ERR_INVALID_ARG, "%s: kv layout sizes must be positive", name);
    Q4_CHECK(kv->stride_b >= 0 && kv->stride_h >= 0 && kv->stride_t >= kv->head_dim,
             Q4_ERR_SHAPE, "%s: kv strides must be >= 0 and stride_t >= head_dim", name);
    Q4_CHECK(kv->head_dim % 2 == 0, Q4_ERR_SHAPE, "%s: head_dim %lld is odd", name,
             (long long)kv->head_dim);
    Q4_CHECK(kv->head_dim <= 512, Q4_ERR_UNSUPPORTED, "%s: head_dim %lld > 512", name,
             (long long)kv->head_dim);
    Q4_CHECK(kv->batch <= 65535 && kv->n_kv_heads <= 4096 && kv->cap <= (int64_t(1) << 30),
             Q4_ERR_UNSUPPORTED, "%s: batch, kv heads or capacity too large", name);
    Q4_CHECK(kv->dtype == Q4_KV_F32 || kv->dtype == Q4_KV_F16, Q4_ERR_INVALID_ARG,
             "%s: kv dtype %lld is neither Q4_KV_F32 nor Q4_KV_F16", name, (long long)kv->dtype);
    return Q4_OK;
}
}  // namespace q4

extern "C" q4_status qk_norm_rope_partial(float *q, int64_t ldq, const float *k, const float *v,
                                          int64_t ldkv, const float *q_norm, const float *k_norm,
                                          int64_t n_q_heads, const q4_kv_layout *kv,
                                          const int64_t *pos_dev, double theta, float eps,
                                          int v_from_k, int64_t rot_dims, void *k_cache,
                                          void *v_cache, void *stream) {
    q4::clear_error();
    q4_status st = q4::check_kv_layout("qk_norm_rope", kv);
    if (st != Q4_OK) return st;
    Q4_CHECK(rot_dims >= 2 && rot_dims <= kv->head_dim && rot_dims % 2 == 0, Q4_ERR_INVALID_ARG,
             "qk_norm_rope: rotated dims %lld must be even and in [2, head_dim]", (long long)rot_dims);
    Q4_CHECK(q && k && q_norm && k_norm && pos_dev && k_cache && v_cache, Q4_ERR_INVALID_ARG,
             "qk_norm_rope: q, k, q_norm, k_norm, pos_dev and the caches must not be NULL");
    Q4_CHECK(v_from_k ? v == nullptr : v != nullptr, Q4_ERR_INVALID_ARG,
             "qk_norm_rope: v must be NULL exactly when v_from_k is set");
    Q4_CHECK(n_q_heads >= 1 && n_q_heads % kv->n_kv_heads == 0, Q4_ERR_SHAPE,
             "qk_norm_rope: n_q_heads %lld is not a multiple of n_kv_heads %lld",
             (long long)n_q_heads, (long long)kv->n_kv_heads);
    Q4_CHECK(ldq >= n_q_heads * kv->head_dim && ldkv >= kv->n_kv_heads * kv->head_dim,
             Q4_ERR_SHAPE, "qk_norm_rope: row strides smaller than the rows");
    Q4_CHECK(theta > 0.0 && eps >= 0.f, Q4_ERR_INVALID_ARG, "qk_norm_rope: theta > 0, eps >= 0");
    Q4_CHECK(n_q_heads + kv->n_kv_heads <= 65535, Q4_ERR_UNSUPPORTED, "qk_norm_rope: too many heads");
    dim3 grid(static_cast<unsigned>(n_q_heads + kv->n_kv_heads), static_cast<unsigned>(kv->batch));
    const double r = std::pow(theta, -2.0 / static_cast<double>(rot_dims));
    if (kv->dtype == Q4_KV_F16)
        hipLaunchKernelGGL(qk_norm_rope_kernel<_Float16>, grid, dim3(64), 0, q4::as_stream(stream), q,
                           ldq, k, v, ldkv, q_norm, k_norm, static_cast<int>(n_q_heads),
                           static_cast<int>(kv->head_dim), pos_dev, r, eps, v_from_k ? 1 : 0,
                           static_cast<_Float16 *>(k_cache), static_cast<_Float16 *>(v_cache), kv->cap,
                           kv->stride_b, kv->stride_h, kv->stride_t, static_cast<int>(rot_dims));
    else
        hipLaunchKernelGGL(qk_norm_rope_kernel<float>, grid, dim3(64), 0, q4::as_stream(stream), q,
                           ldq, k, v, ldkv, q_norm, k_norm, static_cast<int>(n_q_heads),
                           static_cast<int>(kv->head_dim), pos_dev, r, eps, v_from_k ? 1 : 0,
                           static_cast<float *>(k_cache), static_cast<float *>(v_cache), kv->cap,
                           kv->stride_b, kv->stride_h, kv->stride_t, static_cast<int>(rot_dims));
    return q4::launch_status("qk_norm_rope");
}

extern "C" q4_status qk_norm_rope(float *q, int64_t ldq, const float *k, const float *v,
                                  int64_t ldkv, const float *q_norm, const float *k_norm,
                                  int64_t n_q_heads, const q4_kv_layout *kv,
                                  const int64_t *pos_dev, double theta, float eps, int v_from_k,
                                  void *k_cache, void *v_cache, void *stream) {
    q4::clear_error();
    Q4_CHECK(kv, Q4_ERR_INVALID_ARG, "qk_norm_rope: kv layout must not be NULL");
    return qk_norm_rope_partial(q, ldq, k, v, ldkv, q_norm, k_norm, n_q_heads, kv, pos_dev, theta,
                                eps, v_from_k, kv->head_dim, k_cache, v_cache, stream);
}

extern "C" q4_status argmax_rows(const float *logits, int64_t B, int64_t V, int32_t *out,
                                 void *stream) {
    q4::clear_error();
    Q4_CHECK(logits && out, Q4_ERR_INVALID_ARG, "argmax_rows: logits and out must not be NULL");
    Q4_CHECK(B >= 1 && V >= 1, Q4_ERR_INVALID_ARG, "argmax_rows: B and V must be >= 1");
    Q4_CHECK(V <= (1 << 30) && B <= (1 << 30), Q4_ERR_UNSUPPORTED, "argmax_rows: sizes too large");
    Q4_CHECK(q4::aligned(logits, 4) && q4::aligned(out, 4), Q4_ERR_ALIGNMENT,
             "argmax_rows: logits and out must be 4-byte aligned");
    hipLaunchKernelGGL(argmax_kernel, dim3(static_cast<unsigned>(B)), dim3(1024), 0,
                       q4::as_stream(stream), logits, out, V);
    return q4::launch_status("argmax_rows");
}

namespace q4 {
size_t argmax_scratch_bytes(int64_t B) {
    return static_cast<size_t>(B) * kArgParts * (sizeof(float) + sizeof(int));
}

q4_status argmax_rows_scratch(const float *logits, int64_t B, int64_t V, int32_t *out, void *scratch,
                              hipStream_t s) {
    Q4_CHECK(logits && out && scratch, Q4_ERR_INVALID_ARG, "argmax: logits, out, scratch must not be NULL");
    Q4_CHECK(B >= 1 && V >= 1 && B <= 65535 && V <= (1 << 30), Q4_ERR_INVALID_ARG, "argmax: bad sizes");
    Q4_CHECK(aligned(scratch, 4), Q4_ERR_ALIGNMENT, "argmax: scratch must be 4-byte aligned");
    float *pv = static_cast<float *>(scratch);
    int *pi = reinterpret_cast<int *>(pv + B * kArgParts);
    hipLaunchKernelGGL(argmax_part_kernel, dim3(kArgParts, static_cast<unsigned>(B)), dim3(256), 0, s,
                       logits, V, pv, pi);
    q4_status st = launch_status("argmax (parts)");
    if (st != Q4_OK) return st;
    hipLaunchKernelGGL(argmax_final_kernel, dim3(static_cast<unsigned>(B)), dim3(64), 0, s, pv, pi, out);
    return launch_status("argmax (final)");
}
}  // namespace q4

extern "C" size_t argmax_rows_workspace(int64_t B) { return B >= 1 ? q4::argmax_scratch_bytes(B) : 0; }

extern "C" q4_status argmax_rows_ws(const float *logits, int64_t B, int64_t V, int32_t *out, void *ws,
                                    size_t ws_bytes, void *stream) {
    q4::clear_error();
    Q4_CHECK(B >= 1, Q4_ERR_INVALID_ARG, "argmax_rows_ws: B must be >= 1");
    Q4_CHECK(ws && ws_bytes >= q4::argmax_scratch_bytes(B), Q4_ERR_WORKSPACE,
             "argmax_rows_ws: workspace of %zu bytes needed, got %zu", q4::argmax_scratch_bytes(B), ws_bytes);
    Q4_CHECK(q4::aligned(logits, 4) && q4::aligned(out, 4), Q4_ERR_ALIGNMENT,
             "argmax_rows_ws: logits and out must be 4-byte aligned");
    return q4::argmax_rows_scratch(logits, B, V, out, ws, q4::as_stream(stream));
}
