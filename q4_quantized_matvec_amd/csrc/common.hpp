// Internal helpers shared by the HIP sources of libq4dec (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>

#include "q4dec.h"

namespace q4 {

// Records the message for q4dec_last_error() and returns the status.
q4_status fail(q4_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
// Checks hipGetLastError() after a launch.
q4_status launch_status(const char *what);
// Compute units of the current device (cached per device).
int device_cus();
// Host validation of a KV-cache layout shared by the attention-side calls.
q4_status check_kv_layout(const char *name, const q4_kv_layout *kv);
// argmax_rows in two passes with a caller-owned scratch of
// argmax_scratch_bytes(B) bytes (4-byte aligned): many workgroups per row
// instead of one.  Same result as argmax_rows.
size_t argmax_scratch_bytes(int64_t B);
q4_status argmax_rows_scratch(const float *logits, int64_t B, int64_t V, int32_t *out,
                              void *scratch, hipStream_t s);

// The matrix-core matvec without a K split, so without a workspace: every
// workgroup of the tile kernel walks the whole K for its 64 (Q4_0) or 32
// (Q8_0) rows.  For the workspace-free matvec entry points at 3 <= B <= 8;
// the caller has checked K % 256 == 0, 16-byte aligned W, x, x2 and norm_w,
// ld_x % 4 == 0 and y disjoint from x and x2.  fmt: 0 = Q4_0, 1 = Q8_0.
void matvec_mfma_whole_k(int fmt, const void *W, int N, int K, const float *x, const float *x2,
                         const float *norm_w, int64_t ldx, int B, int op_kind, int out_op, float eps,
                         float *y, const float *res, hipStream_t s);

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }
inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace q4

#define Q4_CHECK(cond, status, ...)                                                   \
    do {                                                                              \
        if (!(cond)) return ::q4::fail((status), __VA_ARGS__);                        \
    } while (0)

#define Q4_HIP_CHECK(call)                                                            \
    do {                                                                              \
        hipError_t e_ = (call);                                                       \
        if (e_ != hipSuccess)                                                         \
            return ::q4::fail(Q4_ERR_HIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
    } while (0)

// ------------------------------------------------------------------ device side
namespace q4dev {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
// 16 bytes with only 2-byte alignment: gfx950 serves these as one dwordx4.
typedef uint32_t u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

// KV-cache rows are read once per step: their loads carry the nontemporal
// hint (Q4_NT_KV), measured 5-9 % faster attention.  (The weight windows of
// the matvecs, 4-byte aligned 16-byte loads, measured slower with it and
// stay plain.)  The pointee types fix the alignment: 16 bytes for fp32
// rows, 8 for binary16 ones.
#ifndef Q4_NT_KV
#define Q4_NT_KV 1
#endif
typedef float f32x4_ev __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_ev __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x4_ev ld_kv(const f32x4_ev *p) {
    if constexpr (Q4_NT_KV) return __builtin_nontemporal_load(p);
    else return *p;
}
__device__ __forceinline__ u32x2_ev ld_kv(const u32x2_ev *p) {
    if constexpr (Q4_NT_KV) return __builtin_nontemporal_load(p);
    else return *p;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

// acc + (low / high binary16 half of t) * x, the half widened exactly to fp32
// (folds into v_fma_mix_f32).
__device__ __forceinline__ float fma_lo(uint32_t t, float x, float acc) {
    return __builtin_fmaf(static_cast<float>(__builtin_bit_cast(half2_t, t).x), x, acc);
}
__device__ __forceinline__ float fma_hi(uint32_t t, float x, float acc) {
    return __builtin_fmaf(static_cast<float>(__builtin_bit_cast(half2_t, t).y), x, acc);
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

// Sum over the 64 lanes of a wavefront; every lane receives the total.
// DPP quad permutes, half-row / row mirrors, then row broadcasts 15 and 31.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<0xB1>(v);        // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);        // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);       // row_half_mirror
    v += dpp<0x140>(v);       // row_mirror: every lane holds its 16-lane row sum
    v += dpp<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// DPP move whose lanes without a valid source keep their own value.
template <int CTRL>
__device__ __forceinline__ float dpp_keep(float v) {
    int b = __builtin_bit_cast(int, v);
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, CTRL, 0xF, 0xF, false));
}

// Maximum over the 64 lanes (all lanes must be active); every lane receives it.
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_keep<0xB1>(v));
    v = fmaxf(v, dpp_keep<0x4E>(v));
    v = fmaxf(v, dpp_keep<0x141>(v));
    v = fmaxf(v, dpp_keep<0x140>(v));
    float t = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 15));
    t = fmaxf(t, __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31)));
    t = fmaxf(t, __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 47)));
    t = fmaxf(t, __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63)));
    return t;
}

}  // namespace q4dev
