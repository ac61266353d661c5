// Device helpers for the gfx950 kernels: bf16 / E4M3 conversion, wave-level
// reductions built on DPP and ds_bpermute, order-preserving keys for top-k.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

// ------------------------------------------------------------------ bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round a finite fp32 value to bf16, nearest even (overflow gives inf).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Eight bf16 values held in a 16-byte vector, unpacked to fp32.
__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// ------------------------------------------------------------------ E4M3

// Four fp32 values to four OCP E4M3 codes (byte i = value i), nearest even.
// Inputs are clamped to +-448 first, which equals rounding then saturating.
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
    a = __builtin_amdgcn_fmed3f(a, 448.0f, -448.0f);
    b = __builtin_amdgcn_fmed3f(b, 448.0f, -448.0f);
    c = __builtin_amdgcn_fmed3f(c, 448.0f, -448.0f);
    d = __builtin_amdgcn_fmed3f(d, 448.0f, -448.0f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Value of E4M3 code byte `sel` (0..3) of a word, exact in fp32.
__device__ __forceinline__ float e4m3_to_f32(uint32_t w, int sel) {
    switch (sel) {
        case 0: return __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
        case 1: return __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
        case 2: return __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
        default: return __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
    }
}

// ------------------------------------------------------------------ DPP

// DPP controls (GCN/CDNA encoding).
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <-> 7-i within each 8 lanes

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Maximum over each aligned group of 8 lanes; all 8 lanes must be active.
__device__ __forceinline__ float group8_max(float v) {
    v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
    v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
    v = fmaxf(v, dpp_f32<kDppRowHalfMirror>(v));
    return v;
}

// ------------------------------------------------------------------ shuffles

__device__ __forceinline__ uint32_t shfl_xor_u32(uint32_t v, int mask) {
    const int lane = __lane_id();
    return (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, (int)v);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
    uint32_t lo = shfl_xor_u32((uint32_t)v, mask);
    uint32_t hi = shfl_xor_u32((uint32_t)(v >> 32), mask);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ float shfl_xor_f32(float v, int mask) {
    return __uint_as_float(shfl_xor_u32(__float_as_uint(v), mask));
}

// ------------------------------------------------------------------ buffer loads

// Buffer-descriptor word 3 for raw (untyped, stride 0) buffers on gfx9 parts.
constexpr int kRawBufferConfig = 0x00020000;
// Cache-policy bits of a buffer access: nt marks the data as streaming.
constexpr int kCachePolicyNT = 2;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Descriptor for a wave-uniform byte range [base, base + bytes). Accesses at
// offsets past `bytes` (all of them when bytes == 0) read zeros and drop
// writes instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRawBufferConfig);
}

// 16-byte streaming load at byte `offset` of a range descriptor.
__device__ __forceinline__ uint4 load16_nt(__amdgpu_buffer_rsrc_t rs, int offset) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, offset, 0, kCachePolicyNT);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// 16-byte streaming store (global address).
__device__ __forceinline__ void store16_nt(void* p, const uint4& v) {
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}

// ------------------------------------------------------------------ top-k keys

// Map an fp32 logit to a uint32 whose unsigned order is the numeric order,
// with -0 taken as +0 so that IEEE-equal values give equal keys.
__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t u = __float_as_uint(v);
    if ((u << 1) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// (logit key, expert) packed so that the unsigned maximum is the larger
// logit and, among equal logits, the lower expert index. Never zero for a
// real candidate, so zero marks an empty or already chosen slot.
__device__ __forceinline__ uint64_t topk_pack(float v, int e) {
    return ((uint64_t)order_key(v) << 32) | (uint32_t)(~(uint32_t)e);
}

__device__ __forceinline__ int topk_expert(uint64_t p) { return (int)(~(uint32_t)p); }
__device__ __forceinline__ float topk_value(uint64_t p) { return key_value((uint32_t)(p >> 32)); }

}  // namespace moe
