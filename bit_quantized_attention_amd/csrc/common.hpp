// common.hpp — types and device helpers shared by the gfx950 kernels of libbqa.
//
// Everything here is written for CDNA4 (gfx950) only: 64-lane wavefronts,
// the gfx950 matrix instructions (i8 32x32x32, scaled f8f6f4 32x32x64 /
// 16x16x128, bf16/f16 32x32x16, bf16 16x16x32) and the permlane swaps.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bqa {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------ tensors
// Dense [B, H, N, d] view with element strides (innermost stride 1).
struct Dense {
    void* p;
    int64_t sB, sH, sN;
};

// ------------------------------------------------------------------ lanes
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Value of x held by the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ int partner32(int x) {
    v2i r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (threadIdx.x & 32) ? r[0] : r[1];
}
__device__ __forceinline__ float partner32f(float x) {
    return __builtin_bit_cast(float, partner32(__builtin_bit_cast(int, x)));
}

// ------------------------------------------------------------------ LDS copies
// Direct global -> LDS copies (global_load_lds, scalar base + per-lane 32-bit
// offset): lane i's 16 (4) bytes land at lds + 16 i (4 i).  They are issued
// from inline assembly, so the compiler does not track them (it would
// otherwise wait for every copy in flight before any LDS read): the caller
// waits for them with s_waitcnt vmcnt and makes them visible to the other
// wavefronts with a barrier.  M0 holds the LDS destination, one wait state
// before the copy reads it; M0 is reserved to the compiler, which sets it
// right before each of its own users, so it is not named as a clobber.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}
// The base and the LDS address must be the same in every lane; readfirstlane
// puts them in scalar registers where the compiler cannot prove it itself
// (it folds away for values already known to be uniform).
__device__ __forceinline__ const void* uniform_base(const void* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void lds_copy16(uint32_t voff, const void* sbase, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff),
                 "s"(uniform_base(sbase)), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
}
__device__ __forceinline__ void lds_copy4(uint32_t voff, const void* sbase, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff),
                 "s"(uniform_base(sbase)), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
}
// The same copies with the non-temporal cache policy, for data a kernel
// streams once (a decode step's KV cache): measured on MI355X, 4 GiB read
// this way runs at about 7.1 TB/s against 6.3 TB/s with the default policy.
__device__ __forceinline__ void lds_copy16_nt(uint32_t voff, const void* sbase, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff),
                 "s"(uniform_base(sbase)), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
}
__device__ __forceinline__ void lds_copy4_nt(uint32_t voff, const void* sbase, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1 nt" ::"v"(voff),
                 "s"(uniform_base(sbase)), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
}
// s_waitcnt with vmcnt(n) (n < 64) and lgkmcnt(0), expcnt not waited for
#define BQA_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(0x0070 | ((n) & 15) | (((n) >> 4) << 14))
// A workgroup barrier that does not wait for the copies above (the barrier of
// __syncthreads carries a fence that waits for every memory operation)
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }
// Scalar-cache view of a uniform array (loads become s_load, counted by
// lgkmcnt, so they never wait for the copies above)
template <class T>
__device__ __forceinline__ const __attribute__((address_space(4))) T* uniform_ptr(const T* p) {
    return (const __attribute__((address_space(4))) T*)p;
}

// ------------------------------------------------------------------ MFMA
__device__ __forceinline__ v16i mfma_i8_32x32x32(v4i a, v4i b, v16i c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}
// fp8 e4m3 x fp8 e4m3 with unit scales (E8M0 127 = 2^0)
__device__ __forceinline__ v16f mfma_f8_32x32x64(v8i a, v8i b, v16f c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// MXFP4 x MXFP4: 16 bytes (32 e2m1) per lane, one E8M0 scale byte per lane
__device__ __forceinline__ v16f mfma_f4_32x32x64(v4i a, int sa, v4i b, int sb, v16f c) {
    v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
    v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 0, sa, 0, sb);
}
// The same at 16 x 16 x 128: lane l supplies row (A) or column (B) l % 16,
// elements 32 (l / 16) .. + 31, with that block's scale byte; lane l of the
// result holds column l % 16, rows 4 (l / 16) .. + 3.
__device__ __forceinline__ v4f mfma_f4_16x16x128(v4i a, int sa, v4i b, int sb, v4f c) {
    v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
    v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, 4, 4, 0, sa, 0, sb);
}
// bf16 16 x 16 x 32: lane l supplies row (A) or column (B) l % 16, elements
// 8 (l / 16) .. + 7; the result is laid out as above.
__device__ __forceinline__ v4f mfma_bf16_16x16x32(v8bf a, v8bf b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v16f mfma_bf16_32x32x16(v8bf a, v8bf b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v16f mfma_f16_32x32x16(v8h a, v8h b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ formats
// fp32 <-> bf16 / fp16 with round-to-nearest-even.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}
template <bool IS_F16>
__device__ __forceinline__ float load_half(const uint16_t* p) {
    return IS_F16 ? f16_bits_to_f32(*p) : bf16_bits_to_f32(*p);
}

// Symmetric INT8: nearest-even integer of the fp32 product, clamped to +-127.
__device__ __forceinline__ int enc_i8(float x, float inv) {
    float r = __builtin_rintf(x * inv);
    r = __builtin_fminf(__builtin_fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

// Four values -> four INT8 codes rint(fp32(x * inv)) packed little-endian in
// one word.  The caller guarantees |x * inv| <= 127 (inv comes from the
// largest magnitude), so no clamp is needed: the code is the low byte of
// fp32(x * inv) + 1.5 * 2^23, whose addition rounds to the nearest even
// integer.  inv = 0 gives zero codes.
__device__ __forceinline__ int q8x4(float a, float b, float c, float d, float inv) {
#pragma clang fp contract(off)
    const float M = 12582912.0f;
    const uint32_t wa = __builtin_bit_cast(uint32_t, a * inv + M), wb = __builtin_bit_cast(uint32_t, b * inv + M);
    const uint32_t wc = __builtin_bit_cast(uint32_t, c * inv + M), wd = __builtin_bit_cast(uint32_t, d * inv + M);
    return (int)(__builtin_amdgcn_perm(wb, wa, 0x0c0c0400u) | __builtin_amdgcn_perm(wd, wc, 0x04000c0cu));
}

// OCP MX shared exponent of a block with absolute maximum amax:
// floor(log2 amax) - 2, clamped to [-127, 127]; -127 for 0 and subnormals.
__device__ __forceinline__ int mx_exponent(float amax) {
    uint32_t E = (__builtin_bit_cast(uint32_t, amax) >> 23) & 0xFF;
    if (E == 0) return -127;
    int e = (int)E - 127 - 2;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// ------------------------------------------------------------------ reductions
// Value of x in the lane of the same 32-half 16 positions away.
__device__ __forceinline__ float partner16f(float x) {
    const int b = __builtin_bit_cast(int, x);
    v2i r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    return __builtin_bit_cast(float, (threadIdx.x & 16) ? r[0] : r[1]);
}
// Maxima of values that are never NaN.  Written with the compiler's own
// maximum (which the backend fuses into v_max3_f32), never as inline
// assembly: the hardware does not interlock a vector read of a matrix
// instruction's result, and the compiler inserts the wait states such a read
// needs only for its own instructions.  The kernels that use them are built
// with -fno-honor-nans, so no canonicalising v_max x, x precede them.
__device__ __forceinline__ float max3f(float a, float b, float c) { return __builtin_fmaxf(__builtin_fmaxf(a, b), c); }
__device__ __forceinline__ float max2f(float a, float b) { return __builtin_fmaxf(a, b); }
// Maximum (of values that are never NaN) and sum over the four lanes
// l % 16 + 16 k of a wavefront (whole wavefront active): each swap hands
// every lane its partner's value in one of the two registers, so the result
// needs no select.
__device__ __forceinline__ float quad_max16(float x) {
    int b = __builtin_bit_cast(int, x);
    v2i r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    const int r0 = r[0], r1 = r[1];
    x = max2f(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
    b = __builtin_bit_cast(int, x);
    r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    const int t0 = r[0], t1 = r[1];
    return max2f(__builtin_bit_cast(float, t0), __builtin_bit_cast(float, t1));
}
__device__ __forceinline__ float quad_sum16(float x) {
    int b = __builtin_bit_cast(int, x);
    v2i r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    const int r0 = r[0], r1 = r[1];
    x = __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
    b = __builtin_bit_cast(int, x);
    r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    const int t0 = r[0], t1 = r[1];
    return __builtin_bit_cast(float, t0) + __builtin_bit_cast(float, t1);
}
// x of another lane of the same row of 16 by a DPP pattern (whole wave active)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    const int b = __builtin_bit_cast(int, x);
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, CTRL, 0xF, 0xF, false));
}
// Largest value over the 64 lanes, in every lane: DPP within rows of 16
// (lane xor 1, xor 2, mirror of 8, mirror of 16), then the row swaps of 16
// and 32 lanes; vector instructions only (no LDS round trips).
__device__ __forceinline__ float wave_max(float v) {
    v = __builtin_fmaxf(v, dpp_f<0xB1>(v));    // quad_perm [1,0,3,2]
    v = __builtin_fmaxf(v, dpp_f<0x4E>(v));    // quad_perm [2,3,0,1]
    v = __builtin_fmaxf(v, dpp_f<0x141>(v));   // row_half_mirror
    v = __builtin_fmaxf(v, dpp_f<0x140>(v));   // row_mirror
    v = __builtin_fmaxf(v, partner16f(v));
    return __builtin_fmaxf(v, partner32f(v));
}

// ------------------------------------------------------------------ NVFP4 emulation
// Nearest e4m3 value of x >= 0 (the hardware's nearest-even conversion after
// clamping to 448, i.e. saturating), back in fp32.
__device__ __forceinline__ float e4m3_round(float x) {
    const int b = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(x, -448.0f, 448.0f), 0.0f, 0, false);
    return __builtin_amdgcn_cvt_f32_fp8(b, 0);
}
// Nearest e2m1 value of x and y (nearest-even, saturating at 6; the hardware
// conversion with a unit scale), back in fp32.
__device__ __forceinline__ v2f e2m1_round2(float x, float y) {
    const uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x, y, 1.0f, 0);
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
}
// Power-of-two NVFP4 tensor scale: the smallest 2^k with 2688 2^k >= amax
// (2688 = 448 * 6, the largest block scale times the largest e2m1 value);
// 1 for amax == 0.  With amax = f 2^e, f in [0.5, 1): 2^(e - 12) when
// f <= 2688 / 4096, else 2^(e - 11).
__device__ __forceinline__ float nv_tensor_scale(float amax) {
    if (!(amax > 0.0f)) return 1.0f;
    int e;
    const float f = __builtin_frexpf(amax, &e);
    return __builtin_ldexpf(1.0f, e - 12 + (f > 0.65625f ? 1 : 0));
}

}  // namespace bqa
