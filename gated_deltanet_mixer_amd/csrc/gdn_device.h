// gdn_device.h -- device-side helpers shared by the mixer's gfx950 kernels:
// bf16/fp16 conversion, wave64 reductions and MFMA tile wrappers.
//
// MFMA lane layouts used throughout (CDNA3/CDNA4, wave64):
//   v_mfma_f32_16x16x32_f16  A[16][32]: lane l holds row l%16, 8 k-values
//                            B[32][16]: lane l holds col l%16, 8 k-values
//                            C[16][16]: lane l holds col l%16, rows 4*(l/16)+e, e<4
//   v_mfma_f32_16x16x16_f16  as above with 4 k-values per lane.
// A product is invariant under any permutation of k applied to A and B
// alike, so the kernels only rely on the row/column and C layouts; the lane
// k-slot assignment used here is k = (k-values per lane) * (l/16) + e.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // 16-byte copy unit kept in registers

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    __bf16 h = static_cast<__bf16>(x);
    return __builtin_bit_cast(uint16_t, h);
}

// 8 bf16 packed in a uint4 -> 8 floats.
__device__ __forceinline__ void unpack_bf16x8(const uint4 &p, float (&f)[8]) {
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

__device__ __forceinline__ uint4 pack_bf16x8(const float (&f)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = static_cast<uint32_t>(f32_to_bf16(f[2 * i])) |
               (static_cast<uint32_t>(f32_to_bf16(f[2 * i + 1])) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// ---------------------------------------------------------------- math

// a.lo * b.lo + a.hi * b.hi + c for two bf16 pairs, accumulated in fp32 (v_dot2c_f32_bf16)
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
__device__ __forceinline__ float bf16_dot2(unsigned int a, unsigned int b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// x * sigmoid(x) in fp32 from the hardware base-2 exponential and reciprocal
// (v_exp_f32, v_rcp_f32: about 1 ulp each).  Saturates correctly: a large
// negative x gives exp2 -> inf, rcp -> 0.
__device__ __forceinline__ float silu(float x) {
    const float t = __builtin_amdgcn_exp2f(x * -1.4426950408889634f);
    return x * __builtin_amdgcn_rcpf(1.0f + t);
}

// Gates from their logits ("How Qwen3.5 works" §9.5), in fp32:
// g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b).
__device__ __forceinline__ float gate_g(float a, float A_log, float dt_bias) {
    const float x = a + dt_bias;
    const float sp = x > 20.0f ? x : log1pf(expf(x));  // softplus; ln(1 + e^x) = x to fp32 beyond 20
    return -expf(A_log) * sp;
}
__device__ __forceinline__ float gate_beta(float b) { return 1.0f / (1.0f + expf(-b)); }

// ---------------------------------------------------------------- reductions

// Sum over the 64 lanes of a wave; every lane receives the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v += __shfl_xor(v, o, 64);
    return v;
}

// Sum over aligned groups of `W` lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = W / 2; o >= 1; o >>= 1)
        v += __shfl_xor(v, o, 64);
    return v;
}

// v of another lane of the same 16-lane row, through the DPP operand modifier (no LDS)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over each row of 16 lanes (lanes 16 k .. 16 k + 15), every lane of the row receiving
// the same bits: each step adds two equal partial sums, in either order, across a quad, a
// half-row and the row (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror).
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    v += dpp_f<0x140>(v);
    return v;
}

// ---------------------------------------------------------------- barriers

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for every
// outstanding global load and store of the wave; kernels whose waves exchange
// data through LDS alone use this instead, so prefetches and output stores
// stay in flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------- hardware ids

// Index of the XCD (accelerator complex die) the calling wave runs on.
__device__ __forceinline__ unsigned int xcc_id() {
    unsigned int v;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(v));
    return v;
}

// ---------------------------------------------------------------- MFMA

__device__ __forceinline__ floatx4 mfma16x16x32(const half8 &a, const half8 &b, const floatx4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma16x16x16(const half4 &a, const half4 &b, const floatx4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// Load an operand fragment of 8 consecutive fp16 from LDS (16-byte aligned).
__device__ __forceinline__ half8 lds_half8(const _Float16 *p) {
    return *reinterpret_cast<const half8 *>(p);
}
__device__ __forceinline__ half4 lds_half4(const _Float16 *p) {
    return *reinterpret_cast<const half4 *>(p);
}

} // namespace gdn
