// Device-side helpers shared by the KDA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kHeadDim = 128;
constexpr int kConvTaps = 4;
constexpr int kRingTaps = kConvTaps - 1;

// bf16 travels as its 16-bit pattern: the top half of an IEEE binary32.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even; NaN stays a quiet NaN.
// fp32 -> bf16 bits, round to nearest even (the hardware conversion, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// An io value already in a register, as fp32.
__device__ __forceinline__ float io_to_f32(float x) { return x; }
__device__ __forceinline__ float io_to_f32(bf16_t x) { return bf16_to_f32(x.bits); }

template <typename IO>
__device__ __forceinline__ float load_io(const IO* p, int64_t i);
template <>
__device__ __forceinline__ float load_io<float>(const float* p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float load_io<bf16_t>(const bf16_t* p, int64_t i) {
  return bf16_to_f32(p[i].bits);
}

template <typename IO>
__device__ __forceinline__ void store_io(IO* p, int64_t i, float x);
template <>
__device__ __forceinline__ void store_io<float>(float* p, int64_t i, float x) {
  p[i] = x;
}
template <>
__device__ __forceinline__ void store_io<bf16_t>(bf16_t* p, int64_t i, float x) {
  p[i].bits = f32_to_bf16(x);
}

// Raw buffer access (CDNA buffer instructions): a resource of `bytes` bytes at `base` in
// four SGPRs, one 32-bit VGPR offset per lane and a scalar offset per access, so a
// thread's 16 rows of state cost one address register instead of 16 64-bit pointers.
// Accesses past `bytes` read 0 and are dropped on write; the check covers the lane (VGPR)
// offset, not the scalar one, so code that relies on it keeps the checked part in the
// lane offset.
typedef float f32x4_raw __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_raw __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  // word 3: 32-bit data format, the raw-buffer setting for this architecture family
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes,
                                           0x00020000);
}
__device__ __forceinline__ float4 buffer_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const f32x4_raw v = __builtin_bit_cast(f32x4_raw, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
  return make_float4(v.x, v.y, v.z, v.w);
}
// Non-temporal 16-byte store (cache policy bit 1: nt).
__device__ __forceinline__ void buffer_store16_nt(__amdgpu_buffer_rsrc_t r, int voff, int soff, const float4& v) {
  const f32x4_raw x = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_raw, x), r, voff, soff, 2);
}

// Streaming store of 16 bytes: marked non-temporal so that a buffer written once per
// launch (the decode state) does not displace reusable lines from the caches.
__device__ __forceinline__ void store_streaming(float4* p, const float4& v) {
  typedef float f32x4_nt __attribute__((ext_vector_type(4)));
  const f32x4_nt x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<f32x4_nt*>(p));
}

// e^x, sigmoid and SiLU on the hardware exp2 and reciprocal (v_exp_f32, v_rcp_f32, about
// 1 ulp each): e^x = 2^(x log2 e), whose relative error grows as |x| 6e-8 from the rounding
// of the product (under 2e-6 for |x| < 30); e^x reaches 0 and inf where fp32 does, so the
// sigmoid and SiLU go to their limits.
__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.0f + exp_fast(-x)); }
__device__ __forceinline__ float siluf_(float x) { return x * __builtin_amdgcn_rcpf(1.0f + exp_fast(-x)); }

// Lower-bounded per-channel log decay: lb * sigmoid(exp(A_log) * (z + dt_bias)).
__device__ __forceinline__ float kda_gate(float z, float dt_bias, float a_scale, float lb) {
  return lb * sigmoidf_(a_scale * (z + dt_bias));
}

// The unbounded gate: g = -exp(A_log) * softplus(z + dt_bias), a_scale = exp(A_log);
// softplus(x) = log(1 + e^x), linear in x above 20 (where e^-x is below fp32's epsilon).
__device__ __forceinline__ float kda_gate_softplus(float z, float dt_bias, float a_scale) {
  const float x = z + dt_bias;
  return -a_scale * (x > 20.f ? x + log1pf(expf(-x)) : log1pf(expf(x)));
}

// Inclusive prefix sum over each 16-lane DPP row: row_shr 1, 2, 4, 8 with zero fill for
// the lanes whose source lies before the row.  Lane 15 of a row ends with the row's total.
template <int CTRL>
__device__ __forceinline__ float dpp_shr_zero(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_prefix16(float x) {
  x += dpp_shr_zero<0x111>(x);
  x += dpp_shr_zero<0x112>(x);
  x += dpp_shr_zero<0x114>(x);
  x += dpp_shr_zero<0x118>(x);
  return x;
}
__device__ __forceinline__ float lane_value(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// Sum over the 64 lanes of a wave (all active); every lane receives the total.
__device__ __forceinline__ float wave_sum(float x) {
  x = row_prefix16(x);
  return (lane_value(x, 15) + lane_value(x, 31)) + (lane_value(x, 47) + lane_value(x, 63));
}

// Sum over lanes 0 .. 31 of a wave (active); every lane receives the total.
__device__ __forceinline__ float half_wave_sum(float x) {
  x = row_prefix16(x);
  return lane_value(x, 15) + lane_value(x, 31);
}

}  // namespace kda
