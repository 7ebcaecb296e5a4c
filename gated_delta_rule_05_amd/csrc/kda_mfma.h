// MFMA, DPP and LDS helpers shared by the prefill kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kda_device.h"

namespace kda {
namespace mf {

constexpr int C = 16;  // chunk = exponent tile

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

// exp(x) through the hardware base-2 exponential; relative error ~1e-6 over the ranges
// used here (|x| <= 80).
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float frcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fsigmoid(float x) { return frcp(1.0f + fexp(-x)); }

// Cross-lane moves inside a row of 16 lanes (DPP): row_newbcast:n hands every lane of the
// row the value of its lane n; row_ror:k rotates the row by k lanes.
// Every control used here (row_ror, row_newbcast) reads a valid lane of the same row for
// every lane, so the instruction's old value is never kept; mov_dpp leaves it undefined,
// which lets the compiler fold the move into the consuming add (v_add_f32_dpp) instead of
// first zeroing a temporary.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
// A DPP move whose lanes without a source lane in their row (row_shr past the row start)
// read 0.
template <int CTRL>
__device__ __forceinline__ float dpp_z(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
  return dpp<0x150 + N>(x);
}
// Multiplies the four key rows 16 IT + 4 lq + s (s = 0..3) of a state tile by their
// factors, where lane n of each 16-lane row holds the factors of (it, s) = (n / 2,
// 2 (n % 2)) in e0 and (n / 2, 2 (n % 2) + 1) in e1: row s takes lane 2 IT + s / 2's value.
template <int IT, typename V4>
__device__ __forceinline__ void decay_tile(V4& st, float e0, float e1) {
  st[0] *= row_bcast<2 * IT>(e0);
  st[1] *= row_bcast<2 * IT>(e1);
  st[2] *= row_bcast<2 * IT + 1>(e0);
  st[3] *= row_bcast<2 * IT + 1>(e1);
}
// Sum over the 16 lanes of a row, delivered to every lane of the row.
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0x128>(x);
  x += dpp<0x124>(x);
  x += dpp<0x122>(x);
  x += dpp<0x121>(x);
  return x;
}

// Workgroup barrier for LDS traffic only.  __syncthreads() is also a fence on global
// memory and waits for every outstanding global load, which would drain the next
// chunk's prefetched rows at each barrier; nothing global is exchanged between the
// threads of a workgroup here, so waiting for LDS operations is enough.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16 bytes per lane from global memory straight into LDS (buffer_load_dwordx4 ... lds):
// lane l's bytes land at lds_wave_base + 16 l, so one wave fills 1 KiB.  lds_wave_base is
// an LDS byte address, wave-uniform (it goes to M0).  The source is a buffer resource
// (base and size in SGPRs) with a 32-bit lane offset and a scalar offset, so the per-lane
// address costs no 64-bit arithmetic, and lanes past the resource's size touch no memory
// (what their LDS bytes then hold is not to be used).  The range check covers the lane offset only, not the
// scalar one: an offset that must stay within the resource belongs in voff.  Completion
// is counted by vmcnt, not lgkmcnt: the issuing
// wave waits with wait_vm() before the barrier that publishes the data.  The instruction
// is issued from inline assembly so that the compiler does not track it: it would
// otherwise wait for the transfer before LDS accesses it cannot prove disjoint from the
// target, which stalls on HBM latency.  The vmcnt waits the compiler does compute for its
// own loads stay correct (vector memory operations complete in issue order, so extra
// ones in flight only make those waits longer).  The resource must be in SGPRs: build it
// with uniform_rsrc, which takes its wave-uniform inputs through readfirstlane whatever
// the compiler's divergence analysis concludes about where they came from.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, int bytes) {
  const uint64_t b = reinterpret_cast<uintptr_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
  const void* u = reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return buffer_rsrc(u, __builtin_amdgcn_readfirstlane(bytes));
}
// The LDS byte address of a __shared__ object: the low half of its flat address (the LDS
// aperture puts the offset there), taken without an address-space cast and its null test.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, int voff, int soff, uint32_t lds_wave_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_wave_base);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds), "s"(soff)
               : "memory", "m0");
}
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Waits for this wave's outstanding LDS operations (e.g. reads of a buffer it refills next).
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Hides a value from the optimiser so that address arithmetic is recomputed where it is
// used instead of being kept live (in 64-bit registers) across the whole kernel.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ void split_store(__bf16* hi, __bf16* lo, float x) {
  const __bf16 h = static_cast<__bf16>(x);
  *hi = h;
  *lo = static_cast<__bf16>(x - static_cast<float>(h));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// The bf16 (hi, lo) split of two values, each half packed two to a register: hi rounds x
// to nearest even, lo rounds the exact remainder x - hi.  One packed conversion per half
// and pair; the hi values come back to fp32 by a shift and a mask.  The same values as
// split_store, at three instructions per value instead of four.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){x0, x1}, bf16x2_t));
  const float l0 = x0 - __uint_as_float(h << 16);
  const float l1 = x1 - __uint_as_float(h & 0xffff0000u);
  hi = h;
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){l0, l1}, bf16x2_t));
}
__device__ __forceinline__ __bf16 bf16_lo(uint32_t w) { return __builtin_bit_cast(__bf16, static_cast<uint16_t>(w)); }
__device__ __forceinline__ __bf16 bf16_hi(uint32_t w) {
  return __builtin_bit_cast(__bf16, static_cast<uint16_t>(w >> 16));
}
// split_store of two values at once
__device__ __forceinline__ void split_store2(__bf16* hi0, __bf16* lo0, __bf16* hi1, __bf16* lo1, float x0,
                                             float x1) {
  uint32_t h, l;
  split2(x0, x1, h, l);
  *hi0 = bf16_lo(h);
  *lo0 = bf16_lo(l);
  *hi1 = bf16_hi(h);
  *lo1 = bf16_hi(l);
}

// Splits of N = 4 or 8 consecutive values into bf16 vectors (hi, lo).
template <int N, typename V>
__device__ __forceinline__ void split_vec(const float* x, V& hi, V& lo) {
  static_assert(N == 4 || N == 8, "split_vec: 4 or 8 values");
  uint32_t h[N / 2], l[N / 2];
#pragma unroll
  for (int s = 0; s < N / 2; ++s) split2(x[2 * s], x[2 * s + 1], h[s], l[s]);
  if constexpr (N == 4) {
    hi = __builtin_bit_cast(V, (u32x2_t){h[0], h[1]});
    lo = __builtin_bit_cast(V, (u32x2_t){l[0], l[1]});
  } else {
    hi = __builtin_bit_cast(V, (u32x4_t){h[0], h[1], h[2], h[3]});
    lo = __builtin_bit_cast(V, (u32x4_t){l[0], l[1], l[2], l[3]});
  }
}

__device__ __forceinline__ f32x4_t mma32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// fp16 operands: 3 more mantissa bits than bf16, for the products whose operands stay
// inside fp16's range (the state pass against the state, see the prefill kernel)
__device__ __forceinline__ f32x4_t mma32h(f16x8_t a, f16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma4(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// The same for a 16-long inner dimension on the 16x16x32 instruction, which issues in the
// same time as the 16x16x16 one.  The A operand carries both halves, a = [ah | al] (slots
// j < 4 of a lane hold ah, slots j >= 4 al, for the same four positions of the inner
// dimension), and the two B operands are built once per tile: b_l0 = [bl | 0] and
// b_hh = [bh | bh].  Then a b_l0 = ah bl and a b_hh = ah bh + al bh.  Both steps use the
// same opcode: a 16x16x16 result taken as the accumulator of a 16x16x32 a few instructions
// later gave wrong rows on gfx950, whereas chains of one opcode accumulate correctly.
__device__ __forceinline__ f32x4_t mma16p(bf16x8_t a, bf16x8_t b_l0, bf16x8_t b_hh, f32x4_t c) {
  c = mma32(a, b_l0, c);
  return mma32(a, b_hh, c);
}
// (b_l0, b_hh) from the bf16 halves of a B operand
__device__ __forceinline__ void b_pair(bf16x4_t bh, bf16x4_t bl, bf16x8_t& b_l0, bf16x8_t& b_hh) {
  const bf16x4_t z = {};
  b_l0 = __builtin_shufflevector(bl, z, 0, 1, 2, 3, 4, 5, 6, 7);
  b_hh = __builtin_shufflevector(bh, bh, 0, 1, 2, 3, 4, 5, 6, 7);
}
// Position of element x (0..15) of a row in the interleaved (hi, lo) layout read by
// mma16p: lane group x / 4 takes 8 values, ah then al.  The lo part sits 4 further on.
__device__ __forceinline__ int il16(int x) { return 8 * (x >> 2) + (x & 3); }

template <typename V, typename E>
__device__ __forceinline__ V ld(const E* p) {
  return *reinterpret_cast<const V*>(p);
}

// 4 consecutive values as (hi, lo) bf16 at hi[0..3], lo[0..3] (8-byte writes), or hi only.
__device__ __forceinline__ void store4(__bf16* hi, __bf16* lo, const float* x) {
  bf16x4_t h, l;
  split_vec<4>(x, h, l);
  *reinterpret_cast<bf16x4_t*>(hi) = h;
  *reinterpret_cast<bf16x4_t*>(lo) = l;
}
__device__ __forceinline__ void store4_f16(_Float16* dst, const float* x) {
  f16x4_t h;
#pragma unroll
  for (int v = 0; v < 4; ++v) h[v] = static_cast<_Float16>(x[v]);
  *reinterpret_cast<f16x4_t*>(dst) = h;
}
// One elimination step per row j of the 16x16 unit-lower system: every lane of a 16-lane
// row takes row j's values from lane j of its own row (DPP broadcast).  The row's
// coefficients come negated (nrow = -A[row]), so that a step is one multiply-add with the
// broadcast as its DPP source (v_fmac_f32_dpp) instead of a DPP move and a negated fma.
template <int J>
__device__ __forceinline__ void eliminate(float* tt, const float* nrow) {
  if constexpr (J < C - 1) {
#pragma unroll
    for (int s = 0; s < 4; ++s) tt[s] = fmaf(row_bcast<J>(tt[s]), nrow[J], tt[s]);
    eliminate<J + 1>(tt, nrow);
  }
}

// The same for two of the four strided slots (SA, SB) only: columns never mix in the
// elimination, so two waves can share it, one taking slots {0, 3} and the other {1, 2}
// (18 updates each).
//
// A step is one v_fmac_f32_dpp, t += bcast_J(t) * nrow[J], issued from inline assembly
// (the compiler keeps a separate DPP move in front of the multiply-add, which doubles the
// dependency chain).  The s_nop in front of it provides the two wait states a DPP read
// needs after the VALU write of its source.
template <int J>
__device__ __forceinline__ void elim_step(float& t, float nr) {
  asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %0, %1 row_newbcast:%2 row_mask:0xf bank_mask:0xf"
               : "+v"(t)
               : "v"(nr), "i"(J));
}
template <int J, int SA, int SB>
__device__ __forceinline__ void eliminate_strided2(float* tt, const float* nrow) {
  if constexpr (J < C - 1) {
    if constexpr (SA <= J / 4) elim_step<J>(tt[0], nrow[J]);
    if constexpr (SB <= J / 4) elim_step<J>(tt[1], nrow[J]);
    eliminate_strided2<J + 1, SA, SB>(tt, nrow);
  }
}

}  // namespace mf
}  // namespace kda
