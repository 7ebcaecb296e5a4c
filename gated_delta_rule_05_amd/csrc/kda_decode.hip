// Recurrent decode of the KDA core: one or more consecutive tokens per sequence, the fp32
// state streamed through HBM once per launch.
//
// Math ("Kimi Delta Attention (KDA) -- analysis & C kernel plan", section "Recurrence",
// and its "C kernel plan / Decode" outline): S' = Diag(exp(g)) S; u = S'^T k;
// delta = beta (v - u); S = S' + k delta^T; o = S^T q.  The readout is taken from the
// same pass: o = S'^T q + delta (k . q), so S is read once and written once.
//
// One workgroup of 256 threads per (sequence, head).  Thread t owns value columns
// 4*(t%32) .. +3 and key rows (t/32) + 8m, m = 0..15: 64 fp32 of state in registers,
// loaded and stored 16 bytes at a time (buffer instructions: one offset register) so each
// wave moves two whole 512-byte rows per access.
// The first token's activations and the conv history are loaded right behind the state
// (vector memory completes in order, so the first prologue starts as the state arrives);
// the epilogue is the sigmoid-gated RMSNorm over the head's 128 outputs.  State stores
// are non-temporal: on MI355X that lifts the read+write stream from about 5.0 to about
// 6.6 TB/s for this kernel (measured), with identical results.
//
// Several tokens per launch (the batched verify of speculative decoding, docs.rs
// "memra_engine::kda" kda_verify_rows_cached): the token loop runs over the
// register-resident state and conv history, and its body is compiled once (no unrolling
// or peeling), so each token's arithmetic is the very instruction sequence a one-token
// launch executes.  A t-token launch is therefore bit-identical, row by row, to t chained
// one-token launches, and a rollback is a replay of the same launch from the pre-round
// state over the first `keep` tokens (kda_verify_rollback_rows, kda_scan_replay).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// The low-rank decay gate's pre-activation of one channel, sum_r z_low[r] f_b[c][r] over
// the 128 ranks ("Kimi Delta Attention (KDA) -- analysis & C kernel plan", "The KDA layer,
// precisely", fact 2; the Retention-gate page's f_b_proj(f_a_proj(.))): 16-byte loads of
// both rows, four partial sums.
__device__ __forceinline__ float low_rank_z(const float* zrow, const float* frow) {
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < kHeadDim; r += 4) {
    const float4 z4 = *reinterpret_cast<const float4*>(zrow + r);
    const float4 f4 = *reinterpret_cast<const float4*>(frow + r);
    acc[0] = fmaf(z4.x, f4.x, acc[0]);
    acc[1] = fmaf(z4.y, f4.y, acc[1]);
    acc[2] = fmaf(z4.z, f4.z, acc[2]);
    acc[3] = fmaf(z4.w, f4.w, acc[3]);
  }
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}
__device__ __forceinline__ float low_rank_z(const bf16_t* zrow, const bf16_t* frow) {
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < kHeadDim; r += 8) {
    const uint4 z8 = *reinterpret_cast<const uint4*>(zrow + r);
    const uint4 f8 = *reinterpret_cast<const uint4*>(frow + r);
    const uint32_t zw[4] = {z8.x, z8.y, z8.z, z8.w}, fw[4] = {f8.x, f8.y, f8.z, f8.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[j] = fmaf(__uint_as_float(zw[j] << 16), __uint_as_float(fw[j] << 16), acc[j]);
      acc[j] = fmaf(__uint_as_float(zw[j] & 0xffff0000u), __uint_as_float(fw[j] & 0xffff0000u), acc[j]);
    }
  }
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

template <typename IO>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  const int H = a.L.H;
  const int unit = blockIdx.x;  // (b, h), h fastest
  const int b = unit / H;
  const int h = unit - b * H;
  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int cg = t & 31;
  const int rg = t >> 5;
  const int64_t Hd = static_cast<int64_t>(H) * kHeadDim;
  // rows of this sequence: [row0, row0 + n)
  int64_t row0;
  int n;
  if (a.cu) {
    row0 = a.cu[b];
    n = a.cu[b + 1] - a.cu[b];
  } else {
    row0 = static_cast<int64_t>(b) * a.tokens;
    n = a.ntok ? min(max(a.ntok[b], 0), a.tokens) : a.tokens;
  }

  // the token's vectors; the output gate by token parity, since the last readers of a
  // token's gate run while the next token's prologue writes
  __shared__ float a_q[kHeadDim], a_k[kHeadDim], a_v[kHeadDim], eg[kHeadDim], sg[2][kHeadDim];
  __shared__ float dlt[kHeadDim];
  __shared__ float part[2][3];
  // each half-wave's partial sums of u and w over its 16 key rows
  __shared__ float red[8][2][kHeadDim];
  __shared__ float part2[2];

  const IO* x_q = static_cast<const IO*>(a.q);
  const IO* x_k = static_cast<const IO*>(a.k);
  const IO* x_v = static_cast<const IO*>(a.v);
  const IO* x_z = static_cast<const IO*>(a.z);
  const IO* x_g = static_cast<const IO*>(a.gate);
  const IO* x_b = static_cast<const IO*>(a.beta);
  const int i = t & (kHeadDim - 1);
  const int64_t c = static_cast<int64_t>(h) * kHeadDim + i;

  // 1. the state loads first: the 64 KiB stream bounds the kernel, and issuing it ahead
  // of everything else measured fastest.  Then the first token's activations and the conv
  // history; each later token's activations are fetched one token ahead.  Threads < 128
  // use planes q and k of channel i, the others plane v, the decay pre-activation and the
  // output gate of channel i.  Raw io values are kept (converted only where used), and
  // every thread loads the same way through its own plane pointers, so no load is waited
  // for before it is needed.
  // with the low-rank gate, z holds z_low [rows][128]: read whole in the prologue instead
  const IO* f_b = static_cast<const IO*>(a.L.f_b);
  const IO* pa = t < kHeadDim ? x_q : x_v;
  const IO* pb = t < kHeadDim ? x_k : (f_b ? nullptr : x_z);
  IO xa{}, xb{}, xc{}, xbeta{};
  auto fetch = [&](int tok) __attribute__((always_inline)) {
    const int64_t row = row0 + tok;
    xa = pa[row * Hd + c];
    if (pb) xb = pb[row * Hd + c];
    xc = x_g[row * Hd + c];
    xbeta = x_b[row * H + h];
  };
  // state rows rg + 8 m of this (sequence, head): byte offset 16 (32 rg + cg) + 4096 m
  const int64_t soff = static_cast<int64_t>(unit) * kHeadDim * kHeadDim;
  constexpr int kStateBytes = kHeadDim * kHeadDim * 4;
  const __amdgpu_buffer_rsrc_t Sin = buffer_rsrc(a.state_in ? a.state_in + soff : nullptr, kStateBytes);
  const __amdgpu_buffer_rsrc_t Sout = buffer_rsrc(a.state_out ? a.state_out + soff : nullptr, kStateBytes);
  const int svoff = 16 * (32 * rg + cg);
  float4 s[16];
  if (a.state_in) {
#pragma unroll
    for (int m = 0; m < 16; ++m) s[m] = buffer_load16(Sin, svoff, 4096 * m);
  } else {
#pragma unroll
    for (int m = 0; m < 16; ++m) s[m] = make_float4(0.f, 0.f, 0.f, 0.f);
  }

  if (n > 0) fetch(0);

  const int64_t roff = static_cast<int64_t>(b) * 3 * Hd * kRingTaps;
  const int p0 = t < kHeadDim ? 0 : 2;  // first plane this thread holds
  float hist[2][3] = {{0.f, 0.f, 0.f}, {0.f, 0.f, 0.f}};
#pragma unroll
  for (int pp = 0; pp < 2; ++pp) {
    const int p = p0 + pp;
    if (p < 3 && a.ring_in) {
#pragma unroll
      for (int j = 0; j < 3; ++j) hist[pp][j] = a.ring_in[roff + (p * Hd + c) * kRingTaps + j];
    }
  }
  const float ascale = expf(a.L.A_log[h]);
  const float dtb = a.L.dt_bias[c];
  const float nw = a.L.norm_w[i];

#pragma clang loop unroll(disable)
  for (int tok = 0; tok < n; ++tok) {
    const int64_t xrow = (row0 + tok) * Hd;
    const float beta = sigmoidf_(io_to_f32(xbeta));

    // 2. prologue: conv + SiLU with the history, history roll, gate, beta
    if (t < kHeadDim) {
      float sums[3];
      float act[2];
      const float xs[2] = {io_to_f32(xa), io_to_f32(xb)};
#pragma unroll
      for (int p = 0; p < 2; ++p) {  // planes q, k
        const float x = xs[p];
        // re-read per token (L2): held in registers they cost the one-token step 5%
        const float* w = a.L.conv_w + (p * Hd + c) * kConvTaps;
        const float y = w[3] * x + w[0] * hist[p][0] + w[1] * hist[p][1] + w[2] * hist[p][2];
        hist[p][0] = hist[p][1];
        hist[p][1] = hist[p][2];
        hist[p][2] = x;
        act[p] = siluf_(y);
      }
      a_q[i] = act[0];
      a_k[i] = act[1];
      sums[0] = wave_sum(act[0] * act[0]);
      sums[1] = wave_sum(act[1] * act[1]);
      sums[2] = wave_sum(act[0] * act[1]);
      if ((t & 63) == 0) {
        part[wave][0] = sums[0];
        part[wave][1] = sums[1];
        part[wave][2] = sums[2];
      }
    } else {
      const float x = io_to_f32(xa);
      const float* w = a.L.conv_w + (2 * Hd + c) * kConvTaps;
      const float y = w[3] * x + w[0] * hist[0][0] + w[1] * hist[0][1] + w[2] * hist[0][2];
      hist[0][0] = hist[0][1];
      hist[0][1] = hist[0][2];
      hist[0][2] = x;
      a_v[i] = siluf_(y);
      const float zv = f_b ? low_rank_z(x_z + (row0 + tok) * kHeadDim, f_b + c * kHeadDim) : io_to_f32(xb);
      const float g = a.L.gate_kind == KDA_GATE_SOFTPLUS ? kda_gate_softplus(zv, dtb, ascale)
                                                         : kda_gate(zv, dtb, ascale, a.L.lower_bound);
      eg[i] = exp_fast(g);
      sg[tok & 1][i] = sigmoidf_(io_to_f32(xc));
    }
    if (tok + 1 < n) fetch(tok + 1);
    __syncthreads();

    // 3. decay the state and form both GEMVs, u = S'^T k-hat and w = S'^T q-hat
    const float rq = __builtin_amdgcn_rsqf(part[0][0] + part[1][0] + a.L.l2_eps) * 0.08838834764831845f;
    const float rk = __builtin_amdgcn_rsqf(part[0][1] + part[1][1] + a.L.l2_eps);
    const float qk = (part[0][2] + part[1][2]) * rq * rk;  // k-hat . q-hat
    float kh[16];
    float u0 = 0.f, u1 = 0.f, u2 = 0.f, u3 = 0.f, w0 = 0.f, w1 = 0.f, w2 = 0.f, w3 = 0.f;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int r = rg + 8 * m;
      kh[m] = a_k[r] * rk;
      const float qh = a_q[r] * rq;
      const float e = eg[r];
      s[m].x *= e;
      s[m].y *= e;
      s[m].z *= e;
      s[m].w *= e;
      u0 += s[m].x * kh[m];
      u1 += s[m].y * kh[m];
      u2 += s[m].z * kh[m];
      u3 += s[m].w * kh[m];
      w0 += s[m].x * qh;
      w1 += s[m].y * qh;
      w2 += s[m].z * qh;
      w3 += s[m].w * qh;
    }
    // the two halves of a wave hold different rows of the same columns: both partial sums
    // go to LDS, which is cheaper than combining them through lane exchanges first
    *reinterpret_cast<float4*>(&red[rg][0][cg * 4]) = make_float4(u0, u1, u2, u3);
    *reinterpret_cast<float4*>(&red[rg][1][cg * 4]) = make_float4(w0, w1, w2, w3);
    __syncthreads();

    // 4. delta and the readout for column j = t
    float o = 0.f;
    if (t < kHeadDim) {
      const int j = t;
      const float uj = ((red[0][0][j] + red[1][0][j]) + (red[2][0][j] + red[3][0][j])) +
                       ((red[4][0][j] + red[5][0][j]) + (red[6][0][j] + red[7][0][j]));
      const float wj = ((red[0][1][j] + red[1][1][j]) + (red[2][1][j] + red[3][1][j])) +
                       ((red[4][1][j] + red[5][1][j]) + (red[6][1][j] + red[7][1][j]));
      const float d = beta * (a_v[j] - uj);
      dlt[j] = d;
      o = wj + qk * d;
      const float so = wave_sum(o * o);
      if ((t & 63) == 0) part2[wave] = so;
    }
    __syncthreads();

    // 5. rank-1 update in registers, and after the last token the single state write;
    // gated RMSNorm on the output
    const float4 d4 = *reinterpret_cast<const float4*>(&dlt[cg * 4]);
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      s[m].x += kh[m] * d4.x;
      s[m].y += kh[m] * d4.y;
      s[m].z += kh[m] * d4.z;
      s[m].w += kh[m] * d4.w;
    }
    if (tok + 1 == n && a.state_out) {
#pragma unroll
      for (int m = 0; m < 16; ++m) buffer_store16_nt(Sout, svoff, 4096 * m, s[m]);
    }
    if (t < kHeadDim && a.out) {
      const int j = t;
      const float r = __builtin_amdgcn_rsqf((part2[0] + part2[1]) * (1.0f / kHeadDim) + a.L.rms_eps);
      store_io(static_cast<IO*>(a.out), xrow + static_cast<int64_t>(h) * kHeadDim + j,
               nw * o * r * sg[tok & 1][j]);
    }
    // Three barriers per token, none here: the next token's prologue writes a_q, a_k,
    // a_v, eg and part, all read before this token's last barrier, and the other parity
    // of sg; red, dlt and part2 are rewritten only after the next token's first barrier.
  }

  // 6. no token: the state passes through; then the conv history
  if (n == 0 && a.state_out) {
#pragma unroll
    for (int m = 0; m < 16; ++m) buffer_store16_nt(Sout, svoff, 4096 * m, s[m]);
  }
#pragma unroll
  for (int pp = 0; pp < 2; ++pp) {
    const int p = p0 + pp;
    if (p < 3 && a.ring_out) {
#pragma unroll
      for (int j = 0; j < 3; ++j) a.ring_out[roff + (p * Hd + c) * kRingTaps + j] = hist[pp][j];
    }
  }
}

hipError_t launch_decode(const DecodeArgs& a, kda_dtype io, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.batch) * static_cast<unsigned>(a.L.H));
  const dim3 block(256);
  if (io == KDA_F32)
    hipLaunchKernelGGL(decode_kernel<float>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(decode_kernel<bf16_t>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace kda
