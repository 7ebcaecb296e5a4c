// Chunked prefill of the KDA core on gfx950.
//
// The algebra (docs.rs "memra_engine::kda" header prose: per-channel cumulative log gate
// Gcum, keys scaled by exp(-Gcum), queries by exp(+Gcum); "Kimi Delta Attention (KDA) --
// analysis & C kernel plan", section "Recurrence"): inside a chunk of C tokens with
// Gcum_r = g_1 + ... + g_r per key channel,
//   A[r][j] = beta_r sum_i k_ri k_ji exp(Gcum_ri - Gcum_ji)      (j < r)
//   P[r][j] =        sum_i q_ri k_ji exp(Gcum_ri - Gcum_ji)      (j <= r)
//   (I + A) [W | U~] = Diag(beta) [Ka | V],   Ka_r = k_r exp(Gcum_r)
//   U = U~ - W S;   O = Qa S + P U,           Qa_r = q_r exp(Gcum_r)
//   S <- Diag(exp(Gcum_C)) S + Kl^T U,        Kl_r = k_r exp(Gcum_C - Gcum_r)
// C = 16 here, the tile length of OpenModelAtlas "Kimi K3 - Retention gate" ("Why"):
// with g >= -5, exp(Gcum_r - Gcum_j) inside the Gram matrices is formed from a reference
// at the chunk midpoint, so each factor stays within e^(+-40); Ka, Qa and Kl only carry
// factors <= 1.
//
// Mapping: one workgroup (8 waves) per (sequence, head).  Each wave owns 16 value columns
// of the fp32 128x128 state, held across the whole sequence in MFMA accumulator tiles
// (8 key tiles of 16x16).  Those tiles double as the B operand of W.S and
// Qa.S (the contraction order inside an MFMA is free, so the A operand is read from LDS
// in the matching key order) and as the accumulator of Kl^T.U.  The bf16 instantiation
// uses v_mfma_f32_16x16x32_bf16 / 16x16x16_bf16 with fp32 accumulation; the fp32
// instantiation (fp32 io) the same data flow on v_mfma_f32_16x16x4_f32.
//
// Per chunk: (1) raw q/k/v/z/gate rows -> conv + SiLU with the conv history in registers,
// gate, Gcum, exp(+-Gcum); (2) q/k row norms; (3) scaled operands; (4) Gram tiles A, P;
// (5) forward substitution for W and U~ (fp32, one column per thread); (6) the state pass;
// (7) gated RMSNorm and the output store.
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int C = 16;          // chunk = exponent tile
constexpr int LDP = 132;       // padded row stride of [16][128] LDS arrays
constexpr int KLP = 20;        // padded row stride of the transposed Kl array
constexpr int NWAVES = 8;      // one 16-column value tile of the state per wave
constexpr int NTHREADS = 64 * NWAVES;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct SeqOrder {
  int32_t idx[kMaxOrdered];
};

struct Smem {
  float qa[C][LDP];   // silu(conv q) -> Qp = q-hat exp(Gcum - Gref)
  float ka[C][LDP];   // silu(conv k) -> Kp = k-hat exp(Gcum - Gref)
  float kx[C][LDP];   // Ka = k-hat exp(Gcum) -> W
  float va[C][LDP];   // silu(conv v) -> U~
  float ep[C][LDP];   // exp(+Gcum)
  float em[C][LDP];   // exp(-Gcum) -> Km = k-hat exp(Gref - Gcum)
  float sg[C][LDP];   // sigmoid(gate)
  float klt[kHeadDim][KLP];  // Kl^T: k-hat exp(Gcum_C - Gcum), [key][token]
  float A[C][C + 1];
  float P[C][C + 1];
  float erefp[kHeadDim], erefm[kHeadDim], eglast[kHeadDim];
  float rn[2 * C];    // 1/|q| * d^-1/2 for rows 0..15, 1/|k| for rows 16..31
  float beta[C];
  float ss[NWAVES][C];
};

// ---- MFMA operand helpers -------------------------------------------------------------
// bf16 operands are either rounded once ("hi") or split as x = hi + lo with both parts in
// bf16; a split product takes three MFMAs (hi.hi + hi.lo + lo.hi), which keeps about 16
// significant bits.  The split is used where a single rounding would show in the output
// (Gram tiles, Qa.S, P.U and the state update).

template <int N>
struct SplitBf16;
template <>
struct SplitBf16<8> {
  bf16x8_t hi, lo;
};
template <>
struct SplitBf16<4> {
  bf16x4_t hi, lo;
};

template <int N>
__device__ __forceinline__ void split_bf16(const float* x, SplitBf16<N>& r) {
#pragma unroll
  for (int s = 0; s < N; ++s) {
    const __bf16 hi = static_cast<__bf16>(x[s]);
    r.hi[s] = hi;
    r.lo[s] = static_cast<__bf16>(x[s] - static_cast<float>(hi));
  }
}

__device__ __forceinline__ f32x4_t mma32(const SplitBf16<8>& a, const SplitBf16<8>& b, f32x4_t acc,
                                         bool split) {
  if (split) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
  }
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mma16(const SplitBf16<4>& a, const SplitBf16<4>& b, f32x4_t acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.lo, b.hi, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.lo, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.hi, acc, 0, 0, 0);
}

// Hides a value from the optimiser so that address arithmetic is recomputed where it is
// used instead of being kept live (in 64-bit registers) across the whole kernel.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ f32x4_t mma_f32(float a, float b, f32x4_t acc) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

// acc += X[m][.] . S[.][n] over all 128 keys: X row-major in LDS, times an optional
// per-key scale; S is the wave's value tile (S[it][s] = key 16 it + 4 (l/16) + s).
// bf16: the key order inside each 32-key MFMA block is (l/16, s) -> 4 (l/16) + s for
// s < 4 and 16 + 4 (l/16) + s - 4 otherwise, which matches two consecutive S tiles.
template <bool F32OPS>
__device__ __forceinline__ f32x4_t x_times_s(const float (*X)[LDP], const float* scale,
                                             const f32x4_t* S, const SplitBf16<8>* Sb, bool split,
                                             int lane, f32x4_t acc) {
  const int m = lane & 15;
  const int q = lane >> 4;
  if constexpr (F32OPS) {
#pragma unroll
    for (int it = 0; it < 8; ++it)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int i = 16 * it + 4 * q + s;
        float a = X[m][i];
        if (scale) a *= scale[i];
        acc = mma_f32(a, S[it][s], acc);
      }
  } else {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float a8[8];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int i0 = 32 * kb + 4 * q + s;
        a8[s] = X[m][i0];
        a8[4 + s] = X[m][i0 + 16];
        if (scale) {
          a8[s] *= scale[i0];
          a8[4 + s] *= scale[i0 + 16];
        }
      }
      SplitBf16<8> A;
      split_bf16<8>(a8, A);
      acc = mma32(A, Sb[kb], acc, split);
    }
  }
  return acc;
}

// acc += M[m][r] . U[r][n] over the chunk's 16 tokens; M row-major in LDS (row stride
// ld), U in accumulator layout (token 4 (l/16) + s), always split in bf16.
template <bool F32OPS>
__device__ __forceinline__ f32x4_t m_times_u(const float* M, int ld, const f32x4_t& U,
                                             const SplitBf16<4>& Ub, int lane, f32x4_t acc) {
  const int m = lane & 15;
  const int q = lane >> 4;
  if constexpr (F32OPS) {
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mma_f32(M[m * ld + 4 * q + s], U[s], acc);
  } else {
    float a4[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) a4[s] = M[m * ld + 4 * q + s];
    SplitBf16<4> A;
    split_bf16<4>(a4, A);
    acc = mma16(A, Ub, acc);
  }
  return acc;
}

template <typename IO>
__global__ __launch_bounds__(NTHREADS) void prefill_kernel(PrefillArgs a, SeqOrder order) {
  constexpr bool F32OPS = std::is_same<IO, float>::value;
  __shared__ Smem sm;

  const int H = a.L.H;
  const int rank = blockIdx.x / H;
  const int h = blockIdx.x - rank * H;
  const int n = (a.num_seqs <= kMaxOrdered) ? order.idx[rank] : rank;
  const int64_t t0 = a.cu_seqlens[n];
  const int T = a.cu_seqlens[n + 1] - static_cast<int>(t0);
  const int64_t Hd = static_cast<int64_t>(H) * kHeadDim;

  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lane = t & 63;
  const int lm = lane & 15;
  const int lq = lane >> 4;
  // elementwise roles: 0 = q, 1 = k, 2 = v, 3 = z and gate, each over 128 channels
  const int role = t >> 7;
  const int ch = t & (kHeadDim - 1);
  const int64_t c = static_cast<int64_t>(h) * kHeadDim + ch;
  const int col = 16 * wave + lm;  // the value column this lane holds in the state pass

  const IO* x_b = static_cast<const IO*>(a.beta);
  const IO* x_z = static_cast<const IO*>(a.z);
  const IO* x_g = static_cast<const IO*>(a.gate);
  const IO* x_p = static_cast<const IO*>(role == 0 ? a.q : role == 1 ? a.k : a.v);

  // conv weights and history of the owned channel (roles 0-2: plane = role)
  float w[4] = {0.f, 0.f, 0.f, 0.f}, hist[3] = {0.f, 0.f, 0.f};
  const float* rin = a.ring_in ? a.ring_in + static_cast<int64_t>(n) * 3 * Hd * kRingTaps : nullptr;
  if (role < 3) {
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = a.L.conv_w[(role * Hd + c) * kConvTaps + j];
    if (rin)
#pragma unroll
      for (int j = 0; j < 3; ++j) hist[j] = rin[(role * Hd + c) * kRingTaps + j];
  }
  const float dtb = a.L.dt_bias[c];
  const float ascale = expf(a.L.A_log[h]);
  const float lb = a.L.lower_bound;

  // the wave's state tile: S[it] covers keys 16 it + 4 lq + s, value column `col`
  f32x4_t S[8];
  const int64_t sbase = (static_cast<int64_t>(n) * H + h) * kHeadDim * kHeadDim;
  if (a.state_in) {
    const float* sp = a.state_in + sbase + opaque(4 * lq * kHeadDim + col);
#pragma unroll
    for (int it = 0; it < 8; ++it)
#pragma unroll
      for (int s = 0; s < 4; ++s) S[it][s] = sp[(16 * it + s) * kHeadDim];
  } else {
#pragma unroll
    for (int it = 0; it < 8; ++it) S[it] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const float nw = a.L.norm_w[col];

  for (int c0 = 0; c0 < T; c0 += C) {
    const int L = min(C, T - c0);
    const int64_t row0 = t0 + c0;
    __syncthreads();  // the previous chunk is done with every LDS array

    // (1) elementwise prologue: conv + SiLU per plane, gate and Gcum, sigmoid(gate), beta.
    // Rows are walked with pointer increments so that no per-row 64-bit offsets stay live.
    if (role < 3) {
      float(*dst)[LDP] = role == 0 ? sm.qa : role == 1 ? sm.ka : sm.va;
      const IO* px = x_p + row0 * Hd + c;
#pragma unroll
      for (int r = 0; r < C; ++r) {
        float act = 0.f;
        if (r < L) {
          const float x = load_io(px, 0);
          const float y = w[3] * x + w[0] * hist[0] + w[1] * hist[1] + w[2] * hist[2];
          hist[0] = hist[1];
          hist[1] = hist[2];
          hist[2] = x;
          act = siluf_(y);
        }
        px += Hd;
        dst[r][ch] = act;
      }
      if (role == 0 && t < C) sm.beta[t] = (t < L) ? sigmoidf_(load_io(x_b, (row0 + t) * H + h)) : 0.f;
    } else {
      float G = 0.f;
      const IO* pz = x_z + row0 * Hd + c;
      const IO* pg = x_g + row0 * Hd + c;
#pragma unroll
      for (int r = 0; r < C; ++r) {
        float sgv = 0.f;
        if (r < L) {
          G += kda_gate(load_io(pz, 0), dtb, ascale, lb);
          sgv = sigmoidf_(load_io(pg, 0));
        }
        pz += Hd;
        pg += Hd;
        sm.sg[r][ch] = sgv;
        sm.ep[r][ch] = expf(G);
        sm.em[r][ch] = expf(-G);
        if (r == C / 2 - 1) {
          sm.erefp[ch] = expf(G);
          sm.erefm[ch] = expf(-G);
        }
      }
      sm.eglast[ch] = expf(G);
    }
    __syncthreads();

    // (2) row norms: 16 threads per (plane, row)
    {
      const int task = t >> 4, part = t & 15;
      const float(*X)[LDP] = task < C ? sm.qa : sm.ka;
      const int r = task & (C - 1);
      float ss = 0.f;
#pragma unroll
      for (int m = 0; m < kHeadDim / 16; ++m) {
        const float x = X[r][part + 16 * m];
        ss += x * x;
      }
      ss = group_sum<16>(ss);
      if (part == 0)
        sm.rn[task] = (1.0f / sqrtf(ss + a.L.l2_eps)) * (task < C ? 0.08838834764831845f : 1.0f);
    }
    __syncthreads();

    // (3) scaled operands.  q owners: Qp over qa.  k owners: Kp over ka, Km over em, Kl^T
    // and Ka = k-hat exp(Gcum) for the forward substitution.
    if (role == 0) {
      const float erm = sm.erefm[ch];
#pragma unroll
      for (int r = 0; r < C; ++r) sm.qa[r][ch] = sm.qa[r][ch] * sm.rn[r] * (sm.ep[r][ch] * erm);
    } else if (role == 1) {
      const float erp = sm.erefp[ch], erm = sm.erefm[ch], egl = sm.eglast[ch];
#pragma unroll
      for (int r = 0; r < C; ++r) {
        const float kh = sm.ka[r][ch] * sm.rn[C + r];
        const float ep = sm.ep[r][ch], em = sm.em[r][ch];
        sm.kx[r][ch] = kh * ep;
        sm.ka[r][ch] = kh * (ep * erm);
        sm.em[r][ch] = kh * (em * erp);
        sm.klt[ch][r] = kh * (em * egl);
      }
    }
    __syncthreads();

    // (4) Gram tiles: wave 0 -> A = Kp Km^T (strict lower, times beta_r); wave 1 -> P = Qp Km^T
    if (wave < 2) {
      const float(*X)[LDP] = wave == 0 ? sm.ka : sm.qa;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (F32OPS) {
#pragma unroll 8
        for (int kk = 0; kk < kHeadDim / 4; ++kk)
          acc = mma_f32(X[lm][4 * kk + lq], sm.em[lm][4 * kk + lq], acc);
      } else {
#pragma unroll
        for (int kb = 0; kb < kHeadDim / 32; ++kb) {
          float a8[8], b8[8];
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            a8[s] = X[lm][32 * kb + 8 * lq + s];
            b8[s] = sm.em[lm][32 * kb + 8 * lq + s];
          }
          SplitBf16<8> Af, Bf;
          split_bf16<8>(a8, Af);
          split_bf16<8>(b8, Bf);
          acc = mma32(Af, Bf, acc, true);
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int r = 4 * lq + s, j = lm;
        if (wave == 0)
          sm.A[r][j] = (j < r) ? sm.beta[r] * acc[s] : 0.f;
        else
          sm.P[r][j] = (j <= r) ? acc[s] : 0.f;
      }
    }
    __syncthreads();

    // (5) forward substitution (I + A) X = Diag(beta) [Ka | V], one column per thread and in
    // place in LDS: k owners turn Ka into W, v owners turn V into U~
    if (role == 1 || role == 2) {
      float(*X)[LDP] = role == 1 ? sm.kx : sm.va;
      for (int r = 0; r < C; ++r) {
        float v = sm.beta[r] * X[r][ch];
        for (int j = 0; j < r; ++j) v -= sm.A[r][j] * X[j][ch];
        X[r][ch] = v;
      }
    }
    __syncthreads();

    // (6) state pass on the wave's value tile
    f32x4_t O;
    {
      SplitBf16<8> Sb[4];
      if constexpr (!F32OPS) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          float b8[8];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            b8[s] = S[2 * kb][s];
            b8[4 + s] = S[2 * kb + 1][s];
          }
          split_bf16<8>(b8, Sb[kb]);
        }
      }
      // U = U~ - W S
      f32x4_t ws = {0.f, 0.f, 0.f, 0.f};
      ws = x_times_s<F32OPS>(sm.kx, nullptr, S, Sb, false, lane, ws);
      f32x4_t U;
#pragma unroll
      for (int s = 0; s < 4; ++s) U[s] = sm.va[4 * lq + s][col] - ws[s];
      SplitBf16<4> Ub;
      if constexpr (!F32OPS) {
        float u4[4] = {U[0], U[1], U[2], U[3]};
        split_bf16<4>(u4, Ub);
      }
      // O = Qa S + P U, with Qa = Qp exp(Gref)
      O = f32x4_t{0.f, 0.f, 0.f, 0.f};
      O = x_times_s<F32OPS>(sm.qa, sm.erefp, S, Sb, true, lane, O);
      O = m_times_u<F32OPS>(&sm.P[0][0], C + 1, U, Ub, lane, O);
      // S = Diag(exp(Gcum_C)) S + Kl^T U
#pragma unroll
      for (int it = 0; it < 8; ++it) {
#pragma unroll
        for (int s = 0; s < 4; ++s) S[it][s] *= sm.eglast[16 * it + 4 * lq + s];
        S[it] = m_times_u<F32OPS>(&sm.klt[16 * it][0], KLP, U, Ub, lane, S[it]);
      }
    }

    // (7) gated RMSNorm over each output row and the store
    {
      float ss[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) ss[s] = group_sum<16>(O[s] * O[s]);
      if (lm == 0)
#pragma unroll
        for (int s = 0; s < 4; ++s) sm.ss[wave][4 * lq + s] = ss[s];
    }
    __syncthreads();
    {
      IO* po = static_cast<IO*>(a.out) + (row0 + 4 * lq) * Hd + static_cast<int64_t>(h) * kHeadDim + col;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int r = 4 * lq + s;
        if (r < L) {
          float tot = 0.f;
#pragma unroll
          for (int wv = 0; wv < NWAVES; ++wv) tot += sm.ss[wv][r];
          const float rr = 1.0f / sqrtf(tot * (1.0f / kHeadDim) + a.L.rms_eps);
          store_io(po, 0, nw * O[s] * rr * sm.sg[r][col]);
        }
        po += Hd;
      }
    }
  }

  // final state and ring
  if (a.state_out) {
    float* sp = a.state_out + sbase + opaque(4 * lq * kHeadDim + col);
#pragma unroll
    for (int it = 0; it < 8; ++it)
#pragma unroll
      for (int s = 0; s < 4; ++s) sp[(16 * it + s) * kHeadDim] = S[it][s];
  }
  if (a.ring_out && role < 3) {
    float* rout = a.ring_out + static_cast<int64_t>(n) * 3 * Hd * kRingTaps;
#pragma unroll
    for (int j = 0; j < 3; ++j) rout[(role * Hd + c) * kRingTaps + j] = hist[j];
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, kda_dtype io, const int32_t* order_host,
                          hipStream_t stream) {
  SeqOrder ord;
  const int nord = a.num_seqs < kMaxOrdered ? a.num_seqs : kMaxOrdered;
  for (int i = 0; i < kMaxOrdered; ++i) ord.idx[i] = i < nord ? order_host[i] : 0;
  const dim3 grid(static_cast<unsigned>(a.num_seqs) * static_cast<unsigned>(a.L.H));
  const dim3 block(NTHREADS);
  if (io == KDA_F32)
    hipLaunchKernelGGL(prefill_kernel<float>, grid, block, 0, stream, a, ord);
  else
    hipLaunchKernelGGL(prefill_kernel<bf16_t>, grid, block, 0, stream, a, ord);
  return hipGetLastError();
}

}  // namespace kda
