// Chunked prefill of the KDA core on gfx950.
//
// The algebra (docs.rs "memra_engine::kda" header prose: per-channel cumulative log gate
// Gcum, keys scaled by exp(-Gcum), queries by exp(+Gcum); "Kimi Delta Attention (KDA) --
// analysis & C kernel plan", section "Recurrence"): inside a chunk of C tokens with
// Gcum_r = g_1 + ... + g_r per key channel,
//   A[r][j] = beta_r sum_i k_ri k_ji exp(Gcum_ri - Gcum_ji)      (j < r)
//   P[r][j] =        sum_i q_ri k_ji exp(Gcum_ri - Gcum_ji)      (j <= r)
//   T = (I + A)^-1 Diag(beta);  W = T Ka,  U~ = T V,          Ka_r = k_r exp(Gcum_r)
//   U = U~ - W S;   O = Qa S + P U,                              Qa_r = q_r exp(Gcum_r)
//   S <- Diag(exp(Gcum_C)) S + Kl^T U,                           Kl_r = k_r exp(Gcum_C - Gcum_r)
// C = 16, the tile length of OpenModelAtlas "Kimi K3 - Retention gate" ("Why"): with
// g >= -5, exp(Gcum_r - Gcum_j) inside the Gram tiles is formed from a reference at the
// chunk midpoint, so each factor stays within e^(+-40); Ka, Qa and Kl carry factors <= 1.
//
// Mapping: one workgroup of 8 waves per (sequence, head).  Wave w owns value columns
// 16w .. 16w+15 of the fp32 128x128 state for the whole sequence, as 8 MFMA accumulator
// tiles (key rows 16 it + 4 (lane/16) + s, value column 16 w + lane%16).  Those tiles are
// also the B operand of W.S and Qa.S (the contraction order inside an MFMA is free, so the
// A operand is supplied in the matching key order) and the accumulator of Kl^T.U.
//
// Per chunk, with the raw rows of the next chunk already loading (16-byte loads, parked
// in LDS for the next iteration):
//   (1) q/k/v conv + SiLU (history in registers), gate, Gcum, sigmoid(gate), beta
//   (2) q/k row norms
//   (3) scaled operands, stored once in MFMA-ready form
//   (4) Gram tiles A and P (waves 0 and 1)
//   (5) every wave: T by elimination across lanes (DPP broadcasts); W^T = Ka^T T^T lands directly in the
//       A-operand layout of W.S; U~ = T V for its own value tile; the state pass
//   (6) sigmoid-gated RMSNorm of each output row and the store
// This kernel serves fp32 io: every product runs on v_mfma_f32_16x16x4_f32 (fp32 operands,
// fp32 accumulation).  bf16 io has its own producer/consumer kernel (kda_prefill_pc.hip).

#include "kda_device.h"
#include "kda_internal.h"
#include "kda_mfma.h"

namespace kda {

namespace {

using namespace mf;
constexpr int NWAVES = 8;    // one 16-column value tile of the state per wave
constexpr int NTHREADS = 64 * NWAVES;
constexpr int LDP = 132;     // row stride (floats) of fp32 [16][128] arrays
constexpr int AP = 20;       // row stride (floats) of the A tile

struct SeqOrder {
  int32_t idx[kMaxOrdered];
};

// MFMA operands, fp32.
struct alignas(16) Ops {
  static constexpr int OPP = 132;  // row stride of [16][128] operands
  static constexpr int KTP = 20;   // row stride of [128][16] operands
  static constexpr int PPP = 20;   // row stride of the P tile
  float qp[C][OPP];         // Qp = q-hat exp(Gcum - Gref)
  float qa[C][OPP];         // Qa = q-hat exp(Gcum)
  float kp[C][OPP];         // Kp = k-hat exp(Gcum - Gref)
  float km[C][OPP];         // Km = k-hat exp(Gref - Gcum)
  float kat[kHeadDim][KTP];  // Ka^T
  float klt[kHeadDim][KTP];  // Kl^T
  float p[C][PPP];          // P tile (lower incl.)
};

struct alignas(16) Smem {
  static constexpr int RAWP = kHeadDim + 4;
  float raw[5][C][RAWP];  // raw rows of q, k, v, z, gate
  float braw[C];          // raw beta
  float aq[C][LDP];    // silu(conv q)
  float ak[C][LDP];    // silu(conv k)
  float va[C][LDP];    // silu(conv v) = V
  float gam[C][LDP];   // Gcum
  float sg[2][C][LDP];  // sigmoid(gate), double-buffered across chunks
  Ops op;
  float A[C][AP];      // A tile times beta (strict lower), fp32
  float g7[kHeadDim];  // Gcum at the chunk midpoint (Gram reference)
  float g15[kHeadDim];  // Gcum at the chunk end
  float eg15[kHeadDim];  // exp(Gcum at the chunk end)
  float rn[2 * C];     // 1/|q| * d^-1/2 for rows 0..15, 1/|k| for rows 16..31
  float beta[C];
  float ss[2][NWAVES][C];
};

__global__ __launch_bounds__(NTHREADS) void prefill_kernel(PrefillArgs a, SeqOrder order) {
  using OP = Ops;
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
  const int role = t >> 7;  // elementwise roles: 0 = q, 1 = k, 2 = v, 3 = z and gate
  const int ch = t & (kHeadDim - 1);
  const int64_t c = static_cast<int64_t>(h) * kHeadDim + ch;
  const int col = 16 * wave + lm;  // value column this lane holds in the state pass

  const float* x_b = static_cast<const float*>(a.beta);

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

  // the wave's state tile
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

  // Raw rows of the next chunk (q, k, v, z, gate: 16 rows x 128 channels each) are
  // fetched as 16-byte segments right after the current chunk's prologue, held in
  // registers while the chunk is processed, and parked in LDS just before the chunk's last
  // barrier.  Rows past the end of the sequence re-read its last row (always in bounds)
  // and are masked when used.
  constexpr int E = sizeof(float);
  constexpr int SPR = kHeadDim * E / 16;  // 16-byte segments per row
  constexpr int NSEG = 5 * C * SPR;
  constexpr int NRND = (NSEG + NTHREADS - 1) / NTHREADS;
  uint4 seg0, seg1, seg2, seg3, seg4;
  // plane base pointers (uniform per wave: a wave's segments all fall in one plane)
  const char* const pq = static_cast<const char*>(a.q);
  const char* const pk = static_cast<const char*>(a.k);
  const char* const pv = static_cast<const char*>(a.v);
  const char* const pz = static_cast<const char*>(a.z);
  const char* const pgt = static_cast<const char*>(a.gate);
#define KDA_SEG_SRC(k, c0n, Ln)                                                            \
  ([&]() -> const uint4* {                                                                 \
    const int sidx = t + (k) * NTHREADS;                                                   \
    /* one plane per wave and round: make the plane index scalar */                        \
    const int pl = __builtin_amdgcn_readfirstlane(sidx / (C * SPR));                       \
    const int rem = sidx % (C * SPR);                                                      \
    const int r = rem / SPR, part = rem % SPR;                                             \
    const char* base = pl == 0 ? pq : pl == 1 ? pk : pl == 2 ? pv : pl == 3 ? pz : pgt;    \
    return reinterpret_cast<const uint4*>(                                                 \
        base + ((t0 + (c0n) + min(r, (Ln) - 1)) * Hd + static_cast<int64_t>(h) * kHeadDim) * E + \
        16 * part);                                                                        \
  }())
#define KDA_SEG_DST(k)                                                                     \
  ([&]() -> uint4* {                                                                       \
    const int sidx = t + (k) * NTHREADS;                                                   \
    const int pl = sidx / (C * SPR), rem = sidx % (C * SPR);                               \
    const int r = rem / SPR, part = rem % SPR;                                             \
    return reinterpret_cast<uint4*>(&sm.raw[pl][r][part * (16 / E)]);                      \
  }())
#define KDA_SEG_OK(k) (NSEG % NTHREADS == 0 || t + (k) * NTHREADS < NSEG)
  float braw = 0.f;
  auto prefetch = [&](int c0n) __attribute__((always_inline)) {
    const int Ln = min(C, T - c0n);
    if (KDA_SEG_OK(0)) seg0 = *KDA_SEG_SRC(0, c0n, Ln);
    if (NRND > 1 && KDA_SEG_OK(1)) seg1 = *KDA_SEG_SRC(1, c0n, Ln);
    if (NRND > 2 && KDA_SEG_OK(2)) seg2 = *KDA_SEG_SRC(2, c0n, Ln);
    if (NRND > 3 && KDA_SEG_OK(3)) seg3 = *KDA_SEG_SRC(3, c0n, Ln);
    if (NRND > 4 && KDA_SEG_OK(4)) seg4 = *KDA_SEG_SRC(4, c0n, Ln);
    if (t < C) braw = x_b[(t0 + c0n + min(t, Ln - 1)) * H + h];
  };
  auto stage = [&]() __attribute__((always_inline)) {
    if (KDA_SEG_OK(0)) *KDA_SEG_DST(0) = seg0;
    if (NRND > 1 && KDA_SEG_OK(1)) *KDA_SEG_DST(1) = seg1;
    if (NRND > 2 && KDA_SEG_OK(2)) *KDA_SEG_DST(2) = seg2;
    if (NRND > 3 && KDA_SEG_OK(3)) *KDA_SEG_DST(3) = seg3;
    if (NRND > 4 && KDA_SEG_OK(4)) *KDA_SEG_DST(4) = seg4;
    if (t < C) sm.braw[t] = braw;
  };
  static_assert(NRND <= 5, "five prefetch registers");
  static_assert((C * SPR) % 64 == 0, "a wave's segments must fall in one plane");
  if (T > 0) {
    prefetch(0);
    stage();
    lds_barrier();
  }

  const int last_c0 = T > 0 ? ((T - 1) / C) * C : 0;
  int buf = 0;
  for (int c0 = 0; c0 < T; c0 += C, buf ^= 1) {
    const int L = min(C, T - c0);
    const int64_t row0 = t0 + c0;

    // (1) elementwise prologue
    if (role < 3) {
      float(*dst)[LDP] = role == 0 ? sm.aq : role == 1 ? sm.ak : sm.va;
#pragma unroll
      for (int r = 0; r < C; ++r) {
        const float x = sm.raw[role][r][ch];
        const float y = w[3] * x + w[0] * hist[0] + w[1] * hist[1] + w[2] * hist[2];
        const bool live = r < L;
        if (live) {
          hist[0] = hist[1];
          hist[1] = hist[2];
          hist[2] = x;
        }
        dst[r][ch] = live ? y * fsigmoid(y) : 0.f;
      }
    } else {
      float G = 0.f;
#pragma unroll
      for (int r = 0; r < C; ++r) {
        const bool live = r < L;
        G += live ? lb * fsigmoid(ascale * (sm.raw[3][r][ch] + dtb)) : 0.f;
        sm.gam[r][ch] = G;
        sm.sg[buf][r][ch] = live ? fsigmoid(sm.raw[4][r][ch]) : 0.f;
        if (r == C / 2 - 1) sm.g7[ch] = G;
      }
      sm.g15[ch] = G;
      sm.eg15[ch] = fexp(G);
    }
    if (t < C) sm.beta[t] = (t < L) ? fsigmoid(sm.braw[t]) : 0.f;
    // next chunk's raw rows (the last chunk re-reads itself)
    prefetch(min(c0 + C, last_c0));
    lds_barrier();

    // (2) row norms: 16 threads per (plane, row)
    {
      const int task = t >> 4, part = t & 15;
      const float(*X)[LDP] = task < C ? sm.aq : sm.ak;
      const int r = task & (C - 1);
      float ss = 0.f;
#pragma unroll
      for (int m = 0; m < kHeadDim / 16; ++m) {
        const float x = X[r][part + 16 * m];
        ss += x * x;
      }
      ss = row_sum16(ss);
      if (part == 0)
        sm.rn[task] = (1.0f / sqrtf(ss + a.L.l2_eps)) * (task < C ? 0.08838834764831845f : 1.0f);
    }
    lds_barrier();

    // (3) scaled operands, written once in MFMA-ready form, by 8-channel work items:
    // threads 0..255 take (row, 8 channels) of Qp, Kp, Km; threads 256..511 take
    // (row, one lane group) of Qa in the key order of the .S products, and
    // (channel, 8 rows) of Ka^T and Kl^T
    {
      if (t < 256) {
        const int r = t >> 4, c8 = 8 * (t & 15);
        float q8[8], k8[8], d8[8];
#pragma unroll
        for (int v = 0; v < 8; v += 4) {
          const float4 qv = *reinterpret_cast<const float4*>(&sm.aq[r][c8 + v]);
          const float4 kv = *reinterpret_cast<const float4*>(&sm.ak[r][c8 + v]);
          const float4 gv = *reinterpret_cast<const float4*>(&sm.gam[r][c8 + v]);
          const float4 g7 = *reinterpret_cast<const float4*>(&sm.g7[c8 + v]);
          q8[v] = qv.x; q8[v + 1] = qv.y; q8[v + 2] = qv.z; q8[v + 3] = qv.w;
          k8[v] = kv.x; k8[v + 1] = kv.y; k8[v + 2] = kv.z; k8[v + 3] = kv.w;
          d8[v] = gv.x - g7.x; d8[v + 1] = gv.y - g7.y; d8[v + 2] = gv.z - g7.z; d8[v + 3] = gv.w - g7.w;
        }
        const float rq = sm.rn[r], rk = sm.rn[C + r];
        float qp[8], kp[8], km[8];
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const float el = fexp(d8[v]), er = fexp(-d8[v]);
          qp[v] = q8[v] * rq * el;
          kp[v] = k8[v] * rk * el;
          km[v] = k8[v] * rk * er;
        }
        *reinterpret_cast<float4*>(&sm.op.qp[r][c8]) = make_float4(qp[0], qp[1], qp[2], qp[3]);
        *reinterpret_cast<float4*>(&sm.op.qp[r][c8 + 4]) = make_float4(qp[4], qp[5], qp[6], qp[7]);
        *reinterpret_cast<float4*>(&sm.op.kp[r][c8]) = make_float4(kp[0], kp[1], kp[2], kp[3]);
        *reinterpret_cast<float4*>(&sm.op.kp[r][c8 + 4]) = make_float4(kp[4], kp[5], kp[6], kp[7]);
        *reinterpret_cast<float4*>(&sm.op.km[r][c8]) = make_float4(km[0], km[1], km[2], km[3]);
        *reinterpret_cast<float4*>(&sm.op.km[r][c8 + 4]) = make_float4(km[4], km[5], km[6], km[7]);
      } else {
        const int u = t - 256;
        {
          // Qa: row r, lane group (kb, g): keys 32kb + 4g + 0..3 and 32kb + 16 + 4g + 0..3
          const int r = u >> 4, kb = (u >> 2) & 3, g = u & 3;
          const int k0 = 32 * kb + 4 * g;
          const float rq = sm.rn[r];
          float qa[8];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const float4 qv = *reinterpret_cast<const float4*>(&sm.aq[r][k0 + 16 * half]);
            const float4 gv = *reinterpret_cast<const float4*>(&sm.gam[r][k0 + 16 * half]);
            qa[4 * half + 0] = qv.x * rq * fexp(gv.x);
            qa[4 * half + 1] = qv.y * rq * fexp(gv.y);
            qa[4 * half + 2] = qv.z * rq * fexp(gv.z);
            qa[4 * half + 3] = qv.w * rq * fexp(gv.w);
          }
          // fp32 operands keep the natural key order
          *reinterpret_cast<float4*>(&sm.op.qa[r][k0]) = make_float4(qa[0], qa[1], qa[2], qa[3]);
          *reinterpret_cast<float4*>(&sm.op.qa[r][k0 + 16]) = make_float4(qa[4], qa[5], qa[6], qa[7]);
        }
        {
          // Ka^T and Kl^T: channel cc, rows 8 hf .. 8 hf + 7
          const int cc = u >> 1, hf = u & 1;
          const float gend = sm.g15[cc];
          float ka[8], kl[8];
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            const int r = 8 * hf + v;
            const float kh = sm.ak[r][cc] * sm.rn[C + r];
            const float G = sm.gam[r][cc];
            ka[v] = kh * fexp(G);
            kl[v] = kh * fexp(gend - G);
          }
#pragma unroll
          for (int v = 0; v < 8; v += 4) {
            *reinterpret_cast<float4*>(&sm.op.kat[cc][8 * hf + v]) = make_float4(ka[v], ka[v + 1], ka[v + 2], ka[v + 3]);
            *reinterpret_cast<float4*>(&sm.op.klt[cc][8 * hf + v]) = make_float4(kl[v], kl[v + 1], kl[v + 2], kl[v + 3]);
          }
        }
      }
    }
    lds_barrier();

    // (4) Gram tiles: wave 0 -> A = Kp Km^T (strict lower, times beta_r); wave 1 -> P = Qp Km^T
    if (wave < 2) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      const float(*X)[OP::OPP] = wave == 0 ? sm.op.kp : sm.op.qp;
#pragma unroll 8
      for (int kk = 0; kk < kHeadDim / 4; ++kk) acc = mma4(X[lm][4 * kk + lq], sm.op.km[lm][4 * kk + lq], acc);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int r = 4 * lq + s, j = lm;
        if (wave == 0)
          sm.A[r][j] = (j < r) ? sm.beta[r] * acc[s] : 0.f;
        else
          sm.op.p[r][j] = (j <= r) ? acc[s] : 0.f;
      }
    }
    lds_barrier();

    // (5a) T = (I + A)^-1 Diag(beta), row-elimination with rows spread over lanes: lane
    // (lm, lq) ends up holding T[lm][4 lq + s].  A[r][j] = 0 for j >= r, so the update
    // is unconditional.
    float tt[4];
    {
      float arow[C];
#pragma unroll
      for (int j = 0; j < C; j += 4) {
        const float4 v4 = *reinterpret_cast<const float4*>(&sm.A[lm][j]);
        arow[j] = -v4.x;  // negated: the elimination takes -A[row]
        arow[j + 1] = -v4.y;
        arow[j + 2] = -v4.z;
        arow[j + 3] = -v4.w;
      }
      const float bl = sm.beta[lm];
#pragma unroll
      for (int s = 0; s < 4; ++s) tt[s] = (4 * lq + s == lm) ? bl : 0.f;
      eliminate<0>(tt, arow);
    }

    // (5b) U~ = T V for the wave's value tile (accumulator layout: row 4 lq + s, column col)
    f32x4_t Ut = {0.f, 0.f, 0.f, 0.f};
    {
      float v4[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) v4[s] = sm.va[4 * lq + s][col];
#pragma unroll
      for (int s = 0; s < 4; ++s) Ut = mma4(tt[s], v4[s], Ut);
    }

    // (5c) W^T = Ka^T T^T, tile nt holding W[lm][16 nt + 4 lq + s]: exactly the A operand
    // of W.S in the key order of the state tiles
    f32x4_t Wt[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      Wt[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) Wt[nt] = mma4(sm.op.kat[16 * nt + lm][4 * lq + s], tt[s], Wt[nt]);
    }

    // (5d) the state pass on the wave's value tile
    f32x4_t O = {0.f, 0.f, 0.f, 0.f};
    {
      f32x4_t ws = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int it = 0; it < 8; ++it)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          ws = mma4(Wt[it][s], S[it][s], ws);
          O = mma4(sm.op.qa[lm][16 * it + 4 * lq + s], S[it][s], O);
        }
      f32x4_t U = Ut - ws;
#pragma unroll
      for (int s = 0; s < 4; ++s) O = mma4(sm.op.p[lm][4 * lq + s], U[s], O);
#pragma unroll
      for (int it = 0; it < 8; ++it) {
#pragma unroll
        for (int s = 0; s < 4; ++s) S[it][s] *= sm.eg15[16 * it + 4 * lq + s];
#pragma unroll
        for (int s = 0; s < 4; ++s) S[it] = mma4(sm.op.klt[16 * it + lm][4 * lq + s], U[s], S[it]);
      }
    }

    // (6) gated RMSNorm over each output row and the store
    {
      float ss[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) ss[s] = row_sum16(O[s] * O[s]);
      if (lm == 0)
#pragma unroll
        for (int s = 0; s < 4; ++s) sm.ss[buf][wave][4 * lq + s] = ss[s];
    }
    stage();  // the next chunk's raw rows, for the next iteration's prologue
    lds_barrier();
    {
      float* po = static_cast<float*>(a.out) + (row0 + 4 * lq) * Hd + static_cast<int64_t>(h) * kHeadDim + col;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int r = 4 * lq + s;
        if (r < L) {
          float tot = 0.f;
#pragma unroll
          for (int wv = 0; wv < NWAVES; ++wv) tot += sm.ss[buf][wv][r];
          const float rr = 1.0f / sqrtf(tot * (1.0f / kHeadDim) + a.L.rms_eps);
          *po = nw * O[s] * rr * sm.sg[buf][r][col];
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

#undef KDA_SEG_SRC
#undef KDA_SEG_DST
#undef KDA_SEG_OK

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, kda_dtype io, const int32_t* order_host,
                          hipStream_t stream) {
  if (io == KDA_BF16) return launch_prefill_bf16(a, order_host, stream);
  SeqOrder ord;
  const int nord = a.num_seqs < kMaxOrdered ? a.num_seqs : kMaxOrdered;
  for (int i = 0; i < kMaxOrdered; ++i) ord.idx[i] = i < nord ? order_host[i] : 0;
  const dim3 grid(static_cast<unsigned>(a.num_seqs) * static_cast<unsigned>(a.L.H));
  hipLaunchKernelGGL(prefill_kernel, grid, dim3(NTHREADS), 0, stream, a, ord);
  return hipGetLastError();
}

}  // namespace kda
