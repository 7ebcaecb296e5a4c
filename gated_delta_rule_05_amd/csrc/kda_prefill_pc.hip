// Chunked prefill of the KDA core for bf16 io on gfx950: producer/consumer waves.
//
// Same algebra as the fp32 prefill kernel (kda_prefill.hip; docs.rs "memra_engine::kda"
// header prose for the per-channel Gcum chunk form, "Kimi Delta Attention (KDA) --
// analysis & C kernel plan" section "Recurrence", OpenModelAtlas "Kimi K3 - Retention
// gate" "Why" for the 16-token tile bound), mapped so that the two kinds of work overlap:
//
//   * 8 producer waves build everything chunk c+1 needs from its raw rows alone: short
//     conv + SiLU, gate and Gcum, q/k norms, MFMA-ready operands (bf16 hi/lo) and the
//     Gram tiles A and P, while the next-but-one chunk's raw rows stream from HBM straight
//     into LDS;
//   * 8 consumer waves run chunk c's state pass, one 16-column value tile of the fp32
//     128x128 state each, held in MFMA accumulators for the whole sequence: O = Qa S,
//     beside which two of them form T = (I + A)^-1 Diag(beta) (DPP elimination, once
//     per chunk);
//     then U~ = T V, W^T = Ka^T T^T (landing in the A-operand layout of W.S),
//     U = U~ - W S, O += P U; then the gated RMSNorm epilogue; then
//     S <- Diag(e^Gcum_C) S + Kl^T U.
//
// Operands that cross from producers to consumers are double-buffered by chunk parity.
// Four LDS barriers per chunk.  With 16 waves per workgroup each SIMD holds two producer
// and two consumer waves, so the VALU-heavy and MFMA-heavy halves hide each other's
// latencies.
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_mfma.h"

namespace kda {

namespace {

using namespace mf;

constexpr int PW = 8;                  // producer waves
constexpr int CWN = 8;                 // consumer waves
constexpr int PT = 64 * PW;            // producer threads
// Waves that also run the once-per-chunk jobs (wave w runs on SIMD w % 4): the T
// elimination goes to two consumer waves, whose interval 1 is light; the two Gram tiles
// to the v producer waves (SIMDs 0 and 1), which are otherwise idle in interval 4.
constexpr int kElimCwA = 2;  // consumer waves PW + 2 and PW + 3, on SIMDs 2 and 3
constexpr int kElimCwB = 3;
constexpr int kGramAWave = 4;
constexpr int kGramPWave = 5;
constexpr int NT = 64 * (PW + CWN);
constexpr int LDP = 132;               // fp32 row stride of [16][128] arrays
constexpr int OPP = 136;               // bf16 row stride of [16][128] operands
constexpr int KTP = 24;                // bf16 row stride of [128][16] operands
constexpr int ILP = 40;                // bf16 row stride of interleaved hi/lo [.][16] operands

struct PcOrder {
  int32_t idx[kMaxOrdered];
};

// What consumers read for one chunk (double-buffered by chunk parity).
struct alignas(16) KBuf {
  _Float16 qa[C][OPP];          // Qa = q-hat exp(Gcum), fp16, key order of the .S products
  __bf16 kat[kHeadDim][KTP];    // Ka^T, hi
  __bf16 klt[kHeadDim][ILP];    // Kl^T, hi/lo interleaved (il16)
  __bf16 p[C][ILP];             // P (lower incl.), hi/lo interleaved
  __bf16 tm[C][ILP];            // T = (I + A)^-1 Diag(beta), hi/lo interleaved
  float V[C][LDP];              // V = silu(conv v)
  float eg15[kHeadDim];         // exp(Gcum at the chunk end)
  float beta[C];
};

struct alignas(16) PcSmem {
  KBuf kb[2];
  uint16_t braw[C];             // staged raw beta
  float aq[C][LDP];             // silu(conv q)
  float ak[C][LDP];             // silu(conv k)
  float gam[C][LDP];            // Gcum (log2 units)
  __bf16 qp[2][C][OPP];         // Qp = q-hat exp(Gcum - Gref), hi/lo
  __bf16 kp[2][C][OPP];         // Kp = k-hat exp(Gcum - Gref), hi/lo
  __bf16 km[2][C][OPP];         // Km = k-hat exp(Gref - Gcum), hi/lo
  float g7[kHeadDim];           // Gcum at the chunk midpoint (Gram reference), log2 units
  float g15[kHeadDim];          // Gcum at the chunk end, log2 units
  float eg7[kHeadDim];          // exp(Gcum at the midpoint)
  float e157[kHeadDim];         // exp(Gcum at the end - Gcum at the midpoint)
  float rn[2 * C];              // 1/|q| * d^-1/2, then 1/|k|
  float A[C][20];               // A times beta (strict lower), for the elimination
  float ss[CWN][C];             // per consumer wave, per row: sum of O^2 over its columns
};

// The LDS DMA targets are variables of their own: the compiler then knows that the
// loads in flight cannot alias the other LDS data, and does not wait for them before
// every LDS read.
constexpr int kDmaBytes = (4 + 2) * C * kHeadDim * 2;
static_assert(sizeof(PcSmem) + kDmaBytes <= 160 * 1024, "LDS budget of one workgroup");
// 16-byte LDS accesses (DMA targets, float4 and bf16x8 reads)
static_assert(offsetof(PcSmem, kb) % 16 == 0 && sizeof(KBuf) % 16 == 0 &&
                  offsetof(KBuf, qa) % 16 == 0 && offsetof(KBuf, eg15) % 16 == 0 &&
                  offsetof(KBuf, V) % 16 == 0 && offsetof(PcSmem, ss) % 16 == 0 &&
                  offsetof(KBuf, klt) % 16 == 0 && offsetof(KBuf, p) % 16 == 0 &&
                  offsetof(KBuf, tm) % 16 == 0 && (ILP * 2) % 16 == 0 &&
                  offsetof(PcSmem, A) % 16 == 0 && offsetof(PcSmem, aq) % 16 == 0 &&
                  offsetof(PcSmem, ak) % 16 == 0 && offsetof(PcSmem, gam) % 16 == 0 &&
                  offsetof(PcSmem, g7) % 16 == 0 && offsetof(PcSmem, qp) % 16 == 0 &&
                  offsetof(PcSmem, kp) % 16 == 0 && offsetof(PcSmem, km) % 16 == 0,
              "16-byte aligned LDS members");

__global__ __launch_bounds__(NT) void prefill_pc_kernel(PrefillArgs a, PcOrder order, SplitPlan plan) {
  __shared__ PcSmem sm;
  // raw rows of q, k, v, z of the next-but-one chunk, unpadded
  __shared__ __attribute__((aligned(16))) uint16_t raw_lds[4][C][kHeadDim];
  // raw output-gate rows, double-buffered by chunk parity (read by the epilogue)
  __shared__ __attribute__((aligned(16))) uint16_t graw_lds[2][C][kHeadDim];

  // This workgroup's (sequence n, head h) and tokens [t0, t0 + T): a whole sequence, or
  // segment kseg of nsegs (see the passes in kda_internal.h).
  const int H = a.L.H;
  int n, h, seg = 0, kseg = 0, nsegs = 1;
  bool transfer_m = false;  // Transfer pass, M half: identity start, v = 0
  int64_t t0;
  int T;
  if (a.pass == kPassWhole) {
    const int rank = blockIdx.x / H;
    h = blockIdx.x - rank * H;
    n = (a.num_seqs <= kMaxOrdered) ? order.idx[rank] : rank;
    t0 = a.cu_seqlens[n];
    T = a.cu_seqlens[n + 1] - static_cast<int>(t0);
  } else {
    int blk = blockIdx.x;
    if (a.pass == kPassTransfer && blk >= plan.nseg * H) {
      transfer_m = true;
      blk -= plan.nseg * H;
    }
    seg = blk / H;
    h = blk - seg * H;
    n = 0;
    while (plan.first[n + 1] <= seg) ++n;
    kseg = seg - plan.first[n];
    nsegs = plan.first[n + 1] - plan.first[n];
    t0 = a.cu_seqlens[n] + static_cast<int64_t>(kseg) * plan.seg_len;
    T = min(static_cast<int>(a.cu_seqlens[n + 1] - t0), plan.seg_len);
    // the Transfer pass needs neither the last segment's end state nor the first's M
    if (a.pass == kPassTransfer && (kseg == nsegs - 1 || (transfer_m && kseg == 0))) return;
  }
  const bool write_out = a.pass != kPassTransfer;
  const bool last_seg = kseg == nsegs - 1;
  const int64_t Hd = static_cast<int64_t>(H) * kHeadDim;
  const int nch = (T + C - 1) / C;

  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lane = t & 63;
  const int lm = lane & 15;
  const int lq = lane >> 4;
  const bool producer = wave < PW;
  // producers: role 0 = q, 1 = k, 2 = v, 3 = z and gate, over 128 channels each (two
  // waves per role, so the role is wave-uniform)
  const int role = (t >> 7) & 3;
  const int ch = t & (kHeadDim - 1);
  const int64_t c = static_cast<int64_t>(h) * kHeadDim + ch;
  // consumers: value tile cw, column col
  const int cw = wave - PW;
  const int col = 16 * (cw & (CWN - 1)) + lm;

  if (producer) {
    // ============================================================== producer waves
    const int urole = __builtin_amdgcn_readfirstlane(role);
    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    float w[4] = {0.f, 0.f, 0.f, 0.f}, hist[3] = {0.f, 0.f, 0.f};
    if (urole < 3) {
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = a.L.conv_w[(role * Hd + c) * kConvTaps + j];
      if (kseg > 0) {
        // a later segment: the conv history is the previous segment's last raw rows
        // (segments before the last are at least one chunk long)
        const bf16_t* pl = static_cast<const bf16_t*>(urole == 0 ? a.q : urole == 1 ? a.k : a.v);
#pragma unroll
        for (int j = 0; j < 3; ++j) hist[j] = bf16_to_f32(pl[(t0 - 3 + j) * Hd + c].bits);
      } else if (a.ring_in) {
        const float* rin = a.ring_in + static_cast<int64_t>(n) * 3 * Hd * kRingTaps;
#pragma unroll
        for (int j = 0; j < 3; ++j) hist[j] = rin[(role * Hd + c) * kRingTaps + j];
      }
    }
    // gate: g = lb sigmoid(e^A_log (z + dt_bias)) = lb / (1 + 2^(z ga + gb)); Gcum is kept
    // in log2 units (scaled by log2 e) so that every exponential below is one exp2
    const float ascale = expf(a.L.A_log[h]);
    const float ga = -kLog2e * ascale, gb = -kLog2e * ascale * a.L.dt_bias[c];
    const float lb2 = kLog2e * a.L.lower_bound;

    // Raw rows of a chunk, straight into LDS, as 16 pieces of 16 bytes per row.  Planes q,
    // k, v, z go to sm.raw: piece s (plane s / 256, row (s / 16) % 16, bytes 16 (s % 16) of
    // the row) lands at byte 16 s, so the 64 pieces of one wave instruction are 1 KiB
    // contiguous, as the instruction writes them.  The output-gate plane goes to the
    // consumers' double-buffered copy in the same way.  Rows past the end of a sequence
    // re-read its last row.
    constexpr int SPR = kHeadDim * 2 / 16;
    constexpr int NSEG = 4 * C * SPR;
    static_assert(NSEG == 2 * PT && (C * SPR) % 64 == 0, "two pieces per producer thread");
    static_assert(C * SPR == 4 * 64, "the gate plane is four waves' pieces");
    uint16_t braw = 0;
    const char* const pq = static_cast<const char*>(a.q);
    const char* const pk = static_cast<const char*>(a.k);
    const char* const pv = static_cast<const char*>(a.v);
    const char* const pz = static_cast<const char*>(a.z);
    const char* const pgt = static_cast<const char*>(a.gate);
    const bf16_t* const x_b = static_cast<const bf16_t*>(a.beta);
    const int row_bytes = static_cast<int>(Hd) * 2;
    const int64_t head_bytes = static_cast<int64_t>(h) * kHeadDim * 2;
    // byte offset of this lane's piece k inside a chunk (plane base and first row aside),
    // for a full chunk and for a last chunk of Ln rows
    auto piece_off = [&](int k, int Ln) __attribute__((always_inline)) {
      const int s0 = 64 * wave + k * PT;
      const int rem = (s0 + lane) % (C * SPR);
      return min(rem / SPR, Ln - 1) * row_bytes + 16 * (rem % SPR);
    };
    const int off_full0 = piece_off(0, C), off_full1 = piece_off(1, C);
    auto prefetch = [&](int c0n) __attribute__((always_inline)) {
      const int Ln = min(C, T - c0n);
      const bool full = Ln == C;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int s0 = __builtin_amdgcn_readfirstlane(64 * wave + k * PT);
        const int pl = s0 / (C * SPR);
        const char* base = pl == 0 ? pq : pl == 1 ? pk : pl == 2 ? pv : pz;
        base += (t0 + c0n) * Hd * 2 + head_bytes;
        const int off = full ? (k == 0 ? off_full0 : off_full1) : piece_off(k, Ln);
        lds_dma16(base + off, &raw_lds[0][0][0] + 8 * s0);
      }
      if (t < C) braw = x_b[(t0 + c0n + min(t, Ln - 1)) * H + h].bits;
    };
    auto prefetch_gate = [&](int c0n, int buf) __attribute__((always_inline)) {
      if (__builtin_amdgcn_readfirstlane(wave) < 4) {
        const int Ln = min(C, T - c0n);
        const int s0 = __builtin_amdgcn_readfirstlane(64 * wave);
        const int rem = s0 + lane;
        const char* base = pgt + (t0 + c0n) * Hd * 2 + head_bytes;
        const int off = Ln == C ? off_full0 : min(rem / SPR, Ln - 1) * row_bytes + 16 * (rem % SPR);
        lds_dma16(base + off, &graw_lds[buf][0][0] + 8 * s0);
      }
    };

    if (T > 0) {
      prefetch(0);
      prefetch_gate(0, 0);
      wait_vm();
      if (t < C) sm.braw[t] = braw;
    }
    lds_barrier();

    // iteration i: producers build chunk i + 1
    for (int i = -1; i < nch; ++i) {
      const bool has_next = i + 1 < nch;
      const int Ln = min(C, T - (i + 1) * C);
      KBuf& KN = sm.kb[(i + 1) & 1];

      // ---------------------------------------------------------- interval 1
      if (has_next) {
        // conv + SiLU with the history in registers; gate and Gcum; beta.
        // All raw values are read first (one LDS round trip per chunk).  Every chunk but
        // a sequence's last is full, and takes a path without per-row liveness tests so
        // that the rows' exp/rcp chains interleave.
        uint16_t xr[C];
#pragma unroll
        for (int r = 0; r < C; ++r) xr[r] = raw_lds[urole][r][ch];
        const bool full = Ln == C;
        if (urole == 2 && transfer_m) {
          // the transfer matrix is the end state from the identity with v = 0
#pragma unroll
          for (int r = 0; r < C; ++r) KN.V[r][ch] = 0.f;
        } else if (urole < 3) {
          float(*dst)[LDP] = urole == 0 ? sm.aq : urole == 1 ? sm.ak : KN.V;
          if (full) {
#pragma unroll
            for (int r = 0; r < C; ++r) {
              const float x = bf16_to_f32(xr[r]);
              const float y = w[3] * x + w[0] * hist[0] + w[1] * hist[1] + w[2] * hist[2];
              hist[0] = hist[1];
              hist[1] = hist[2];
              hist[2] = x;
              dst[r][ch] = y * fsigmoid(y);
            }
          } else {
#pragma unroll
            for (int r = 0; r < C; ++r) {
              const float x = bf16_to_f32(xr[r]);
              const float y = w[3] * x + w[0] * hist[0] + w[1] * hist[1] + w[2] * hist[2];
              const bool live = r < Ln;
              if (live) {
                hist[0] = hist[1];
                hist[1] = hist[2];
                hist[2] = x;
              }
              dst[r][ch] = live ? y * fsigmoid(y) : 0.f;
            }
          }
        } else {
          float G = 0.f, G7 = 0.f;
          if (full) {
#pragma unroll
            for (int r = 0; r < C; ++r) {
              G += lb2 * frcp(1.0f + fexp2(fmaf(bf16_to_f32(xr[r]), ga, gb)));
              sm.gam[r][ch] = G;
              if (r == C / 2 - 1) G7 = G;
            }
          } else {
#pragma unroll
            for (int r = 0; r < C; ++r) {
              const bool live = r < Ln;
              G += live ? lb2 * frcp(1.0f + fexp2(fmaf(bf16_to_f32(xr[r]), ga, gb))) : 0.f;
              sm.gam[r][ch] = G;
              if (r == C / 2 - 1) G7 = G;
            }
          }
          sm.g7[ch] = G7;
          sm.g15[ch] = G;
          KN.eg15[ch] = fexp2(G);
          sm.eg7[ch] = fexp2(G7);
          sm.e157[ch] = fexp2(G - G7);
        }
        if (t < C) KN.beta[t] = (t < Ln) ? fsigmoid(bf16_to_f32(sm.braw[t])) : 0.f;
      }
      lds_barrier();

      // ---------------------------------------------------------- interval 2
      // raw rows of chunk i + 2 (chunk i + 1's were consumed in interval 1)
      if (i + 2 < nch) prefetch((i + 2) * C);
      if (has_next) {
        // q/k row norms: 16 threads per (plane, row)
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

      // ---------------------------------------------------------- interval 3
      if (has_next) {
        // Every operand of chunk i + 1 for row r, channels c4 .. c4 + 3 (rows run fastest
        // across lanes, so the transposed Ka / Kl writes are 32 contiguous bytes per
        // channel).  With d = Gcum - Gcum_mid: Qp = q-hat e^d, Kp = k-hat e^d,
        // Km = k-hat e^-d; Qa = Qp e^Gcum_mid, Ka = Kp e^Gcum_mid, Kl = Km e^(Gcum_end -
        // Gcum_mid).
        const int r = t & (C - 1), c4 = 4 * (t >> 4);
        const float4 qv = ld<float4>(&sm.aq[r][c4]);
        const float4 kv = ld<float4>(&sm.ak[r][c4]);
        const float4 gv = ld<float4>(&sm.gam[r][c4]);
        const float4 g7 = ld<float4>(&sm.g7[c4]);
        const float4 e7 = ld<float4>(&sm.eg7[c4]);
        const float4 e157 = ld<float4>(&sm.e157[c4]);
        const float rq = sm.rn[r], rk = sm.rn[C + r];
        const float q4[4] = {qv.x * rq, qv.y * rq, qv.z * rq, qv.w * rq};
        const float k4[4] = {kv.x * rk, kv.y * rk, kv.z * rk, kv.w * rk};
        const float d4[4] = {gv.x - g7.x, gv.y - g7.y, gv.z - g7.z, gv.w - g7.w};
        const float m7[4] = {e7.x, e7.y, e7.z, e7.w};
        const float m157[4] = {e157.x, e157.y, e157.z, e157.w};
        float qp[4], kp[4], km[4], qa[4], ka[4], kl[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float el = fexp2(d4[v]), er = fexp2(-d4[v]);
          qp[v] = q4[v] * el;
          kp[v] = k4[v] * el;
          km[v] = k4[v] * er;
          qa[v] = qp[v] * m7[v];
          ka[v] = kp[v] * m7[v];
          kl[v] = km[v] * m157[v];
        }
        store4(&sm.qp[0][r][c4], &sm.qp[1][r][c4], qp);
        store4(&sm.kp[0][r][c4], &sm.kp[1][r][c4], kp);
        store4(&sm.km[0][r][c4], &sm.km[1][r][c4], km);
        // Qa in the key order of the .S products: channels 32 kb + 4 m .. + 3 sit at
        // 32 kb + 8 (m % 4) + 4 (m / 4)
        const int pa = 32 * (c4 >> 5) + 8 * ((c4 >> 2) & 3) + 4 * ((c4 >> 4) & 1);
        store4_f16(&KN.qa[r][pa], qa);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          KN.kat[c4 + v][r] = static_cast<__bf16>(ka[v]);
          split_store(&KN.klt[c4 + v][il16(r)], &KN.klt[c4 + v][il16(r) + 4], kl[v]);
        }
      }
      lds_barrier();

      // ---------------------------------------------------------- interval 4
      if (has_next && (uwave == kGramAWave || uwave == kGramPWave)) {
        const bool gram_a = uwave == kGramAWave;
        // Gram tiles of chunk i + 1: A = Kp Km^T (strict lower, times beta_r), eliminated
        // by consumer waves kElimCwA/B in the next interval 1; P = Qp Km^T (lower incl.)
        const __bf16(*Xh)[OPP] = gram_a ? sm.kp[0] : sm.qp[0];
        const __bf16(*Xl)[OPP] = gram_a ? sm.kp[1] : sm.qp[1];
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < kHeadDim / 32; ++kb) {
          const int o = 32 * kb + 8 * lq;
          const bf16x8_t xh = ld<bf16x8_t>(&Xh[lm][o]), xl = ld<bf16x8_t>(&Xl[lm][o]);
          const bf16x8_t mh = ld<bf16x8_t>(&sm.km[0][lm][o]), ml = ld<bf16x8_t>(&sm.km[1][lm][o]);
          acc = mma32(xh, mh, acc);
          a1 = mma32(xh, ml, a1);
          a1 = mma32(xl, mh, a1);
        }
        acc += a1;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int r = 4 * lq + s, j = lm;
          if (gram_a) {
            sm.A[r][j] = (j < r) ? KN.beta[r] * acc[s] : 0.f;
          } else {
            split_store(&KN.p[r][il16(j)], &KN.p[r][il16(j) + 4], (j <= r) ? acc[s] : 0.f);
          }
        }
      }
      if (i + 2 < nch) {
        wait_vm();  // this wave's pieces of chunk i + 2 are in LDS
        if (t < C) sm.braw[t] = braw;
        // chunk i's output gate has been read by now; its buffer takes chunk i + 2's
        prefetch_gate((i + 2) * C, (i + 2) & 1);
      }
      lds_barrier();
    }

    // conv history of q, k, v -> ring
    if (a.ring_out && urole < 3 && write_out && last_seg) {
      float* rout = a.ring_out + static_cast<int64_t>(n) * 3 * Hd * kRingTaps;
#pragma unroll
      for (int j = 0; j < 3; ++j) rout[(role * Hd + c) * kRingTaps + j] = hist[j];
    }
  } else {
    // ============================================================== consumer waves
    f32x4_t S[8];
    constexpr int64_t kDD = kHeadDim * kHeadDim;
    const int64_t nbase = (static_cast<int64_t>(n) * H + h) * kDD;    // [N][H] planes
    const int64_t sgbase = (static_cast<int64_t>(seg) * H + h) * kDD; // [segments][H] planes
    const float* src = nullptr;
    if (a.pass == kPassFinal && kseg > 0)
      src = a.seg_start + sgbase;
    else if (kseg == 0 && !transfer_m && a.state_in)
      src = a.state_in + nbase;
    if (src) {
      const float* sp = src + opaque(4 * lq * kHeadDim + col);
#pragma unroll
      for (int it = 0; it < 8; ++it)
#pragma unroll
        for (int s = 0; s < 4; ++s) S[it][s] = sp[(16 * it + s) * kHeadDim];
    } else {
#pragma unroll
      for (int it = 0; it < 8; ++it)
#pragma unroll
        for (int s = 0; s < 4; ++s) S[it][s] = (transfer_m && 16 * it + 4 * lq + s == col) ? 1.f : 0.f;
    }
    const float nw = a.L.norm_w[col];
    lds_barrier();

    bf16x8_t u_l0 = {}, u_hh = {};  // U as the B operands of mma16p
    // S = Diag(exp(Gcum_C)) S + Kl^T U, once chunk i's U is known
    auto update_state = [&](const KBuf& K) __attribute__((always_inline)) {
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const float4 e4 = ld<float4>(&K.eg15[16 * it + 4 * lq]);
        S[it][0] *= e4.x;
        S[it][1] *= e4.y;
        S[it][2] *= e4.z;
        S[it][3] *= e4.w;
        S[it] = mma16p(ld<bf16x8_t>(&K.klt[16 * it + lm][8 * lq]), u_l0, u_hh, S[it]);
      }
    };

    // iteration i: consumers run chunk i
    for (int i = -1; i < nch; ++i) {
      const bool has_next = i + 1 < nch;
      KBuf& K = sm.kb[i & 1];
      KBuf& KN = sm.kb[(i + 1) & 1];
      f32x4_t O = {0.f, 0.f, 0.f, 0.f};
      f16x8_t sf[4];

      // ---------------------------------------------------------- interval 1
      if (i >= 0) {
        if (cw == kElimCwA || cw == kElimCwB) {
          // T = (I + A)^-1 Diag(beta) by elimination with rows spread over lanes (DPP
          // broadcasts inside each 16-lane row); A[r][j] = 0 for j >= r, so the update
          // is unconditional.  Lane (lm, lq) holds T[lm][lq + 4 s]; wave kElimCwA takes
          // slots s = 0, 3 and wave kElimCwB slots 1, 2.
          float arow[C], tt[2];
#pragma unroll
          for (int j = 0; j < C; j += 4) {
            const float4 v4 = *reinterpret_cast<const float4*>(&sm.A[lm][j]);
            arow[j] = v4.x;
            arow[j + 1] = v4.y;
            arow[j + 2] = v4.z;
            arow[j + 3] = v4.w;
          }
          const float bl = K.beta[lm];
          const bool wa = cw == kElimCwA;
          const int s0 = wa ? 0 : 1, s1 = wa ? 3 : 2;
          tt[0] = (lq + 4 * s0 == lm) ? bl : 0.f;
          tt[1] = (lq + 4 * s1 == lm) ? bl : 0.f;
          if (wa)
            eliminate_strided2<0, 0, 3>(tt, arow);
          else
            eliminate_strided2<0, 1, 2>(tt, arow);
          split_store(&K.tm[lm][il16(lq + 4 * s0)], &K.tm[lm][il16(lq + 4 * s0) + 4], tt[0]);
          split_store(&K.tm[lm][il16(lq + 4 * s1)], &K.tm[lm][il16(lq + 4 * s1) + 4], tt[1]);
        }
        // S as fp16 B operands (per 32 keys: 4 lq + s, then 16 + 4 lq + s)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            sf[kb][s] = static_cast<_Float16>(S[2 * kb][s]);
            sf[kb][4 + s] = static_cast<_Float16>(S[2 * kb + 1][s]);
          }
        }
        // O = Qa S
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          O = mma32h(ld<f16x8_t>(&K.qa[lm][32 * kb + 8 * lq]), sf[kb], O);
      }
      lds_barrier();

      // ---------------------------------------------------------- interval 2
      if (i >= 0) {
        // T, split into bf16 hi/lo: lane (lm, lq) holds T[lm][4 lq + s]
        const bf16x8_t tq = ld<bf16x8_t>(&K.tm[lm][8 * lq]);
        const bf16x4_t th = __builtin_shufflevector(tq, tq, 0, 1, 2, 3);
        // U~ = T V for this wave's value tile
        f32x4_t Ut = {0.f, 0.f, 0.f, 0.f};
        {
          float v4[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) v4[s] = K.V[4 * lq + s][col];
          bf16x4_t vh, vl;
          split_vec<4>(v4, vh, vl);
          bf16x8_t v_l0, v_hh;
          b_pair(vh, vl, v_l0, v_hh);
          Ut = mma16p(tq, v_l0, v_hh, Ut);
        }
        // W S, with W^T = Ka^T T^T computed two 16-key tiles at a time
        f32x4_t ws = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const f32x4_t w0 = mma16(ld<bf16x4_t>(&K.kat[32 * kb + lm][4 * lq]), th,
                                   f32x4_t{0.f, 0.f, 0.f, 0.f});
          const f32x4_t w1 = mma16(ld<bf16x4_t>(&K.kat[32 * kb + 16 + lm][4 * lq]), th,
                                   f32x4_t{0.f, 0.f, 0.f, 0.f});
          f16x8_t wb;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            wb[s] = static_cast<_Float16>(w0[s]);
            wb[4 + s] = static_cast<_Float16>(w1[s]);
          }
          ws = mma32h(wb, sf[kb], ws);
        }
        const f32x4_t U = Ut - ws;
        {
          float u4[4] = {U[0], U[1], U[2], U[3]};
          bf16x4_t uh, ul;
          split_vec<4>(u4, uh, ul);
          b_pair(uh, ul, u_l0, u_hh);
        }
        // O += P U
        O = mma16p(ld<bf16x8_t>(&K.p[lm][8 * lq]), u_l0, u_hh, O);
        float ss[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) ss[s] = row_sum16(O[s] * O[s]);
        if (lm == 0)
          *reinterpret_cast<float4*>(&sm.ss[cw][4 * lq]) = make_float4(ss[0], ss[1], ss[2], ss[3]);
      }
      lds_barrier();

      // ---------------------------------------------------------- interval 3
      if (i >= 0 && write_out) {
        // gated RMSNorm of the chunk's output rows and the store
        const int L = min(C, T - i * C);
        float tot[4];
        {
          const float4 s4 = ld<float4>(&sm.ss[0][4 * lq]);
          tot[0] = s4.x;
          tot[1] = s4.y;
          tot[2] = s4.z;
          tot[3] = s4.w;
        }
#pragma unroll
        for (int wv = 1; wv < CWN; ++wv) {
          const float4 s4 = ld<float4>(&sm.ss[wv][4 * lq]);
          tot[0] += s4.x;
          tot[1] += s4.y;
          tot[2] += s4.z;
          tot[3] += s4.w;
        }
        float y[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float rr = __builtin_amdgcn_rsqf(tot[s] * (1.0f / kHeadDim) + a.L.rms_eps);
          const float g = fsigmoid(bf16_to_f32(graw_lds[i & 1][4 * lq + s][col]));
          y[s] = nw * O[s] * rr * g;
        }
        bf16_t* po = static_cast<bf16_t*>(a.out) + (t0 + i * C + 4 * lq) * Hd +
                     static_cast<int64_t>(h) * kHeadDim + col;
        if (L == C) {
#pragma unroll
          for (int s = 0; s < 4; ++s) po[s * Hd].bits = f32_to_bf16(y[s]);
        } else {
#pragma unroll
          for (int s = 0; s < 4; ++s)
            if (4 * lq + s < L) po[s * Hd].bits = f32_to_bf16(y[s]);
        }
      }
      lds_barrier();

      // ---------------------------------------------------------- interval 4
      if (i >= 0) update_state(K);
      lds_barrier();
    }

    float* dst = nullptr;
    if (a.pass == kPassTransfer)
      dst = (transfer_m ? a.seg_m : a.seg_b) + sgbase;
    else if (last_seg && a.state_out)
      dst = a.state_out + nbase;
    if (dst) {
      float* sp = dst + opaque(4 * lq * kHeadDim + col);
#pragma unroll
      for (int it = 0; it < 8; ++it)
#pragma unroll
        for (int s = 0; s < 4; ++s) sp[(16 * it + s) * kHeadDim] = S[it][s];
    }
  }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, const int32_t* order_host, hipStream_t stream) {
  PcOrder ord;
  const int nord = a.num_seqs < kMaxOrdered ? a.num_seqs : kMaxOrdered;
  for (int i = 0; i < kMaxOrdered; ++i) ord.idx[i] = i < nord ? order_host[i] : 0;
  SplitPlan none{};
  PrefillArgs w = a;
  w.pass = kPassWhole;
  const dim3 grid(static_cast<unsigned>(a.num_seqs) * static_cast<unsigned>(a.L.H));
  hipLaunchKernelGGL(prefill_pc_kernel, grid, dim3(NT), 0, stream, w, ord, none);
  return hipGetLastError();
}

namespace {

// S_{k+1} = M_k S_k + B_k over the segments of each sequence, for one 16-column block of
// one head's state (value columns never mix, so the blocks are independent).  S_1 = B_0:
// segment 0 started from the true state.  256 threads: thread t forms rows t / 2, columns
// 8 (t % 2) .. + 7 of the block; the block itself sits in LDS.  fp32 FMAs in a fixed order.
__global__ __launch_bounds__(256) void combine_kernel(PrefillArgs a, SplitPlan plan) {
  constexpr int CB = 16;
  __shared__ float sblk[kHeadDim][CB];
  const int H = a.L.H;
  const int nb = kHeadDim / CB;
  const int unit = blockIdx.x / nb;
  const int cb = blockIdx.x - unit * nb;
  const int n = unit / H;
  const int h = unit - n * H;
  const int t = threadIdx.x;
  const int r = t >> 1, c0 = 8 * (t & 1);
  const int first = plan.first[n], nsegs = plan.first[n + 1] - plan.first[n];
  if (nsegs < 2) return;
  constexpr int64_t kDD = kHeadDim * kHeadDim;
  auto plane = [&](float* base, int k) { return base + ((static_cast<int64_t>(first + k)) * H + h) * kDD; };
  // S_1 = B_0
  float acc[8];
  {
    const float* b0 = plane(a.seg_b, 0) + r * kHeadDim + cb * CB + c0;
    float* s1 = plane(a.seg_start, 1) + r * kHeadDim + cb * CB + c0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[j] = b0[j];
      s1[j] = acc[j];
      sblk[r][c0 + j] = acc[j];
    }
  }
  for (int k = 1; k + 1 < nsegs; ++k) {
    __syncthreads();
    const float* mrow = plane(a.seg_m, k) + r * kHeadDim;
    const float* brow = plane(a.seg_b, k) + r * kHeadDim + cb * CB + c0;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.f;
    for (int l = 0; l < kHeadDim; l += 4) {
      const float4 m4 = *reinterpret_cast<const float4*>(mrow + l);
      const float mv[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = fmaf(mv[u], sblk[l + u][c0 + j], acc[j]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += brow[j];
    __syncthreads();
    float* snext = plane(a.seg_start, k + 1) + r * kHeadDim + cb * CB + c0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      sblk[r][c0 + j] = acc[j];
      snext[j] = acc[j];
    }
  }
}

}  // namespace

hipError_t launch_prefill_bf16_split(const PrefillArgs& a, const SplitPlan& plan, hipStream_t stream) {
  PcOrder none{};
  const unsigned H = static_cast<unsigned>(a.L.H);
  PrefillArgs w = a;
  w.pass = kPassTransfer;
  hipLaunchKernelGGL(prefill_pc_kernel, dim3(2u * plan.nseg * H), dim3(NT), 0, stream, w, none, plan);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(static_cast<unsigned>(a.num_seqs) * H * (kHeadDim / 16)),
                     dim3(256), 0, stream, w, plan);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  w.pass = kPassFinal;
  hipLaunchKernelGGL(prefill_pc_kernel, dim3(plan.nseg * H), dim3(NT), 0, stream, w, none, plan);
  return hipGetLastError();
}

}  // namespace kda
