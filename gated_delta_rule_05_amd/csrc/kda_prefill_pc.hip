// Chunked prefill of the KDA core for bf16 io on gfx950: producer/consumer waves.
//
// Same algebra as the fp32 prefill kernel (kda_prefill.hip; docs.rs "memra_engine::kda"
// header prose for the per-channel Gcum chunk form, "Kimi Delta Attention (KDA) --
// analysis & C kernel plan" section "Recurrence", OpenModelAtlas "Kimi K3 - Retention
// gate" "Why" for the 16-token tile bound), mapped so that the two kinds of work overlap.
//
// The keys enter unnormalised.  With k-hat = a / |a|' (|a|' = sqrt(|a|^2 + eps)), the update
// beta k-hat (v - S^T k-hat)^T equals beta' a (v' - S^T a)^T with beta' = beta / |a|'^2 and
// v' = |a|' v, so the recurrence is the same one over the raw SiLU outputs a with beta'
// and v'; likewise o = S^T q-hat is S^T a_q scaled per row.  The operands of a chunk are
// therefore built before its row norms are known; the norms only touch beta', V' and the
// output rows.
//
//   * 8 producer waves build everything chunk c+1 needs from its raw rows alone: short
//     conv + SiLU (two waves per plane of q, k, v, one channel per lane over the 16 rows),
//     gate and Gcum (two z waves) (interval 1); the MFMA-ready operands (bf16 hi/lo,
//     fp16) and partial sums of squares of the q and k rows (interval 2); the Gram tiles
//     G = Kp Km^T and P = Qp Km^T on two waves and the row norms on a third (interval 3).
//     Each wave reads its own slice of the chunk's raw rows from LDS at the start of
//     interval 1 and at once refills it with the chunk after, straight from HBM.
//   * The consumer waves run chunk c's state pass on the fp32 128x128 state, held in MFMA
//     accumulators for the whole sequence, 16 value columns per tile: O = Qa S and
//     X = Ka S, beside which two of them form T = (I + A)^-1 Diag(beta') with
//     A = Diag(beta') G (DPP elimination, once per chunk) (interval 1); then
//     U = U~ - W S = T (V' - X) (with U~ = T V' and W = T Ka) and O += P U (interval 2);
//     then S <- Diag(e^Gcum_C) S + Kl^T U (interval 3).
//   * The gated RMSNorm epilogue of chunk c: with the bounded full-rank gate on the four
//     q and k producer waves in interval 3 (the consumers leave O in the chunk's V buffer;
//     4 consumer waves of two tiles each, 12 waves per workgroup); with the softplus or
//     the low-rank gate, whose producers have interval-3 work of their own, on the
//     consumers one chunk late, from row factors the norm wave forms (8 consumer waves of
//     one tile each, 16 waves per workgroup).
//
// With the low-rank decay gate (kFb below) every producer wave also forms one 16-channel
// tile of chunk c+2's gate in interval 3.
//
// Operands that cross from producers to consumers are double-buffered by chunk parity.
// Three LDS barriers per chunk.  Each SIMD holds two producer waves and one or two
// consumer waves, so the VALU-heavy and MFMA-heavy work hide each other's latencies.
#include <type_traits>

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
// to the v producer waves (SIMDs 0 and 1) and the row norms to a z producer wave (SIMD 2),
// which are otherwise idle in interval 3.
constexpr int kElimCwA = 2;  // consumer waves PW + 2 and PW + 3, on SIMDs 2 and 3
constexpr int kElimCwB = 3;
constexpr int kGramAWave = 4;
constexpr int kGramPWave = 5;
// Producer wave that forms the row norms and the RMSNorm row factors (also with the
// low-rank gate, where every producer wave forms a tile of the gate in interval 3).
constexpr int kNormWave = 6;
constexpr int NT = 64 * (PW + CWN);
// With the bounded full-rank gate the state pass runs on 4 consumer waves of two 16-column
// value tiles each (12 waves per workgroup): every A operand a consumer reads from LDS (Qa,
// Ka, T, P, Kl^T) then serves two tiles, which halves those reads, and with 3 waves per
// SIMD a wave may hold 168 registers, room for the 64 state values.  The other variants
// keep 8 consumer waves of one tile (16 waves).
// The Transfer pass of that variant forms both end states of a segment in one workgroup
// (kMerged): a second set of 4 consumer waves runs M (identity start, v = 0) beside the
// first set's B, on the same operands, so each segment's rows are read and its operands
// built once (16 waves).
template <bool kSp, bool kFb, bool kXfer = false>
struct PcShape {
  static constexpr bool kWide = !kSp && !kFb;
  static constexpr int kCT = kWide ? 2 : 1;                // value tiles per consumer wave
  static constexpr int kCwn = CWN / kCT;                   // consumer waves per state
  static constexpr bool kMerged = kWide && kXfer;
  static constexpr int kNt = 64 * (PW + (kMerged ? 2 : 1) * kCwn);  // threads per workgroup
};
constexpr int LDP = 132;               // fp32 row stride of [16][128] arrays
constexpr int OPP = 136;               // bf16 row stride of [16][128] operands
constexpr int ILP = 40;                // bf16 row stride of interleaved hi/lo [.][16] operands
constexpr int NSP = 36;                // fp32 row stride of the [16][32] partial sums of squares
constexpr float kQScale = 0.08838834764831845f;  // d^-1/2
// The producers keep the SiLU conv outputs of q, k and v scaled by kCs = -log2 e: with
// conv weights scaled by kCs, the conv sum is the exponent of SiLU's sigmoid in base 2,
// and kCs a = ys / (1 + 2^ys).  The constant cancels in the per-row factors: with
// a~ = kCs a, |a|'^2 = |a~|^2 / kCs^2 + eps, beta' = beta / (kCs^2 |a_k|'^2),
// V' = |a_k|' (kCs v) and the q scale d^-1/2 / (kCs |a_q|') = -ln 2 d^-1/2 / |a_q|'.
constexpr float kCs = -1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;  // 1 / |kCs|

struct PcOrder {
  int32_t idx[kMaxOrdered];
};

// What consumers read for one chunk (double-buffered by chunk parity).
struct alignas(16) KBuf {
  _Float16 qa[C][OPP];          // Qa = a_q exp(Gcum), fp16, key order of the .S products
  _Float16 ka[C][OPP];          // Ka = a_k exp(Gcum), fp16, key order of the .S products
  __bf16 klt[kHeadDim][ILP];    // Kl^T, hi/lo interleaved (il16)
  __bf16 p[C][ILP];             // P (lower incl.), hi/lo interleaved
  __bf16 tm[C][ILP];            // T = (I + A)^-1 Diag(beta'), hi/lo interleaved
  float V[C][LDP];              // kCs v, v = silu(conv v)
  float eg15[kHeadDim];         // exp(Gcum at the chunk end)
  float beta[C];                // sigmoid(raw beta), then beta' (for the scaled keys kCs a_k)
  float vk[C];                  // |a_k|' = sqrt(|a_k|^2 + eps): V' = vk V
  float rq[C];                  // q scale of the scaled rows kCs a_q: d^-1/2 / (kCs |a_q|')
};

struct alignas(16) PcSmem {
  KBuf kb[2];
  float aq[C][LDP];             // kCs a_q, a_q = silu(conv q)
  float ak[C][LDP];             // kCs a_k, a_k = silu(conv k)
  float gam[C][LDP];            // Gcum (log2 units)
  __bf16 qp[2][C][OPP];         // Qp = a_q exp(Gcum - Gref), hi/lo
  __bf16 kp[2][C][OPP];         // Kp = a_k exp(Gcum - Gref), hi/lo
  __bf16 km[2][C][OPP];         // Km = a_k exp(Gref - Gcum), hi/lo
  float g7[kHeadDim];           // Gcum at the chunk midpoint (Gram reference), log2 units
  float eg7[kHeadDim];          // exp(Gcum at the midpoint)
  float e157[kHeadDim];         // exp(Gcum at the end - Gcum at the midpoint)
  float nsq[2][C][NSP];         // per row: sums of squares of a_q (0) and a_k (1), per 4 channels
  float A[C][20];               // G = Kp Km^T (strict lower), for the elimination
  float ss[CWN][C];             // per consumer wave, per row: sum of O^2 over its columns
  float rr[2][C];               // per row: the RMSNorm factor, by chunk parity
  float nw[kHeadDim];           // the RMSNorm weight (producer epilogue)
  float gbias[kHeadDim];        // low-rank gate: -log2 e exp(A_log) dt_bias per channel
  float eg15n[kHeadDim];        // low-rank gate: e^Gcum_end of the chunk formed ahead
};

// The LDS DMA targets are variables of their own: the compiler then knows that the
// loads in flight cannot alias the other LDS data, and does not wait for them before
// every LDS read.
constexpr int kDmaBytes = (4 + 3) * C * kHeadDim * 2;
constexpr int kZlowBytes = 2 * C * kHeadDim * 2;  // low-rank gate: two z_low chunks
static_assert(sizeof(PcSmem) + kDmaBytes + kZlowBytes <= 160 * 1024, "LDS budget of one workgroup");
// 16-byte LDS accesses (DMA targets, float4 and bf16x8 reads)
static_assert(offsetof(PcSmem, kb) % 16 == 0 && sizeof(KBuf) % 16 == 0 &&
                  offsetof(KBuf, qa) % 16 == 0 && offsetof(KBuf, eg15) % 16 == 0 &&
                  offsetof(KBuf, V) % 16 == 0 && offsetof(PcSmem, ss) % 16 == 0 &&
                  offsetof(KBuf, klt) % 16 == 0 && offsetof(KBuf, p) % 16 == 0 &&
                  offsetof(KBuf, tm) % 16 == 0 && (ILP * 2) % 16 == 0 &&
                  offsetof(PcSmem, A) % 16 == 0 && offsetof(PcSmem, aq) % 16 == 0 &&
                  offsetof(PcSmem, ak) % 16 == 0 && offsetof(PcSmem, gam) % 16 == 0 &&
                  offsetof(PcSmem, g7) % 16 == 0 && offsetof(PcSmem, qp) % 16 == 0 &&
                  offsetof(PcSmem, nsq) % 16 == 0 && offsetof(KBuf, beta) % 16 == 0 &&
                  offsetof(KBuf, vk) % 16 == 0 && offsetof(KBuf, rq) % 16 == 0 &&
                  offsetof(PcSmem, kp) % 16 == 0 && offsetof(PcSmem, km) % 16 == 0 &&
                  offsetof(PcSmem, rr) % 16 == 0 && offsetof(PcSmem, gbias) % 16 == 0 &&
                  offsetof(PcSmem, nw) % 16 == 0,
              "16-byte aligned LDS members");

// Softplus gate: the Gram operands of one level, bf16 hi and lo, 24 rows each (the level's
// earlier-half rows Y, then its later-half rows as Xk, then as Xq), stored where the bounded
// gate keeps Qp, Kp and Km (the same 26 KB).
struct LevelOps {
  __bf16 h[3 * C / 2][OPP];
  __bf16 l[3 * C / 2][OPP];
};
static_assert(offsetof(PcSmem, kp) == offsetof(PcSmem, qp) + sizeof(PcSmem::qp) &&
                  offsetof(PcSmem, km) == offsetof(PcSmem, kp) + sizeof(PcSmem::kp) &&
                  2 * sizeof(LevelOps) == 3 * sizeof(PcSmem::qp) && offsetof(PcSmem, qp) % 16 == 0,
              "the two levels' operands fill Qp, Kp and Km exactly");
__device__ __forceinline__ LevelOps* level_ops(PcSmem& sm) {
  return reinterpret_cast<LevelOps*>(&sm.qp[0][0][0]);
}

// The softplus gate's per-token log2 decay, log2 e g = -e^A_log log2 e softplus(z + dt_bias):
// with u = (z + dt_bias) log2 e (spb = dt_bias log2 e), log2 e softplus = log2(1 + 2^u),
// one exp2 and one log2 (u beyond 24: u itself).  The absolute error stays near 1e-7 (the
// rounding of 1 + 2^u), which is what the decay factors 2^Gcum see.
__device__ __forceinline__ float softplus_gate2(float z, float spb, float ascale) {
  const float u = fmaf(z, kLog2e, spb);
  return -ascale * (u > 24.f ? u : __builtin_amdgcn_logf(1.0f + fexp2(u)));
}

// kFb: the low-rank decay gate (z is z_low [T][128] and the pre-activation z_low f_b^T;
// "Kimi Delta Attention (KDA) -- analysis & C kernel plan", "The KDA layer, precisely",
// fact 2; the Retention-gate page's f_b_proj(f_a_proj(.))).  The q waves then also copy
// z_low rows into a buffer by chunk parity, three chunks ahead, in place of the z waves'
// raw z rows; every producer wave forms one 16-channel tile of a chunk's gate on MFMA in
// interval 3 two chunks ahead, with its f_b rows fetched from L2 as operands; and the z
// waves only move the chunk's e^Gcum_end into its buffer.  The rest is unchanged.
//
// kSp: the unbounded softplus decay gate, g = -e^A_log softplus(z + dt_bias) (Kimi-Linear's
// gate, "Kimi Delta Attention (KDA) -- analysis & C kernel plan", status note).  Without a
// lower bound the in-chunk decay range of a channel is unbounded, so the Gram tiles cannot
// take one reference row (OpenModelAtlas "Kimi K3 - Retention gate", "Why": the unbounded
// form needs position pairs on the diagonal tiles).  Here every pair i > j of a chunk is
// formed relative to a boundary row that lies between them, so that both factors
// x_i 2^(Gcum_i - Gcum_b) and k_j 2^(Gcum_b - Gcum_j) are at most |x_i| and |k_j|:
//   level 1, rows 8..15 against rows 0..7, boundary row 7 (MFMA);
//   level 2, rows 4..7 against 0..3 and 12..15 against 8..11, boundary rows 3 and 11 (MFMA);
//   the pairs inside aligned groups of four rows and P's diagonal, one exponential per pair
//   and channel on the vector ALU (on the four q and k waves: interval 3, or interval 2
//   with the low-rank gate).
// Qa, Ka and Kl take their factors directly (2^Gcum, 2^(Gcum_end - Gcum), both <= 1).
//
// kXfer: the Transfer pass of the segment-parallel path, which forms end states only: the
// q plane and everything built from it (Qa, P, O, the output rows) are left out.
template <bool kFb, bool kSp, bool kXfer>
__global__ __launch_bounds__((PcShape<kSp, kFb, kXfer>::kNt)) void prefill_pc_kernel(PrefillArgs a, PcOrder order, SplitPlan plan) {
  using Shape = PcShape<kSp, kFb, kXfer>;
  constexpr int kCT = Shape::kCT;
  __shared__ PcSmem sm;
  // raw rows of q, k, v, z of the next chunk, as [plane][channel half][row][64]: producer
  // wave w reads and refills slice [w / 2][w % 2] only
  __shared__ __attribute__((aligned(16))) uint16_t raw_lds[4][2][C][kHeadDim / 2];
  // raw output-gate rows, three buffers by chunk index mod 3: the epilogue reads chunk c's
  // in interval 3 of iteration c + 1, while chunk c + 2's arrives
  __shared__ __attribute__((aligned(16))) uint16_t graw_lds[3][C][kHeadDim];
  // low-rank gate: the z_low rows of a chunk, by chunk parity, 16-byte pieces XOR-swizzled
  // by row (piece p of row r holds piece p ^ r) so that the MFMA operand reads of 16 rows
  // hit distinct banks
  __shared__ __attribute__((aligned(16))) uint16_t zlow_lds[kFb ? 2 : 1][kFb ? C : 1][kHeadDim];

  // This workgroup's (sequence n, head h) and tokens [t0, t0 + T): a whole sequence, or
  // segment kseg of nsegs (see the passes in kda_internal.h).
  const int H = a.L.H;
  int n, h, seg = 0, kseg = 0, nsegs = 1;
  bool transfer_m = false;  // Transfer pass, M half: identity start, v = 0 (not kMerged)
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
  constexpr bool write_out = !kXfer;  // a.pass == kPassTransfer exactly when kXfer
  // Where the gated RMSNorm epilogue runs.  With the bounded full-rank gate it runs on the
  // four q and k producer waves in interval 3, where they are otherwise idle: the consumers
  // leave each chunk's O rows in the chunk's V buffer (each lane over the very elements of
  // V it has just read) and go straight on to the state update.  With the softplus or the
  // low-rank gate those waves have interval-3 work of their own (position pairs, gate
  // tiles), and the consumers run the epilogue themselves, one chunk late, from per-wave
  // partial sums of squares that the norm wave turns into row factors.
  constexpr bool kProdEpi = !kSp && !kFb;
  const bool last_seg = kseg == nsegs - 1;
  const int64_t Hd = static_cast<int64_t>(H) * kHeadDim;
  const int nch = (T + C - 1) / C;

  // With the softplus gate alone, the v and z producer waves (logical waves 4..7) are
  // dispatched first, so that they are the oldest waves in each SIMD's issue arbitration
  // (measured 3% faster there; the other variants gain nothing or lose); t and wave below
  // are the logical numbering.  The swap moves waves by 4, so every wave keeps its SIMD.
  constexpr bool kVzFirst = kSp && !kFb;
  const int pwave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int t = kVzFirst ? ((pwave < 4 ? pwave + 4 : pwave < 8 ? pwave - 4 : pwave) << 6) | (threadIdx.x & 63)
                         : static_cast<int>(threadIdx.x);
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
  // (value column of tile j: col + 16 j)
  const int col = 16 * kCT * (cw & (Shape::kCwn - 1)) + lm;

  if (producer) {
    // ============================================================== producer waves
    const int urole = __builtin_amdgcn_readfirstlane(role);
    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    const int hf = uwave & 1;  // channel half of this wave's raw slice
    float w[4] = {0.f, 0.f, 0.f, 0.f}, hist[3] = {0.f, 0.f, 0.f};
    if (urole < 3) {
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = kCs * a.L.conv_w[(role * Hd + c) * kConvTaps + j];
      if (kseg > 0) {
        // a later segment: the conv history is the previous segment's last raw rows
        // (segments before the last are at least one chunk long)
        const bf16_t* pl = static_cast<const bf16_t*>(urole == 0 ? a.q : urole == 1 ? a.k : a.v);
#pragma unroll
        for (int j = 0; j < 3; ++j) hist[j] = bf16_to_f32(pl[(t0 - 3 + j) * Hd + c].bits);
      } else if (a.ring_in) {
        // segment 0 of a sequence cut into several: the Final pass reads the copy of the
        // ring that the Transfer pass left in the unused M plane of segment 0, since the
        // sequence's last segment may write ring_out == ring_in in the same launch
        float* const copy = a.pass == kPassWhole ? nullptr
                                                 : a.seg_m + (static_cast<int64_t>(seg) * H + h) * kHeadDim * kHeadDim +
                                                       (role * kHeadDim + ch) * kRingTaps;
        const float* const hp = (a.pass == kPassFinal && nsegs > 1)
                                    ? copy
                                    : a.ring_in + (static_cast<int64_t>(n) * 3 * Hd + role * Hd + c) * kRingTaps;
#pragma unroll
        for (int j = 0; j < 3; ++j) hist[j] = hp[j];
        if (a.pass == kPassTransfer && !transfer_m) {
#pragma unroll
          for (int j = 0; j < 3; ++j) copy[j] = hist[j];
        }
      }
    }
    // gate: g = lb sigmoid(e^A_log (z + dt_bias)) = lb / (1 + 2^(z ga + gb)); Gcum is kept
    // in log2 units (scaled by log2 e) so that every exponential below is one exp2
    const float ascale = expf(a.L.A_log[h]);
    const float ga = -kLog2e * ascale, gb = -kLog2e * ascale * a.L.dt_bias[c];
    const float lb2 = kLog2e * a.L.lower_bound;
    const float spb = kLog2e * a.L.dt_bias[c];  // softplus gate: (z + dt_bias) log2 e = z log2 e + spb
    if (kFb && urole == 3) sm.gbias[ch] = kSp ? spb : gb;
    if (kProdEpi && write_out && urole == 3) sm.nw[ch] = a.L.norm_w[ch];  // both z waves: 128 channels

    // Raw rows of a chunk, straight into LDS.  Each wave fetches exactly the slice it reads
    // itself in interval 1 (plane urole, channels 64 hf .. + 63, all 16 rows) as two
    // instructions of 64 pieces of 16 bytes: piece (k, lane) is row 8 k + lane / 8, bytes
    // 16 (lane % 8) of the slice's row, and one instruction's pieces land contiguously at
    // raw_lds[urole][hf][8 k].  No other wave touches the slice, so the wave orders its
    // reads and refills by itself.  The output-gate plane goes to the consumers'
    // double-buffered copy: four waves, piece s = 64 wave + lane is row s / 16, bytes
    // 16 (s % 16).  Both go through a buffer resource that starts at the chunk's first row
    // and spans its rows within the sequence: the lane offsets stay the same from chunk to
    // chunk (only the resource's SGPRs move), and rows past the end of a sequence are not
    // fetched; no arithmetic of a ragged chunk uses their slots.
    const char* const pq = static_cast<const char*>(a.q);
    const char* const pk = static_cast<const char*>(a.k);
    const char* const pv = static_cast<const char*>(a.v);
    const char* const pz = static_cast<const char*>(a.z);
    const char* const pgt = static_cast<const char*>(a.gate);
    const bf16_t* const x_b = static_cast<const bf16_t*>(a.beta);
    const int row_bytes = static_cast<int>(Hd) * 2;
    const int head_bytes = h * kHeadDim * 2;
    const char* const plane = urole == 0 ? pq : urole == 1 ? pk : urole == 2 ? pv : pz;
    uint16_t braw = 0;  // raw beta of row t (threads t < C), one chunk ahead
    // this wave's slice of raw_lds (wave-uniform)
    const uint32_t raw_slice = lds_addr(&raw_lds[0][0][0][0]) + (2 * urole + hf) * (C * kHeadDim);
    auto prefetch = [&](int c0n) __attribute__((always_inline)) {
      const int Ln = min(C, T - c0n);
      if (kFb && urole == 3) return;  // the z plane is z_low, fetched by prefetch_zlow
      if (t < C) {
        const __amdgpu_buffer_rsrc_t rb = uniform_rsrc(x_b + (t0 + c0n) * H, Ln * H * 2);
        braw = __builtin_amdgcn_raw_buffer_load_b16(rb, (t * H + h) * 2, 0, 0);
      }
      if (urole == 0 && !write_out) return;  // the Transfer pass has no use for q
      const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(plane + (t0 + c0n) * row_bytes, Ln * row_bytes);
      const int vo = opaque((lane >> 3) * row_bytes + head_bytes + (kHeadDim / 2) * 2 * hf + 16 * (lane & 7));
#pragma unroll
      for (int k = 0; k < 2; ++k) lds_dma16(rs, vo + 8 * k * row_bytes, 0, raw_slice + 8 * k * kHeadDim);
    };
    auto prefetch_gate = [&](int c0n, int buf) __attribute__((always_inline)) {
      if (uwave < 4) {
        const int Ln = min(C, T - c0n);
        const int sg = 64 * uwave + lane;
        const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(pgt + (t0 + c0n) * row_bytes, Ln * row_bytes);
        lds_dma16(rs, (sg >> 4) * row_bytes + head_bytes + 16 * (sg & 15), 0,
                      lds_addr(&graw_lds[buf][0][0]) + 2 * 8 * 64 * uwave);
      }
    };

    // low-rank gate: z_low rows 8 hf .. + 7 of chunk c0n / C into its parity's buffer (the q
    // waves, at the end of their interval 1 like their own rows): row 8 hf + 4 j + lane / 16,
    // swizzled piece lane % 16 (lane-dependent parts recomputed here rather than kept live
    // across the loop)
    auto prefetch_zlow = [&](int c0n) __attribute__((always_inline)) {
      const int Ln = min(C, T - c0n);
      // rows past the end of the sequence are not fetched (their gate is masked)
      const __amdgpu_buffer_rsrc_t rz = uniform_rsrc(pz + (t0 + c0n) * (kHeadDim * 2), Ln * (kHeadDim * 2));
      const int ln = opaque(lane);
      const int buf = (c0n / C) & 1;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = 8 * hf + 4 * j + (ln >> 4);
        lds_dma16(rz, row * (kHeadDim * 2) + 16 * ((ln & 15) ^ row), 0, lds_addr(&zlow_lds[buf][8 * hf + 4 * j][0]));
      }
    };

    // Low-rank gate of a chunk for channels 16 w .. + 15 of this head on producer wave w
    // (interval 3, beside the Gram tiles and the norms): the tile z^T = f_b[tile] z_low^T on
    // four MFMAs, so lane (lm, lq) holds row lm of channels 4 lq + s, with the f_b operands
    // fetched from L2 by buffer loads off one lane offset; then g per element, the
    // cumulative sum over the rows (the 16 lanes of a DPP row) and the per-channel factors,
    // as the full-rank path.  e^Gcum_end goes to eg15n: the chunk's KBuf is still the
    // consumers' when this runs, and the z waves copy it over one interval later.
    const bool gate_wave = kFb;
    auto gate_fetch = [&](bf16x8_t* fa) __attribute__((always_inline)) {
      const __amdgpu_buffer_rsrc_t fbr =
          buffer_rsrc(static_cast<const __bf16*>(a.L.f_b) + static_cast<int64_t>(h) * kHeadDim * kHeadDim,
                      kHeadDim * kHeadDim * 2);
      const int fvo = opaque(((16 * uwave + lm) * kHeadDim + 8 * lq) * 2);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        fa[kb] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(fbr, fvo, 32 * kb * 2, 0));
    };
    auto gate_low_rank = [&](int cidx, const bf16x8_t* fa) __attribute__((always_inline)) {
      const int Ln = min(C, T - cidx * C);
      const uint16_t(*zl)[kHeadDim] = zlow_lds[cidx & 1];
      f32x4_t zt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) zt = mma32(fa[kb], ld<bf16x8_t>(&zl[lm][8 * ((4 * kb + lq) ^ lm)]), zt);
      const int cb = 16 * uwave + 4 * lq;
      const float4 g4 = ld<float4>(&sm.gbias[cb]);
      const float gbv[4] = {g4.x, g4.y, g4.z, g4.w};
      // lanes lm < 4 own channel cb + lm for the per-channel factors
      float G[4], g7 = 0.f, g15 = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float g = kSp ? softplus_gate2(zt[s], gbv[s], ascale) : lb2 * frcp(1.0f + fexp2(fmaf(zt[s], ga, gbv[s])));
        g = lm < Ln ? g : 0.f;
        g += dpp_z<0x111>(g);  // inclusive prefix over the rows: row_shr 1, 2, 4, 8
        g += dpp_z<0x112>(g);
        g += dpp_z<0x114>(g);
        g += dpp_z<0x118>(g);
        G[s] = g;
        const float b7 = row_bcast<C / 2 - 1>(g), b15 = row_bcast<C - 1>(g);
        g7 = lm == s ? b7 : g7;
        g15 = lm == s ? b15 : g15;
      }
      *reinterpret_cast<float4*>(&sm.gam[lm][opaque(cb)]) = make_float4(G[0], G[1], G[2], G[3]);
      const float e15 = fexp2(g15), e7 = fexp2(g7), e157 = fexp2(g15 - g7);
      if (lm < 4) {
        const int cc = opaque(cb + lm);  // recomputed here, not kept live across the loop
        sm.eg15n[cc] = e15;
        if (!kSp) {
          sm.g7[cc] = g7;
          sm.eg7[cc] = e7;
          sm.e157[cc] = e157;
        }
      }
    };

    // softplus gate: the 4x4 diagonal blocks of chunk i + 1's G and P as position pairs,
    // on the four q and k waves: in interval 3, where they have no other job, or with the
    // low-rank gate in interval 2, since there interval 3 overwrites Gcum with chunk i + 2's.
    // Wave w takes rows 4w .. 4w + 3 (local rows 0..3): the first half-wave the pairs
    // (1,0), (2,0), (2,1) and P's diagonal at rows 0..2, the second the pairs (3,0), (3,1),
    // (3,2) and the diagonal at row 3; lane l of a half takes channels 4 (l % 32) .. + 3.  A
    // pair (a, b) costs one exponential 2^(Gcum_a - Gcum_b) <= 1 per channel.  The sums over
    // the half's 32 lanes (DPP row sums, then the two rows) are written by its first 12
    // (rows 0..2) or 4 (row 3) lanes, one entry of G and of P each.
    auto pair_blocks = [&](int kbuf) __attribute__((always_inline)) {
      KBuf& KP = sm.kb[kbuf];
      const int hh = lane >> 5, pc = 4 * (lane & 31), r0 = 4 * uwave;
      auto row4 = [&](const float(*arr)[LDP], int row, float* x) __attribute__((always_inline)) {
        const float4 v = ld<float4>(&arr[r0 + row][pc]);
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
      };
      float ps[9];  // G and P of the half's three pairs, then three diagonal entries
#pragma unroll
      for (int sl = 0; sl < 3; ++sl) {
        // pair sl of this half: (1, 0), (2, 0), (2, 1) in the first, (3, sl) in the second
        const int ra = hh ? 3 : (sl == 0 ? 1 : 2), rb = hh ? sl : (sl == 2 ? 1 : 0);
        float qa[4], ka[4], ga[4], kb[4], gb[4];
        row4(sm.aq, ra, qa);
        row4(sm.ak, ra, ka);
        row4(sm.gam, ra, ga);
        row4(sm.ak, rb, kb);
        row4(sm.gam, rb, gb);
        float sg = 0.f, sp = 0.f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float kf = kb[v] * fexp2(ga[v] - gb[v]);
          sg = fmaf(ka[v], kf, sg);
          sp = fmaf(qa[v], kf, sp);
        }
        ps[sl] = sg;
        ps[3 + sl] = sp;
      }
#pragma unroll
      for (int dg = 0; dg < 3; ++dg) {
        float qd[4], kd[4];
        row4(sm.aq, hh ? 3 : dg, qd);
        row4(sm.ak, hh ? 3 : dg, kd);
        ps[6 + dg] = (qd[0] * kd[0] + qd[1] * kd[1]) + (qd[2] * kd[2] + qd[3] * kd[3]);
      }
#pragma unroll
      for (int x = 0; x < 9; ++x) {
        ps[x] = row_sum16(ps[x]);
        ps[x] += __shfl_xor(ps[x], 16, 64);
      }
      const int cl = lane & 31;
      if (cl < (hh ? 4 : 12)) {
        const int a = hh ? 3 : cl >> 2, b = cl & 3;
        // pair (a, b), b < a: its slot in this half
        const int sl = hh ? b : (a == 1 ? 0 : 1 + b);
        const float gsel = sl == 0 ? ps[0] : sl == 1 ? ps[1] : ps[2];
        const float psel = sl == 0 ? ps[3] : sl == 1 ? ps[4] : ps[5];
        const float dsel = hh ? ps[6] : (a == 0 ? ps[6] : a == 1 ? ps[7] : ps[8]);
        const float gv_ = b < a ? gsel : 0.f;
        const float pv_ = b < a ? psel : (b == a ? dsel : 0.f);
        sm.A[r0 + a][r0 + b] = gv_;
        split_store(&KP.p[r0 + a][il16(r0 + b)], &KP.p[r0 + a][il16(r0 + b) + 4], pv_);
      }
    };

    // The gated RMSNorm epilogue of chunk ic (kProdEpi) on the q and k waves in interval 3:
    // wave w takes rows 4 w .. 4 w + 3, lane l row 4 w + l / 16 and channels 8 (l % 16) ..
    // + 7.  The consumers left the chunk's rows of O = Qa S + P U in its V buffer; the true
    // output row is rq O (rq the q row factor), and rq O / sqrt(mean (rq O)^2 + eps) = O rr
    // with rr = rq / sqrt(rq^2 mean O^2 + eps), the sum of squares taken over the 16 lanes
    // of a DPP row.  Then times the norm weight and sigmoid(gate), rounded to bf16 and
    // stored as one 16-byte piece per lane through a buffer resource over the chunk's rows.
    auto epilogue = [&](int ic) __attribute__((always_inline)) {
      const KBuf& K = sm.kb[ic & 1];
      const int r = 4 * uwave + (lane >> 4), c8 = 8 * (lane & 15);
      const float4 o0 = ld<float4>(&K.V[r][c8]), o1 = ld<float4>(&K.V[r][c8 + 4]);
      const float o[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
      const uint4 gr = ld<uint4>(&graw_lds[ic % 3][r][c8]);
      const float4 w0 = ld<float4>(&sm.nw[c8]), w1 = ld<float4>(&sm.nw[c8 + 4]);
      const float nw8[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      const uint32_t g2[4] = {gr.x, gr.y, gr.z, gr.w};
      float ss = 0.f;
#pragma unroll
      for (int v = 0; v < 8; ++v) ss = fmaf(o[v], o[v], ss);
      ss = row_sum16(ss);
      const float rq = K.rq[r];
      const float rr = rq * __builtin_amdgcn_rsqf(rq * rq * ss * (1.0f / kHeadDim) + a.L.rms_eps);
      uint32_t packed[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float ga0 = __uint_as_float(g2[j] << 16), ga1 = __uint_as_float(g2[j] & 0xffff0000u);
        const float y0 = nw8[2 * j] * o[2 * j] * rr * fsigmoid(ga0);
        const float y1 = nw8[2 * j + 1] * o[2 * j + 1] * rr * fsigmoid(ga1);
        packed[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){y0, y1}, bf16x2_t));
      }
      // rows past the end of the sequence fall outside the resource and are not written
      const __amdgpu_buffer_rsrc_t ro =
          uniform_rsrc(static_cast<char*>(a.out) + (t0 + ic * C) * row_bytes, min(C, T - ic * C) * row_bytes);
      const u32x4_raw pk4 = {packed[0], packed[1], packed[2], packed[3]};
      __builtin_amdgcn_raw_buffer_store_b128(pk4, ro, r * row_bytes + head_bytes + 2 * c8, 0, 0);
    };

    if (T > 0) {
      prefetch(0);
      if (kFb && urole == 0) {
        prefetch_zlow(0);
        if (nch > 1) prefetch_zlow(C);
      }
      wait_vm();
    }
    lds_barrier();
    // low-rank gate: the gate waves form chunk c's gate in interval 3 of iteration c - 2,
    // the interval before the one in which the other producers build chunk c, from z_low
    // rows fetched in interval 1 of iteration c - 3; chunk 0's here (the consumers keep the
    // barrier count with a barrier of their own)
    if (kFb) {
      if (gate_wave && T > 0) {
        bf16x8_t fa[4];
        gate_fetch(fa);
        gate_low_rank(0, fa);
      }
      lds_barrier();
    }

    // With two value tiles per consumer wave (the 12-wave layout, which has registers to
    // spare), the raw rows are read straight into the high halves of registers whose low
    // halves stay zero from one chunk to the next (ds_read_u16_d16_hi): each value is then
    // already the fp32 of its bf16, and the 16 shifts per chunk and wave are saved.
    uint32_t xw[C];
#pragma unroll
    for (int r = 0; r < C; ++r) xw[r] = 0u;

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
        if (!(kFb && urole == 3) && !(urole == 0 && !write_out)) {
          if constexpr (Shape::kWide) {
            const uint32_t ra = lds_addr(&raw_lds[urole][hf][0][lane]);
#pragma unroll
            for (int r = 0; r < C; ++r)
              asm volatile("ds_read_u16_d16_hi %0, %1 offset:%2" : "+v"(xw[r]) : "v"(ra), "i"(r * kHeadDim) : "memory");
            lds_wait();  // the compiler does not track these reads
          } else {
#pragma unroll
            for (int r = 0; r < C; ++r) xr[r] = raw_lds[urole][hf][r][lane];
          }
        }
        // raw value of row r as fp32
        auto raw = [&](int r) __attribute__((always_inline)) {
          return Shape::kWide ? __uint_as_float(xw[r]) : bf16_to_f32(xr[r]);
        };
        if (t < C) KN.beta[t] = (t < Ln) ? fsigmoid(bf16_to_f32(braw)) : 0.f;
        // this wave's raw slice is read: refill it with chunk i + 2 at once (the reads are
        // complete before the transfer is issued), so that the transfer's issue overlaps
        // the arithmetic below instead of following it
        if (i + 2 < nch && !(kFb && urole == 3)) {
          lds_wait();
          prefetch((i + 2) * C);
        }
        const bool full = Ln == C;
        if (urole == 2 && transfer_m) {
          // the transfer matrix is the end state from the identity with v = 0
#pragma unroll
          for (int r = 0; r < C; ++r) KN.V[r][ch] = 0.f;
        } else if (urole == 0 && !write_out) {
          // the Transfer pass forms end states only: q and everything built from it (Qa,
          // P, the output rows) go unused, and their work is skipped
        } else if (urole < 3) {
          float(*dst)[LDP] = urole == 0 ? sm.aq : urole == 1 ? sm.ak : KN.V;
          if (full) {
            // Staged over the 16 rows: every conv sum, then every exponential, then every
            // reciprocal, then the products.  The history is a pure shift, so the rows are
            // independent and 16 chains interleave instead of the few a row-by-row loop
            // leaves the scheduler.
            float xs[C + 3], ys[C], ev[C];
            xs[0] = hist[0];
            xs[1] = hist[1];
            xs[2] = hist[2];
#pragma unroll
            for (int r = 0; r < C; ++r) xs[r + 3] = raw(r);
#pragma unroll
            for (int r = 0; r < C; ++r) ys[r] = w[3] * xs[r + 3] + w[0] * xs[r] + w[1] * xs[r + 1] + w[2] * xs[r + 2];
            hist[0] = xs[C];
            hist[1] = xs[C + 1];
            hist[2] = xs[C + 2];
#pragma unroll
            for (int r = 0; r < C; ++r) ev[r] = fexp2(ys[r]);
#pragma unroll
            for (int r = 0; r < C; ++r) ev[r] = frcp(1.0f + ev[r]);
#pragma unroll
            for (int r = 0; r < C; ++r) dst[r][ch] = ys[r] * ev[r];
          } else {
#pragma unroll
            for (int r = 0; r < C; ++r) {
              const float x = raw(r);
              const float ys = w[3] * x + w[0] * hist[0] + w[1] * hist[1] + w[2] * hist[2];
              const bool live = r < Ln;
              if (live) {
                hist[0] = hist[1];
                hist[1] = hist[2];
                hist[2] = x;
              }
              dst[r][ch] = live ? ys * frcp(1.0f + fexp2(ys)) : 0.f;
            }
          }
        } else if (kFb) {
          // this chunk's gate was formed one interval 3 earlier (or before the loop)
          const int cc = opaque(ch);  // recomputed here, not kept live across the loop
          KN.eg15[cc] = sm.eg15n[cc];
        } else {
          // the per-token log2 decay of either gate
          auto gate2 = [&](float xz) __attribute__((always_inline)) {
            return kSp ? softplus_gate2(xz, spb, ascale) : lb2 * frcp(1.0f + fexp2(fmaf(xz, ga, gb)));
          };
          float G = 0.f, G7 = 0.f;
          if (full) {
            // every row's decay first (independent chains), then the running sum
            float gv[C];
#pragma unroll
            for (int r = 0; r < C; ++r) gv[r] = gate2(raw(r));
#pragma unroll
            for (int r = 0; r < C; ++r) {
              G += gv[r];
              sm.gam[r][ch] = G;
              if (r == C / 2 - 1) G7 = G;
            }
          } else {
#pragma unroll
            for (int r = 0; r < C; ++r) {
              const bool live = r < Ln;
              G += live ? gate2(raw(r)) : 0.f;
              sm.gam[r][ch] = G;
              if (r == C / 2 - 1) G7 = G;
            }
          }
          KN.eg15[ch] = fexp2(G);
          if (!kSp) {
            sm.g7[ch] = G7;
            sm.eg7[ch] = fexp2(G7);
            sm.e157[ch] = fexp2(G - G7);
          }
        }
        // low-rank gate: chunk i + 3's z_low rows (their buffer's chunk i + 1 was read in the
        // previous interval 3), waited for with this wave's other transfers
        if (kFb && urole == 0 && i + 3 < nch) prefetch_zlow((i + 3) * C);

      }
      lds_barrier();

      // ---------------------------------------------------------- interval 2
      if (has_next) {
        // chunk i + 1's output gate, into the buffer of chunk i - 2, whose epilogue ran in
        // the previous interval 3
        if (write_out) prefetch_gate((i + 1) * C, (i + 1) % 3);
        // Every operand of chunk i + 1 for row r, channels c4 .. c4 + 3 (rows run fastest
        // across lanes, so the transposed Ka / Kl writes are 32 contiguous bytes per
        // channel).  With d = Gcum - Gcum_mid: Qp = a_q e^d, Kp = a_k e^d, Km = a_k e^-d;
        // Qa = Qp e^Gcum_mid, Ka = Kp e^Gcum_mid, Kl = Km e^(Gcum_end - Gcum_mid).  Also the
        // rows' sums of squares over these 4 channels.
        const int r = t & (C - 1), c4 = 4 * (t >> 4);
        const float4 qv = ld<float4>(&sm.aq[r][c4]);
        const float4 kv = ld<float4>(&sm.ak[r][c4]);
        const float4 gv = ld<float4>(&sm.gam[r][c4]);
        const float q4[4] = {qv.x, qv.y, qv.z, qv.w};
        const float k4[4] = {kv.x, kv.y, kv.z, kv.w};
        float qa[4], ka[4], kl[4], sq = 0.f, sk = 0.f;
        if constexpr (kSp) {
          // Qa, Ka and Kl from 2^Gcum and 2^(Gcum_end - Gcum); the level operands of the
          // Gram tiles (see the kernel's kSp note): at level l a row r in the later half of
          // its block (of 16 or 8 rows) gives Xk = a_k 2^(Gcum - Gcum_b) and Xq = a_q 2^(.)
          // (rows 8 + x and 16 + x of the level's [24] operand rows), a row in the earlier
          // half Y = a_k 2^(Gcum_b - Gcum) (row x), with b the block's boundary row and x the
          // row's index among the level's later or earlier rows
          const float4 ge = ld<float4>(&sm.gam[C - 1][c4]);
          const float4 b1 = ld<float4>(&sm.gam[C / 2 - 1][c4]);
          const float4 b2 = ld<float4>(&sm.gam[(r & 8) + 3][c4]);
          const float gr[4] = {gv.x, gv.y, gv.z, gv.w}, gend[4] = {ge.x, ge.y, ge.z, ge.w};
          const float gb1[4] = {b1.x, b1.y, b1.z, b1.w}, gb2[4] = {b2.x, b2.y, b2.z, b2.w};
          const bool late1 = r >= 8, late2 = (r & 4) != 0;
          float x1k[4], x1q[4], x2k[4], x2q[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float e = fexp2(gr[v]);
            qa[v] = q4[v] * e;
            ka[v] = k4[v] * e;
            kl[v] = k4[v] * fexp2(gend[v] - gr[v]);
            const float f1 = fexp2(late1 ? gr[v] - gb1[v] : gb1[v] - gr[v]);
            const float f2 = fexp2(late2 ? gr[v] - gb2[v] : gb2[v] - gr[v]);
            x1k[v] = k4[v] * f1;
            x1q[v] = q4[v] * f1;
            x2k[v] = k4[v] * f2;
            x2q[v] = q4[v] * f2;
            sq = fmaf(q4[v], q4[v], sq);
            sk = fmaf(k4[v], k4[v], sk);
          }
          LevelOps& L1 = level_ops(sm)[0];
          LevelOps& L2 = level_ops(sm)[1];
          const int x1 = r & 7, x2 = ((r >> 3) << 2) + (r & 3);
          store4(&L1.h[late1 ? 8 + x1 : x1][c4], &L1.l[late1 ? 8 + x1 : x1][c4], x1k);
          store4(&L2.h[late2 ? 8 + x2 : x2][c4], &L2.l[late2 ? 8 + x2 : x2][c4], x2k);
          if (late1 && write_out) store4(&L1.h[16 + x1][c4], &L1.l[16 + x1][c4], x1q);
          if (late2 && write_out) store4(&L2.h[16 + x2][c4], &L2.l[16 + x2][c4], x2q);
        } else {
          const float4 g7 = ld<float4>(&sm.g7[c4]);
          const float4 e7 = ld<float4>(&sm.eg7[c4]);
          const float4 e157 = ld<float4>(&sm.e157[c4]);
          const float d4[4] = {gv.x - g7.x, gv.y - g7.y, gv.z - g7.z, gv.w - g7.w};
          const float m7[4] = {e7.x, e7.y, e7.z, e7.w};
          const float m157[4] = {e157.x, e157.y, e157.z, e157.w};
          float qp[4], kp[4], km[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float el = fexp2(d4[v]), er = fexp2(-d4[v]);
            qp[v] = q4[v] * el;
            kp[v] = k4[v] * el;
            km[v] = k4[v] * er;
            qa[v] = qp[v] * m7[v];
            ka[v] = kp[v] * m7[v];
            kl[v] = km[v] * m157[v];
            sq = fmaf(q4[v], q4[v], sq);
            sk = fmaf(k4[v], k4[v], sk);
          }
          if (write_out) store4(&sm.qp[0][r][c4], &sm.qp[1][r][c4], qp);
          store4(&sm.kp[0][r][c4], &sm.kp[1][r][c4], kp);
          store4(&sm.km[0][r][c4], &sm.km[1][r][c4], km);
        }
        sm.nsq[0][r][t >> 4] = sq;
        sm.nsq[1][r][t >> 4] = sk;
        // Qa and Ka in the key order of the .S products: channels 32 kb + 4 m .. + 3 sit
        // at 32 kb + 8 (m % 4) + 4 (m / 4)
        const int pa = 32 * (c4 >> 5) + 8 * ((c4 >> 2) & 3) + 4 * ((c4 >> 4) & 1);
        if (write_out) store4_f16(&KN.qa[r][pa], qa);
        store4_f16(&KN.ka[r][pa], ka);
#pragma unroll
        for (int v = 0; v < 4; v += 2)
          split_store2(&KN.klt[c4 + v][il16(r)], &KN.klt[c4 + v][il16(r) + 4], &KN.klt[c4 + v + 1][il16(r)],
                       &KN.klt[c4 + v + 1][il16(r) + 4], kl[v], kl[v + 1]);
        if (kSp && kFb && uwave < 4) pair_blocks((i + 1) & 1);
      }
      lds_barrier();

      // ---------------------------------------------------------- interval 3
      if (kSp && !kFb && has_next && uwave < 4) pair_blocks((i + 1) & 1);
      if (kProdEpi && write_out && i >= 0 && uwave < 4) epilogue(i);
      // (softplus gate: level 1 of G and P on the Gram waves, level 2 on waves 7 and 6,
      // so that each SIMD issues one level tile)
      const bool gram_a = uwave == kGramAWave || uwave == 7;
      if (has_next && (uwave == kGramAWave || uwave == kGramPWave || (kSp && uwave >= 6)) && (gram_a || write_out)) {
        const int lv = kSp && uwave >= 6 ? 1 : 0;  // softplus gate: this wave's level
        // Gram tiles of chunk i + 1: G = Kp Km^T (strict lower; the elimination of consumer
        // waves kElimCwA/B in the next interval 1 scales its rows by beta') and
        // P = Qp Km^T (lower incl.)
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (kSp) {
          // level lv + 1 as the product of its operands (lane row lm: Xk or Xq if lm is in
          // the later half of its block, else Y); a lane's rows 4 lq .. + 3 and column lm
          // belong to level 1 if lm is in the other half of the 16 rows, to level 2 if in
          // the other group of four of the same half, else to the pair waves
          const LevelOps& L = level_ops(sm)[lv];
          const bool late = (lm & (8 >> lv)) != 0;
          const int x = lv == 0 ? (lm & 7) : ((lm >> 3) << 2) + (lm & 3);
          const int ra = late ? (gram_a ? 8 : 16) + x : x, rb = late ? 8 + x : x;
          f32x4_t x1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < kHeadDim / 32; ++kb) {
            const int o = 32 * kb + 8 * lq;
            const bf16x8_t xh = ld<bf16x8_t>(&L.h[ra][o]), xl = ld<bf16x8_t>(&L.l[ra][o]);
            const bf16x8_t mh = ld<bf16x8_t>(&L.h[rb][o]), ml = ld<bf16x8_t>(&L.l[rb][o]);
            acc = mma32(xh, mh, acc);
            x1 = mma32(xh, ml, x1);
            x1 = mma32(xl, mh, x1);
          }
          acc += x1;
        } else {
          const __bf16(*Xh)[OPP] = gram_a ? sm.kp[0] : sm.qp[0];
          const __bf16(*Xl)[OPP] = gram_a ? sm.kp[1] : sm.qp[1];
          f32x4_t a1 = {0.f, 0.f, 0.f, 0.f};
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
        }
        if (kSp && (lv == 0 ? (lm >> 3) == (lq >> 1) : ((lm >> 3) != (lq >> 1) || (lm >> 2) == lq))) {
          // entries of another level or of the pair waves
        } else if (gram_a) {
#pragma unroll
          for (int s = 0; s < 4; ++s) sm.A[4 * lq + s][lm] = (lm < 4 * lq + s) ? acc[s] : 0.f;
        } else {
#pragma unroll
          for (int s = 0; s < 4; s += 2) {
            const int r = 4 * lq + s, j = lm;
            split_store2(&KN.p[r][il16(j)], &KN.p[r][il16(j) + 4], &KN.p[r + 1][il16(j)], &KN.p[r + 1][il16(j) + 4],
                         (j <= r) ? acc[s] : 0.f, (j <= r + 1) ? acc[s + 1] : 0.f);
          }
        }
      }
      if (uwave == kNormWave) {
        const int r = lane & (C - 1);
        if (lane < 2 * C) {
          if (has_next) {
            // Row norms of chunk i + 1 from the 32 partial sums of squares of each row (of
            // the scaled rows kCs a): lanes 0..15 form |a_k|' and beta', lanes 16..31 the
            // q scale.
            const bool kk = lane < C;
            const float(*ns)[NSP] = sm.nsq[kk ? 1 : 0];
            float tot = 0.f;
#pragma unroll
            for (int g = 0; g < kHeadDim / 4; g += 4) {
              const float4 v4 = ld<float4>(&ns[r][g]);
              tot += (v4.x + v4.y) + (v4.z + v4.w);
            }
            // |a|'^2 = |kCs a|^2 / kCs^2 + eps
            const float den = fmaf(tot, kLn2 * kLn2, a.L.l2_eps);
            if (kk) {
              KN.vk[r] = __builtin_amdgcn_sqrtf(den);
              KN.beta[r] = KN.beta[r] * frcp(den) * (kLn2 * kLn2);
            } else {
              KN.rq[r] = __builtin_amdgcn_rsqf(den) * (-kQScale * kLn2);
            }
          }
        } else if (lane < 3 * C) {
          if (!kProdEpi && i >= 0 && write_out) {
            // RMSNorm factor of chunk i's output row r from the consumers' partial sums:
            // the true row is rq O, and rq O / sqrt(mean (rq O)^2 + eps) = O rr with
            // rr = rq / sqrt(rq^2 mean O^2 + eps)
            float tot = sm.ss[0][r];
#pragma unroll
            for (int wv = 1; wv < CWN; ++wv) tot += sm.ss[wv][r];
            const float rq = sm.kb[i & 1].rq[r];
            sm.rr[i & 1][r] = rq * __builtin_amdgcn_rsqf(rq * rq * tot * (1.0f / kHeadDim) + a.L.rms_eps);
          }
        }
      }
      // low-rank gate of chunk i + 2 (the readers of gam and of the per-channel factors of
      // chunk i + 1 ran in interval 2)
      if (gate_wave && i + 2 < nch) {
        bf16x8_t fa[4];
        gate_fetch(fa);
        gate_low_rank(i + 2, fa);
      }
      // this wave's transfers (raw rows of chunk i + 2, output gate of chunk i + 1) are
      // in LDS before the barrier that publishes them
      wait_vm();
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
    // kCT value tiles of 16 columns per wave (tile j: columns col + 16 j), each the fp32
    // 128 x 16 block of the state as 8 MFMA accumulator tiles.  mstate: this wave forms a
    // transfer matrix M (the M half of the Transfer pass, or its second wave set)
    const bool mstate = Shape::kMerged ? cw >= Shape::kCwn : transfer_m;
    f32x4_t S[kCT][8];
    constexpr int64_t kDD = kHeadDim * kHeadDim;
    const int64_t nbase = (static_cast<int64_t>(n) * H + h) * kDD;    // [N][H] planes
    const int64_t sgbase = (static_cast<int64_t>(seg) * H + h) * kDD; // [segments][H] planes
    const float* src = nullptr;
    if (a.pass == kPassFinal && kseg > 0)
      src = a.seg_start + sgbase;
    else if (a.pass == kPassFinal && nsegs > 1)
      // segment 0 of a sequence cut into several: the Transfer pass's copy of the start
      // state (the sequence's last segment may write state_out == state_in in this launch)
      src = a.state_in ? a.seg_start + sgbase : nullptr;
    else if (kseg == 0 && !mstate && a.state_in)
      src = a.state_in + nbase;
    if (src) {
      const float* sp = src + opaque(4 * lq * kHeadDim + col);
#pragma unroll
      for (int j = 0; j < kCT; ++j)
#pragma unroll
        for (int it = 0; it < 8; ++it)
#pragma unroll
          for (int s = 0; s < 4; ++s) S[j][it][s] = sp[(16 * it + s) * kHeadDim + 16 * j];
      if (a.pass == kPassTransfer && !mstate) {
        // segment 0 (the Transfer pass skips a sequence's last segment, so the sequence
        // has several): keep the start state where the Final pass reads it, in segment
        // 0's start plane, which the combine never writes
        float* cp = a.seg_start + sgbase + opaque(4 * lq * kHeadDim + col);
#pragma unroll
        for (int j = 0; j < kCT; ++j)
#pragma unroll
          for (int it = 0; it < 8; ++it)
#pragma unroll
            for (int s = 0; s < 4; ++s) cp[(16 * it + s) * kHeadDim + 16 * j] = S[j][it][s];
      }
    } else {
#pragma unroll
      for (int j = 0; j < kCT; ++j)
#pragma unroll
        for (int it = 0; it < 8; ++it)
#pragma unroll
          for (int s = 0; s < 4; ++s) S[j][it][s] = (mstate && 16 * it + 4 * lq + s == col + 16 * j) ? 1.f : 0.f;
    }
    lds_barrier();
    if (kFb) lds_barrier();  // the producers' low-rank gate of chunk 0

    const float nw = kProdEpi ? 0.f : a.L.norm_w[col];
    bf16x8_t u_l0[kCT] = {}, u_hh[kCT] = {};  // U of each tile as the B operands of mma16p
    // S = Diag(exp(Gcum_C)) S + Kl^T U, once chunk i's U is known.  The factors of key rows
    // 16 it + 4 lq + s (it = 0..7, s = 0..3) are the same for the 16 lanes of a DPP row:
    // lane lm reads those of (it, s) = (lm / 2, 2 (lm % 2)) and (lm / 2, 2 (lm % 2) + 1)
    // (one 8-byte LDS read instead of eight 16-byte ones), and every lane takes each factor
    // from its owner by row_newbcast inside the multiply.  Each Kl^T operand serves every
    // tile of the wave.
    auto update_state = [&](const KBuf& K) __attribute__((always_inline)) {
      const float2 e2 = ld<float2>(&K.eg15[16 * (lm >> 1) + 4 * lq + 2 * (lm & 1)]);
      auto mm = [&](int it) __attribute__((always_inline)) {
        const bf16x8_t kl = ld<bf16x8_t>(&K.klt[16 * it + lm][8 * lq]);
#pragma unroll
        for (int j = 0; j < kCT; ++j) S[j][it] = mma16p(kl, u_l0[j], u_hh[j], S[j][it]);
      };
      auto dec = [&](auto tag) __attribute__((always_inline)) {
        constexpr int IT = decltype(tag)::value;
#pragma unroll
        for (int j = 0; j < kCT; ++j) decay_tile<IT>(S[j][IT], e2.x, e2.y);
        mm(IT);
      };
      dec(std::integral_constant<int, 0>{});
      dec(std::integral_constant<int, 1>{});
      dec(std::integral_constant<int, 2>{});
      dec(std::integral_constant<int, 3>{});
      dec(std::integral_constant<int, 4>{});
      dec(std::integral_constant<int, 5>{});
      dec(std::integral_constant<int, 6>{});
      dec(std::integral_constant<int, 7>{});
    };

    // Gated RMSNorm of chunk ic's output rows O and the store, with the row factors rr
    // that the norm wave formed from every consumer wave's partial sums (the variants
    // whose epilogue runs on the consumers; one tile per wave there).
    auto emit = [&](int ic, const f32x4_t& Oc) __attribute__((always_inline)) {
      const int L = min(C, T - ic * C);
      const float4 r4 = ld<float4>(&sm.rr[ic & 1][4 * lq]);
      const float rr[4] = {r4.x, r4.y, r4.z, r4.w};
      float y[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float g = fsigmoid(bf16_to_f32(graw_lds[ic % 3][4 * lq + s][col]));
        y[s] = nw * Oc[s] * rr[s] * g;
      }
      bf16_t* po = static_cast<bf16_t*>(a.out) + (t0 + ic * C + 4 * lq) * Hd + static_cast<int64_t>(h) * kHeadDim + col;
      if (L == C) {
#pragma unroll
        for (int s = 0; s < 4; ++s) po[s * Hd].bits = f32_to_bf16(y[s]);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          if (4 * lq + s < L) po[s * Hd].bits = f32_to_bf16(y[s]);
      }
    };

    // iteration i: consumers run chunk i, and emit chunk i - 1's output rows
    f32x4_t Oprev = {0.f, 0.f, 0.f, 0.f};
    for (int i = -1; i < nch; ++i) {
      KBuf& K = sm.kb[i & 1];
      f32x4_t O[kCT], X[kCT];  // Qa S + P U, and Ka S, per tile
#pragma unroll
      for (int j = 0; j < kCT; ++j) O[j] = X[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

      // ---------------------------------------------------------- interval 1
      if (i >= 0) {
        if (cw == kElimCwA || cw == kElimCwB) {
          // T = (I + A)^-1 Diag(beta') by elimination with rows spread over lanes (DPP
          // broadcasts inside each 16-lane row); A[r][j] = 0 for j >= r, so the update
          // is unconditional.  Lane (lm, lq) holds T[lm][lq + 4 s]; wave kElimCwA takes
          // slots s = 0, 3 and wave kElimCwB slots 1, 2.
          // -A = -Diag(beta') G, row lm (the elimination takes the row negated)
          float arow[C], tt[2];
          const float bl = K.beta[lm], nbl = -bl;
#pragma unroll
          for (int j = 0; j < C; j += 4) {
            const float4 v4 = *reinterpret_cast<const float4*>(&sm.A[lm][j]);
            arow[j] = nbl * v4.x;
            arow[j + 1] = nbl * v4.y;
            arow[j + 2] = nbl * v4.z;
            arow[j + 3] = nbl * v4.w;
          }
          const bool wa = cw == kElimCwA;
          const int s0 = wa ? 0 : 1, s1 = wa ? 3 : 2;
          tt[0] = (lq + 4 * s0 == lm) ? bl : 0.f;
          tt[1] = (lq + 4 * s1 == lm) ? bl : 0.f;
          // five wait states ahead of the first DPP step, whatever the compiler placed
          // before it (a VALU write of EXEC needs five; a VGPR write two)
          asm volatile("s_nop 4" ::: "memory");
          if (wa)
            eliminate_strided2<0, 0, 3>(tt, arow);
          else
            eliminate_strided2<0, 1, 2>(tt, arow);
          split_store2(&K.tm[lm][il16(lq + 4 * s0)], &K.tm[lm][il16(lq + 4 * s0) + 4], &K.tm[lm][il16(lq + 4 * s1)],
                       &K.tm[lm][il16(lq + 4 * s1) + 4], tt[0], tt[1]);
        }
        // O = Qa S (rows still to be scaled by the q scale rq) and X = Ka S, with S as
        // fp16 B operands (per 32 keys: 4 lq + s, then 16 + 4 lq + s); each Qa and Ka
        // operand serves every tile
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const f16x8_t qa = write_out ? ld<f16x8_t>(&K.qa[lm][32 * kb + 8 * lq]) : f16x8_t{};
          const f16x8_t ka = ld<f16x8_t>(&K.ka[lm][32 * kb + 8 * lq]);
#pragma unroll
          for (int j = 0; j < kCT; ++j) {
            f16x8_t sf;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              sf[s] = static_cast<_Float16>(S[j][2 * kb][s]);
              sf[4 + s] = static_cast<_Float16>(S[j][2 * kb + 1][s]);
            }
            if (write_out) O[j] = mma32h(qa, sf, O[j]);
            X[j] = mma32h(ka, sf, X[j]);
          }
        }
      }
      lds_barrier();

      // ---------------------------------------------------------- interval 2
      if (i >= 0) {
        // U = U~ - W S = T (V' - Ka S) for each value tile, V' = |a_k|' V by rows
        const bf16x8_t tq = ld<bf16x8_t>(&K.tm[lm][8 * lq]);
        const float4 k4 = ld<float4>(&K.vk[4 * lq]);
        const float vk[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
        for (int j = 0; j < kCT; ++j) {
          f32x4_t U = {0.f, 0.f, 0.f, 0.f};
          float y4[4];
#pragma unroll
          for (int s = 0; s < 4; ++s)
            y4[s] = fmaf(Shape::kMerged && mstate ? 0.f : K.V[4 * lq + s][col + 16 * j], vk[s], -X[j][s]);
          bf16x4_t yh, yl;
          split_vec<4>(y4, yh, yl);
          bf16x8_t y_l0, y_hh;
          b_pair(yh, yl, y_l0, y_hh);
          U = mma16p(tq, y_l0, y_hh, U);
          float u4[4] = {U[0], U[1], U[2], U[3]};
          bf16x4_t uh, ul;
          split_vec<4>(u4, uh, ul);
          b_pair(uh, ul, u_l0[j], u_hh[j]);
        }
        // O += P U and the rows' partial sums of squares (not in the Transfer pass).
        // Accumulator hand-off between opcodes: O was last written by the fp16 16x16x32
        // MFMA of interval 1 and is accumulated here by the bf16 16x16x32 one.  The rule
        // this kernel keeps (see mma16p) is that a dependent accumulation chain never mixes
        // instructions of different shapes (a 16x16x16 result taken as the accumulator of a
        // 16x16x32 a few instructions later gave wrong rows); these two have the same shape
        // and pass count, and a barrier and the U product lie between them.  Every other
        // chain in the kernel uses a single opcode.
        if (write_out) {
          const bf16x8_t pp = ld<bf16x8_t>(&K.p[lm][8 * lq]);
#pragma unroll
          for (int j = 0; j < kCT; ++j) O[j] = mma16p(pp, u_l0[j], u_hh[j], O[j]);
          if constexpr (kProdEpi) {
            // the O rows go to the producers' epilogue, over the elements of V this lane
            // read above (no other lane touches them)
#pragma unroll
            for (int j = 0; j < kCT; ++j)
#pragma unroll
              for (int s = 0; s < 4; ++s) K.V[4 * lq + s][col + 16 * j] = O[j][s];
          } else {
            float ss[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) ss[s] = row_sum16(O[0][s] * O[0][s]);
            if (lm == 0)
              *reinterpret_cast<float4*>(&sm.ss[cw][4 * lq]) = make_float4(ss[0], ss[1], ss[2], ss[3]);
          }
        }

      }
      lds_barrier();

      // ---------------------------------------------------------- interval 3
      if (!kProdEpi && i >= 1 && write_out) emit(i - 1, Oprev);
      if (i >= 0) {
        update_state(K);
      }
      lds_barrier();
      Oprev = O[0];
    }
    if (!kProdEpi && nch > 0 && write_out) emit(nch - 1, Oprev);

    float* dst = nullptr;
    if (a.pass == kPassTransfer) {
      // (segment 0 needs no M, and its M plane holds the Transfer pass's copy of the ring)
      if (!(mstate && kseg == 0)) dst = (mstate ? a.seg_m : a.seg_b) + sgbase;
    } else if (last_seg && a.state_out) {
      dst = a.state_out + nbase;
    }
    if (dst) {
      float* sp = dst + opaque(4 * lq * kHeadDim + col);
#pragma unroll
      for (int j = 0; j < kCT; ++j)
#pragma unroll
        for (int it = 0; it < 8; ++it)
#pragma unroll
          for (int s = 0; s < 4; ++s) sp[(16 * it + s) * kHeadDim + 16 * j] = S[j][it][s];
    }
  }
}

}  // namespace

// The kernel variant for the layer's decay gate (low-rank or full-rank pre-activation,
// bounded or softplus gate) and the pass (Transfer, or one with outputs).
using PcKernel = void (*)(PrefillArgs, PcOrder, SplitPlan);
template <bool kXfer>
static PcKernel pc_kernel_for(const PrefillArgs& a) {
  const bool sp = a.L.gate_kind == KDA_GATE_SOFTPLUS;
  if (a.L.f_b) return sp ? prefill_pc_kernel<true, true, kXfer> : prefill_pc_kernel<true, false, kXfer>;
  return sp ? prefill_pc_kernel<false, true, kXfer> : prefill_pc_kernel<false, false, kXfer>;
}
// Threads per workgroup of the variant pc_kernel_for picks.
static unsigned pc_threads(const PrefillArgs& a, bool xfer) {
  const bool sp = a.L.gate_kind == KDA_GATE_SOFTPLUS, fb = a.L.f_b != nullptr;
  if (sp || fb) return static_cast<unsigned>(PcShape<true, true>::kNt);
  return static_cast<unsigned>(xfer ? PcShape<false, false, true>::kNt : PcShape<false, false>::kNt);
}
// Whether the Transfer pass forms B and M in one workgroup (kMerged) for this layer.
static bool pc_merged(const PrefillArgs& a) {
  return a.L.gate_kind != KDA_GATE_SOFTPLUS && a.L.f_b == nullptr;
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, const int32_t* order_host, hipStream_t stream) {
  PcOrder ord;
  const int nord = a.num_seqs < kMaxOrdered ? a.num_seqs : kMaxOrdered;
  for (int i = 0; i < kMaxOrdered; ++i) ord.idx[i] = i < nord ? order_host[i] : 0;
  SplitPlan none{};
  PrefillArgs w = a;
  w.pass = kPassWhole;
  const dim3 grid(static_cast<unsigned>(a.num_seqs) * static_cast<unsigned>(a.L.H));
  hipLaunchKernelGGL(pc_kernel_for<false>(a), grid, dim3(pc_threads(a, false)), 0, stream, w, ord, none);
  return hipGetLastError();
}

namespace {

// S_{k+1} = M_k S_k + B_k over the segments of each sequence, for one 16-column block of
// one head's state (value columns never mix, so the blocks are independent).  S_1 = B_0:
// segment 0 started from the true state.  The products run on fp32 MFMA (16x16x4): wave w
// forms rows 32w .. 32w + 31 of the block as two 16-row tiles, and lane (lm, lq) feeds
// M[row lm][32 lq + kk] and S[32 lq + kk][column lm] at step kk = 0..31, so the 128-long
// contraction runs as four contiguous quarters, one per lane group; a lane's quarter-rows
// of M and its entries of B are loaded one step ahead.  S_k sits in LDS.
__global__ __launch_bounds__(256, 1) void combine_kernel(PrefillArgs a, SplitPlan plan) {
  constexpr int CB = 16;
  constexpr int SP = CB + 1;  // padded LDS row
  __shared__ float sblk[kHeadDim][SP];
  const int H = a.L.H;
  constexpr int nb = kHeadDim / CB;
  // The eight column blocks of a (sequence, head) go to one XCD (workgroups are dealt
  // round-robin over the 8 XCDs), so that M_k comes from HBM once per unit and from that
  // XCD's L2 for the other seven blocks.
  int unit, cb;
  const int nunits = static_cast<int>(gridDim.x) / nb;
  if (nunits % 8 == 0) {
    const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    unit = (slot / nb) * 8 + xcd;
    cb = slot % nb;
  } else {
    unit = blockIdx.x / nb;
    cb = blockIdx.x - unit * nb;
  }
  const int n = unit / H;
  const int h = unit - n * H;
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63, lm = lane & 15, lq = lane >> 4;
  const int first = plan.first[n], nsegs = plan.first[n + 1] - plan.first[n];
  if (nsegs < 2) return;
  constexpr int64_t kDD = kHeadDim * kHeadDim;
  auto plane = [&](float* base, int k) { return base + ((static_cast<int64_t>(first + k)) * H + h) * kDD; };
  // this lane's output rows: 32 wave + 16 tile + 4 lq + s, column cb * 16 + lm
  auto row_of = [&](int tile, int s) { return 32 * wave + 16 * tile + 4 * lq + s; };
  const int col = cb * CB + lm;
  // S_1 = B_0
  {
    const float* b0 = plane(a.seg_b, 0) + col;
    float* s1 = plane(a.seg_start, 1) + col;
    float v[2][4];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile)
#pragma unroll
      for (int s = 0; s < 4; ++s) v[tile][s] = b0[row_of(tile, s) * kHeadDim];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        s1[row_of(tile, s) * kHeadDim] = v[tile][s];
        sblk[row_of(tile, s)][lm] = v[tile][s];
      }
  }
  // M_k's quarter-rows of this lane: rows 32 wave + 16 tile + lm, columns 32 lq .. + 31
  float4 mq[2][8];
  auto load_m = [&](int k) __attribute__((always_inline)) {
    const float* m = plane(a.seg_m, k) + 32 * lq;
#pragma unroll
    for (int tile = 0; tile < 2; ++tile)
#pragma unroll
      for (int q = 0; q < 8; ++q)
        mq[tile][q] = *reinterpret_cast<const float4*>(m + (32 * wave + 16 * tile + lm) * kHeadDim + 4 * q);
  };
  // B_k at this lane's output entries, also one step ahead
  float bv[2][4];
  auto load_b = [&](int k) __attribute__((always_inline)) {
    const float* bk = plane(a.seg_b, k) + col;
#pragma unroll
    for (int tile = 0; tile < 2; ++tile)
#pragma unroll
      for (int s = 0; s < 4; ++s) bv[tile][s] = bk[row_of(tile, s) * kHeadDim];
  };
  if (nsegs > 2) {
    load_m(1);
    load_b(1);
  }
  for (int k = 1; k + 1 < nsegs; ++k) {
    __syncthreads();
    // all 32 B operands from LDS first (one LDS round trip), then the MFMA chain
    float bs[32];
#pragma unroll
    for (int kk = 0; kk < 32; ++kk) bs[kk] = sblk[32 * lq + kk][lm];
    __builtin_amdgcn_sched_barrier(0);
    f32x4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc[0] = mma4(mq[0][q][u], bs[4 * q + u], acc[0]);
        acc[1] = mma4(mq[1][q][u], bs[4 * q + u], acc[1]);
      }
    }
#pragma unroll
    for (int tile = 0; tile < 2; ++tile)
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[tile][s] += bv[tile][s];
    if (k + 2 < nsegs) {
      load_m(k + 1);
      load_b(k + 1);
    }
    __syncthreads();
    float* snext = plane(a.seg_start, k + 1) + col;
#pragma unroll
    for (int tile = 0; tile < 2; ++tile)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sblk[row_of(tile, s)][lm] = acc[tile][s];
        snext[row_of(tile, s) * kHeadDim] = acc[tile][s];
      }
  }
}

}  // namespace

hipError_t launch_prefill_bf16_split(const PrefillArgs& a, const SplitPlan& plan, hipStream_t stream) {
  PcOrder none{};
  const unsigned H = static_cast<unsigned>(a.L.H);
  PrefillArgs w = a;
  w.pass = kPassTransfer;
  const unsigned halves = pc_merged(a) ? 1u : 2u;  // B and M in one workgroup, or in two
  hipLaunchKernelGGL(pc_kernel_for<true>(a), dim3(halves * plan.nseg * H), dim3(pc_threads(a, true)), 0, stream, w,
                     none, plan);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(static_cast<unsigned>(a.num_seqs) * H * (kHeadDim / 16)),
                     dim3(256), 0, stream, w, plan);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  w.pass = kPassFinal;
  hipLaunchKernelGGL(pc_kernel_for<false>(a), dim3(plan.nseg * H), dim3(pc_threads(a, false)), 0, stream, w, none,
                     plan);
  return hipGetLastError();
}

}  // namespace kda
