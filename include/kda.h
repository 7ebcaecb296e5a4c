/*
 * kda.h -- C ABI of libkda.so, the MI355X (gfx950) Kimi Delta Attention (KDA) mixer core.
 *
 * The library takes one layer's already-projected activations and runs, per (sequence,
 * head): the short causal depthwise conv (kernel 4, no bias) with SiLU on q, k and v;
 * L2 normalisation of q and k (eps l2_eps) and the head_dim^-1/2 scale on q; the
 * lower-bounded per-channel log decay g = lower_bound * sigmoid(exp(A_log) * (z + dt_bias));
 * beta = sigmoid(raw beta); the gated delta-rule recurrence; and the sigmoid-gated RMSNorm
 * on the output.  Sources, by page and section:
 *   - docs.rs "ferrox_models::kda" module page: conv (depthwise causal Conv1d, padding
 *     kernel_size-1, no bias), q/k L2 norm with eps 1e-6 then q * head_dim^-1/2, the
 *     per-channel gate and the sigmoid output gate;
 *   - "Kimi Delta Attention (KDA) -- analysis & C kernel plan", sections "The KDA layer,
 *     precisely" and "Recurrence": S' = Diag(exp(g_t)) S_{t-1};
 *     S_t = S' + beta_t k_t (v_t - S'^T k_t)^T; o_t = S_t^T q_t;
 *   - OpenModelAtlas "Kimi K3 - Retention gate": formula and gate.py excerpt for g;
 *     "Why": lower bound -5 keeps a 16-token tile's rescale below e^80;
 *   - docs.rs "memra_engine::kda": fused conv weights and ring (plane offset
 *     plane * H * d), token-major channel c = h * d + i, head_dim 128 only, stateless /
 *     stateful prefill and the T = 1 decode step.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is device memory owned by the caller, unless named *_host.
 *     The library allocates nothing, keeps no pointer after returning, and never
 *     synchronises: work is enqueued on `stream` and completes asynchronously.
 *   - Errors are reported by status code only, and arguments are checked before any
 *     work is enqueued: on a non-OK return nothing has been written.  Faults inside a
 *     kernel surface at the caller's next synchronisation.  kda_last_error() returns a
 *     thread-local description of the last failure.
 *   - Activations are token-major: q, k, v, z (decay pre-activation) and gate (output
 *     gate pre-activation) are [T][H * d] with channel c = h * d + i; raw beta is [T][H].
 *     They are all of the io dtype; out has the io dtype and the [T][H * d] layout.
 *   - The recurrent state is fp32 [N][H][d_k = d][d_v = d], row-major with the key index
 *     (the decayed axis) first.
 *   - The conv ring is fp32 [N][3 * H * d][kernel - 1]: planes q, k, v (plane offset
 *     plane * H * d), then channel, then taps oldest first; it holds the most recent
 *     kernel - 1 raw (pre-conv) inputs of each channel.
 *   - conv_w is fp32 [3 * H * d][kernel], same plane order; tap kernel - 1 multiplies the
 *     current token, tap 0 the oldest.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 5

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARG = 1, /* null or misaligned pointer, bad size, inconsistent cu_seqlens */
  KDA_ERR_UNSUPPORTED = 2, /* head_dim != 128, conv kernel != 4, chunked lower bound below -5 */
  KDA_ERR_WORKSPACE = 3,   /* workspace NULL with a nonzero size, or not 256-byte aligned */
  KDA_ERR_HIP = 4          /* the HIP runtime refused a launch */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* Decay-gate formula. */
typedef enum {
  /* g = lower_bound * sigmoid(exp(A_log) * (z + dt_bias)) (OpenModelAtlas "Kimi K3 -
     Retention gate", gate.py; Kimi K3) */
  KDA_GATE_BOUNDED = 0,
  /* g = -exp(A_log) * softplus(z + dt_bias), unbounded (Kimi-Linear, per the analysis
     page's status note); lower_bound is ignored.  Without the bound a chunk's decay range
     is unbounded; the bf16 chunked prefill forms every intra-chunk pair against a boundary
     row between its two rows (two MFMA levels, position pairs on the 4x4 diagonal blocks;
     OpenModelAtlas "Kimi K3 - Retention gate", "Why"), also together with the low-rank
     gate (f_b).  With fp32 io, kda_prefill runs the sequential scan for it. */
  KDA_GATE_SOFTPLUS = 1
} kda_gate_kind;

/*
 * One layer's shape and parameters (device pointers, fp32):
 *   conv_w  [3 * H * d][conv_kernel]   fused short-conv weights, planes q, k, v
 *   dt_bias [H * d]                    added to z before the gate
 *   A_log   [H]                        per-head log scale of the gate
 *   norm_w  [d]                        gated-RMSNorm weight, shared by all heads
 * lower_bound is the gate's lower bound (-5 in the pages' models); l2_eps the q/k L2
 * epsilon (1e-6); rms_eps the output RMSNorm epsilon; gate_kind selects the decay-gate
 * formula (kda_gate_kind).
 *
 * f_b selects the low-rank decay gate ("Kimi Delta Attention (KDA) -- analysis & C kernel
 * plan", "The KDA layer, precisely", fact 2: hidden -> head_dim -> H * head_dim; the
 * Retention-gate page: g = f_b_proj(f_a_proj(hidden)), a 7,168 -> 128 -> 12,288 pair).
 * NULL: the z argument of every entry point is the full pre-activation [rows][H * d].
 * Otherwise f_b is the second projection's weight, [H * d][d] row-major in the io dtype
 * (device memory, 16-byte aligned, owned by the caller), the z argument is the rank-d
 * input z_low [rows][d] (io dtype), and the pre-activation of channel c is
 * sum_r z_low[row][r] * f_b[c][r], accumulated in fp32.  The full-rank z plane then never
 * passes through memory.  With fp32 io, kda_prefill runs the sequential scan for it.
 */
typedef struct kda_layer {
  int32_t num_heads;
  int32_t head_dim;    /* must be 128 */
  int32_t conv_kernel; /* must be 4 */
  float lower_bound;
  float l2_eps;
  float rms_eps;
  const float* conv_w;
  const float* dt_bias;
  const float* A_log;
  const float* norm_w;
  int32_t gate_kind;   /* kda_gate_kind */
  const void* f_b;     /* NULL, or the low-rank gate's [H * d][d] weight (io dtype) */
} kda_layer;

/*
 * Bytes of device workspace with which kda_prefill() takes its fastest path for this
 * problem (0 when that path needs none).  With few (sequence, head) units -- bf16 io,
 * fewer than 96 of them, at most 64 sequences -- the fastest path cuts the sequences into
 * segments that run in parallel (the state recurrence is affine in its start state); the
 * workspace then holds three fp32 states per (segment, head).  Returns 0 also for invalid
 * arguments (kda_prefill reports those).
 */
size_t kda_prefill_workspace_bytes(const kda_layer* layer, kda_dtype io, int32_t num_seqs,
                                   const int32_t* cu_seqlens_host, int64_t total_tokens);

/*
 * Chunked prefill over num_seqs packed sequences (stateless when state_in / ring_in are
 * NULL, stateful otherwise; memra_engine::kda kda_attn / kda_attn_prime).
 *   cu_seqlens_dev / cu_seqlens_host  int32 [num_seqs + 1], the same offsets in device and
 *       host memory, non-decreasing, starting at 0 and ending at total_tokens.  Empty
 *       sequences are allowed (their state and ring pass through unchanged).
 *   q, k, v, z, gate  [total_tokens][H * d] io (z: [total_tokens][d] with layer->f_b);
 *                     beta [total_tokens][H] io (raw, pre-sigmoid)
 *   state_in  fp32 [num_seqs][H][d][d] or NULL (zero initial state)
 *   ring_in   fp32 [num_seqs][3 * H * d][kernel - 1] or NULL (zero history)
 *   out       [total_tokens][H * d] io
 *   state_out fp32 [num_seqs][H][d][d] or NULL (not written); may equal state_in
 *   ring_out  fp32 [num_seqs][3 * H * d][kernel - 1] or NULL; may equal ring_in
 *   workspace device buffer, 256-byte aligned, or NULL with workspace_bytes = 0.  With at
 *             least kda_prefill_workspace_bytes() bytes the segment-parallel path may run;
 *             with less, the whole-sequence path runs (same results up to rounding).  The
 *             library keeps nothing in it after the call's work completes.
 * Partial overlap between inputs and outputs is invalid.  State pointers and q, k, v, z,
 * gate and out must be 16-byte aligned (the kernels move activation rows in 16-byte
 * pieces).
 * Range (bf16 io): the state pass multiplies fp16 operands, so every state entry (start,
 * intermediate and final) and log2(e) times every SiLU conv output of q and k must stay
 * below 65504 in magnitude -- about 45,000 for the conv outputs themselves.  Past that
 * the outputs and the final state are not finite (inf or NaN, never finite wrong
 * values); nothing is checked on the host.  State entries are bounded by about
 * sqrt(d) * max |v| plus the start state's, since the keys are unit vectors and beta <= 1.
 * fp32 io and the decode entry points compute in fp32 throughout and have fp32's range.
 */
kda_status kda_prefill(const kda_layer* layer, kda_dtype io, int32_t num_seqs,
                       const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                       int64_t total_tokens, const void* q, const void* k, const void* v,
                       const void* z, const void* beta, const void* gate, const float* state_in,
                       const float* ring_in, void* out, float* state_out, float* ring_out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_prefill for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments, checks
 * and results as kda_prefill, without the workspace: when the segment-parallel path
 * applies, its per-segment states live in a device array the library holds, of
 * KDA_NOALLOC_SCRATCH_BYTES per GPU (allocated when the library's code is loaded on that
 * GPU, kept until the process ends; every plan of the path fits in it, and a plan that
 * would need more -- none does -- returns KDA_ERR_WORKSPACE with nothing written).
 * Results are bit-identical to kda_prefill given a large enough workspace.  The call
 * makes no device allocation; its first call on each GPU looks up that GPU's array
 * (hipGetSymbolAddress), which must not happen during graph capture, so make one
 * call per GPU before capturing.  All calls on one GPU share its array: calls that
 * overlap on one GPU (concurrent streams, or host threads) race and must be serialised
 * by the caller.  The stream's device is the GPU used.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)
kda_status kda_prefill_noalloc(const kda_layer* layer, kda_dtype io, int32_t num_seqs,
                               const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                               int64_t total_tokens, const void* q, const void* k, const void* v,
                               const void* z, const void* beta, const void* gate,
                               const float* state_in, const float* ring_in, void* out,
                               float* state_out, float* ring_out, hipStream_t stream);

/*
 * Sequential-scan prefill: the same packed problem and buffers as kda_prefill (no
 * workspace), run token by token by the decode kernel over register-resident state
 * (memra_engine::kda's prefill arrangement, memra_kda_scan_s128, which serves prefill and
 * decode alike).  An A/B comparator for the chunked path (which measures faster on this
 * hardware even for 64-token prompts), and the path kda_prefill takes for fp32 io with the
 * softplus or the low-rank gate.  Each sequence's outputs, final state and ring are
 * bit-identical to running its tokens through kda_decode_step one at a time.  Any
 * lower_bound <= 0 is accepted (there
 * is no tile bound).  state_in / ring_in may be NULL (zeros), state_out / ring_out NULL
 * (not written); state_out may equal state_in and ring_out ring_in.
 */
kda_status kda_prefill_scan(const kda_layer* layer, kda_dtype io, int32_t num_seqs,
                            const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                            int64_t total_tokens, const void* q, const void* k, const void* v,
                            const void* z, const void* beta, const void* gate,
                            const float* state_in, const float* ring_in, void* out,
                            float* state_out, float* ring_out, hipStream_t stream);

/*
 * One decode token for each of `batch` sequences (memra_engine::kda kda_attn_decode: the
 * same math as a one-token prime).  q, k, v, z, gate [batch][H * d] io; beta [batch][H] io.
 * state fp32 [batch][H][d][d] and ring fp32 [batch][3 * H * d][kernel - 1] are read and
 * updated in place (the ring shifts by one token).  out [batch][H * d] io.  batch = 0 is a
 * no-op.  state must be 16-byte aligned.  Runs the kernel of kda_decode_multi with one row.
 */
kda_status kda_decode_step(const kda_layer* layer, kda_dtype io, int32_t batch, const void* q,
                           const void* k, const void* v, const void* z, const void* beta,
                           const void* gate, float* state, float* ring, void* out,
                           hipStream_t stream);

/*
 * Several consecutive decode tokens per sequence in one launch: the batched verify of
 * speculative decoding, and its rollback by replay (docs.rs "memra_engine::kda":
 * kda_verify_rows_cached runs t = K + 1 rows of every sequence with the recurrence
 * sequential inside one launch over register-resident state; kda_verify_rollback_rows and
 * kda_scan_replay rebuild the state after the first `keep` rows by replaying the same
 * launch from the pre-round state).
 *   tokens     rows per sequence, >= 0; activations are [batch][tokens][H * d] io (row
 *              b * tokens + s), beta [batch][tokens][H] io.
 *   ntok_dev   int32 [batch] device, the number of rows to run for each sequence (values
 *              are clamped to [0, tokens]); NULL runs all `tokens` rows.
 *   state_in / ring_in    fp32 [batch][H][d][d] / [batch][3 * H * d][kernel - 1]: the state
 *              and conv history before the first row (read only).
 *   state_out / ring_out  the same shapes: after the sequence's last row run.  They may
 *              equal state_in / ring_in (in place); partial overlap is invalid.
 *   out        [batch][tokens][H * d] io, or NULL to skip the outputs (a replay); rows at or
 *              past a sequence's count are not written.
 * Each row's arithmetic is the same instruction sequence a one-token launch executes, so
 * the outputs and final states are bit-identical to chaining one-token steps; that is what
 * makes rollback exact: keep the pre-round buffers (ping-pong: state_out != state_in), run
 * all rows, and if sequence b accepts only keep[b] rows, call again from the pre-round
 * buffers with ntok = keep.  kda_decode_step is this call with tokens = 1.  batch = 0 is a
 * no-op; a sequence with 0 rows copies its state and ring through.  state buffers must be
 * 16-byte aligned.
 */
kda_status kda_decode_multi(const kda_layer* layer, kda_dtype io, int32_t batch, int32_t tokens,
                            const int32_t* ntok_dev, const void* q, const void* k, const void* v,
                            const void* z, const void* beta, const void* gate,
                            const float* state_in, const float* ring_in, float* state_out,
                            float* ring_out, void* out, hipStream_t stream);

/* Short name of a status code. */
const char* kda_status_string(kda_status status);

/* Thread-local description of the calling thread's last non-OK status ("" if none). */
const char* kda_last_error(void);

/* KDA_ABI_VERSION of the loaded library. */
int32_t kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
