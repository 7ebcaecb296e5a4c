// Internal interface between the C ABI layer (kda_api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/kda.h"

namespace kda {

constexpr int kHeadDimHost = 128;

struct LayerParams {
  int32_t H;
  int32_t gate_kind;  // KDA_GATE_BOUNDED or KDA_GATE_SOFTPLUS
  float lower_bound, l2_eps, rms_eps;
  const float* conv_w;
  const float* dt_bias;
  const float* A_log;
  const float* norm_w;
  const void* f_b;    // low-rank decay gate: [H d][d] io, or null (z is full rank)
};

// Decode of up to `tokens` consecutive tokens per sequence (one token: the decode step).
// Activations are [batch][tokens][...]; ntok (device, or null for all) gives each
// sequence's count.  With cu (device, [batch + 1]) the rows are packed instead: sequence b
// has rows cu[b] .. cu[b + 1] - 1 (the sequential-scan prefill).  state_out / ring_out may
// equal state_in / ring_in; a null state_in / ring_in starts from zeros, a null state_out /
// ring_out / out is not written.
struct DecodeArgs {
  LayerParams L;
  int32_t batch;
  int32_t tokens;
  const int32_t* ntok;
  const int32_t* cu;
  const void *q, *k, *v, *z, *beta, *gate;
  const float* state_in;
  const float* ring_in;
  float* state_out;
  float* ring_out;
  void* out;
};

// Longest-first order of the sequences for the prefill grid, passed by value.
constexpr int kMaxOrdered = 512;

// Prefill passes.  Whole: one workgroup per (sequence, head).  With few (sequence, head)
// units the sequences are cut into segments that run in parallel, using that the state
// recurrence is affine in its start state, S_end = M S_start + B:
//   Transfer: for every segment but a sequence's last, B (from a zero start; the first
//             segment from the true start) and M (from the identity start with v = 0),
//             no outputs;
//   Final:    every segment from its true start state (segment 0: the sequence's, later
//             ones: S_{k+1} = M_k S_k + B_k, formed in between), with outputs; the last
//             segment writes the final state and ring.
enum : int32_t { kPassWhole = 0, kPassTransfer = 1, kPassFinal = 2 };

struct PrefillArgs {
  LayerParams L;
  int32_t num_seqs;
  const int32_t* cu_seqlens;
  const void *q, *k, *v, *z, *beta, *gate;
  const float* state_in;
  const float* ring_in;
  void* out;
  float* state_out;
  float* ring_out;
  int32_t pass;
  float* seg_b;            // [segments][H][d][d]
  float* seg_m;            // [segments][H][d][d]
  float* seg_start;        // [segments][H][d][d]
};

// Segment k of sequence n covers tokens [cu[n] + k L, min(cu[n + 1], cu[n] + (k + 1) L)).
constexpr int kMaxSplitSeqs = 64;
struct SplitPlan {
  int32_t seg_len;                   // L, a multiple of the 16-token chunk
  int32_t nseg;                      // segments in total
  int32_t first[kMaxSplitSeqs + 1];  // first segment of each sequence; first[N] = nseg
};

// The scratch array of kda_prefill_noalloc: the largest workspace any segment-parallel
// plan needs (3 states of 64 KiB for at most 340 (segment, head) pairs, since the plan
// only applies below 96 (sequence, head) units and cuts each into ceil(256 / units)
// segments at most), rounded up.
constexpr size_t kNoAllocScratchBytes = size_t{64} << 20;
static_assert(kNoAllocScratchBytes == KDA_NOALLOC_SCRATCH_BYTES, "the header's figure");
// Device address of the calling stream's GPU's copy of that array (looked up once per device).
hipError_t noalloc_scratch(hipStream_t stream, void** ptr);

hipError_t launch_decode(const DecodeArgs& a, kda_dtype io, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, kda_dtype io, const int32_t* order_host,
                          hipStream_t stream);
// bf16 io: the producer/consumer kernel of kda_prefill_pc.hip
hipError_t launch_prefill_bf16(const PrefillArgs& a, const int32_t* order_host, hipStream_t stream);
// bf16 io, split into segments: Transfer pass, combine, Final pass (a.seg_* set)
hipError_t launch_prefill_bf16_split(const PrefillArgs& a, const SplitPlan& plan, hipStream_t stream);

}  // namespace kda
