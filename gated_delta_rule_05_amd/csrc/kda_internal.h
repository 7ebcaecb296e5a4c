// Internal interface between the C ABI layer (kda_api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/kda.h"

namespace kda {

constexpr int kHeadDimHost = 128;

struct LayerParams {
  int32_t H;
  float lower_bound, l2_eps, rms_eps;
  const float* conv_w;
  const float* dt_bias;
  const float* A_log;
  const float* norm_w;
};

// Decode of up to `tokens` consecutive tokens per sequence (one token: the decode step).
// Activations are [batch][tokens][...]; ntok (device, or null for all) gives each
// sequence's count.  state_out / ring_out may equal state_in / ring_in; out may be null.
struct DecodeArgs {
  LayerParams L;
  int32_t batch;
  int32_t tokens;
  const int32_t* ntok;
  const void *q, *k, *v, *z, *beta, *gate;
  const float* state_in;
  const float* ring_in;
  float* state_out;
  float* ring_out;
  void* out;
};

// Longest-first order of the sequences for the prefill grid, passed by value.
constexpr int kMaxOrdered = 512;

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
};

hipError_t launch_decode(const DecodeArgs& a, kda_dtype io, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, kda_dtype io, const int32_t* order_host,
                          hipStream_t stream);
// bf16 io: the producer/consumer kernel of kda_prefill_pc.hip
hipError_t launch_prefill_bf16(const PrefillArgs& a, const int32_t* order_host, hipStream_t stream);

}  // namespace kda
