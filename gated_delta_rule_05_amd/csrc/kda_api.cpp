// C ABI of libkda.so: argument validation, then one launch per call on the caller's
// stream.  Nothing here allocates device memory or synchronises.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "kda_internal.h"

namespace {

thread_local std::string g_last_error;

kda_status fail(kda_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

kda_status ok() {
  g_last_error.clear();
  return KDA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

kda_status check_layer(const kda_layer* L, bool chunked) {
  if (!L) return fail(KDA_ERR_INVALID_ARG, "layer is NULL");
  if (L->num_heads <= 0) return fail(KDA_ERR_INVALID_ARG, "num_heads must be positive");
  if (L->head_dim != kda::kHeadDimHost)
    return fail(KDA_ERR_UNSUPPORTED, "head_dim %d is not supported (only 128)", L->head_dim);
  if (L->conv_kernel != 4)
    return fail(KDA_ERR_UNSUPPORTED, "conv_kernel %d is not supported (only 4)", L->conv_kernel);
  if (!L->conv_w || !L->dt_bias || !L->A_log || !L->norm_w)
    return fail(KDA_ERR_INVALID_ARG, "a layer parameter pointer is NULL");
  if (!(L->l2_eps >= 0.f) || !(L->rms_eps >= 0.f) || !std::isfinite(L->l2_eps) ||
      !std::isfinite(L->rms_eps))
    return fail(KDA_ERR_INVALID_ARG, "epsilons must be finite and non-negative");
  if (L->gate_kind != KDA_GATE_BOUNDED && L->gate_kind != KDA_GATE_SOFTPLUS)
    return fail(KDA_ERR_INVALID_ARG, "unknown gate_kind %d", L->gate_kind);
  if (L->f_b && !aligned16(L->f_b)) return fail(KDA_ERR_INVALID_ARG, "f_b must be 16-byte aligned");
  if (L->gate_kind == KDA_GATE_SOFTPLUS) return KDA_OK;  // lower_bound unused
  if (!std::isfinite(L->lower_bound) || L->lower_bound > 0.f)
    return fail(KDA_ERR_INVALID_ARG, "lower_bound must be finite and <= 0");
  // The chunked kernel forms exp(+-Gcum) over 16-token tiles from a mid-tile reference:
  // with g >= -5 every factor stays within e^(+-40), far inside fp32 and bf16 range.
  if (chunked && L->lower_bound < -5.f)
    return fail(KDA_ERR_UNSUPPORTED, "prefill needs lower_bound >= -5 (16-token tile bound)");
  return KDA_OK;
}

kda::LayerParams layer_params(const kda_layer* L) {
  kda::LayerParams p;
  p.H = L->num_heads;
  p.gate_kind = L->gate_kind;
  p.lower_bound = L->lower_bound;
  p.l2_eps = L->l2_eps;
  p.rms_eps = L->rms_eps;
  p.conv_w = L->conv_w;
  p.dt_bias = L->dt_bias;
  p.A_log = L->A_log;
  p.norm_w = L->norm_w;
  p.f_b = L->f_b;
  return p;
}

bool io_ok(kda_dtype io) { return io == KDA_F32 || io == KDA_BF16; }

// Packed varlen inputs of the prefill entry points (num_seqs > 0).
kda_status check_packed(int32_t num_seqs, const int32_t* cu_dev, const int32_t* cu_host,
                        int64_t total_tokens, const void* q, const void* k, const void* v,
                        const void* z, const void* beta, const void* gate, const void* out,
                        const float* state_in, const float* state_out) {
  if (!cu_dev || !cu_host)
    return fail(KDA_ERR_INVALID_ARG, "cu_seqlens (device and host copies) are required");
  if (cu_host[0] != 0) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens[0] must be 0");
  for (int32_t n = 0; n < num_seqs; ++n)
    if (cu_host[n + 1] < cu_host[n])
      return fail(KDA_ERR_INVALID_ARG, "cu_seqlens must be non-decreasing (at %d)", n);
  if (static_cast<int64_t>(cu_host[num_seqs]) != total_tokens)
    return fail(KDA_ERR_INVALID_ARG, "cu_seqlens[num_seqs] = %d != total_tokens = %lld",
                cu_host[num_seqs], static_cast<long long>(total_tokens));
  if (total_tokens > 0 && (!q || !k || !v || !z || !beta || !gate || !out))
    return fail(KDA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if ((state_in && !aligned16(state_in)) || (state_out && !aligned16(state_out)))
    return fail(KDA_ERR_INVALID_ARG, "state buffers must be 16-byte aligned");
  if (total_tokens > 0 && (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(z) ||
                           !aligned16(gate) || !aligned16(out)))
    return fail(KDA_ERR_INVALID_ARG, "q, k, v, z, gate and out must be 16-byte aligned");
  return KDA_OK;
}

// Splitting sequences into segments pays when there are too few (sequence, head) units to
// fill the chip's 256 compute units: each sequence is cut into about 256 / units segments
// of at least 256 tokens (a multiple of the 16-token chunk), and the three passes then run
// about 3 segment-times instead of one sequence-time.
constexpr int64_t kSplitMaxUnits = 96;
constexpr int32_t kSplitMinSeg = 256;
constexpr int32_t kSplitTarget = 256;

bool make_split_plan(const kda_layer* L, kda_dtype io, int32_t N, const int32_t* cu,
                     kda::SplitPlan* plan, size_t* bytes) {
  *bytes = 0;
  if (io != KDA_BF16 || N <= 0 || N > kda::kMaxSplitSeqs || !L || L->num_heads <= 0) return false;
  const int64_t units = static_cast<int64_t>(N) * L->num_heads;
  if (units >= kSplitMaxUnits) return false;
  int32_t tmax = 0;
  for (int32_t n = 0; n < N; ++n) tmax = std::max(tmax, cu[n + 1] - cu[n]);
  const int64_t kwant = (kSplitTarget + units - 1) / units;
  int64_t seg = (tmax + kwant - 1) / kwant;
  seg = std::max<int64_t>(kSplitMinSeg, (seg + 15) / 16 * 16);
  if (seg >= tmax) return false;  // nothing would be split
  plan->seg_len = static_cast<int32_t>(seg);
  int32_t total = 0;
  for (int32_t n = 0; n < N; ++n) {
    plan->first[n] = total;
    const int32_t len = cu[n + 1] - cu[n];
    total += std::max<int32_t>(1, static_cast<int32_t>((len + seg - 1) / seg));
  }
  plan->first[N] = total;
  plan->nseg = total;
  *bytes = 3ull * static_cast<size_t>(total) * static_cast<size_t>(L->num_heads) *
           kda::kHeadDimHost * kda::kHeadDimHost * sizeof(float);
  return true;
}

// kda_prefill and kda_prefill_noalloc: the same checks and launches; they differ only in
// where the segment-parallel path's workspace comes from (the caller's buffer, or the
// library's scratch array).  No device memory is allocated, and on success no host heap
// memory either (the launch order lives on the stack).
kda_status prefill_impl(const kda_layer* layer, kda_dtype io, int32_t num_seqs,
                        const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                        int64_t total_tokens, const void* q, const void* k, const void* v,
                        const void* z, const void* beta, const void* gate, const float* state_in,
                        const float* ring_in, void* out, float* state_out, float* ring_out,
                        void* workspace, size_t workspace_bytes, bool noalloc, hipStream_t stream) {
  kda_status st = check_layer(layer, true);
  if (st != KDA_OK) return st;
  if (!io_ok(io)) return fail(KDA_ERR_INVALID_ARG, "unknown io dtype %d", static_cast<int>(io));
  if (num_seqs < 0) return fail(KDA_ERR_INVALID_ARG, "num_seqs must be >= 0");
  if (num_seqs == 0) {
    if (total_tokens != 0) return fail(KDA_ERR_INVALID_ARG, "no sequences but total_tokens != 0");
    return ok();
  }
  st = check_packed(num_seqs, cu_seqlens_dev, cu_seqlens_host, total_tokens, q, k, v, z, beta,
                    gate, out, state_in, state_out);
  if (st != KDA_OK) return st;
  if (workspace_bytes > 0 && !workspace)
    return fail(KDA_ERR_WORKSPACE, "workspace is NULL but workspace_bytes = %zu", workspace_bytes);
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return fail(KDA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (static_cast<int64_t>(num_seqs) * layer->num_heads > 0x7fffffffLL)
    return fail(KDA_ERR_INVALID_ARG, "num_seqs * num_heads exceeds the grid limit");

  kda::PrefillArgs a;
  a.L = layer_params(layer);
  a.num_seqs = num_seqs;
  a.cu_seqlens = cu_seqlens_dev;
  a.q = q; a.k = k; a.v = v; a.z = z; a.beta = beta; a.gate = gate;
  a.state_in = state_in;
  a.ring_in = ring_in;
  a.out = out;
  a.state_out = state_out;
  a.ring_out = ring_out;
  // The fp32-io chunked kernel has neither the softplus gate nor the low-rank gate: with
  // either, fp32 io runs the scan.
  if (io == KDA_F32 && (layer->gate_kind == KDA_GATE_SOFTPLUS || layer->f_b))
    return kda_prefill_scan(layer, io, num_seqs, cu_seqlens_dev, cu_seqlens_host, total_tokens,
                            q, k, v, z, beta, gate, state_in, ring_in, out, state_out, ring_out,
                            stream);
  a.pass = kda::kPassWhole;
  a.seg_b = a.seg_m = a.seg_start = nullptr;

  kda::SplitPlan plan;
  size_t need = 0;
  hipError_t e;
  bool split = make_split_plan(layer, io, num_seqs, cu_seqlens_host, &plan, &need);
  if (split && noalloc) {
    if (need > kda::kNoAllocScratchBytes)
      return fail(KDA_ERR_WORKSPACE, "the segment-parallel plan needs %zu bytes of scratch, more than the %zu "
                  "bytes kda_prefill_noalloc holds", need, kda::kNoAllocScratchBytes);
    e = kda::noalloc_scratch(stream, &workspace);
    if (e != hipSuccess)
      return fail(KDA_ERR_HIP, "scratch lookup failed: %s", hipGetErrorString(e));
    workspace_bytes = kda::kNoAllocScratchBytes;
  }
  split = split && workspace_bytes >= need;
  if (split) {
    const size_t plane = static_cast<size_t>(plan.nseg) * layer->num_heads * kda::kHeadDimHost *
                         kda::kHeadDimHost;
    float* ws = static_cast<float*>(workspace);
    a.seg_b = ws;
    a.seg_m = ws + plane;
    a.seg_start = ws + 2 * plane;
    e = kda::launch_prefill_bf16_split(a, plan, stream);
  } else {
    // Longest sequences first, so the long serial chains start early (the launch orders
    // at most kMaxOrdered of them; ties keep their index order).
    int32_t order[kda::kMaxOrdered];
    const int32_t nord = std::min<int32_t>(num_seqs, kda::kMaxOrdered);
    for (int32_t i = 0; i < nord; ++i) order[i] = i;
    if (num_seqs <= kda::kMaxOrdered)
      std::sort(order, order + nord, [&](int32_t x, int32_t y) {
        const int32_t lx = cu_seqlens_host[x + 1] - cu_seqlens_host[x];
        const int32_t ly = cu_seqlens_host[y + 1] - cu_seqlens_host[y];
        return lx != ly ? lx > ly : x < y;
      });
    e = kda::launch_prefill(a, io, order, stream);
  }
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int32_t kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
  }
  return "KDA_ERR_UNKNOWN";
}

const char* kda_last_error(void) { return g_last_error.c_str(); }

kda_status kda_decode_step(const kda_layer* layer, kda_dtype io, int32_t batch, const void* q,
                           const void* k, const void* v, const void* z, const void* beta,
                           const void* gate, float* state, float* ring, void* out,
                           hipStream_t stream) {
  if (!out && batch > 0) return fail(KDA_ERR_INVALID_ARG, "out is NULL");
  return kda_decode_multi(layer, io, batch, 1, nullptr, q, k, v, z, beta, gate, state, ring,
                          state, ring, out, stream);
}

kda_status kda_decode_multi(const kda_layer* layer, kda_dtype io, int32_t batch, int32_t tokens,
                            const int32_t* ntok_dev, const void* q, const void* k, const void* v,
                            const void* z, const void* beta, const void* gate,
                            const float* state_in, const float* ring_in, float* state_out,
                            float* ring_out, void* out, hipStream_t stream) {
  kda_status st = check_layer(layer, false);
  if (st != KDA_OK) return st;
  if (!io_ok(io)) return fail(KDA_ERR_INVALID_ARG, "unknown io dtype %d", static_cast<int>(io));
  if (batch < 0) return fail(KDA_ERR_INVALID_ARG, "batch must be >= 0");
  if (tokens < 0) return fail(KDA_ERR_INVALID_ARG, "tokens must be >= 0");
  if (batch == 0) return ok();
  if (!state_in || !ring_in || !state_out || !ring_out)
    return fail(KDA_ERR_INVALID_ARG, "a state or ring pointer is NULL");
  if (tokens > 0 && (!q || !k || !v || !z || !beta || !gate))
    return fail(KDA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned16(state_in) || !aligned16(state_out))
    return fail(KDA_ERR_INVALID_ARG, "state buffers must be 16-byte aligned");
  const int64_t units = static_cast<int64_t>(batch) * layer->num_heads;
  if (units > 0x7fffffffLL)
    return fail(KDA_ERR_INVALID_ARG, "batch * num_heads exceeds the grid limit");
  {
    // exact aliasing is allowed (in place); partial overlap is not
    const int64_t sbytes = units * kda::kHeadDimHost * kda::kHeadDimHost * 4;
    const int64_t rbytes = static_cast<int64_t>(batch) * 3 * layer->num_heads * kda::kHeadDimHost * 3 * 4;
    auto overlap = [](const void* a, const void* b, int64_t n) {
      const char* x = static_cast<const char*>(a);
      const char* y = static_cast<const char*>(b);
      return x != y && x < y + n && y < x + n;
    };
    if (overlap(state_in, state_out, sbytes) || overlap(ring_in, ring_out, rbytes))
      return fail(KDA_ERR_INVALID_ARG, "state or ring buffers overlap partially");
  }
  kda::DecodeArgs a;
  a.L = layer_params(layer);
  a.batch = batch;
  a.tokens = tokens;
  a.ntok = ntok_dev;
  a.cu = nullptr;
  a.q = q; a.k = k; a.v = v; a.z = z; a.beta = beta; a.gate = gate;
  a.state_in = state_in;
  a.ring_in = ring_in;
  a.state_out = state_out;
  a.ring_out = ring_out;
  a.out = out;
  hipError_t e = kda::launch_decode(a, io, stream);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t kda_prefill_workspace_bytes(const kda_layer* layer, kda_dtype io, int32_t num_seqs,
                                   const int32_t* cu_seqlens_host, int64_t total_tokens) {
  (void)total_tokens;
  if (!cu_seqlens_host || num_seqs <= 0) return 0;
  kda::SplitPlan plan;
  size_t bytes = 0;
  return make_split_plan(layer, io, num_seqs, cu_seqlens_host, &plan, &bytes) ? bytes : 0;
}

kda_status kda_prefill(const kda_layer* layer, kda_dtype io, int32_t num_seqs,
                       const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                       int64_t total_tokens, const void* q, const void* k, const void* v,
                       const void* z, const void* beta, const void* gate, const float* state_in,
                       const float* ring_in, void* out, float* state_out, float* ring_out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return prefill_impl(layer, io, num_seqs, cu_seqlens_dev, cu_seqlens_host, total_tokens, q, k, v, z,
                      beta, gate, state_in, ring_in, out, state_out, ring_out, workspace,
                      workspace_bytes, false, stream);
}

kda_status kda_prefill_noalloc(const kda_layer* layer, kda_dtype io, int32_t num_seqs,
                               const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                               int64_t total_tokens, const void* q, const void* k, const void* v,
                               const void* z, const void* beta, const void* gate,
                               const float* state_in, const float* ring_in, void* out,
                               float* state_out, float* ring_out, hipStream_t stream) {
  return prefill_impl(layer, io, num_seqs, cu_seqlens_dev, cu_seqlens_host, total_tokens, q, k, v, z,
                      beta, gate, state_in, ring_in, out, state_out, ring_out, nullptr, 0, true,
                      stream);
}

kda_status kda_prefill_scan(const kda_layer* layer, kda_dtype io, int32_t num_seqs,
                            const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                            int64_t total_tokens, const void* q, const void* k, const void* v,
                            const void* z, const void* beta, const void* gate,
                            const float* state_in, const float* ring_in, void* out,
                            float* state_out, float* ring_out, hipStream_t stream) {
  kda_status st = check_layer(layer, false);
  if (st != KDA_OK) return st;
  if (!io_ok(io)) return fail(KDA_ERR_INVALID_ARG, "unknown io dtype %d", static_cast<int>(io));
  if (num_seqs < 0) return fail(KDA_ERR_INVALID_ARG, "num_seqs must be >= 0");
  if (num_seqs == 0) {
    if (total_tokens != 0) return fail(KDA_ERR_INVALID_ARG, "no sequences but total_tokens != 0");
    return ok();
  }
  st = check_packed(num_seqs, cu_seqlens_dev, cu_seqlens_host, total_tokens, q, k, v, z, beta,
                    gate, out, state_in, state_out);
  if (st != KDA_OK) return st;
  if (static_cast<int64_t>(num_seqs) * layer->num_heads > 0x7fffffffLL)
    return fail(KDA_ERR_INVALID_ARG, "num_seqs * num_heads exceeds the grid limit");
  kda::DecodeArgs a;
  a.L = layer_params(layer);
  a.batch = num_seqs;
  a.tokens = 0;
  a.ntok = nullptr;
  a.cu = cu_seqlens_dev;
  a.q = q; a.k = k; a.v = v; a.z = z; a.beta = beta; a.gate = gate;
  a.state_in = state_in;
  a.ring_in = ring_in;
  a.state_out = state_out;
  a.ring_out = ring_out;
  a.out = out;
  hipError_t e = kda::launch_decode(a, io, stream);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "prefill scan launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
