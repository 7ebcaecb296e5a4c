"""MI355X (gfx950) Kimi Delta Attention (KDA) mixer core.

The compute runs in libkda.so (hand-written HIP, C ABI in include/kda.h); this package
is the thin Python binding used by the tests and the benchmark.

    layer = Layer(num_heads, conv_w, dt_bias, A_log, norm_w)
    out, state, ring = prefill(layer, q, k, v, z, beta, gate, cu_seqlens)
    out = decode_step(layer, q, k, v, z, beta, gate, state, ring)
    out = decode_multi(layer, q, k, v, z, beta, gate, state_in, ring_in, state_out, ring_out, ntok)
"""
from ._binding import (ABI_VERSION, EXPORTED, GATE_BOUNDED, GATE_SOFTPLUS, HEAD_DIM, CONV_KERNEL,
                       KdaError, Layer, LIB_PATH, NOALLOC_SCRATCH_BYTES,
                       decode_multi, decode_step, load, prefill, prefill_workspace_bytes)

__all__ = ["ABI_VERSION", "EXPORTED", "GATE_BOUNDED", "GATE_SOFTPLUS", "HEAD_DIM", "CONV_KERNEL",
           "KdaError", "Layer", "LIB_PATH", "NOALLOC_SCRATCH_BYTES", "decode_multi", "decode_step", "load", "prefill",
           "prefill_workspace_bytes"]
