"""ctypes binding of libkda.so (argument marshalling only; every step runs in HIP).

PyTorch supplies device memory and the stream; each call checks tensor placement, dtype,
shape and contiguity, then passes raw pointers through the C ABI declared in
include/kda.h.  There is no fallback: if the library is missing or refuses the call, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE, KDA_ERR_HIP = range(5)
KDA_F32, KDA_BF16 = 0, 1
ABI_VERSION = 5
HEAD_DIM = 128
NOALLOC_SCRATCH_BYTES = 64 << 20  # KDA_NOALLOC_SCRATCH_BYTES
CONV_KERNEL = 4

EXPORTED = ("kda_prefill_workspace_bytes", "kda_prefill", "kda_prefill_noalloc", "kda_prefill_scan",
            "kda_decode_step", "kda_decode_multi",
            "kda_status_string", "kda_last_error", "kda_abi_version")


class KdaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class KdaLayerC(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("conv_kernel", ctypes.c_int32), ("lower_bound", ctypes.c_float),
                ("l2_eps", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("conv_w", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
                ("A_log", ctypes.c_void_p), ("norm_w", ctypes.c_void_p),
                ("gate_kind", ctypes.c_int32), ("f_b", ctypes.c_void_p)]

GATE_BOUNDED, GATE_SOFTPLUS = 0, 1


_lib = None
_lock = threading.Lock()


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python __graft_entry__.py build` "
                               "(or gated_delta_rule_05_amd/_build.py)")
        lib = ctypes.CDLL(path)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        lp = ctypes.POINTER(KdaLayerC)
        lib.kda_abi_version.restype = i32
        lib.kda_abi_version.argtypes = []
        lib.kda_status_string.restype = ctypes.c_char_p
        lib.kda_status_string.argtypes = [ctypes.c_int]
        lib.kda_last_error.restype = ctypes.c_char_p
        lib.kda_last_error.argtypes = []
        lib.kda_prefill_workspace_bytes.restype = sz
        lib.kda_prefill_workspace_bytes.argtypes = [lp, ctypes.c_int, i32, vp, i64]
        lib.kda_prefill.restype = ctypes.c_int
        lib.kda_prefill.argtypes = [lp, ctypes.c_int, i32, vp, vp, i64] + [vp] * 11 + [vp, sz, vp]
        lib.kda_prefill_noalloc.restype = ctypes.c_int
        lib.kda_prefill_noalloc.argtypes = [lp, ctypes.c_int, i32, vp, vp, i64] + [vp] * 11 + [vp]
        lib.kda_decode_step.restype = ctypes.c_int
        lib.kda_decode_step.argtypes = [lp, ctypes.c_int, i32] + [vp] * 9 + [vp]
        lib.kda_prefill_scan.restype = ctypes.c_int
        lib.kda_prefill_scan.argtypes = [lp, ctypes.c_int, i32, vp, vp, i64] + [vp] * 11 + [vp]
        lib.kda_decode_multi.restype = ctypes.c_int
        lib.kda_decode_multi.argtypes = [lp, ctypes.c_int, i32, i32, vp] + [vp] * 6 + [vp] * 5 + [vp]
        if lib.kda_abi_version() != ABI_VERSION:
            raise RuntimeError(f"libkda ABI {lib.kda_abi_version()} != binding ABI {ABI_VERSION}")
        _lib = lib
        return lib


def _check(status: int):
    if status != KDA_OK:
        lib = load()
        raise KdaError(status, "%s: %s" % (lib.kda_status_string(status).decode(),
                                           lib.kda_last_error().decode()))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def io_code(dtype: torch.dtype) -> int:
    if dtype == torch.float32:
        return KDA_F32
    if dtype == torch.bfloat16:
        return KDA_BF16
    raise TypeError(f"io dtype must be float32 or bfloat16, got {dtype}")


def _need(t, name, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must live on {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class Layer:
    """One layer's parameters on the GPU: conv_w [3*H*128, 4], dt_bias [H*128], A_log [H],
    norm_w [128], all fp32; the gate's lower bound, the two epsilons, and the gate formula
    (GATE_BOUNDED, or GATE_SOFTPLUS for the unbounded softplus gate).  f_b (optional,
    [H*128, 128] in the io dtype) selects the low-rank decay gate: the z argument of every
    call is then z_low [rows, 128] and the gate's pre-activation z_low f_b^T."""

    def __init__(self, num_heads, conv_w, dt_bias, A_log, norm_w, lower_bound=-5.0,
                 l2_eps=1e-6, rms_eps=1e-5, head_dim=HEAD_DIM, conv_kernel=CONV_KERNEL,
                 gate_kind=GATE_BOUNDED, f_b=None, **_):
        self.H = int(num_heads)
        dev = conv_w.device
        Hd = self.H * HEAD_DIM
        _need(conv_w, "conv_w", (3 * Hd, CONV_KERNEL), torch.float32, dev)
        _need(dt_bias, "dt_bias", (Hd,), torch.float32, dev)
        _need(A_log, "A_log", (self.H,), torch.float32, dev)
        _need(norm_w, "norm_w", (HEAD_DIM,), torch.float32, dev)
        if f_b is not None:
            _need(f_b, "f_b", (Hd, HEAD_DIM), f_b.dtype, dev)
            io_code(f_b.dtype)
        self.f_b = f_b
        self.device = dev
        self.tensors = (conv_w, dt_bias, A_log, norm_w, f_b)  # keep alive
        self.c = KdaLayerC(self.H, int(head_dim), int(conv_kernel), float(lower_bound),
                           float(l2_eps), float(rms_eps), conv_w.data_ptr(), dt_bias.data_ptr(),
                           A_log.data_ptr(), norm_w.data_ptr(), int(gate_kind),
                           None if f_b is None else f_b.data_ptr())

    def z_width(self, dt) -> int:
        """Columns of the z argument: 128 (z_low) with the low-rank gate, else H*128."""
        if self.f_b is None:
            return self.H * HEAD_DIM
        if self.f_b.dtype != dt:
            raise TypeError(f"f_b has dtype {self.f_b.dtype}, the activations {dt}")
        return HEAD_DIM


def prefill_workspace_bytes(layer: Layer, io_dtype: torch.dtype, cu_seqlens_host) -> int:
    cu = torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous()
    return int(load().kda_prefill_workspace_bytes(ctypes.byref(layer.c), io_code(io_dtype),
                                                   cu.numel() - 1, _ptr(cu), int(cu[-1])))


def prefill(layer: Layer, q, k, v, z, beta, gate, cu_seqlens, cu_seqlens_host=None,
            state_in=None, ring_in=None, out=None, state_out=None, ring_out=None,
            final_state: bool = True, workspace=None, allow_split: bool = True, scan: bool = False,
            noalloc: bool = False, stream=None):
    """Chunked prefill over packed sequences (see kda_prefill in include/kda.h).

    q, k, v, z, gate: [T, H*128] io (fp32 or bf16); beta: [T, H] io.  cu_seqlens: int32
    [N+1] on the GPU; cu_seqlens_host: the same on the CPU (copied from the GPU, with a
    sync, when omitted).  Returns (out, state_out, ring_out); the last two are None when
    final_state is False and no buffers were passed.  The workspace the library asks for
    (segment-parallel path for few (sequence, head) units) is allocated when not given;
    allow_split=False passes none, so the whole-sequence path runs.  scan=True runs the
    sequential-scan arm instead (kda_prefill_scan: token by token, bit-identical to decode
    steps).  noalloc=True calls kda_prefill_noalloc: no workspace; the segment-parallel path
    uses the library's own scratch array.
    """
    lib = load()
    dev = layer.device
    H = layer.H
    Hd = H * HEAD_DIM
    dt = q.dtype
    io = io_code(dt)
    if cu_seqlens_host is None:
        cu_seqlens_host = cu_seqlens.to("cpu")
    cu_h = torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous()
    N = cu_h.numel() - 1
    T = int(cu_h[-1]) if N >= 0 else 0
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    for name, x in (("q", q), ("k", k), ("v", v), ("gate", gate)):
        _need(x, name, (T, Hd), dt, dev)
    _need(z, "z", (T, layer.z_width(dt)), dt, dev)
    _need(beta, "beta", (T, H), dt, dev)
    if state_in is not None:
        _need(state_in, "state_in", (N, H, HEAD_DIM, HEAD_DIM), torch.float32, dev)
    if ring_in is not None:
        _need(ring_in, "ring_in", (N, 3 * Hd, CONV_KERNEL - 1), torch.float32, dev)
    if out is None:
        out = torch.empty((T, Hd), dtype=dt, device=dev)
    _need(out, "out", (T, Hd), dt, dev)
    if final_state and state_out is None:
        state_out = torch.empty((N, H, HEAD_DIM, HEAD_DIM), dtype=torch.float32, device=dev)
    if final_state and ring_out is None:
        ring_out = torch.empty((N, 3 * Hd, CONV_KERNEL - 1), dtype=torch.float32, device=dev)
    if state_out is not None:
        _need(state_out, "state_out", (N, H, HEAD_DIM, HEAD_DIM), torch.float32, dev)
    if ring_out is not None:
        _need(ring_out, "ring_out", (N, 3 * Hd, CONV_KERNEL - 1), torch.float32, dev)
    if noalloc:
        _check(lib.kda_prefill_noalloc(ctypes.byref(layer.c), io, N, _ptr(cu_seqlens), _ptr(cu_h), T,
                                       _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta), _ptr(gate),
                                       _ptr(state_in), _ptr(ring_in), _ptr(out), _ptr(state_out),
                                       _ptr(ring_out), _stream_handle(stream)))
        return out, state_out, ring_out
    if scan:
        _check(lib.kda_prefill_scan(ctypes.byref(layer.c), io, N, _ptr(cu_seqlens), _ptr(cu_h), T,
                                    _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta), _ptr(gate),
                                    _ptr(state_in), _ptr(ring_in), _ptr(out), _ptr(state_out),
                                    _ptr(ring_out), _stream_handle(stream)))
        return out, state_out, ring_out
    need = int(lib.kda_prefill_workspace_bytes(ctypes.byref(layer.c), io, N, _ptr(cu_h), T))
    if not allow_split:
        workspace = None
    elif need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.kda_prefill(ctypes.byref(layer.c), io, N, _ptr(cu_seqlens), _ptr(cu_h), T,
                           _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta), _ptr(gate),
                           _ptr(state_in), _ptr(ring_in), _ptr(out), _ptr(state_out),
                           _ptr(ring_out), _ptr(workspace), ws_bytes, _stream_handle(stream)))
    return out, state_out, ring_out


def decode_step(layer: Layer, q, k, v, z, beta, gate, state, ring, out=None, stream=None):
    """One decode token per sequence; state [B, H, 128, 128] fp32 and ring
    [B, 3*H*128, 3] fp32 are updated in place.  q, k, v, z, gate [B, H*128] io,
    beta [B, H] io.  Returns out [B, H*128] io."""
    lib = load()
    dev = layer.device
    H = layer.H
    Hd = H * HEAD_DIM
    dt = q.dtype
    io = io_code(dt)
    B = q.shape[0]
    for name, x in (("q", q), ("k", k), ("v", v), ("gate", gate)):
        _need(x, name, (B, Hd), dt, dev)
    _need(z, "z", (B, layer.z_width(dt)), dt, dev)
    _need(beta, "beta", (B, H), dt, dev)
    _need(state, "state", (B, H, HEAD_DIM, HEAD_DIM), torch.float32, dev)
    _need(ring, "ring", (B, 3 * Hd, CONV_KERNEL - 1), torch.float32, dev)
    if out is None:
        out = torch.empty((B, Hd), dtype=dt, device=dev)
    _need(out, "out", (B, Hd), dt, dev)
    _check(lib.kda_decode_step(ctypes.byref(layer.c), io, B, _ptr(q), _ptr(k), _ptr(v), _ptr(z),
                               _ptr(beta), _ptr(gate), _ptr(state), _ptr(ring), _ptr(out),
                               _stream_handle(stream)))
    return out


def decode_multi(layer: Layer, q, k, v, z, beta, gate, state_in, ring_in, state_out=None,
                 ring_out=None, ntok=None, out=None, write_out=True, stream=None):
    """Several consecutive decode tokens per sequence in one launch (batched verify of
    speculative decoding; also its rollback by replay).

    q, k, v, z, gate [B, t, H*128] io, beta [B, t, H] io.  state_in [B, H, 128, 128] fp32 and
    ring_in [B, 3*H*128, 3] fp32 are the state and conv history before the first token;
    state_out / ring_out receive them after each sequence's last token (default: in place,
    i.e. the input buffers).  ntok: int32 [B] on the device with each sequence's token count
    (clamped to [0, t]), or None for all t.  Returns out [B, t, H*128] io (rows past a
    sequence's count are left as they were), or None when write_out is False.  Bit-identical
    row by row to chaining decode_step."""
    lib = load()
    dev = layer.device
    H = layer.H
    Hd = H * HEAD_DIM
    dt = q.dtype
    io = io_code(dt)
    B, t = q.shape[0], q.shape[1]
    for name, x in (("q", q), ("k", k), ("v", v), ("gate", gate)):
        _need(x, name, (B, t, Hd), dt, dev)
    _need(z, "z", (B, t, layer.z_width(dt)), dt, dev)
    _need(beta, "beta", (B, t, H), dt, dev)
    _need(state_in, "state_in", (B, H, HEAD_DIM, HEAD_DIM), torch.float32, dev)
    _need(ring_in, "ring_in", (B, 3 * Hd, CONV_KERNEL - 1), torch.float32, dev)
    state_out = state_in if state_out is None else state_out
    ring_out = ring_in if ring_out is None else ring_out
    _need(state_out, "state_out", (B, H, HEAD_DIM, HEAD_DIM), torch.float32, dev)
    _need(ring_out, "ring_out", (B, 3 * Hd, CONV_KERNEL - 1), torch.float32, dev)
    if ntok is not None:
        _need(ntok, "ntok", (B,), torch.int32, dev)
    if write_out:
        if out is None:
            out = torch.empty((B, t, Hd), dtype=dt, device=dev)
        _need(out, "out", (B, t, Hd), dt, dev)
    else:
        out = None
    _check(lib.kda_decode_multi(ctypes.byref(layer.c), io, B, t, _ptr(ntok), _ptr(q), _ptr(k),
                                _ptr(v), _ptr(z), _ptr(beta), _ptr(gate), _ptr(state_in),
                                _ptr(ring_in), _ptr(state_out), _ptr(ring_out), _ptr(out),
                                _stream_handle(stream)))
    return out
