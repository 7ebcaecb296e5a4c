"""fp64 CPU oracle for the KDA mixer core -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
package.  It shares no code with the HIP library and never imports it.

The arithmetic lives in ``kda_oracle.c`` (plain C, double precision, token by token);
this module compiles it on first use with gcc and marshals numpy arrays in and out.
Page citations are in the C file's header; in short:

* short conv + SiLU, L2 norm, q scale  -- docs.rs "ferrox_models::kda" module page;
* the recurrence                         -- "Kimi Delta Attention (KDA) -- analysis & C
  kernel plan", section "Recurrence";
* the lower-bounded gate                 -- OpenModelAtlas "Kimi K3 - Retention gate",
  gate.py excerpt;
* the chunk form (Gcum, 16-token tiles)  -- docs.rs "memra_engine::kda" header prose and
  the Retention-gate page's "Why".

Decode is the same definition with one token per sequence, the conv history taken from
the ring and the ring shifted ("Same math as a one-token prime", memra_engine::kda,
kda_attn_decode).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lock = threading.Lock()
_lib = None

F32, BF16 = 0, 1


def build(force: bool = False) -> str:
    """Compile the C oracle into ``oracle/libkda_oracle.so`` (gcc, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                               _SRC, "-o", tmp, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build())
            dp = ctypes.POINTER(ctypes.c_double)
            vp = ctypes.c_void_p
            lib.kdao_sigmoid.restype = ctypes.c_double
            lib.kdao_sigmoid.argtypes = [ctypes.c_double]
            lib.kdao_silu.restype = ctypes.c_double
            lib.kdao_silu.argtypes = [ctypes.c_double]
            lib.kdao_gate.restype = ctypes.c_double
            lib.kdao_gate.argtypes = [ctypes.c_double] * 4
            lib.kdao_gate_softplus.restype = ctypes.c_double
            lib.kdao_gate_softplus.argtypes = [ctypes.c_double] * 3
            lib.kdao_l2norm.restype = None
            lib.kdao_l2norm.argtypes = [vp, ctypes.c_int, ctypes.c_double, ctypes.c_double]
            lib.kdao_gated_rmsnorm.restype = None
            lib.kdao_gated_rmsnorm.argtypes = [vp, vp, vp, ctypes.c_int, ctypes.c_double, vp]
            lib.kdao_core.restype = None
            lib.kdao_core.argtypes = [ctypes.c_int] * 3 + [vp] * 8
            lib.kdao_core_chunked.restype = None
            lib.kdao_core_chunked.argtypes = [ctypes.c_int] * 5 + [vp] * 7
            lib.kdao_prefill_units.restype = ctypes.c_int
            lib.kdao_prefill_units.argtypes = (
                [ctypes.c_int32] * 4 + [ctypes.c_double] * 3 + [vp] * 4 + [ctypes.c_int]
                + [vp] * 7 + [vp] + [vp, vp] + [ctypes.c_int32, vp, vp, vp, vp, vp, ctypes.c_int]
                + [vp] * 7)
            lib.kdao_gate_projection.restype = None
            lib.kdao_gate_projection.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int64,
                                                 ctypes.c_int32, ctypes.c_int64, vp]
            del dp
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def _io_array(a, io: int):
    """Accept numpy or torch-CPU arrays; bf16 travels as its uint16 bit pattern."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous()
            if a.dtype == torch.bfloat16:
                return a.view(torch.int16).numpy().view(np.uint16)
            return a.numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(a)
    if io == BF16:
        if a.dtype != np.uint16:
            raise TypeError("bf16 io must be passed as uint16 bit patterns or a torch bfloat16 tensor")
    elif a.dtype != np.float32:
        raise TypeError("fp32 io must be float32")
    return a


def _np(a, dtype=None):
    if a is None:
        return None
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(a, dtype=dtype) if dtype is not None else np.ascontiguousarray(a)


# --------------------------------------------------------------------------- elementwise

def sigmoid(x: float) -> float:
    return _load().kdao_sigmoid(float(x))


def silu(x: float) -> float:
    return _load().kdao_silu(float(x))


def gate(z: float, dt_bias: float, A_log: float, lower_bound: float = -5.0) -> float:
    """g = lower_bound * sigmoid(exp(A_log) * (z + dt_bias))  (Retention gate page, gate.py)."""
    return _load().kdao_gate(float(z), float(dt_bias), float(A_log), float(lower_bound))


def gate_softplus(z: float, dt_bias: float, A_log: float) -> float:
    """g = -exp(A_log) * softplus(z + dt_bias): Kimi-Linear's unbounded gate (the analysis
    page's status note on the decay-gate formula)."""
    return _load().kdao_gate_softplus(float(z), float(dt_bias), float(A_log))


GATE_BOUNDED, GATE_SOFTPLUS = 0, 1


def gate_projection(z_low, f_b, io: int) -> np.ndarray:
    """The low-rank decay-gate projection z = z_low f_b^T in fp64: z_low [rows, r] and
    f_b [channels, r] in the io dtype ("Kimi Delta Attention (KDA) -- analysis & C kernel
    plan", "The KDA layer, precisely", fact 2; Retention-gate page, f_b_proj(f_a_proj(.)))."""
    zl = _io_array(z_low, io)
    fb = _io_array(f_b, io)
    rows, r = zl.shape
    ch, r2 = fb.shape
    assert r == r2
    z = np.empty((rows, ch))
    _load().kdao_gate_projection(_ptr(zl), _ptr(fb), io, rows, r, ch, _ptr(z))
    return z


def l2norm(x, eps: float = 1e-6, scale: float = 1.0) -> np.ndarray:
    y = _f64(x).copy()
    _load().kdao_l2norm(_ptr(y), y.shape[-1], eps, scale)
    return y


def gated_rmsnorm(o, gate_pre, w, eps: float = 1e-5) -> np.ndarray:
    o = _f64(o)
    g = _f64(gate_pre)
    w = _f32(w)
    y = np.empty_like(o)
    _load().kdao_gated_rmsnorm(_ptr(o), _ptr(g), _ptr(w), o.shape[-1], eps, _ptr(y))
    return y


# --------------------------------------------------------------------------- recurrence

def core(qh, kh, v, g, beta, S0=None, trace: bool = False):
    """Bare token recurrence on prepared inputs (qh, kh, g: [T, dk]; v: [T, dv]; beta: [T]).

    Returns (o [T, dv], S_final [dk, dv]) and, with ``trace``, the state after every token.
    """
    qh, kh, v, g, beta = map(_f64, (qh, kh, v, g, beta))
    T, dk = kh.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.empty((T, dv))
    Str = np.empty((T, dk, dv)) if trace else None
    _load().kdao_core(T, dk, dv, _ptr(qh), _ptr(kh), _ptr(v), _ptr(g), _ptr(beta), _ptr(S),
                      _ptr(o), _ptr(Str))
    return (o, S, Str) if trace else (o, S)


def core_chunked(qh, kh, v, g, beta, S0=None, chunk: int = 64, tile: int = 16):
    """The chunk form of the same recurrence (fp64), for the chunked == recurrent pin."""
    qh, kh, v, g, beta = map(_f64, (qh, kh, v, g, beta))
    T, dk = kh.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.empty((T, dv))
    _load().kdao_core_chunked(T, dk, dv, chunk, tile, _ptr(qh), _ptr(kh), _ptr(v), _ptr(g),
                              _ptr(beta), _ptr(S), _ptr(o))
    return o, S


# --------------------------------------------------------------------------- full mixer core

class Layer:
    """Per-layer parameters (fp32): conv_w [3*H*d, kconv], dt_bias [H*d], A_log [H], norm_w [d].

    ``f_b`` (optional, io dtype [H*d, d]) selects the low-rank decay gate: the z argument of
    every call is then z_low [T, d] and the gate's pre-activation z_low f_b^T."""

    def __init__(self, num_heads, head_dim, conv_w, dt_bias, A_log, norm_w, conv_kernel=4,
                 lower_bound=-5.0, l2_eps=1e-6, rms_eps=1e-5, gate_kind=GATE_BOUNDED, f_b=None):
        self.H = int(num_heads)
        self.f_b = f_b
        self.gate_kind = int(gate_kind)
        self.d = int(head_dim)
        self.kconv = int(conv_kernel)
        self.lower_bound = float(lower_bound)
        self.l2_eps = float(l2_eps)
        self.rms_eps = float(rms_eps)
        self.conv_w = _np(conv_w, np.float32)
        self.dt_bias = _np(dt_bias, np.float32)
        self.A_log = _np(A_log, np.float32)
        self.norm_w = _np(norm_w, np.float32)
        Hd = self.H * self.d
        assert self.conv_w.shape == (3 * Hd, self.kconv)
        assert self.dt_bias.shape == (Hd,) and self.A_log.shape == (self.H,)
        assert self.norm_w.shape == (self.d,)


def prefill_units(layer: Layer, io: int, cu_seqlens, q, k, v, z, beta, gate_pre,
                  state_in=None, ring_in=None, units=None, nthreads=None, trace=False):
    """Run the full core for the listed (sequence, head) units.

    Inputs are token-major [T_tot, H*d] (beta [T_tot, H]) in the io dtype (fp32 or bf16).
    state_in [N, H, d, d] (converted to fp64 exactly) and ring_in [N, 3*H*d, kconv-1] fp32
    may be None (zeros).  Returns a dict with per-unit results:
      out   list of [T_n, d] fp64 arrays (normed, gated output),
      state [n_units, d, d] fp64,  ring [n_units, 3, d, kconv-1] fp64 (exact copies).
    With ``trace`` (one unit only) also the per-token q-hat, k-hat, v, g, beta, the raw
    readout o = S^T q-hat and the state after every token.
    """
    lib = _load()
    H, d, R = layer.H, layer.d, layer.kconv - 1
    cu = _np(cu_seqlens, np.int64)
    N = cu.shape[0] - 1
    if units is None:
        units = [(n, h) for n in range(N) for h in range(H)]
    units = np.ascontiguousarray(np.asarray(units, dtype=np.int32).reshape(-1, 2))
    lens = cu[units[:, 0] + 1] - cu[units[:, 0]]
    offs = np.zeros(len(units), dtype=np.int64)
    offs[1:] = np.cumsum(lens)[:-1]
    out = np.empty((int(lens.sum()), d))
    st = np.empty((len(units), d, d))
    rg = np.empty((len(units), 3, d, R))
    arrs = [_io_array(a, io) for a in (q, k, v, z, beta, gate_pre)]
    f_b = None if layer.f_b is None else _io_array(layer.f_b, io)
    if f_b is not None:
        assert f_b.shape == (H * d, d) and arrs[3].shape[-1] == d
    s_in = None if state_in is None else _np(state_in, np.float64)
    r_in = None if ring_in is None else _np(ring_in, np.float32)
    tr = {}
    if trace:
        assert len(units) == 1
        T = int(lens[0])
        tr = dict(q=np.empty((T, d)), k=np.empty((T, d)), v=np.empty((T, d)),
                  g=np.empty((T, d)), beta=np.empty(T), o_raw=np.empty((T, d)),
                  S=np.empty((T, d, d)))
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    rc = lib.kdao_prefill_units(
        H, d, layer.kconv, layer.gate_kind, layer.lower_bound, layer.l2_eps, layer.rms_eps,
        _ptr(layer.conv_w), _ptr(layer.dt_bias), _ptr(layer.A_log), _ptr(layer.norm_w),
        io, _ptr(cu), *[_ptr(a) for a in arrs], _ptr(f_b), _ptr(s_in), _ptr(r_in),
        len(units), _ptr(units), _ptr(offs), _ptr(out), _ptr(st), _ptr(rg), int(nthreads),
        *[_ptr(tr.get(key)) for key in ("q", "k", "v", "g", "beta", "o_raw", "S")])
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    outs = [out[offs[i]:offs[i] + lens[i]] for i in range(len(units))]
    res = dict(units=units, out=outs, state=st, ring=rg)
    if trace:
        res["trace"] = tr
    return res


def prefill(layer: Layer, io: int, cu_seqlens, q, k, v, z, beta, gate_pre, state_in=None,
            ring_in=None, nthreads=None):
    """Whole-problem prefill; returns out [T_tot, H*d], state [N, H, d, d] and
    ring [N, 3*H*d, kconv-1], all fp64."""
    H, d, R = layer.H, layer.d, layer.kconv - 1
    cu = _np(cu_seqlens, np.int64)
    N = cu.shape[0] - 1
    res = prefill_units(layer, io, cu, q, k, v, z, beta, gate_pre, state_in, ring_in,
                        nthreads=nthreads)
    T_tot = int(cu[-1])
    out = np.empty((T_tot, H * d))
    state = res["state"].reshape(N, H, d, d)
    ring = np.empty((N, 3, H, d, R))
    for u, (n, h) in enumerate(res["units"]):
        out[cu[n]:cu[n + 1], h * d:(h + 1) * d] = res["out"][u]
        ring[n, :, h] = res["ring"][u]
    return out, state, ring.reshape(N, 3 * H * d, R)


def decode_step(layer: Layer, io: int, q, k, v, z, beta, gate_pre, state, ring, units=None,
                nthreads=None):
    """One decode token per sequence: the same definition with T = 1 per sequence, the
    conv history read from ``ring`` and the ring shifted.  q..gate are [B, H*d] (beta
    [B, H]); state [B, H, d, d] (fp64 or fp32), ring [B, 3*H*d, kconv-1] fp32.
    Returns (out [B, H*d], state [B, H, d, d], ring [B, 3*H*d, kconv-1]) in fp64 for all
    units, or the per-unit dict of ``prefill_units`` when ``units`` is given."""
    st = _np(state, np.float64)
    B = st.shape[0]
    cu = np.arange(B + 1, dtype=np.int64)
    if units is not None:
        return prefill_units(layer, io, cu, q, k, v, z, beta, gate_pre, st, ring, units=units,
                             nthreads=nthreads)
    return prefill(layer, io, cu, q, k, v, z, beta, gate_pre, st, ring, nthreads=nthreads)
