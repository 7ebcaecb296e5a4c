"""Seeded synthetic inputs for the KDA mixer core.

This module only draws random numbers and rounds them to the io dtype; it holds none of
the method's arithmetic.  Both the HIP path and the oracle take their inputs from here.

Workloads (all head_dim 128, short-conv kernel 4, lower bound -5):

* ``tiny_prefill_fp32``   -- 1 sequence x 64 tokens, 2 heads, fp32 io, zero state and ring;
* ``decode_b256_h32``     -- 256 sequences x 1 token, 32 heads, bf16 io, fp32 state
  ~ N(0, 0.02) and rings ~ N(0, 1), run as 128 consecutive steps;
* ``prefill_t4096_h32``   -- 1 sequence x 4096 tokens, 32 heads, bf16 io;
* ``prefill_2x8192_h96``  -- 2 sequences x 8192 tokens, 96 heads, bf16 io, final states;
* ``varlen16_h64``        -- 16 sequences with lengths ~ U[512, 16384], 64 heads, bf16 io,
  initial state ~ N(0, 0.02) and ring ~ N(0, 1), then 32 decode steps;
* ``short256x64_h32``     -- 256 prompts x 64 tokens, 32 heads, bf16 io, carried state and
  ring: the short-prompt case on which the chunked and the sequential-scan prefill are
  compared;
* ``prefill_2x8192_h96_lowrank`` -- ``prefill_2x8192_h96`` with the low-rank decay gate:
  z_low [T, 128] and f_b [96*128, 128] in place of the full-rank z;
* ``prefill_2x8192_h96_softplus`` -- ``prefill_2x8192_h96`` with Kimi-Linear's unbounded
  softplus decay gate (layer["gate_kind"] = GATE_SOFTPLUS, the ABI's value) in place of the
  lower-bounded one; with A_log = log U(1, 16) and z ~ N(0, 1) a token's decay reaches
  tens of nats, so a 16-token chunk spans up to several hundred;
* ``prefill_2x8192_h96_softplus_lowrank`` -- both: Kimi-Linear's pairing of the softplus gate
  with the low-rank pre-activation.

Distributions: raw q/k/v, decay pre-activation z and output-gate pre-activation ~ N(0, 1);
raw beta ~ N(0, 1); conv weights ~ U(-0.5, 0.5); dt_bias ~ N(0, 0.1); A_log = log U(1, 16)
per head; RMSNorm weight = 1 + N(0, 0.02).  With the low-rank decay gate, z_low ~ N(0, 1)
and f_b ~ N(0, 128^-1/2), so that the gate's pre-activation z_low f_b^T keeps unit
variance; they take z's place in the draw order and f_b is drawn last.  N(0, s) means
standard deviation s.  Values
are drawn in fp32 by torch's generator on the requested device and rounded once (round to
nearest even) to the io dtype.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

HEAD_DIM = 128
CONV_KERNEL = 4
LOWER_BOUND = -5.0
GATE_SOFTPLUS = 1  # kda_layer.gate_kind of the unbounded gate (include/kda.h)
L2_EPS = 1e-6
RMS_EPS = 1e-5


@dataclass
class Workload:
    name: str
    kind: str                      # "prefill" or "decode"
    io: str                        # "f32" or "bf16"
    heads: int
    seqlens: list = field(default_factory=list)   # prefill sequence lengths
    batch: int = 0                 # decode batch
    steps: int = 0                 # decode steps
    init_state: bool = False
    init_ring: bool = False
    decode_after: int = 0          # decode steps that continue a prefill
    seed: int = 0
    low_rank_gate: bool = False    # z_low [T, 128] and f_b [H*128, 128] instead of z
    softplus_gate: bool = False    # the unbounded softplus decay gate

    @property
    def total_tokens(self) -> int:
        return sum(self.seqlens) if self.kind == "prefill" else self.batch * self.steps


def _varlen_lengths(seed: int, n: int = 16, lo: int = 512, hi: int = 16384) -> list:
    g = torch.Generator(device="cpu").manual_seed(seed)
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=g)]


WORKLOADS = {
    "tiny_prefill_fp32": Workload("tiny_prefill_fp32", "prefill", "f32", 2, [64], seed=20260),
    "decode_b256_h32": Workload("decode_b256_h32", "decode", "bf16", 32, batch=256, steps=128,
                                init_state=True, init_ring=True, seed=20261),
    "prefill_t4096_h32": Workload("prefill_t4096_h32", "prefill", "bf16", 32, [4096], seed=20262),
    "prefill_2x8192_h96": Workload("prefill_2x8192_h96", "prefill", "bf16", 96, [8192, 8192],
                                   seed=20263),
    "varlen16_h64": Workload("varlen16_h64", "prefill", "bf16", 64, _varlen_lengths(20264 + 7),
                             init_state=True, init_ring=True, decode_after=32, seed=20264),
    # a batch of short prompts for the chunked-versus-scan comparison (not one of the
    # reference's configurations)
    "short256x64_h32": Workload("short256x64_h32", "prefill", "bf16", 32, [64] * 256,
                                init_state=True, init_ring=True, seed=20265),
    "prefill_2x8192_h96_lowrank": Workload("prefill_2x8192_h96_lowrank", "prefill", "bf16", 96,
                                           [8192, 8192], seed=20266, low_rank_gate=True),
    "prefill_2x8192_h96_softplus": Workload("prefill_2x8192_h96_softplus", "prefill", "bf16", 96,
                                            [8192, 8192], seed=20267, softplus_gate=True),
    "prefill_2x8192_h96_softplus_lowrank": Workload("prefill_2x8192_h96_softplus_lowrank", "prefill",
                                                    "bf16", 96, [8192, 8192], seed=20268,
                                                    low_rank_gate=True, softplus_gate=True),
}


def torch_io_dtype(io: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[io]


def gen(seed: int, device="cpu") -> torch.Generator:
    return torch.Generator(device=device).manual_seed(int(seed))


def layer_params(H: int, g: torch.Generator, device="cpu", d: int = HEAD_DIM,
                 kconv: int = CONV_KERNEL) -> dict:
    """conv_w [3*H*d, kconv] ~ U(-0.5, 0.5); dt_bias [H*d] ~ N(0, 0.1);
    A_log [H] = log U(1, 16); norm_w [d] = 1 + N(0, 0.02); all fp32."""
    Hd = H * d
    conv_w = torch.rand(3 * Hd, kconv, generator=g, device=device) - 0.5
    dt_bias = torch.randn(Hd, generator=g, device=device) * 0.1
    A_log = torch.log(torch.rand(H, generator=g, device=device) * 15.0 + 1.0)
    norm_w = 1.0 + 0.02 * torch.randn(d, generator=g, device=device)
    return dict(num_heads=H, head_dim=d, conv_kernel=kconv, lower_bound=LOWER_BOUND,
                l2_eps=L2_EPS, rms_eps=RMS_EPS, conv_w=conv_w.contiguous(),
                dt_bias=dt_bias.contiguous(), A_log=A_log.contiguous(), norm_w=norm_w.contiguous())


def activations(T: int, H: int, io: str, g: torch.Generator, device="cpu", d: int = HEAD_DIM,
                lead=(), low_rank_gate: bool = False) -> dict:
    """Raw q, k, v, z, gate [*lead, T, H*d] and raw beta [*lead, T, H] ~ N(0, 1) in io dtype;
    with the low-rank gate z is z_low [*lead, T, d]."""
    dt = torch_io_dtype(io)
    shp = tuple(lead) + (T, H * d)
    out = {}
    for name in ("q", "k", "v", "z", "gate"):
        s = tuple(lead) + (T, d) if (name == "z" and low_rank_gate) else shp
        out[name] = torch.randn(s, generator=g, device=device).to(dt)
    out["beta"] = torch.randn(tuple(lead) + (T, H), generator=g, device=device).to(dt)
    return out


def initial_state(N: int, H: int, g: torch.Generator, device="cpu", d: int = HEAD_DIM,
                  std: float = 0.02) -> torch.Tensor:
    return torch.randn(N, H, d, d, generator=g, device=device) * std


def initial_ring(N: int, H: int, g: torch.Generator, device="cpu", d: int = HEAD_DIM,
                 kconv: int = CONV_KERNEL, std: float = 1.0) -> torch.Tensor:
    return torch.randn(N, 3 * H * d, kconv - 1, generator=g, device=device) * std


def cu_seqlens(seqlens) -> torch.Tensor:
    cu = [0]
    for L in seqlens:
        cu.append(cu[-1] + int(L))
    return torch.tensor(cu, dtype=torch.int32)


def low_rank_weight(H: int, io: str, g: torch.Generator, device="cpu", d: int = HEAD_DIM):
    """f_b [H*d, d] ~ N(0, d^-1/2) in the io dtype."""
    return (torch.randn(H * d, d, generator=g, device=device) * d ** -0.5).to(torch_io_dtype(io))


def make_prefill(seqlens, H: int, io: str, seed: int, device="cpu", init_state=False,
                 init_ring=False, d: int = HEAD_DIM, low_rank_gate: bool = False,
                 softplus_gate: bool = False) -> dict:
    """A packed varlen prefill problem.  Draw order: layer params, activations, state, ring,
    then f_b with the low-rank gate (layer["f_b"]; z is then z_low [T, d]).  The softplus
    gate draws nothing of its own."""
    g = gen(seed, device)
    p = layer_params(H, g, device, d)
    if softplus_gate:
        p["gate_kind"] = GATE_SOFTPLUS
    T = int(sum(seqlens))
    a = activations(T, H, io, g, device, d, low_rank_gate=low_rank_gate)
    N = len(seqlens)
    st = initial_state(N, H, g, device, d) if init_state else None
    rg = initial_ring(N, H, g, device, d) if init_ring else None
    if low_rank_gate:
        p["f_b"] = low_rank_weight(H, io, g, device, d)
    return dict(layer=p, io=io, seqlens=list(map(int, seqlens)), cu_seqlens=cu_seqlens(seqlens),
                state_in=st, ring_in=rg, **a)


def make_decode(B: int, H: int, io: str, steps: int, seed: int, device="cpu",
                d: int = HEAD_DIM, low_rank_gate: bool = False) -> dict:
    """A decode problem: params, per-step activations [steps, B, ...], state, ring (then
    f_b with the low-rank gate)."""
    g = gen(seed, device)
    p = layer_params(H, g, device, d)
    a = activations(B, H, io, g, device, d, lead=(steps,), low_rank_gate=low_rank_gate)
    st = initial_state(B, H, g, device, d)
    rg = initial_ring(B, H, g, device, d)
    if low_rank_gate:
        p["f_b"] = low_rank_weight(H, io, g, device, d)
    return dict(layer=p, io=io, batch=B, steps=steps, state=st, ring=rg, **a)


def make_workload(name: str, device="cpu") -> dict:
    w = WORKLOADS[name]
    if w.kind == "decode":
        return make_decode(w.batch, w.heads, w.io, w.steps, w.seed, device)
    return make_prefill(w.seqlens, w.heads, w.io, w.seed, device, w.init_state, w.init_ring,
                        low_rank_gate=w.low_rank_gate, softplus_gate=w.softplus_gate)
