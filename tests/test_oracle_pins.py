"""Pins for the fp64 oracle, against what the pages and the mathematics fix.

None of these re-types the oracle's own formula: each check is a closed form, a special
case that reduces to a library routine (torch's Conv1d / rms_norm / sigmoid, scipy's
expit), an invariant of the recurrence, a brute-force expansion on three tokens, or the
agreement of two different algorithms (token recurrence vs chunk form).

Sources: docs.rs "ferrox_models::kda" (conv, L2 norm, q scale, sigmoid output gate);
"Kimi Delta Attention (KDA) -- analysis & C kernel plan", section "Recurrence";
docs.rs "memra_engine::kda" header prose (Gcum chunk form; fused conv ring);
OpenModelAtlas "Kimi K3 - Retention gate" (lower-bounded gate, 16-token tile bound).
"""
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle

RNG = np.random.default_rng(1234)


def rel(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(np.max(np.abs(b)), 1e-300))


# --------------------------------------------------------------------------- elementwise

def test_sigmoid_matches_scipy_expit():
    xs = [-700.0, -30.0, -1.5, -1e-3, 0.0, 1e-3, 0.7, 12.0, 700.0]
    for x in xs:
        assert oracle.sigmoid(x) == pytest.approx(scipy.special.expit(x), rel=1e-15, abs=1e-300)
    # saturations used by the beta = 0 / beta = 1 pins
    assert oracle.sigmoid(-1e4) == 0.0 and oracle.sigmoid(1e4) == 1.0


def test_silu_matches_torch():
    x = torch.linspace(-12, 12, 97, dtype=torch.float64)
    ref = F.silu(x).numpy()
    got = np.array([oracle.silu(float(v)) for v in x])
    assert rel(got, ref) < 1e-15


def test_gate_special_values():
    """Retention gate: g = -5 * sigmoid(exp(A_log) * (z + dt_bias)).

    z + dt_bias = 0 gives sigmoid(0) = 1/2 whatever A_log is; a large positive argument
    reaches the lower bound; a large negative one gives no decay; A_log = 0 and
    z = ln 3 give sigmoid(ln 3) = 3/4.  The softplus gate of the earlier
    parameterisation, or a missing exp on A_log, fails these."""
    for A_log in (0.0, math.log(1.0), math.log(16.0), 1.3):
        assert oracle.gate(0.25, -0.25, A_log) == -2.5
    assert oracle.gate(1e4, 0.0, 0.0) == -5.0
    assert oracle.gate(-1e4, 0.0, 0.0) == 0.0
    assert oracle.gate(math.log(3.0), 0.0, 0.0) == pytest.approx(-3.75, rel=1e-15)
    # exp(A_log) multiplies: A_log = ln 2 and z = ln(3)/2 also give 3/4
    assert oracle.gate(math.log(3.0) / 2, 0.0, math.log(2.0)) == pytest.approx(-3.75, rel=1e-14)
    # the lower bound scales the whole range
    assert oracle.gate(0.0, 0.0, 0.0, lower_bound=-3.0) == -1.5


def test_gate_range_stays_inside_the_bound():
    """Every retention factor exp(g) stays at or above e^-5 (Retention gate page, "Why";
    mathematically strictly above, but sigmoid rounds to 1 in floating point once its
    argument passes about 37, which the configs' distributions reach)."""
    z = RNG.normal(0, 1, 2000)
    dt = RNG.normal(0, 0.1, 2000)
    A = np.log(RNG.uniform(1, 16, 2000))
    g = np.array([oracle.gate(a, b, c) for a, b, c in zip(z, dt, A)])
    assert np.all(g <= 0) and np.all(g >= -5)
    # 16 tokens at the bound rescale by less than e^80
    assert 16 * 5 == 80


def test_softplus_gate_against_library_routines():
    """Kimi-Linear's unbounded gate, -exp(A_log) softplus(z + dt_bias): softplus is
    numpy's logaddexp(0, x) and torch's softplus; z + dt = 0 gives -exp(A_log) ln 2; large
    arguments grow linearly and very negative ones vanish, without overflow."""
    for A in (0.0, math.log(3.0), math.log(16.0)):
        assert oracle.gate_softplus(-0.25, 0.25, A) == pytest.approx(-math.exp(A) * math.log(2.0), rel=1e-15)
        for x in (-60.0, -5.0, -0.3, 0.0, 0.7, 4.0, 29.0, 31.0, 200.0):
            ref_np = -math.exp(A) * float(np.logaddexp(0.0, x))
            ref_t = -math.exp(A) * float(F.softplus(torch.tensor(x, dtype=torch.float64), threshold=1e9))
            got = oracle.gate_softplus(x - 0.5, 0.5, A)
            assert got == pytest.approx(ref_np, rel=1e-14, abs=1e-300)
            assert got == pytest.approx(ref_t, rel=1e-14, abs=1e-300)


def test_l2norm_closed_form_and_library():
    x = np.zeros(128)
    x[0], x[1] = 3.0, 4.0
    y = oracle.l2norm(x, eps=1e-6)
    assert y[0] == pytest.approx(3.0 / math.sqrt(25.0 + 1e-6), rel=1e-15)
    assert y[1] == pytest.approx(4.0 / math.sqrt(25.0 + 1e-6), rel=1e-15)
    # the q path also scales by head_dim^-1/2
    yq = oracle.l2norm(x, eps=1e-6, scale=128 ** -0.5)
    assert rel(yq, y / math.sqrt(128.0)) < 1e-15
    # against torch's normalize (eps placed differently: x / max(|x|, eps));
    # the two differ by at most eps / (2 |x|^2) relative
    v = RNG.normal(0, 1, 128)
    s = float(np.sum(v * v))
    ref = F.normalize(torch.from_numpy(v), dim=0, eps=1e-12).numpy()
    assert rel(oracle.l2norm(v, eps=1e-6), ref) <= 1e-6 / (2 * s) * 1.01 + 1e-15


def test_gated_rmsnorm_matches_torch_rms_norm():
    o = RNG.normal(0, 0.3, 128)
    w = (1 + RNG.normal(0, 0.02, 128)).astype(np.float32)
    gate = RNG.normal(0, 1, 128)
    got = oracle.gated_rmsnorm(o, gate, w, eps=1e-5)
    ref = (F.rms_norm(torch.from_numpy(o), [128], torch.from_numpy(w.astype(np.float64)), eps=1e-5)
           * torch.sigmoid(torch.from_numpy(gate))).numpy()
    assert rel(got, ref) < 1e-14
    # a fully open gate leaves the plain RMSNorm
    got1 = oracle.gated_rmsnorm(o, np.full(128, 1e4), w, eps=1e-5)
    ref1 = F.rms_norm(torch.from_numpy(o), [128], torch.from_numpy(w.astype(np.float64)),
                      eps=1e-5).numpy()
    assert rel(got1, ref1) < 1e-14


# --------------------------------------------------------------------------- recurrence

def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_core(T, dk, dv, g_lo=-5.0, seed=0):
    r = np.random.default_rng(seed)
    qh = _unit(r.normal(size=(T, dk))) / math.sqrt(dk)
    kh = _unit(r.normal(size=(T, dk)))
    v = r.normal(size=(T, dv))
    g = r.uniform(g_lo, 0.0, size=(T, dk))
    beta = r.uniform(0, 1, size=T)
    S0 = r.normal(0, 0.02, size=(dk, dv))
    return qh, kh, v, g, beta, S0


def test_beta_one_unit_key_writes_v_exactly():
    """With beta = 1 and |k| = 1 the delta rule stores v: S_t^T k_t = v_t
    (Recurrence: S_t = S' + beta k (v - S'^T k)^T, so S_t^T k = S'^T k + (v - S'^T k))."""
    qh, kh, v, g, beta, S0 = _rand_core(24, 32, 16, seed=1)
    beta[:] = 1.0
    _, _, Str = oracle.core(qh, kh, v, g, beta, S0, trace=True)
    for t in range(24):
        assert rel(Str[t].T @ kh[t], v[t]) < 1e-13


def test_beta_zero_no_decay_is_identity():
    qh, kh, v, g, beta, S0 = _rand_core(10, 16, 12, seed=2)
    beta[:] = 0.0
    g[:] = 0.0
    o, S = oracle.core(qh, kh, v, g, beta, S0)
    assert np.array_equal(S, S0)
    assert rel(o, qh @ S0) < 1e-15


def test_beta_zero_is_pure_decay():
    """beta = 0 leaves only the decay: S_T = Diag(exp(sum_t g_t)) S_0."""
    qh, kh, v, g, beta, S0 = _rand_core(12, 16, 8, seed=3)
    beta[:] = 0.0
    _, S = oracle.core(qh, kh, v, g, beta, S0)
    ref = np.exp(g.sum(axis=0))[:, None] * S0
    assert rel(S, ref) < 1e-13


def test_three_token_brute_force():
    """Three tokens from S_0 = 0, expanded by hand (memra_engine::kda pins its arithmetic
    with a hand-derived three-token recurrence):
      S_1 = b1 k1 v1^T
      S_2 = D2 S_1 + b2 k2 (v2 - (D2 S_1)^T k2)^T
      S_3 = D3 S_2 + b3 k3 (v3 - (D3 S_2)^T k3)^T,   D_t = Diag(e^{g_t}),
    written with explicit scalar sums over indices."""
    dk, dv = 5, 4
    qh, kh, v, g, beta, _ = _rand_core(3, dk, dv, seed=4)
    o, S = oracle.core(qh, kh, v, g, beta, np.zeros((dk, dv)))
    b1, b2, b3 = beta
    k1, k2, k3 = kh
    v1, v2, v3 = v
    e2, e3 = np.exp(g[1]), np.exp(g[2])
    # token 1
    S1 = [[b1 * k1[i] * v1[j] for j in range(dv)] for i in range(dk)]
    o1 = [sum(S1[i][j] * qh[0][i] for i in range(dk)) for j in range(dv)]
    # token 2: a = (D2 S1)^T k2 = b1 (sum_i k2_i e2_i k1_i) v1
    c12 = sum(k2[i] * e2[i] * k1[i] for i in range(dk))
    S2 = [[e2[i] * S1[i][j] + b2 * k2[i] * (v2[j] - b1 * c12 * v1[j]) for j in range(dv)]
          for i in range(dk)]
    o2 = [sum(S2[i][j] * qh[1][i] for i in range(dk)) for j in range(dv)]
    # token 3
    u3 = [sum(e3[i] * S2[i][j] * k3[i] for i in range(dk)) for j in range(dv)]
    S3 = [[e3[i] * S2[i][j] + b3 * k3[i] * (v3[j] - u3[j]) for j in range(dv)] for i in range(dk)]
    o3 = [sum(S3[i][j] * qh[2][i] for i in range(dk)) for j in range(dv)]
    assert rel(o, np.array([o1, o2, o3])) < 1e-14
    assert rel(S, np.array(S3)) < 1e-14
    # o_1 = b1 (q1 . k1) v1: the readout sees the updated state
    assert rel(o[0], b1 * float(qh[0] @ k1) * v1) < 1e-14


def test_orthonormal_keys_closed_form():
    """With k_t = e_t (t < dk) and S_0 = 0, later writes never touch row t, so
    S_T[t, :] = beta_t v_t prod_{s > t} e^{g_{s, t}} exactly."""
    T, dk, dv = 8, 8, 6
    qh, _, v, g, beta, _ = _rand_core(T, dk, dv, seed=5)
    kh = np.eye(T, dk)
    _, S = oracle.core(qh, kh, v, g, beta, np.zeros((dk, dv)))
    for t in range(T):
        ref = beta[t] * v[t] * np.exp(g[t + 1:, t].sum())
        assert rel(S[t], ref) < 1e-14


@pytest.mark.parametrize("T,C,tau", [(64, 64, 16), (100, 64, 16), (37, 16, 16), (96, 32, 16),
                                     (128, 64, 8), (5, 64, 16)])
def test_chunk_form_equals_token_recurrence(T, C, tau):
    """Two different algorithms, one answer: the chunk form with per-channel Gcum and
    tile-local reference points (memra_engine::kda; Retention gate page "Why") against
    the token recurrence, including ragged tails."""
    qh, kh, v, g, beta, S0 = _rand_core(T, 32, 24, seed=T + C)
    o_r, S_r = oracle.core(qh, kh, v, g, beta, S0)
    o_c, S_c = oracle.core_chunked(qh, kh, v, g, beta, S0, chunk=C, tile=tau)
    assert rel(o_c, o_r) < 1e-12
    assert rel(S_c, S_r) < 1e-12


def test_chunk_form_at_the_lower_bound():
    """g close to -5 on every channel: a 64-token chunk spans e^-320, far outside fp32,
    and the tile-local references keep every factor finite."""
    qh, kh, v, g, beta, S0 = _rand_core(128, 16, 8, seed=9)
    g[:] = -4.999
    o_r, S_r = oracle.core(qh, kh, v, g, beta, S0)
    o_c, S_c = oracle.core_chunked(qh, kh, v, g, beta, S0, chunk=64, tile=16)
    assert np.all(np.isfinite(o_c))
    assert rel(o_c, o_r) < 1e-12 and rel(S_c, S_r) < 1e-12


# --------------------------------------------------------------------------- full core

def _layer(H, d, seed, dt_scale=0.1):
    r = np.random.default_rng(seed)
    return oracle.Layer(H, d, conv_w=r.uniform(-0.5, 0.5, (3 * H * d, 4)).astype(np.float32),
                        dt_bias=(r.normal(0, dt_scale, H * d)).astype(np.float32),
                        A_log=np.log(r.uniform(1, 16, H)).astype(np.float32),
                        norm_w=(1 + r.normal(0, 0.02, d)).astype(np.float32))


def _acts(T, H, d, seed):
    r = np.random.default_rng(seed)
    a = {n: r.normal(0, 1, (T, H * d)).astype(np.float32) for n in ("q", "k", "v", "z", "gate")}
    a["beta"] = r.normal(0, 1, (T, H)).astype(np.float32)
    return a


def _conv_ref(x, w, hist=None):
    """torch Conv1d, depthwise, padding kernel-1 on the left, no bias; x [T, C], w [C, 4],
    hist [C, 3] prepended when given (the ring)."""
    xt = torch.from_numpy(x.astype(np.float64)).T[None]  # [1, C, T]
    C = xt.shape[1]
    if hist is not None:
        xt = torch.cat([torch.from_numpy(hist.astype(np.float64))[None], xt], dim=2)
        y = F.conv1d(xt, torch.from_numpy(w.astype(np.float64))[:, None, :], groups=C)
    else:
        y = F.conv1d(xt, torch.from_numpy(w.astype(np.float64))[:, None, :], padding=3, groups=C)
        y = y[..., :x.shape[0]]
    return y[0].T.numpy()


@pytest.mark.parametrize("with_ring", [False, True])
def test_conv_silu_norm_against_torch_conv1d(with_ring):
    """Short causal conv (k = 4, no bias) + SiLU per plane, then L2 norm and q scale:
    checked against torch's depthwise Conv1d.  Without a ring the first three positions
    see zero padding; with one they see the ring's raw history."""
    H, d, T = 2, 8, 7
    L = _layer(H, d, 10)
    a = _acts(T, H, d, 11)
    ring = np.random.default_rng(12).normal(0, 1, (1, 3 * H * d, 3)).astype(np.float32)
    cu = np.array([0, T])
    Hd = H * d
    for h in range(H):
        res = oracle.prefill_units(L, oracle.F32, cu, a["q"], a["k"], a["v"], a["z"], a["beta"],
                                   a["gate"], ring_in=ring if with_ring else None,
                                   units=[(0, h)], trace=True)
        tr = res["trace"]
        cols = slice(h * d, (h + 1) * d)
        for p, name in enumerate(("q", "k", "v")):
            w = L.conv_w[p * Hd:(p + 1) * Hd][cols]
            hist = ring[0, p * Hd:(p + 1) * Hd][cols] if with_ring else None
            y = _conv_ref(a[name][:, cols], w, hist)
            act = F.silu(torch.from_numpy(y)).numpy()
            if name == "v":
                assert rel(tr["v"], act) < 1e-14
            else:
                scale = d ** -0.5 if name == "q" else 1.0
                ref = act / np.sqrt(np.sum(act * act, axis=1, keepdims=True) + 1e-6) * scale
                assert rel(tr[name], ref) < 1e-14
        if not with_ring:
            # position 0 sees only the current tap: y_0 = W[3] x_0
            w = L.conv_w[2 * Hd:3 * Hd][cols]
            x0 = a["v"][0, cols].astype(np.float64)
            assert rel(tr["v"][0], F.silu(torch.from_numpy(w[:, 3] * x0)).numpy()) < 1e-15
        # ring out = the last three raw inputs of each plane, exactly
        for p, name in enumerate(("q", "k", "v")):
            assert np.array_equal(res["ring"][0][p], a[name][T - 3:, cols].T.astype(np.float64))


def test_short_sequence_shifts_the_ring():
    H, d, T = 1, 4, 2
    L = _layer(H, d, 13)
    a = _acts(T, H, d, 14)
    ring = np.arange(3 * H * d * 3, dtype=np.float32).reshape(1, 3 * H * d, 3)
    res = oracle.prefill_units(L, oracle.F32, [0, T], a["q"], a["k"], a["v"], a["z"], a["beta"],
                               a["gate"], ring_in=ring, units=[(0, 0)])
    for p, name in enumerate(("q", "k", "v")):
        exp_ring = np.concatenate([ring[0, p * d:(p + 1) * d, 2:], a[name][:, :d].T], axis=1)
        assert np.array_equal(res["ring"][0][p], exp_ring)


def test_full_path_gate_beta_and_readout():
    """Through the full path: z = dt_bias = 0 gives g = -2.5 on every channel; raw beta 0
    gives beta = 1/2; the raw readout is S_t^T q-hat_t from the UPDATED state; the output
    is torch's rms_norm of that readout times sigmoid(gate)."""
    H, d, T = 1, 16, 6
    L = _layer(H, d, 15)
    L.dt_bias[:] = 0
    a = _acts(T, H, d, 16)
    a["z"][:] = 0
    a["beta"][:] = 0
    res = oracle.prefill_units(L, oracle.F32, [0, T], a["q"], a["k"], a["v"], a["z"], a["beta"],
                               a["gate"], units=[(0, 0)], trace=True)
    tr = res["trace"]
    assert np.all(tr["g"] == -2.5)
    assert np.all(tr["beta"] == 0.5)
    for t in range(T):
        assert rel(tr["o_raw"][t], tr["S"][t].T @ tr["q"][t]) < 1e-14
    ref = (F.rms_norm(torch.from_numpy(tr["o_raw"]), [d],
                      torch.from_numpy(L.norm_w.astype(np.float64)), eps=1e-5)
           * torch.sigmoid(torch.from_numpy(a["gate"].astype(np.float64)))).numpy()
    assert rel(res["out"][0], ref) < 1e-14


def test_full_path_beta_one_stores_v():
    """Raw beta = +1e4 gives beta = 1 exactly; k-hat has |k-hat|^2 = s / (s + 1e-6), so
    S_t^T k-hat_t = v_t up to about 1e-6 / s relative."""
    H, d, T = 1, 16, 9
    L = _layer(H, d, 17)
    a = _acts(T, H, d, 18)
    a["beta"][:] = 1e4
    res = oracle.prefill_units(L, oracle.F32, [0, T], a["q"], a["k"], a["v"], a["z"], a["beta"],
                               a["gate"], units=[(0, 0)], trace=True)
    tr = res["trace"]
    for t in range(T):
        assert np.max(np.abs(tr["S"][t].T @ tr["k"][t] - tr["v"][t])) < 1e-5 * max(
            1.0, np.max(np.abs(tr["v"][t])))


def test_beta_zero_full_path_decays_the_initial_state():
    """Raw beta = -1e4 gives beta = 0 exactly: the final state is the initial one decayed
    by exp(sum g), with g at the closed-form value -2.5 (z = -dt_bias)."""
    H, d, T = 2, 8, 5
    L = _layer(H, d, 19)
    a = _acts(T, H, d, 20)
    a["beta"][:] = -1e4
    a["z"][:] = -L.dt_bias[None, :]
    S0 = np.random.default_rng(21).normal(0, 0.02, (1, H, d, d))
    out, S, _ = oracle.prefill(L, oracle.F32, [0, T], a["q"], a["k"], a["v"], a["z"], a["beta"],
                               a["gate"], state_in=S0)
    assert rel(S, S0 * math.exp(-2.5 * T)) < 1e-13


def test_beta_zero_full_path_decays_with_the_softplus_gate():
    """The gate kind reaches the full path: with beta = 0 the final state is the initial
    one decayed per key channel by exp(sum_t g_t), g_t = -exp(A_log) logaddexp(0, z + dt)
    computed here with numpy (the bounded gate would give a different decay)."""
    H, d, T = 2, 8, 5
    L = _layer(H, d, 22)
    L.gate_kind = oracle.GATE_SOFTPLUS
    a = _acts(T, H, d, 23)
    a["beta"][:] = -1e4
    S0 = np.random.default_rng(24).normal(0, 0.02, (1, H, d, d))
    out, S, _ = oracle.prefill(L, oracle.F32, [0, T], a["q"], a["k"], a["v"], a["z"], a["beta"],
                               a["gate"], state_in=S0)
    x = a["z"].astype(np.float64) + L.dt_bias.astype(np.float64)[None, :]       # [T, H*d]
    g = -np.exp(np.repeat(L.A_log.astype(np.float64), d))[None, :] * np.logaddexp(0.0, x)
    decay = np.exp(g.sum(axis=0)).reshape(H, d)                                   # per (h, key)
    assert rel(S[0], S0[0] * decay[:, :, None]) < 1e-12


def _split(a, lo, hi):
    return {n: x[lo:hi] for n, x in a.items()}


def test_prefill_equals_repeated_decode_and_split_prefill():
    """State and ring carry: one prefill over T tokens == T one-token decode steps ==
    two prefills split at any point (memra_engine::kda: decode is the same math as a
    one-token prime; the stateful prime carries ring and state forward)."""
    H, d, T = 2, 8, 11
    L = _layer(H, d, 22)
    a = _acts(T, H, d, 23)
    r = np.random.default_rng(24)
    S0 = r.normal(0, 0.02, (1, H, d, d))
    ring0 = r.normal(0, 1, (1, 3 * H * d, 3)).astype(np.float32)
    out, S, ring = oracle.prefill(L, oracle.F32, [0, T], *[a[n] for n in
                                  ("q", "k", "v", "z", "beta", "gate")], S0, ring0)
    # T decode steps
    st, rg = S0, ring0
    outs = []
    for t in range(T):
        s = _split(a, t, t + 1)
        o1, st, rg = oracle.decode_step(L, oracle.F32, s["q"], s["k"], s["v"], s["z"], s["beta"],
                                        s["gate"], st, rg.astype(np.float32))
        outs.append(o1[0])
    assert rel(np.array(outs), out) < 1e-12
    assert rel(st, S) < 1e-12 and np.array_equal(rg, ring)
    # split prefill at 4
    s1, s2 = _split(a, 0, 4), _split(a, 4, T)
    o1, st1, rg1 = oracle.prefill(L, oracle.F32, [0, 4], *[s1[n] for n in
                                  ("q", "k", "v", "z", "beta", "gate")], S0, ring0)
    o2, st2, rg2 = oracle.prefill(L, oracle.F32, [0, T - 4], *[s2[n] for n in
                                  ("q", "k", "v", "z", "beta", "gate")], st1,
                                  rg1.astype(np.float32))
    assert rel(np.concatenate([o1, o2]), out) < 1e-12
    assert rel(st2, S) < 1e-12 and np.array_equal(rg2, ring)


def test_varlen_packing_equals_separate_runs():
    """Conv and state never cross a cu_seqlens boundary."""
    H, d = 2, 8
    lens = [5, 1, 9, 2]
    L = _layer(H, d, 25)
    T = sum(lens)
    a = _acts(T, H, d, 26)
    r = np.random.default_rng(27)
    S0 = r.normal(0, 0.02, (len(lens), H, d, d))
    ring0 = r.normal(0, 1, (len(lens), 3 * H * d, 3)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)])
    out, S, ring = oracle.prefill(L, oracle.F32, cu, *[a[n] for n in
                                  ("q", "k", "v", "z", "beta", "gate")], S0, ring0)
    for n in range(len(lens)):
        s = _split(a, cu[n], cu[n + 1])
        o1, s1, r1 = oracle.prefill(L, oracle.F32, [0, lens[n]], *[s[m] for m in
                                    ("q", "k", "v", "z", "beta", "gate")], S0[n:n + 1],
                                    ring0[n:n + 1])
        assert np.array_equal(o1, out[cu[n]:cu[n + 1]])
        assert np.array_equal(s1[0], S[n]) and np.array_equal(r1[0], ring[n])


def test_bf16_inputs_are_read_exactly():
    """bf16 io is widened exactly: the same values passed as bf16 and as fp32 agree bit
    for bit."""
    H, d, T = 1, 8, 6
    L = _layer(H, d, 28)
    a32 = _acts(T, H, d, 29)
    abf = {n: torch.from_numpy(x).to(torch.bfloat16) for n, x in a32.items()}
    a32r = {n: x.float().numpy() for n, x in abf.items()}
    names = ("q", "k", "v", "z", "beta", "gate")
    o_b, s_b, _ = oracle.prefill(L, oracle.BF16, [0, T], *[abf[n] for n in names])
    o_f, s_f, _ = oracle.prefill(L, oracle.F32, [0, T], *[a32r[n] for n in names])
    assert np.array_equal(o_b, o_f) and np.array_equal(s_b, s_f)


# --------------------------------------------------------------------------- low-rank decay gate

def test_gate_projection_against_numpy_and_orientation():
    """The low-rank decay gate's pre-activation z = z_low f_b^T ("Kimi Delta Attention (KDA)
    -- analysis & C kernel plan", "The KDA layer, precisely", fact 2: hidden -> head_dim ->
    H * head_dim; Retention-gate page: f_b_proj(f_a_proj(.)), f_b a linear layer's weight
    [out][in]).  The oracle's loops against numpy's fp64 matmul in fp32 and bf16 io, and
    one-hot rows of f_b select columns of z_low, so a transposed f_b fails."""
    zl = RNG.standard_normal((7, 128)).astype(np.float32)
    fb = RNG.standard_normal((256, 128)).astype(np.float32)
    z = oracle.gate_projection(zl, fb, oracle.F32)
    assert rel(z, zl.astype(np.float64) @ fb.astype(np.float64).T) < 1e-14
    zlb = torch.from_numpy(zl).to(torch.bfloat16)
    fbb = torch.from_numpy(fb).to(torch.bfloat16)
    z = oracle.gate_projection(zlb, fbb, oracle.BF16)
    assert rel(z, zlb.double().numpy() @ fbb.double().numpy().T) < 1e-14
    sel = RNG.integers(0, 128, 256)
    onehot = np.zeros((256, 128), np.float32)
    onehot[np.arange(256), sel] = 1.0
    z = oracle.gate_projection(zl, onehot, oracle.F32)
    assert np.array_equal(z, zl[:, sel].astype(np.float64))


def _sparse_int_gate(H, d, T, seed):
    """z_low with small integers and f_b with at most four entries of +-1, +-2 per row, so
    that every z = z_low f_b^T is an integer of magnitude <= 32: exact in bf16 and fp32."""
    r = np.random.default_rng(seed)
    zl = r.integers(-4, 5, (T, d)).astype(np.float32)
    fb = np.zeros((H * d, d), np.float32)
    for c in range(H * d):
        cols = r.choice(d, size=4, replace=False)
        fb[c, cols] = r.choice([-2.0, -1.0, 1.0, 2.0], size=4)
    z = zl.astype(np.float64) @ fb.astype(np.float64).T
    assert np.all(np.abs(z) <= 32) and np.array_equal(z, np.round(z))
    return zl, fb, z.astype(np.float32)


@pytest.mark.parametrize("io", [oracle.F32, oracle.BF16])
def test_low_rank_gate_full_path_equals_materialised_z(io):
    """The full path with f_b equals the full path given z = z_low f_b^T directly, on inputs
    where that z is exact in the io dtype; two heads, so that the head offset of f_b's rows
    (channel c = h d + i) matters; varlen prefill with carried state and ring, then a decode
    step from the returned state."""
    H, d = 2, 8
    lens = [6, 3]
    T = sum(lens)
    L = _layer(H, d, 41)
    a = _acts(T, H, d, 42)
    zl, fb, z = _sparse_int_gate(H, d, T + 1, 43)
    r = np.random.default_rng(44)
    S0 = r.normal(0, 0.02, (len(lens), H, d, d))
    ring0 = r.normal(0, 1, (len(lens), 3 * H * d, 3)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)])
    if io == oracle.BF16:
        conv = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)
    else:
        conv = lambda x: np.ascontiguousarray(x)
    Lf = oracle.Layer(H, d, L.conv_w, L.dt_bias, L.A_log, L.norm_w, f_b=conv(fb))
    names = ("q", "k", "v", "beta", "gate")
    aa = {n: conv(a[n]) for n in names}
    o_f, s_f, r_f = oracle.prefill(Lf, io, cu, aa["q"], aa["k"], aa["v"], conv(zl[:T]), aa["beta"],
                                   aa["gate"], S0, ring0)
    o_m, s_m, r_m = oracle.prefill(L, io, cu, aa["q"], aa["k"], aa["v"], conv(z[:T]), aa["beta"],
                                   aa["gate"], S0, ring0)
    assert np.array_equal(o_f, o_m) and np.array_equal(s_f, s_m) and np.array_equal(r_f, r_m)
    # the gate is not trivial on these inputs
    assert np.std(z) > 1.0
    # one decode step from the returned state of both sequences
    B = len(lens)
    r2 = np.random.default_rng(45)
    d1 = {n: r2.normal(0, 1, (B, H * d if n != "beta" else H)).astype(np.float32) for n in names}
    d1 = {n: conv(x) for n, x in d1.items()}
    zl1, _, _ = _sparse_int_gate(H, d, B, 46)
    z1 = (zl1.astype(np.float64) @ fb.astype(np.float64).T).astype(np.float32)
    of, sf, rf = oracle.decode_step(Lf, io, d1["q"], d1["k"], d1["v"], conv(zl1), d1["beta"],
                                    d1["gate"], s_f, r_f.astype(np.float32))
    om, sm, rm = oracle.decode_step(L, io, d1["q"], d1["k"], d1["v"], conv(z1), d1["beta"],
                                    d1["gate"], s_m, r_m.astype(np.float32))
    assert np.array_equal(of, om) and np.array_equal(sf, sm) and np.array_equal(rf, rm)
