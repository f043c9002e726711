"""Pins of the oracle's attention scale and of its Fast AR loop.

The attention the oracle computes is scaled dot-product attention with grouped
key/value heads: for q head h of KV group g = floor(h / (Hq / Hkv)),
o_h = softmax(q_h . K_g^T / sqrt(D)) . V_g (Qwen3-style decoder with GQA:
"SGLang Day-0 Support for FishAudio S2", Architecture; the page's Engineering
Appendix, Attention Backend Divergence, is about exactly these numerics).  The
tests below hold ``orc_attention`` to that formula in matrix form on general
inputs, and to closed forms in which the 1/sqrt(D) scale decides the value.

The Fast AR runs nine greedy steps on the Slow hidden state with a cache that is
fresh every frame, at Fast positions 0..8 (same page, Architecture, Stage 2;
"s2pro-native", What happens to a sentence).  The tests below rebuild one frame
of the Fast stack in numpy as a single causal forward over the nine-row
sequence [h, E_1[c_1], ..., E_8[c_8]] (no KV cache, every output projection
non-zero) and require the oracle's per-step taps to match it.
"""
import math

import numpy as np
import pytest

import oracle
from dual_ar_codec_amd import synth


@pytest.fixture(scope="module", autouse=True)
def _build(oracle_lib):
    synth.build_lib()
    yield


def _textbook_attention(q, kc, vc, Hq, Hkv, D):
    """softmax(Q K^T / sqrt(D)) V per q head, in numpy matrix form (no max subtraction: the
    inputs are O(1), so exp never overflows and the plain definition is exact to rounding)."""
    ctx = kc.shape[0]
    K = kc.reshape(ctx, Hkv, D)
    V = vc.reshape(ctx, Hkv, D)
    out = np.zeros(Hq * D)
    probs = np.zeros((Hq, ctx))
    for h in range(Hq):
        g = h // (Hq // Hkv)
        s = K[:, g, :] @ q[h * D:(h + 1) * D] / math.sqrt(D)
        e = np.exp(s)
        p = e / e.sum()
        probs[h] = p
        out[h * D:(h + 1) * D] = p @ V[:, g, :]
    return out, probs


@pytest.mark.parametrize("D", [16, 64, 128])
@pytest.mark.parametrize("heads", [(8, 2), (4, 4), (8, 1), (32, 8)])
def test_attention_equals_textbook_scaled_dot_product(D, heads):
    Hq, Hkv = heads
    r = np.random.default_rng(1000 + D + 7 * Hq + Hkv)
    for ctx in (1, 2, 7, 50):
        # O(1) scores: q and k of unit-ish norm per dimension, so 1/sqrt(D) visibly shapes the softmax
        q = r.standard_normal(Hq * D)
        kc = r.standard_normal((ctx, Hkv * D))
        vc = r.standard_normal((ctx, Hkv * D))
        o, p = oracle.attention(q, kc, vc, Hq, Hkv, D)
        o_ref, p_ref = _textbook_attention(q, kc, vc, Hq, Hkv, D)
        assert np.allclose(p, p_ref, rtol=1e-12, atol=1e-14)
        assert np.allclose(o, o_ref, rtol=1e-12, atol=1e-12)


def test_attention_scale_closed_form():
    """Two keys, one along q and one orthogonal to it: the scores are |q|^2 / sqrt(D) and 0, so
    the first key's weight is the logistic function of |q|^2 / sqrt(D).  With D = 16 and
    q = 2 e_0, k_1 = e_0 * 2: score 4 / 4 = 1, weight 1 / (1 + e^-1) = 0.7310585786300049."""
    D = 16
    q = np.zeros(D)
    q[0] = 2.0
    kc = np.zeros((2, D))
    kc[0, 0] = 2.0
    vc = np.zeros((2, D))
    vc[0, 3] = 1.0   # o[3] is the weight of key 0
    vc[1, 5] = 1.0   # o[5] is the weight of key 1
    o, p = oracle.attention(q, kc, vc, 1, 1, D)
    assert p[0, 0] == pytest.approx(0.7310585786300049, rel=1e-15)
    assert o[3] == pytest.approx(0.7310585786300049, rel=1e-15)
    assert o[5] == pytest.approx(0.2689414213699951, rel=1e-14)
    # the same score at D = 64 needs |q||k| = 8: the weight does not depend on D once q.k = sqrt(D)
    D = 64
    q = np.zeros(D)
    q[1] = 4.0
    kc = np.zeros((2, D))
    kc[0, 1] = 2.0
    vc = np.zeros((2, D))
    vc[0, 0] = 1.0
    o, _ = oracle.attention(q, kc, vc, 1, 1, D)
    assert o[0] == pytest.approx(0.7310585786300049, rel=1e-15)
    # and an unscaled softmax (score 8) would have given 0.99966..., far from this value
    assert abs(o[0] - 1.0 / (1.0 + math.exp(-8.0))) > 0.2


def test_attention_scale_with_equal_keys_and_values_of_ramp():
    """ctx keys all equal to q's direction scaled j = 0..n-1: the weights are a geometric series
    w_j proportional to exp(j |q| / sqrt(D)); with V = j the output is its mean, a closed form."""
    D, n = 64, 9
    q = np.zeros(D)
    q[0] = 0.5
    kc = np.zeros((n, D))
    kc[:, 0] = np.arange(n)
    vc = np.zeros((n, D))
    vc[:, 0] = np.arange(n)
    o, _ = oracle.attention(q, kc, vc, 1, 1, D)
    a = 0.5 / 8.0  # per-step score increment |q| / sqrt(64)
    w = np.array([math.exp(a * j) for j in range(n)])
    want = float((w * np.arange(n)).sum() / w.sum())
    assert o[0] == pytest.approx(want, rel=1e-14)


# ------------------------------------------------------------------ Fast AR in matrix form

def _bf16(x32):
    """Round float32 values to bfloat16 (round to nearest even), returned as float64."""
    u = np.asarray(x32, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _rope_tables(theta, D, n_pos, bf16):
    i = np.arange(D // 2, dtype=np.float64)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * theta ** (-2.0 * i / D)[None, :]
    if bf16:  # fp64 -> fp32 -> bf16 (the model's bf16 RoPE table)
        return _bf16(np.cos(ang).astype(np.float32)), _bf16(np.sin(ang).astype(np.float32))
    return np.cos(ang), np.sin(ang)


def _fast_matrix_form(cfg, w, h, forced, pos0=0):
    """One frame of the Fast AR as a single causal forward over the nine input rows, which sit at
    Fast positions pos0 .. pos0 + 8."""
    names = [n for n, _, _ in synth.tensor_specs(cfg)]
    W = lambda n: synth.as_f32(w[names.index(n)]).astype(np.float64)  # noqa: E731
    s = cfg["fast"]
    H, Hq, Hkv, D, eps = s["hidden"], s["n_q_heads"], s["n_kv_heads"], s["head_dim"], cfg["rms_eps"]
    n = cfg["n_codebooks"] - 1
    cb = W("codebook.embed")
    X = np.stack([h] + [cb[j, forced[j - 1]] for j in range(1, n)])  # rows: Fast positions 0..8
    cos, sin = (t[pos0:] for t in _rope_tables(cfg["rope_theta"], D, pos0 + n, cfg["rope_bf16"]))

    def rms(a, g):
        return a / np.sqrt(np.mean(a * a, axis=-1, keepdims=True) + eps) * g

    def rope(a):  # a: [n][heads][D], rotate-half pairs (i, i + D/2) at the row's position
        lo, hi = a[..., :D // 2], a[..., D // 2:]
        c, sn = cos[:, None, :], sin[:, None, :]
        return np.concatenate([lo * c - hi * sn, hi * c + lo * sn], axis=-1)

    resid = np.zeros((n, s["n_layers"], H))
    mask = np.triu(np.full((n, n), -np.inf), 1)
    for l in range(s["n_layers"]):
        p = f"fast.layers.{l}."
        xn = rms(X, W(p + "attn_norm"))
        Q = (xn @ W(p + "wq").T).reshape(n, Hq, D)
        Kx = (xn @ W(p + "wk").T).reshape(n, Hkv, D)
        Vx = (xn @ W(p + "wv").T).reshape(n, Hkv, D)
        Q = rope(rms(Q, W(p + "q_norm")))
        Kx = rope(rms(Kx, W(p + "k_norm")))
        O = np.zeros((n, Hq, D))
        for hq in range(Hq):
            g = hq // (Hq // Hkv)
            S = Q[:, hq, :] @ Kx[:, g, :].T / math.sqrt(D) + mask
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            O[:, hq, :] = P @ Vx[:, g, :]
        X = X + O.reshape(n, Hq * D) @ W(p + "wo").T
        xn = rms(X, W(p + "mlp_norm"))
        G = xn @ W(p + "w_gate").T
        U = xn @ W(p + "w_up").T
        X = X + (G / (1 + np.exp(-G)) * U) @ W(p + "w_down").T
        resid[:, l] = X
    Z = rms(X, W("fast.final_norm"))
    logits = Z @ W("fast.head").T
    return resid, Z, logits


@pytest.mark.parametrize("heads,layers,bf16", [((4, 2), 2, 1), ((4, 4), 1, 0), ((8, 1), 3, 1)])
def test_fast_loop_equals_causal_matrix_form_over_nine_positions(heads, layers, bf16):
    """Every output projection is non-zero, so the Fast attention over positions 0..j-1 shapes
    each step's residual; the matrix form has no cache and one causal mask over nine rows."""
    Hq, Hkv = heads
    cfg = synth.micro_config(seed=40 + layers, slow_layers=1, fast_layers=layers, hidden=64, n_q_heads=Hq,
                             n_kv_heads=Hkv, head_dim=16, ffn=96, rope_bf16=bf16)
    cfg["rope_theta"] = 10.0  # a small base makes the nine positions' rotations large
    w = synth.make_weights(cfg, gains="random", std=0.2)
    m = oracle.Model(cfg, w)
    r = np.random.default_rng(50 + layers)
    h = r.standard_normal(cfg["slow"]["hidden"])
    forced = r.integers(0, cfg["codebook_size"], 9).astype(np.int32)
    fl = m.fast_loop(h, forced=forced, taps=True)
    resid, Z, logits = _fast_matrix_form(cfg, w, h, forced)
    assert np.allclose(fl["resid"], resid, rtol=1e-10, atol=1e-11)
    assert np.allclose(fl["z"], Z, rtol=1e-10, atol=1e-11)
    assert np.allclose(fl["logits"], logits, rtol=1e-10, atol=1e-11)
    # the picks are the argmax of each step's logits (ties to the lowest index)
    assert np.array_equal(fl["codes"], np.argmax(logits, axis=1))


def test_fast_loop_cache_is_fresh_every_frame():
    """A second frame sees none of the first frame's keys: its taps equal the matrix form of its
    own nine rows, whatever ran before."""
    cfg = synth.micro_config(seed=47, slow_layers=1, fast_layers=2, hidden=64, n_q_heads=4, n_kv_heads=2,
                             head_dim=16, ffn=96)
    cfg["rope_theta"] = 10.0
    w = synth.make_weights(cfg, gains="random", std=0.2)
    m = oracle.Model(cfg, w)
    r = np.random.default_rng(47)
    h1, h2 = r.standard_normal((2, cfg["slow"]["hidden"]))
    f1 = r.integers(0, cfg["codebook_size"], 9).astype(np.int32)
    f2 = r.integers(0, cfg["codebook_size"], 9).astype(np.int32)
    m.fast_loop(h1, forced=f1, taps=True)
    second = m.fast_loop(h2, forced=f2, taps=True)
    resid, Z, logits = _fast_matrix_form(cfg, w, h2, f2)
    assert np.allclose(second["resid"], resid, rtol=1e-10, atol=1e-11)
    assert np.allclose(second["logits"], logits, rtol=1e-10, atol=1e-11)


def test_fast_positions_matter():
    """The same nine rows placed at positions 1..9 instead of 0..8 give different taps: rotations
    are relative only in exact arithmetic, and the bf16-rounded cos/sin table is not, so the pin
    above fixes the absolute positions 0..8 and not only their spacing."""
    cfg = synth.micro_config(seed=48, slow_layers=1, fast_layers=1, hidden=64, n_q_heads=4, n_kv_heads=2,
                             head_dim=16, ffn=96, rope_bf16=1)
    cfg["rope_theta"] = 10.0
    w = synth.make_weights(cfg, gains="random", std=0.2)
    m = oracle.Model(cfg, w)
    r = np.random.default_rng(48)
    h = r.standard_normal(cfg["slow"]["hidden"])
    forced = r.integers(0, cfg["codebook_size"], 9).astype(np.int32)
    fl = m.fast_loop(h, forced=forced, taps=True)
    at0, _, _ = _fast_matrix_form(cfg, w, h, forced, pos0=0)
    at1, _, _ = _fast_matrix_form(cfg, w, h, forced, pos0=1)
    assert np.allclose(fl["resid"], at0, rtol=1e-10, atol=1e-11)
    assert np.max(np.abs(fl["resid"] - at1)) > 1e-6
