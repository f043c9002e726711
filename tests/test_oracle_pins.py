"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: closed forms,
exact rational arithmetic, special cases that reduce to textbook operations,
invariants of the method, and the figures the pages print.
"""
import cmath
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from dual_ar_codec_amd import metrics, synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _build(oracle_lib):
    synth.build_lib()
    yield


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_closed_forms():
    # constant vector: y = c / sqrt(c^2 + eps) * g
    for c in (2.0, -0.5, 1e-3):
        x = np.full(8, c)
        y = oracle.rmsnorm(x, np.ones(8), 1e-6)
        assert np.allclose(y, c / math.sqrt(c * c + 1e-6), rtol=1e-15, atol=0)
    # [3, 4] with eps = 0: mean square 12.5
    y = oracle.rmsnorm([3.0, 4.0], [1.0, 1.0], 0.0)
    assert y == pytest.approx([3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rel=1e-15)


def test_rmsnorm_invariants():
    r = _rng(0)
    x = r.standard_normal(64)
    g = r.uniform(0.5, 1.5, 64)
    y = oracle.rmsnorm(x, g, 0.0)
    # unit output mean-square with unit gain, scale invariance, elementwise gain
    assert np.mean(oracle.rmsnorm(x, np.ones(64), 0.0) ** 2) == pytest.approx(1.0, rel=1e-14)
    assert np.allclose(oracle.rmsnorm(7.5 * x, g, 0.0), y, rtol=1e-14)
    assert np.allclose(oracle.rmsnorm(x, np.ones(64), 0.0) * g, y, rtol=1e-14)
    # epsilon sits inside the root: tiny input is damped, not blown up
    tiny = oracle.rmsnorm(np.full(4, 1e-6), np.ones(4), 1e-6)
    assert np.allclose(tiny, 1e-6 / math.sqrt(1e-12 + 1e-6))


# ---------------------------------------------------------------- RoPE

def test_rope_position_zero_is_identity():
    for bf16 in (0, 1):
        c, s = oracle.rope_row(1e6, 128, 0, bf16)
        assert np.all(c == 1.0) and np.all(s == 0.0)
        v = _rng(1).standard_normal(128)
        assert np.array_equal(oracle.rope_apply(v, c, s), v)


def test_rope_matches_complex_rotation():
    """Rotary embedding as complex multiplication (RoFormer, eq. for 2-D
    rotation): the pair (v_i, v_{i+D/2}) is the complex number v_i + i v_{i+D/2}
    multiplied by exp(i * pos * theta^(-2i/D))."""
    D, theta = 64, 1.0e6
    v = _rng(2).standard_normal(D)
    for pos in (1, 5, 97, 4000):
        c, s = oracle.rope_row(theta, D, pos, 0)
        out = oracle.rope_apply(v, c, s)
        for i in range(D // 2):
            z = complex(v[i], v[i + D // 2]) * cmath.exp(1j * pos * theta ** (-2.0 * i / D))
            assert out[i] == pytest.approx(z.real, abs=1e-12)
            assert out[i + D // 2] == pytest.approx(z.imag, abs=1e-12)


def test_rope_relative_position_and_norm():
    D = 128
    r = _rng(3)
    q, k = r.standard_normal(D), r.standard_normal(D)

    def rot(v, p):
        c, s = oracle.rope_row(1e6, D, p, 0)
        return oracle.rope_apply(v, c, s)

    for m, n, sh in ((3, 1, 10), (50, 7, 333), (0, 0, 4095)):
        assert np.dot(rot(q, m), rot(k, n)) == pytest.approx(np.dot(rot(q, m + sh), rot(k, n + sh)), abs=1e-10)
    qr = rot(q, 123)
    for i in range(D // 2):
        assert math.hypot(qr[i], qr[i + D // 2]) == pytest.approx(math.hypot(q[i], q[i + D // 2]), rel=1e-13)


def test_rope_table_rounds_to_bf16():
    """The cos/sin table is rounded to bf16 (S2 page, Engineering Appendix).
    Worked by hand: cos(1) = 0.5403023 lies in [0.5, 1), where bf16 (8
    significant bits) has a step of 2^-8, so it rounds to 138/256 = 0.5390625;
    sin(1) = 0.8414710 rounds to 215/256 = 0.83984375."""
    c, s = oracle.rope_row(1e6, 128, 1, 1)  # i = 0 has inverse frequency 1, angle 1 rad
    # bf16 keeps 8 significant bits: in [0.5, 1) the step is 2^-8
    assert c[0] == 0.5390625 == round(math.cos(1.0) * 256) / 256
    assert s[0] == 0.83984375 == round(math.sin(1.0) * 256) / 256
    for pos in (2, 17, 1000):
        c, s = oracle.rope_row(1e6, 128, pos, 1)
        for v in np.concatenate([c, s]):
            bits = np.array([v], np.float32).view(np.uint32)[0]
            assert bits & 0xFFFF == 0
        c64, s64 = oracle.rope_row(1e6, 128, pos, 0)
        assert np.all(np.abs(c - c64) <= np.abs(c64) * 2 ** -8 + 1e-45)


# ---------------------------------------------------------------- attention

def test_attention_probabilities_sum_to_one_and_single_key():
    r = _rng(4)
    Hq, Hkv, D, ctx = 8, 2, 16, 37
    q = r.standard_normal(Hq * D)
    kc, vc = r.standard_normal((ctx, Hkv * D)), r.standard_normal((ctx, Hkv * D))
    o, p = oracle.attention(q, kc, vc, Hq, Hkv, D)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-12)
    assert np.all(p > 0)
    o1, p1 = oracle.attention(q, kc[:1], vc[:1], Hq, Hkv, D)
    group = Hq // Hkv
    for h in range(Hq):
        assert np.array_equal(o1[h * D:(h + 1) * D], vc[0, (h // group) * D:(h // group + 1) * D])


def test_attention_uniform_and_dominant_limits():
    r = _rng(5)
    Hq, Hkv, D, ctx = 4, 4, 8, 11
    kc, vc = r.standard_normal((ctx, Hkv * D)), r.standard_normal((ctx, Hkv * D))
    o, p = oracle.attention(np.zeros(Hq * D), kc, vc, Hq, Hkv, D)
    assert np.allclose(p, 1.0 / ctx)
    assert np.allclose(o, vc.mean(axis=0), atol=1e-14)
    # one key aligned with a huge query wins
    q = np.zeros(Hq * D)
    for h in range(Hq):
        q[h * D:(h + 1) * D] = 1e3 * kc[6, h * D:(h + 1) * D]
    o, _ = oracle.attention(q, kc, vc, Hq, Hkv, D)
    assert np.allclose(o, vc[6], atol=1e-9)


def test_gqa_equals_mha_with_repeat_interleaved_kv():
    r = _rng(6)
    Hq, Hkv, D, ctx = 8, 2, 16, 21
    q = r.standard_normal(Hq * D)
    kc, vc = r.standard_normal((ctx, Hkv, D)), r.standard_normal((ctx, Hkv, D))
    o, _ = oracle.attention(q, kc.reshape(ctx, -1), vc.reshape(ctx, -1), Hq, Hkv, D)
    kr = np.repeat(kc, Hq // Hkv, axis=1).reshape(ctx, -1)
    vr = np.repeat(vc, Hq // Hkv, axis=1).reshape(ctx, -1)
    o_mha, _ = oracle.attention(q, kr, vr, Hq, Hq, D)
    assert np.allclose(o, o_mha, rtol=0, atol=1e-14)


def test_attention_key_permutation_invariance():
    r = _rng(7)
    Hq, Hkv, D, ctx = 4, 2, 8, 13
    q = r.standard_normal(Hq * D)
    kc, vc = r.standard_normal((ctx, Hkv * D)), r.standard_normal((ctx, Hkv * D))
    perm = r.permutation(ctx)
    o, _ = oracle.attention(q, kc, vc, Hq, Hkv, D)
    o2, _ = oracle.attention(q, kc[perm], vc[perm], Hq, Hkv, D)
    assert np.allclose(o, o2, atol=1e-13)


# ---------------------------------------------------------------- GEMV, SwiGLU, argmax

def test_matvec_against_exact_rational_sums():
    r = _rng(8)
    N, K = 5, 300
    w = r.standard_normal((N, K)).astype(np.float32)
    x = r.standard_normal(K)
    y = oracle.matvec_f32(w, x)
    gamma = K * 2.0 ** -53 / (1 - K * 2.0 ** -53)
    for n in range(N):
        exact = sum(Fraction(float(w[n, k])) * Fraction(float(x[k])) for k in range(K))
        bound = gamma * float(np.sum(np.abs(w[n].astype(np.float64) * x)))
        assert abs(Fraction(y[n]) - exact) <= Fraction(bound) + Fraction(1, 10 ** 300)


def test_matvec_several_vectors_bitwise_equal_to_one_at_a_time():
    r = _rng(9)
    w = r.standard_normal((33, 70)).astype(np.float32)
    X = r.standard_normal((6, 70))
    Y = oracle.matvec_f32(w, X)
    for p in range(6):
        assert np.array_equal(Y[p], oracle.matvec_f32(w, X[p]))


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-16)
    assert oracle.silu(1.0) == pytest.approx(0.7310585786300049, rel=1e-15)
    assert oracle.silu(60.0) == pytest.approx(60.0, rel=1e-20)
    assert abs(oracle.silu(-60.0)) < 1e-24
    for z in (0.3, 2.5, -4.0):  # silu(-z) = silu(z) - z
        assert oracle.silu(-z) == pytest.approx(oracle.silu(z) - z, abs=1e-15)


def test_argmax_brute_force_ties_and_ranges():
    r = _rng(10)
    for trial in range(200):
        n = int(r.integers(1, 50))
        v = r.integers(-3, 4, n).astype(np.float64)  # many ties
        lo = int(r.integers(0, n))
        hi = int(r.integers(lo + 1, n + 1))
        i, mg = oracle.argmax(v, lo, hi)
        sub = v[lo:hi]
        assert i == lo + int(np.argmax(sub))  # numpy: first occurrence of the maximum
        if hi - lo > 1:
            srt = np.sort(sub)
            assert mg == srt[-1] - srt[-2]


# ---------------------------------------------------------------- model-level pins

def _micro(**kw):
    cfg = synth.micro_config(**kw)
    return cfg


def _model(cfg, weights=None, gains="random"):
    w = synth.make_weights(cfg, gains=gains) if weights is None else weights
    return oracle.Model(cfg, w), w


def _idx(cfg, name):
    return [n for n, _, _ in synth.tensor_specs(cfg)].index(name)


def test_gather_sum_picks_the_right_rows():
    cfg = _micro(seed=11)
    w = synth.make_weights(cfg)
    ci = _idx(cfg, "codebook.embed")
    r = _rng(11)
    w[ci] = r.integers(-1000, 1000, w[ci].shape).astype(np.float32)  # integer rows: sums are exact
    m = oracle.Model(cfg, w)
    for _ in range(20):
        codes = r.integers(0, cfg["codebook_size"], 10).astype(np.int32)
        want = sum(w[ci][k, codes[k]].astype(np.int64) for k in range(10))
        assert np.array_equal(m.embed_codes(codes), want.astype(np.float64))
    with pytest.raises(ValueError):
        m.embed_codes(np.full(10, cfg["codebook_size"], np.int32))


def test_single_position_layer_reduces_to_plain_matmuls():
    """With one position, attention weights are exactly 1, so o_h = v of head
    h's KV group regardless of QK-norm and RoPE, and the whole Slow stack is a
    chain of matrix products, norms and SwiGLU that numpy evaluates directly."""
    cfg = _micro(seed=12, slow_layers=2)
    m, w = _model(cfg)
    s = cfg["slow"]
    H, Hq, Hkv, D = s["hidden"], s["n_q_heads"], s["n_kv_heads"], s["head_dim"]
    tok = 17
    x = w[0][tok].astype(np.float64)

    def rms(v, g):
        return v / np.sqrt(np.mean(v * v) + cfg["rms_eps"]) * g

    for l in range(s["n_layers"]):
        base = 1 + 11 * l
        an, wq, wk, wv, qn, kn, wo, mn, wg, wu, wd = [w[base + i].astype(np.float64) for i in range(11)]
        v = wv @ rms(x, an)
        o = np.concatenate([v[(h // (Hq // Hkv)) * D:(h // (Hq // Hkv) + 1) * D] for h in range(Hq)])
        x = x + wo @ o
        xn = rms(x, mn)
        g, u = wg @ xn, wu @ xn
        x = x + wd @ (g / (1 + np.exp(-g)) * u)
    fin = w[1 + 11 * s["n_layers"]].astype(np.float64)
    h_want = rms(x, fin)
    st = m.new_state()
    out = st.prefill(np.array([tok], np.int32))
    assert np.allclose(out["h"], h_want, rtol=1e-11, atol=1e-12)
    head = w[2 + 11 * s["n_layers"]].astype(np.float64)
    logits_want = head @ h_want
    assert np.allclose(out["logits"], logits_want, rtol=1e-11, atol=1e-12)
    Vt = cfg["vocab_text"]
    assert out["c0"] == int(np.argmax(logits_want[Vt:]))


def test_identity_layers_reduce_to_head_and_codebook_chain():
    """With every output projection (wo, w_down) zero, each layer leaves the
    residual unchanged.  The frame then reduces to: h = RMSNorm(sum of codebook
    rows), c0 = argmax of the semantic slice of head.h, and a Fast chain where
    step j's input is codebook table j-1 at c_{j-1}."""
    cfg = _micro(seed=13, slow_layers=2, fast_layers=2)
    w = synth.make_weights(cfg, gains="random")
    names = [n for n, _, _ in synth.tensor_specs(cfg)]
    for i, n in enumerate(names):
        if n.endswith(".wo") or n.endswith(".w_down"):
            w[i] = np.zeros_like(w[i])
    m = oracle.Model(cfg, w)
    K, Vt, eps = cfg["codebook_size"], cfg["vocab_text"], cfg["rms_eps"]
    cb = w[names.index("codebook.embed")].astype(np.float64)
    sfin = w[names.index("slow.final_norm")].astype(np.float64)
    shead = w[names.index("slow.head")].astype(np.float64)
    ffin = w[names.index("fast.final_norm")].astype(np.float64)
    fhead = w[names.index("fast.head")].astype(np.float64)

    def rms(v, g):
        return v / np.sqrt(np.mean(v * v) + eps) * g

    r = _rng(13)
    st = m.new_state()
    st.prefill(r.integers(0, Vt, 4).astype(np.int32))
    codes = r.integers(0, K, 10).astype(np.int32)
    out = st.slow_step(codes)
    h = rms(sum(cb[k, codes[k]] for k in range(10)), sfin)
    assert np.allclose(out["h"], h, rtol=1e-12, atol=1e-13)
    assert out["c0"] == int(np.argmax((shead @ h)[Vt:]))
    fl = m.fast_loop(out["h"], taps=True)
    y = out["h"]
    for j in range(1, 10):
        logits = fhead @ rms(y, ffin)
        assert np.allclose(fl["logits"][j - 1], logits, rtol=1e-11, atol=1e-12)
        c = int(np.argmax(logits))
        assert fl["codes"][j - 1] == c
        y = cb[j, c]


def test_qk_norm_makes_attention_invariant_to_per_head_scaling():
    """QK-norm normalises each q and k head before RoPE, so scaling the rows
    of one head of wq or wk changes nothing downstream (epsilon set negligible
    so that the normalisation is exactly scale-free)."""
    cfg = _micro(seed=14, slow_layers=1)
    cfg["rms_eps"] = 1e-30
    w = synth.make_weights(cfg, gains="random")
    toks = np.array([3, 9, 27, 81, 5], np.int32)
    base = oracle.Model(cfg, w).new_state().prefill(toks)
    D = cfg["slow"]["head_dim"]
    w2 = [a.copy() for a in w]
    w2[_idx(cfg, "slow.layers.0.wq")][D:2 * D] *= 4.0   # q head 1
    w2[_idx(cfg, "slow.layers.0.wk")][0:D] *= 0.25      # k head 0
    other = oracle.Model(cfg, w2).new_state().prefill(toks)
    assert np.allclose(base["h"], other["h"], rtol=1e-9, atol=1e-10)
    # a global (not per-head) scale of q would also cancel; a scale of v must not
    w3 = [a.copy() for a in w]
    w3[_idx(cfg, "slow.layers.0.wv")][0:D] *= 4.0
    changed = oracle.Model(cfg, w3).new_state().prefill(toks)
    assert not np.allclose(base["h"], changed["h"], rtol=1e-6)


def test_kv_cached_decode_equals_full_causal_recompute():
    for seed, kw in ((15, {}), (16, dict(n_q_heads=4, n_kv_heads=4)), (17, dict(n_q_heads=4, n_kv_heads=1))):
        cfg = _micro(seed=seed, slow_layers=2, **kw)
        m, w = _model(cfg)
        r = _rng(seed)
        n = 12
        toks = r.integers(0, cfg["vocab_slow"], n).astype(np.int32)
        mask = (r.random(n) < 0.4).astype(np.uint8)
        codes = r.integers(0, cfg["codebook_size"], (n, 10)).astype(np.int32)
        full = m.full_recompute(toks, mask, codes)
        st = m.new_state()
        for i in range(n):
            h = st.prefill(toks[i:i + 1], mask[i:i + 1], codes[i:i + 1])["h"]
            assert np.allclose(h, full[i], rtol=1e-11, atol=1e-12), (seed, i)


def test_prefill_block_equals_one_position_at_a_time():
    cfg = _micro(seed=18)
    m, w = _model(cfg)
    r = _rng(18)
    n = 9
    toks = r.integers(0, cfg["vocab_slow"], n).astype(np.int32)
    mask = (r.random(n) < 0.5).astype(np.uint8)
    codes = r.integers(0, cfg["codebook_size"], (n, 10)).astype(np.int32)
    a = m.new_state().prefill(toks, mask, codes)
    st = m.new_state()
    for i in range(n):
        b = st.prefill(toks[i:i + 1], mask[i:i + 1], codes[i:i + 1])
    assert np.array_equal(a["h"], b["h"]) and np.array_equal(a["logits"], b["logits"])
    assert a["c0"] == b["c0"]


def test_frame_counts_and_code_ranges():
    cfg = _micro(seed=19, fast_layers=2)
    m, w = _model(cfg)
    r = _rng(19)
    toks = r.integers(0, cfg["vocab_text"], 5).astype(np.int32)
    oracle.reset_counters()
    st = m.new_state()
    pre = st.prefill(toks)
    n_frames = 6
    codes = st.generate(pre["h"], pre["c0"], n_frames)
    c = oracle.counters()
    assert codes.shape == (n_frames, 10)
    assert c["codes_emitted"] == 10 * n_frames
    assert c["fast_steps"] == 9 * n_frames            # 9 Fast steps per Slow step
    assert c["fast_layer_passes"] == 9 * 2 * n_frames
    assert c["slow_steps"] == len(toks) + n_frames - 1
    assert np.all((codes >= 0) & (codes < cfg["codebook_size"]))
    assert st.pos == len(toks) + n_frames - 1


def test_generate_matches_primitives_in_page_order():
    """Frame 1 comes from the prefill's hidden; frame t >= 2 first feeds frame
    t-1's ten codes to the Slow AR, then runs the Fast loop."""
    cfg = _micro(seed=20)
    m, w = _model(cfg)
    toks = _rng(20).integers(0, cfg["vocab_text"], 4).astype(np.int32)
    st1 = m.new_state()
    pre = st1.prefill(toks)
    codes = st1.generate(pre["h"], pre["c0"], 4)
    st2 = m.new_state()
    p2 = st2.prefill(toks)
    h, c0 = p2["h"], p2["c0"]
    for t in range(4):
        if t:
            s = st2.slow_step(codes[t - 1])
            h, c0 = s["h"], s["c0"]
        f = m.fast_loop(h)
        assert codes[t, 0] == c0 and np.array_equal(codes[t, 1:], f["codes"])


def test_teacher_forcing_only_changes_inputs():
    cfg = _micro(seed=21)
    m, _ = _model(cfg)
    h = _rng(21).standard_normal(cfg["slow"]["hidden"])
    own = m.fast_loop(h, taps=True)
    same = m.fast_loop(h, forced=own["codes"], taps=True)
    assert np.array_equal(own["logits"], same["logits"])
    forced = (own["codes"] + 1) % cfg["codebook_size"]
    other = m.fast_loop(h, forced=forced, taps=True)
    assert np.array_equal(other["logits"][0], own["logits"][0])   # step 1 sees only h
    assert not np.allclose(other["logits"][1], own["logits"][1])
    with pytest.raises(ValueError):
        m.fast_loop(h, forced=np.full(9, -1, np.int32))


def test_thread_count_never_changes_a_bit():
    cfg = _micro(seed=22, hidden=128, ffn=256)
    m, _ = _model(cfg)
    toks = _rng(22).integers(0, cfg["vocab_text"], 7).astype(np.int32)
    outs = []
    for nt in (1, 4):
        oracle.set_threads(nt)
        st = m.new_state()
        pre = st.prefill(toks)
        outs.append((pre["logits"], st.generate(pre["h"], pre["c0"], 3)))
    oracle.set_threads(os.cpu_count() or 1)
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


def test_tiny_workload_runs_end_to_end():
    cfg = synth.config("tiny")
    m, _ = _model(cfg, gains="unit")
    toks, mask, codes = synth.make_prompt(cfg)
    st = m.new_state()
    pre = st.prefill(toks, mask, codes)
    out = st.generate(pre["h"], pre["c0"], cfg["frames"])
    assert out.shape == (cfg["frames"], 10)
    assert np.all((out >= 0) & (out < cfg["codebook_size"]))
    # logits have the scale the recipe predicts: std ~ 0.02 * sqrt(H) for a unit-RMS h
    assert 0.5 * 0.02 * 16 < np.std(pre["logits"]) < 2.0 * 0.02 * 16


# ---------------------------------------------------------------- page figures

def _golden():
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        return json.load(f)


def test_frame_duration_and_rtf_reproduce_page_figures():
    g = _golden()
    assert metrics.FRAME_SAMPLES == g["frame_samples"]["value"]
    assert metrics.SAMPLE_RATE == g["sample_rate_hz"]["value"]
    assert round(metrics.frame_seconds() * 1000, g["frame_ms"]["digits"]) == g["frame_ms"]["value"]
    assert abs(1 / metrics.frame_seconds() - g["frame_rate_hz_about"]["value"]) < 1.0  # 21.53 Hz
    pair = g["h200_pair"]
    assert round(metrics.rtf(pair["tok_per_s"]), 2) == pair["rtf"]
    assert metrics.N_CODEBOOKS == g["codes_per_frame"]["value"]
    assert metrics.N_FAST_STEPS == g["fast_steps_per_frame"]["value"]


def test_byte_model_reproduces_params_per_frame():
    g = _golden()
    cfg = synth.config("full")
    assert cfg["slow"]["n_layers"] == g["stack_depths"]["slow_layers"]
    assert cfg["fast"]["n_layers"] == g["stack_depths"]["fast_layers"]
    n = metrics.params_per_frame(cfg, head_rows=cfg["vocab_text"])
    assert n == 7_749_304_320
    assert round(n / 1e9, 2) == g["params_per_frame_about"]["value"] / 1e9
    assert abs(metrics.params_per_frame(cfg) / g["params_per_frame_about"]["value"] - 1) < 0.002
    s = cfg["slow"]
    slow = s["n_layers"] * metrics.layer_matrix_params(s) + cfg["vocab_slow"] * s["hidden"]
    fast = cfg["fast"]["n_layers"] * metrics.layer_matrix_params(cfg["fast"])
    assert abs(slow / g["param_split"]["slow_about"] - 1) < 0.12
    assert abs(fast / g["param_split"]["fast_about"] - 1) < 0.02
    fb = metrics.frame_bytes(cfg, 100)
    assert fb["weights"] > 15.5e9 and fb["kv"] == 294_912 * 101  # fp32 K and V, 36 layers x 8 heads x 128
    assert metrics.kv_bytes_per_position(dict(cfg, kv_dtype="bf16")) == 147_456


# ------------------------------------------------ int8 weights with per-row scales

def _bf16_bits(v):
    """bf16 bit patterns of values that bf16 holds exactly."""
    return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_int8_rows_closed_form():
    # max |w| = 2 maps to -127; 1 / (2/127) = 63.5 rounds to the even 64; 0.5 / (2/127) = 31.75 -> 32
    q, s = oracle.quantize_rows_i8(_bf16_bits([[1.0, -2.0, 0.5, 0.0], [0.0, 0.0, 0.0, 0.0], [3.0, 3.0, -3.0, 1.5]]))
    assert q[0].tolist() == [64, -127, 32, 0]
    assert s[0] == np.float32(2.0) / np.float32(127.0) and abs(float(s[0]) * 127 - 2.0) < 1e-6
    assert q[1].tolist() == [0, 0, 0, 0] and s[1] == 0.0  # a zero row: scale 0, no division
    assert q[2].tolist() == [127, 127, -127, 64]          # 1.5 / (3/127) = 63.5 -> 64
    deq = oracle.dequantize_rows_i8(q, s)
    assert deq[1].tolist() == [0.0] * 4 and deq[0][1] == -np.float32(2.0) / np.float32(127.0) * 127


def test_int8_rows_invariants():
    r = np.random.default_rng(11)
    w = (r.standard_normal((64, 300)) * 0.02).astype(np.float32)
    w[5] *= 1000.0                       # rows of very different magnitude
    w[9, :] = 0.0
    bits = _bf16_bits(np.array([[oracle.bf16_round(v) for v in row] for row in w], np.float32))
    wf = (bits.astype(np.uint32) << 16).view(np.float32)
    q, s = oracle.quantize_rows_i8(bits)
    deq = oracle.dequantize_rows_i8(q, s)
    nz = np.any(wf != 0, axis=1)
    # every non-zero row reaches +-127 at its largest element, and no element leaves [-127, 127]
    assert np.all(np.max(np.abs(q[nz].astype(np.int32)), axis=1) == 127) and np.all(q[~nz] == 0)
    # the rounding error of each weight is at most half a step (plus fp32 rounding of the product)
    err = np.abs(deq.astype(np.float64) - wf.astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 1e-5) + 1e-30)
    # the scale is the row's max |w| / 127 and does not depend on the other rows
    assert np.allclose(s[nz] * 127.0, np.max(np.abs(wf[nz]), axis=1), rtol=1e-6)
    q1, s1 = oracle.quantize_rows_i8(bits[5:6])
    assert np.array_equal(q1[0], q[5]) and s1[0] == s[5]
    # sign symmetry: -w quantises to -q with the same scale
    qn, sn = oracle.quantize_rows_i8(bits ^ np.uint16(0x8000))
    assert np.array_equal(qn.astype(np.int32), -q.astype(np.int32)) and np.array_equal(sn, s)


# ------------------------------------------------ FP8 E4M3 weights with per-row scales

def test_f8_values_follow_the_e4m3_encoding():
    # OCP FP8 E4M3: bias 7, 3 mantissa bits, subnormals m * 2^-9, largest finite 448, S.1111.111 NaN
    want = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2.0 ** -6,
            0x30: 0.5, 0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for b, v in want.items():
        assert oracle.f8_value(b) == v, hex(b)
    assert math.isnan(oracle.f8_value(0x7F)) and math.isnan(oracle.f8_value(0xFF))
    # the finite magnitudes are strictly increasing in the code, so code order is value order
    mags = [oracle.f8_value(b) for b in range(0x7F)]
    assert all(a < b for a, b in zip(mags, mags[1:]))
    # every E4M3 value has at most 4 significant bits, so bf16 (8) holds each one exactly
    assert all(oracle.bf16_round(v) == v for v in mags)


def test_f8_rows_exact_values_and_ties_to_even():
    # max |w| = 448 gives s = 1, so representable values come back unchanged; halfway values go to
    # the even code: 1.0625 lies between 1.0 (0x38) and 1.125 (0x39) -> 1.0; 1.1875 between 1.125
    # and 1.25 (0x3A) -> 1.25; 2^-10 between 0 and 2^-9 -> 0; 3 * 2^-10 between 2^-9 and 2^-8 -> 2^-8
    row = [448.0, -1.0, 0.5, 2.0 ** -9, 1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, -240.0, 0.0]
    q, s = oracle.quantize_rows_f8(_bf16_bits([row, [0.0] * 10]))
    assert s[0] == 1.0 and s[1] == 0.0 and q[1].tolist() == [0] * 10
    deq = oracle.dequantize_rows_f8(q, s)
    assert deq[0].tolist() == [448.0, -1.0, 0.5, 2.0 ** -9, 1.0, 1.25, 0.0, 2.0 ** -8, -240.0, 0.0]
    assert q[0][0] == 0x7E and q[0][1] == 0xB8 and q[0][4] == 0x38 and q[0][5] == 0x3A


def test_f8_rows_invariants():
    r = np.random.default_rng(12)
    w = (r.standard_normal((48, 260)) * 0.02).astype(np.float32)
    w[3] *= 500.0
    w[7, :] = 0.0
    bits = _bf16_bits(np.array([[oracle.bf16_round(v) for v in row] for row in w], np.float32))
    wf = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q, s = oracle.quantize_rows_f8(bits)
    deq = oracle.dequantize_rows_f8(q, s).astype(np.float64)
    nz = np.any(wf != 0, axis=1)
    # each non-zero row's largest element maps to +-448, and the scale is max |w| / 448
    assert np.all(np.max(q[nz] & 0x7F, axis=1) == 0x7E)
    assert np.allclose(s[nz].astype(np.float64) * 448.0, np.max(np.abs(wf[nz]), axis=1), rtol=1e-6)
    # error within half a step of the E4M3 grid at the scaled magnitude (step 2^(floor(log2 v) - 3)
    # for normals, 2^-9 below 2^-6), plus fp32 rounding of the quotient and the product
    v = np.abs(wf[nz]) / s[nz][:, None]
    step = np.where(v >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(v, 1e-300))) - 3), 2.0 ** -9)
    err = np.abs(deq[nz] - wf[nz]) / s[nz][:, None]
    assert np.all(err <= 0.5 * step * (1 + 1e-5) + 448.0 * 2.0 ** -23)
    # sign symmetry and row independence
    qn, sn = oracle.quantize_rows_f8(bits ^ np.uint16(0x8000))
    nzc = (q & 0x7F) != 0
    assert np.array_equal(qn[nzc], q[nzc] ^ 0x80) and np.array_equal(sn, s)
    q1, s1 = oracle.quantize_rows_f8(bits[3:4])
    assert np.array_equal(q1[0], q[3]) and s1[0] == s[3]


# ------------------------------------------------ stop token (EOS) in the Slow pick

def test_slow_pick_with_stop_brute_force():
    r = _rng(30)
    Vt, K = 40, 24
    for trial in range(300):
        v = r.integers(-3, 4, Vt + K).astype(np.float64)  # many ties
        eos = int(r.integers(-1, Vt))
        c0, mg = oracle.slow_pick(v, Vt, K, eos)
        cand = ([eos] if eos >= 0 else []) + list(range(Vt, Vt + K))
        # the largest logit wins; among equal logits the lowest id
        best = min(cand, key=lambda i: (-v[i], i))
        assert c0 == (-1 if best == eos else best - Vt)
        others = sorted((v[i] for i in cand if i != best), reverse=True)
        assert mg == v[best] - others[0]
        if eos < 0:  # no stop token: the plain constrained argmax
            i, m2 = oracle.argmax(v, Vt, Vt + K)
            assert c0 == i - Vt and mg == m2
    # a tie between the EOS logit and the best semantic logit goes to EOS (the lower id)
    v = np.zeros(Vt + K)
    v[Vt + 5] = 2.0
    v[7] = 2.0
    assert oracle.slow_pick(v, Vt, K, 7) == (-1, 0.0)
    v[7] = np.nextafter(2.0, 0.0)
    assert oracle.slow_pick(v, Vt, K, 7)[0] == 5


def test_generate_stops_at_the_first_eos_pick_and_keeps_earlier_frames():
    """A stop id that wins at some Slow step ends the stream there; the frames before it are those
    of the run without a stop id, and every frame from it on is -1."""
    cfg = _micro(seed=31)
    m, w = _model(cfg)
    Vt, K, n_frames = cfg["vocab_text"], cfg["codebook_size"], 6
    toks = _rng(31).integers(0, Vt, 5).astype(np.int32)
    st = m.new_state()
    pre = st.prefill(toks)
    free = st.generate(pre["h"], pre["c0"], n_frames)
    # the Slow logits of every frame's pick: prefill's, then each Slow step's on the free codes
    st2 = m.new_state()
    logits = [st2.prefill(toks)["logits"]]
    for t in range(1, n_frames):
        logits.append(st2.slow_step(free[t - 1])["logits"])
    # stop id: the text id with the largest logit at frame 3's pick, where it beats every semantic id
    eos = int(np.argmax(logits[3][:Vt]))
    if logits[3][eos] < np.max(logits[3][Vt:Vt + K]):
        pytest.skip("no text id beats the semantic ids at this seed")
    stop = next(t for t in range(n_frames) if logits[t][eos] >= np.max(logits[t][Vt:Vt + K]))
    assert stop <= 3
    me = oracle.Model(dict(cfg, eos_id=eos), w)
    st3 = me.new_state()
    pre3 = st3.prefill(toks)
    assert (pre3["c0"] == -1) == (stop == 0)
    got = st3.generate(pre3["h"], pre3["c0"], n_frames)
    assert np.array_equal(got[:stop], free[:stop])
    assert np.all(got[stop:] == -1)
    with pytest.raises(ValueError):
        oracle.Model(dict(cfg, eos_id=Vt), w)  # a semantic id cannot be the stop id
