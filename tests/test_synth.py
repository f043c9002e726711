"""The seeded input generator: deterministic, counter-based, right distributions."""
import numpy as np
import pytest

from dual_ar_codec_amd import synth


@pytest.fixture(scope="module", autouse=True)
def _build():
    synth.build_lib()


def test_counter_based_prefix_property_and_determinism():
    a = synth.normals_f32(5, 77, 10_000)
    b = synth.normals_f32(5, 77, 1234)
    assert np.array_equal(a[:1234], b)
    assert np.array_equal(a, synth.normals_f32(5, 77, 10_000))
    assert not np.array_equal(a, synth.normals_f32(6, 77, 10_000))
    assert not np.array_equal(a, synth.normals_f32(5, 78, 10_000))


def test_normal_moments():
    a = synth.normals_f32(1, 2, 400_000).astype(np.float64)
    assert abs(a.mean()) < 0.01 and abs(a.std() - 1) < 0.01
    assert abs(np.mean(a ** 4) - 3) < 0.05  # kurtosis of a normal


def test_bf16_weights_are_rne_of_fp32_draws():
    cfg = synth.micro_config(weight_dtype="bf16")
    w16 = synth.make_weights(cfg)
    cfg32 = dict(cfg, weight_dtype="f32")
    w32 = synth.make_weights(cfg32)
    for a, b in zip(w16, w32):
        assert a.dtype == np.uint16 and b.dtype == np.float32
        wide = synth.bf16_bits_to_f32(a)
        # round-to-nearest: within half a bf16 step (2^(e-8) for |b| in [2^e, 2^(e+1)))
        half = np.exp2(np.floor(np.log2(np.abs(b) + 1e-38)) - 8)
        assert np.all(np.abs(wide - b) <= half)
    specs = synth.tensor_specs(cfg)
    assert all(w.shape == s for w, (_, s, _) in zip(w32, specs))


def test_uniform_ints_and_permutation():
    v = synth.uniform_ints(3, 9, 100_000, 10, 20)
    assert v.min() == 10 and v.max() == 19
    assert abs(np.bincount(v - 10).std() / 10_000) < 0.05
    p = synth.page_permutation(dict(seed=4), 1000)
    assert np.array_equal(np.sort(p), np.arange(1000))


def test_workload_recipes():
    full = synth.config("full")
    assert full["vocab_slow"] == 151680 + 4096
    toks, mask, codes = synth.make_prompt(full)
    assert len(toks) == 41 and not mask.any() and toks.max() < 151680
    vc = synth.config("voice_clone")
    toks, mask, codes = synth.make_prompt(vc)
    assert len(toks) == 1200 and mask[:1000].all() and not mask[1000:].any()
    assert codes[:1000].max() < 4096 and codes[1000:].max() == 0
    ms = synth.config("multi_stream")
    lens = synth.prompt_lengths(ms)
    assert len(lens) == 16 and min(lens) >= 256 and max(lens) <= 4096
    assert ms["max_context"] >= max(lens) + ms["frames"] + 1
