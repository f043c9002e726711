"""HIP path vs the CPU oracle, through the C ABI, on an MI355X."""
import gc
import sys

import numpy as np
import pytest

import oracle
from dual_ar_codec_amd import s2ar, synth

from parity_util import Report, compare_frames, oracle_run, remember_codebook

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    s2ar.lib()
    yield


def _ctx(cfg, w, **kw):
    ctx = s2ar.Context(cfg, w, **kw)
    remember_codebook(ctx, cfg, w)
    return ctx


def _teacher_forced(name, n_frames=None, gains="unit", prompt=None, **over):
    cfg = synth.config(name, **over)
    _say(f"[parity] {name}: generating weights")
    w = synth.make_weights(cfg, gains=gains)
    toks, mask, codes = prompt if prompt is not None else synth.make_prompt(cfg)
    n = n_frames or cfg["frames"]
    _say(f"[parity] {name}: oracle prefill {len(toks)} + {n} frames")
    frames = oracle_run(cfg, w, toks, mask if mask.any() else None, codes if mask.any() else None, n)
    _say(f"[parity] {name}: GPU")
    ctx = _ctx(cfg, w)
    del w
    gc.collect()
    ctx.prefill(0, toks, mask if mask.any() else None, codes if mask.any() else None)
    rep = compare_frames(ctx, 0, frames, cfg).finish()
    _say(f"[parity] {name}: {rep}")
    ctx.close()
    return rep


def test_tiny_teacher_forced_all_frames():
    rep = _teacher_forced("tiny")
    assert rep["tokens_checked"] > 0


def test_tiny_random_gains_teacher_forced():
    _teacher_forced("tiny", n_frames=3, gains="random")


def test_mid_teacher_forced_all_frames():
    rep = _teacher_forced("mid")
    assert rep["tokens_checked"] > 0


@pytest.mark.timeout(1200)
def test_full_teacher_forced_first_frames():
    """Full FishAudio S2 shape: 41-token prompt, the first 3 frames checked layer by layer."""
    rep = _teacher_forced("full", n_frames=3)
    assert rep["tokens_checked"] > 10


@pytest.mark.timeout(1500)
def test_voice_clone_prefill_teacher_forced():
    """1000 VQ positions (sum of ten codebook rows) + 200 text positions at the full S2 shape,
    prefilled on the matrix cores in chunks, then the first 2 frames checked layer by layer."""
    rep = _teacher_forced("voice_clone", n_frames=2)
    assert rep["tokens_checked"] > 5


def test_prefill_in_two_calls_matches_one_prefill():
    cfg = synth.config("mid")
    w = synth.make_weights(cfg)
    toks, _, _ = synth.make_prompt(cfg)
    frames = oracle_run(cfg, w, toks, None, None, 3)
    ctx = _ctx(cfg, w)
    ctx.prefill(0, toks[:23])
    ctx.prefill(0, toks[23:])
    assert ctx.position(0) == len(toks)
    compare_frames(ctx, 0, frames, cfg).finish()
    ctx.close()


def test_mid_bf16_kv_cache_teacher_forced():
    """The optional bf16 KV cache (half the KV bytes) on the mid shape."""
    rep = _teacher_forced("mid", n_frames=8, kv_dtype="bf16")
    assert rep["tokens_checked"] > 0


def test_vq_masked_prefill_teacher_forced():
    cfg = synth.config("mid")
    r = np.random.default_rng(5)
    n = 40
    toks = r.integers(0, cfg["vocab_text"], n).astype(np.int32)
    mask = np.zeros(n, np.uint8)
    mask[:25] = 1
    codes = r.integers(0, cfg["codebook_size"], (n, 10)).astype(np.int32)
    _teacher_forced("mid", n_frames=2, prompt=(toks, mask, codes))


@pytest.mark.parametrize("n_prompt", [1, 15, 16, 17, 63, 64, 65, 255, 256, 300])
def test_page_chunk_and_split_boundaries(n_prompt):
    """Pages of 16, LDS chunks of 64 and attention splits of 256 positions."""
    cfg = synth.config("tiny", max_context=320)
    w = synth.make_weights(cfg)
    toks = synth.uniform_ints(9, 77, n_prompt, 0, cfg["vocab_slow"])
    frames = oracle_run(cfg, w, toks, None, None, 3)
    ctx = _ctx(cfg, w)
    ctx.prefill(0, toks)
    compare_frames(ctx, 0, frames, cfg).finish()
    ctx.close()


def test_graph_replay_equals_debug_path_and_is_deterministic():
    cfg = synth.config("mid")
    w = synth.make_weights(cfg)
    toks, _, _ = synth.make_prompt(cfg)
    n = 12
    runs = []
    for _ in range(2):
        ctx = _ctx(cfg, w)
        ctx.prefill(0, toks)
        runs.append(ctx.decode_frames([0], n)[:, 0])
        ctx.release(0)
        ctx.prefill(0, toks)
        dbg = np.stack([ctx.debug_frame(0)["own_codes"] for _ in range(n)])
        assert np.array_equal(dbg, runs[-1]), "graph replay and the eager path disagree"
        ctx.close()
    assert np.array_equal(runs[0], runs[1]), "two runs differ"
    # free-running against the oracle, up to the first decision with a thin margin
    frames = oracle_run(cfg, w, toks, None, None, n)
    for t, f in enumerate(frames):
        margins = [f["c0_margin"], *f["fast"]["margins"]]
        if min(margins) <= 5e-2:
            break
        assert np.array_equal(runs[0][t], f["codes"]), f"frame {t}"


def test_decode_frame_one_call_per_frame_matches_batched_call():
    cfg = synth.config("tiny")
    w = synth.make_weights(cfg)
    toks, _, _ = synth.make_prompt(cfg)
    ctx = _ctx(cfg, w, max_streams=3)
    for s in range(3):
        ctx.prefill(s, toks if s != 1 else toks[:5])
    one = np.stack([ctx.decode_frame([0, 1, 2]) for _ in range(4)])
    for s in range(3):
        ctx.release(s)
        ctx.prefill(s, toks if s != 1 else toks[:5])
    many = ctx.decode_frames([0, 1, 2], 4)
    assert np.array_equal(one, many)
    assert np.array_equal(one[:, 0], one[:, 2])  # same prompt, same codes
    assert ctx.position(1) == 5 + 4
    ctx.close()


def test_errors_leave_state_unchanged():
    cfg = synth.config("tiny", max_context=32)
    w = synth.make_weights(cfg)
    ctx = _ctx(cfg, w, max_streams=2)
    with pytest.raises(s2ar.S2arError) as e:
        ctx.decode_frame([0])
    assert e.value.code == -4  # decode before prefill
    with pytest.raises(s2ar.S2arError) as e:
        ctx.prefill(0, np.array([cfg["vocab_slow"]], np.int32))
    assert e.value.code == -2
    with pytest.raises(s2ar.S2arError) as e:
        ctx.prefill(2, np.array([1], np.int32))
    assert e.value.code == -2
    with pytest.raises(s2ar.S2arError) as e:
        ctx.prefill(0, np.arange(33, dtype=np.int32))
    assert e.value.code == -3
    assert ctx.position(0) == 0
    ctx.prefill(0, np.arange(30, dtype=np.int32))
    ctx.decode_frames([0], 2)  # positions 30, 31 fill the context
    with pytest.raises(s2ar.S2arError) as e:
        ctx.decode_frame([0])
    assert e.value.code == -3 and ctx.position(0) == 32
    with pytest.raises(s2ar.S2arError) as e:
        ctx.decode_frame([0, 0])
    assert e.value.code == -1
    with pytest.raises(s2ar.S2arError) as e:
        ctx.debug_frame(0, forced=np.full(10, cfg["codebook_size"], np.int32))
    assert e.value.code in (-2, -3)
    ctx.close()
