"""HIP path vs the CPU oracle, through the C ABI, on an MI355X."""
import gc
import sys

import numpy as np
import pytest

import oracle
from dual_ar_codec_amd import s2ar, synth

from parity_util import (Report, compare_frames, oracle_run, own_slow_pick, quant_reference, remember_codebook,
                         slow_rows)

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


# oracle frames of the default prompts, shared by the cases that differ only on the GPU side (the
# full-shape voice clone at both prefill precisions runs its 1200-position oracle prefill once)
_ORACLE_FRAMES = {}


def _teacher_forced(name, n_frames=None, gains="unit", prompt=None, prefill_precision=0, **over):
    cfg = synth.config(name, **over)
    _say(f"[parity] {name}: generating weights")
    w = synth.make_weights(cfg, gains=gains)
    toks, mask, codes = prompt if prompt is not None else synth.make_prompt(cfg)
    n = n_frames or cfg["frames"]
    key = (name, n, gains, tuple(sorted(over.items()))) if prompt is None else None
    if key is not None and key in _ORACLE_FRAMES:
        frames = _ORACLE_FRAMES[key]
    else:
        _say(f"[parity] {name}: oracle prefill {len(toks)} + {n} frames")
        frames = oracle_run(cfg, w, toks, mask if mask.any() else None, codes if mask.any() else None, n)
        if key is not None and name == "voice_clone":
            _ORACLE_FRAMES[key] = frames
    _say(f"[parity] {name}: GPU")
    ctx = _ctx(cfg, w)
    del w
    gc.collect()
    if prefill_precision:
        ctx.set_prefill_precision(prefill_precision)
    ctx.prefill(0, toks, mask if mask.any() else None, codes if mask.any() else None)
    rep = compare_frames(ctx, 0, frames, cfg).finish()
    _say(f"[parity] {name} (prefill precision {prefill_precision}): {rep}")
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


def test_attention_merge_over_more_than_64_splits():
    """A 4200-position context at batch 1: 66 attention splits of 64 positions, so the split merge
    takes its (max, sum) pairs in two rounds of 64 lanes."""
    cfg = synth.config("tiny", max_context=4288)
    toks = synth.uniform_ints(78, 0, 4200, 0, cfg["vocab_text"])
    mask = np.zeros(len(toks), np.uint8)
    codes = np.zeros((len(toks), cfg["n_codebooks"]), np.int32)
    rep = _teacher_forced("tiny", n_frames=2, prompt=(toks, mask, codes), max_context=4288)
    assert rep["tokens_checked"] > 5


def test_prefill_longer_than_one_row_block():
    """A 2100-position prompt at the mid shape: the matrix-core prefill runs it as two row blocks
    (2048 + 52), the second attending over the first block's cached keys."""
    cfg = synth.config("mid", max_context=2176)
    toks = synth.uniform_ints(77, 0, 2100, 0, cfg["vocab_text"])
    mask = np.zeros(len(toks), np.uint8)
    codes = np.zeros((len(toks), cfg["n_codebooks"]), np.int32)
    rep = _teacher_forced("mid", n_frames=2, prompt=(toks, mask, codes), max_context=2176)
    assert rep["tokens_checked"] > 5


def test_prefill_key_splits_unaligned_second_call():
    """A 23-token prefill, then 1180 more positions in a second call at the mid shape.  The second
    call's causal key ranges reach 1203 keys, so its row blocks are served by up to three key-split
    workgroups, and because the rows start at position 23 the 512-key split boundaries fall inside
    row blocks: some rows have no key in a split and must contribute nothing to it."""
    cfg = synth.config("mid", max_context=1280)
    w = synth.make_weights(cfg)
    toks = synth.uniform_ints(78, 0, 1203, 0, cfg["vocab_text"])
    frames = oracle_run(cfg, w, toks, None, None, 2)
    ctx = _ctx(cfg, w)
    ctx.prefill(0, toks[:23])
    ctx.prefill(0, toks[23:])
    assert ctx.position(0) == len(toks)
    rep = compare_frames(ctx, 0, frames, cfg).finish()
    _say(f"[parity] mid, 23 + 1180 prompt: {rep}")
    ctx.close()


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


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("kv", ["k_bf16", "v_bf16"])
def test_full_mixed_kv_cache_teacher_forced(kv):
    """bf16 keys with fp32 values, and fp32 keys with bf16 values, at the full S2 shape: each keeps a
    quarter fewer KV bytes than fp32 and stays inside the acceptance bar (both halves in bf16 do not:
    the oracle itself, with its keys and values rounded to bf16, drifts 1 - cos = 1.2e-4)."""
    rep = _teacher_forced("full", n_frames=3, kv_dtype=kv)
    assert rep["tokens_checked"] > 0


@pytest.mark.parametrize("kv,precision", [("k_bf16", 0), ("v_bf16", 0), ("k_bf16", 1), ("v_bf16", 1)])
def test_batched_mixed_kv_cache_mid_ragged(kv, precision):
    """Mixed KV caches through the batched kernels, five ragged streams; precision 1 prefills them
    with the fp16 products (its attention converts the bf16 or fp32 cache entries to fp16)."""
    cfg = synth.config("mid", max_context=640, kv_dtype=kv)
    w = synth.make_weights(cfg)
    prompts = _ragged_prompts(cfg, [64, 17, 300, 130, 5], 31)
    per_stream = _oracle_frames_per_stream(cfg, w, prompts, 3)
    ctx = _ctx(cfg, w, max_streams=6)
    if precision:
        ctx.set_prefill_precision(precision)
    ids = [0, 2, 3, 4, 5]
    for s_, p in zip(ids, prompts):
        ctx.prefill(s_, p)
    rep = _compare_batch(ctx, ids, per_stream, cfg, Report()).finish()
    _say(f"[parity] batched mid, {kv} KV, prefill precision {precision}: {rep}")
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


@pytest.mark.timeout(900)
def test_full_workload_graph_replay_in_the_bench_configuration():
    """The timed workload as bench.py runs it (full shape, 41-token prompt, context capacity 1408 and
    three stream slots, so the split merges are live): 60 graph-replayed frames, the first 8 equal
    to the eager path bit for bit and the free-running frames equal to the oracle's up to the first
    decision with a thin margin."""
    cfg = synth.config("full", max_context=1408)
    w = synth.make_weights(cfg)
    toks, _, _ = synth.make_prompt(cfg)
    ctx = _ctx(cfg, w, max_streams=3)
    ctx.prefill(0, toks)
    graph = ctx.decode_frames([0], 60)[:, 0]
    assert np.all((graph >= 0) & (graph < cfg["codebook_size"]))
    ctx.prefill(1, toks)
    eager = np.stack([ctx.debug_frame(1)["own_codes"] for _ in range(8)])
    assert np.array_equal(eager, graph[:8]), "graph replay and the eager path disagree"
    ctx.close()
    frames = oracle_run(cfg, w, toks, None, None, 4)
    checked = 0  # picks in decode order (c0, c1 .. c9 of frame 0, then frame 1 ..) up to a thin margin
    done = False
    for t, f in enumerate(frames):
        for k, m in enumerate([f["c0_margin"], *f["fast"]["margins"]]):
            if m <= 5e-2:
                done = True
                break
            assert graph[t][k] == f["codes"][k], f"frame {t} code {k}"
            checked += 1
        if done:
            break
    assert checked > 0
    _say(f"[parity] full workload, bench configuration: {checked} free-running picks equal to the oracle's")


@pytest.mark.parametrize("n_shared", [64, 37])
def test_shared_prefix_streams(n_shared):
    """Two streams share the first n_shared positions of a VQ-masked prompt (whole pages by
    reference, the partial last page copied when n_shared is not a multiple of 16), then each
    prefills its own text.  Both match the oracle run on their full prompts, before and after the
    other stream decodes, and the sharer keeps working after the source is released."""
    cfg = synth.config("mid", max_context=256)
    w = synth.make_weights(cfg)
    r = np.random.default_rng(17)
    n_vq, n_text = 70, 24
    codes = r.integers(0, cfg["codebook_size"], (n_vq + n_text, 10)).astype(np.int32)
    mask = np.zeros(n_vq + n_text, np.uint8)
    mask[:n_vq] = 1
    prompts = []
    for s_ in range(2):
        toks = r.integers(0, cfg["vocab_text"], n_vq + n_text).astype(np.int32)
        toks[:n_shared] = prompts[0][0][:n_shared] if prompts else toks[:n_shared]
        m, c = mask.copy(), codes.copy()
        prompts.append((toks, m, c))
    refs = [oracle_run(cfg, w, t, m, c, 3) for t, m, c in prompts]
    ctx = _ctx(cfg, w, max_streams=2)
    t0, m0, c0 = prompts[0]
    ctx.prefill(0, t0, m0, c0)
    ctx.share_prefix(0, 1, n_shared)
    assert ctx.position(1) == n_shared
    with pytest.raises(s2ar.S2arError):
        ctx.decode_frame([1])  # not ready until its own positions are prefilled
    t1, m1, c1 = prompts[1]
    ctx.prefill(1, t1[n_shared:], m1[n_shared:], c1[n_shared:])
    assert ctx.position(1) == len(t1)
    rep1 = compare_frames(ctx, 1, refs[1][:2], cfg).finish()
    rep0 = compare_frames(ctx, 0, refs[0], cfg).finish()
    ctx.release(0)
    rep1b = compare_frames(ctx, 1, refs[1][2:], cfg).finish()
    _say(f"[parity] shared prefix {n_shared}: {rep0} {rep1} {rep1b}")
    ctx.close()


def test_shared_prefix_streams_batched():
    """Two streams sharing the first 37 positions (two whole pages by reference and a copied partial
    page) decode together through the batched kernels and match the oracle on their full prompts."""
    cfg = synth.config("mid", max_context=256)
    w = synth.make_weights(cfg)
    r = np.random.default_rng(19)
    n, n_shared = 90, 37
    base = r.integers(0, cfg["vocab_text"], n).astype(np.int32)
    other = r.integers(0, cfg["vocab_text"], n).astype(np.int32)
    other[:n_shared] = base[:n_shared]
    refs = [oracle_run(cfg, w, t, None, None, 3) for t in (base, other)]
    ctx = _ctx(cfg, w, max_streams=2)
    ctx.prefill(0, base)
    ctx.share_prefix(0, 1, n_shared)
    ctx.prefill(1, other[n_shared:])
    rep = _compare_batch(ctx, [0, 1], refs, cfg, Report()).finish()
    _say(f"[parity] shared prefix, batched: {rep}")
    ctx.close()


def test_shared_prefix_errors_leave_state_unchanged():
    cfg = synth.config("tiny")
    w = synth.make_weights(cfg)
    toks, _, _ = synth.make_prompt(cfg)
    ctx = _ctx(cfg, w, max_streams=3)
    ctx.prefill(0, toks)
    ctx.prefill(2, toks[:5])
    for args in [(0, 0, 4), (0, 2, 4), (0, 1, 0), (0, 1, len(toks) + 1), (0, 7, 4), (-1, 1, 4)]:
        with pytest.raises(s2ar.S2arError):
            ctx.share_prefix(*args)
    assert ctx.position(1) == 0 and ctx.position(2) == 5
    ctx.share_prefix(0, 1, len(toks))  # the whole prompt: still needs one more position
    ctx.prefill(1, toks[-1:])
    ctx.close()


def _int8_teacher_forced(name, n_frames, fmt="i8", prompt=None, prefill_precision=0, **over):
    cfg = synth.config(name, **over)
    _say(f"[parity] {name} {fmt}: generating weights")
    w = synth.make_weights(cfg)
    ocfg, ow = quant_reference(cfg, w, fmt)
    toks, mask, codes = prompt if prompt is not None else synth.make_prompt(cfg)
    mk, cd = (mask, codes) if mask.any() else (None, None)
    _say(f"[parity] {name} {fmt}: oracle prefill {len(toks)} + {n_frames} frames")
    frames = oracle_run(ocfg, ow, toks, mk, cd, n_frames)
    del ow
    gc.collect()
    _say(f"[parity] {name} {fmt}: GPU")
    ctx = _ctx(dict(cfg, weight_dtype=fmt), w)
    del w
    gc.collect()
    if prefill_precision:
        ctx.set_prefill_precision(prefill_precision)
    ctx.prefill(0, toks, mk, cd)
    rep = compare_frames(ctx, 0, frames, cfg).finish()
    _say(f"[parity] {name} {fmt} (prefill precision {prefill_precision}): {rep}")
    ctx.close()
    return rep


def test_int8_vq_prompt_prefill_on_the_matrix_cores_mid():
    """A 300-position VQ-masked prompt (200 VQ positions, then text) prefilled with int8 weights: the
    matrix-core GEMMs widen the codes to bf16 in LDS and scale each output column."""
    cfg = synth.config("mid", max_context=384)
    r = np.random.default_rng(71)
    n = 300
    toks = r.integers(0, cfg["vocab_text"], n).astype(np.int32)
    codes = r.integers(0, cfg["codebook_size"], (n, 10)).astype(np.int32)
    mask = np.zeros(n, np.uint8)
    mask[:200] = 1
    for fmt in ("i8", "f8"):
        rep = _int8_teacher_forced("mid", 3, fmt, prompt=(toks, mask, codes), max_context=384)
        assert rep["tokens_checked"] > 0


@pytest.mark.timeout(1500)
def test_int8_voice_clone_prefill_teacher_forced():
    """The 1200-position voice-clone prompt (1000 VQ + 200 text) at the full S2 shape with int8 weights,
    prefilled on the matrix cores in one row block, then 2 frames against the oracle on the same
    quantisation."""
    assert _int8_teacher_forced("voice_clone", 2)["tokens_checked"] > 0


# ------------------------------------------------------------------ fp16 prefill (precision 1)

@pytest.mark.timeout(1500)
def test_voice_clone_prefill_fp16_teacher_forced():
    """The 1200-position voice-clone prompt at the full S2 shape prefilled with one fp16 activation
    plane per product (fp16 matrix cores), then 2 frames checked layer by layer against the oracle."""
    rep = _teacher_forced("voice_clone", n_frames=2, prefill_precision=1)
    assert rep["tokens_checked"] > 5


@pytest.mark.parametrize("case", ["split_k", "two_row_blocks", "int8", "fp8"])
def test_fp16_prefill_mid(case):
    """fp16 prefill at the mid shape: a 41-token prompt (its GEMMs split K, the SwiGLU written by
    the split reduction), a 2100-position prompt (two row blocks of 2048 + 52), and a VQ-masked
    300-position prompt with int8 and FP8 weights (codes widened to fp16 in LDS)."""
    if case == "split_k":
        rep = _teacher_forced("mid", n_frames=4, prefill_precision=1)
    elif case == "two_row_blocks":
        cfg = synth.config("mid", max_context=2176)
        toks = synth.uniform_ints(77, 0, 2100, 0, cfg["vocab_text"])
        mask = np.zeros(len(toks), np.uint8)
        codes = np.zeros((len(toks), cfg["n_codebooks"]), np.int32)
        rep = _teacher_forced("mid", n_frames=2, prompt=(toks, mask, codes), max_context=2176,
                              prefill_precision=1)
    else:
        cfg = synth.config("mid", max_context=384)
        r = np.random.default_rng(71)
        n = 300
        toks = r.integers(0, cfg["vocab_text"], n).astype(np.int32)
        codes = r.integers(0, cfg["codebook_size"], (n, 10)).astype(np.int32)
        mask = np.zeros(n, np.uint8)
        mask[:200] = 1
        rep = _int8_teacher_forced("mid", 3, "i8" if case == "int8" else "f8", prompt=(toks, mask, codes),
                                   max_context=384, prefill_precision=1)
    assert rep["tokens_checked"] > 0


@pytest.mark.parametrize("G,D", [(1, 128), (2, 64), (8, 64), (8, 128)])
def test_fp16_prefill_attention_group_sizes(G, D):
    """The fp16 prefill attention at 1, 2 and 8 q heads per KV head (two 16-row tiles per workgroup
    below 8, one at 8; the 128-VGPR form only from 4 up): a 530-position prompt, so row blocks of
    every height and key ranges split over workgroups, then 2 frames against the oracle."""
    hq = 4 if (G, D) == (1, 128) else 8
    cfg = synth.micro_config(seed=90 + G + D, slow_layers=2, fast_layers=1, hidden=512, n_q_heads=hq,
                             n_kv_heads=hq // G, head_dim=D, ffn=1024, vocab_text=1000, codebook_size=256,
                             weight_dtype="bf16", max_context=576)
    w = synth.make_weights(cfg)
    toks = synth.uniform_ints(91, 0, 530, 0, cfg["vocab_text"])
    frames = oracle_run(cfg, w, toks, None, None, 2)
    ctx = _ctx(cfg, w)
    ctx.set_prefill_precision(1)
    ctx.prefill(0, toks)
    rep = compare_frames(ctx, 0, frames, cfg).finish()
    _say(f"[parity] fp16 prefill G {G} D {D}: {rep}")
    ctx.close()


def _scaled_bf16(a, k):
    """bf16 bits of the tensor times 2^k (exact: a power-of-two scale keeps every bf16 value)."""
    f = synth.as_f32(a) * np.float32(2.0 ** k)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("where", ["norm", "swiglu_split", "swiglu", "attention"])
def test_fp16_prefill_out_of_range_is_an_error(where):
    """A first Slow layer whose prefill activations leave fp16's range, at each kind of producer: an
    attention-norm gain of 30000 (the RMSNorm split), gate and up rows scaled by 256 (the SwiGLU
    written by the split-K reduction for a 64-token prompt, and by the GEMM epilogue for 600 tokens),
    value rows scaled by 2^17 (values beyond 65504 reach the fp16 attention and its output).  The
    fp16 prefill fails with S2AR_E_NUMERIC, keeps the stream's position and leaves it not ready to
    decode; the default precision then prefills the same prompt and decodes."""
    cfg = synth.config("mid", max_context=704)
    w = synth.make_weights(cfg)
    names = [n for n, _, _ in synth.tensor_specs(cfg)]
    pre = "slow.layers.0."
    if where == "norm":
        big = np.array([30000.0], np.float32).view(np.uint32) >> 16  # bf16 bits of 30000 (exact)
        w[names.index(pre + "attn_norm")][:] = np.uint16(big[0])
    elif where.startswith("swiglu"):
        for t in ("w_gate", "w_up"):
            w[names.index(pre + t)] = _scaled_bf16(w[names.index(pre + t)], 8)
    else:
        w[names.index(pre + "wv")] = _scaled_bf16(w[names.index(pre + "wv")], 17)
    if where == "swiglu":
        toks = synth.uniform_ints(79, 0, 600, 0, cfg["vocab_text"])
    else:
        toks, _, _ = synth.make_prompt(cfg)
    ctx = _ctx(cfg, w)
    with pytest.raises(s2ar.S2arError) as e:
        ctx.set_prefill_precision(2)
    assert e.value.code == -1
    ctx.set_prefill_precision(1)
    with pytest.raises(s2ar.S2arError) as e:
        ctx.prefill(0, toks)
    assert e.value.code == -7 and ctx.position(0) == 0
    with pytest.raises(s2ar.S2arError) as e:
        ctx.decode_frames([0], 1)
    assert e.value.code == -4
    ctx.set_prefill_precision(0)
    ctx.prefill(0, toks)
    assert ctx.position(0) == len(toks)
    out = ctx.decode_frames([0], 2)
    assert out.shape == (2, 1, cfg["n_codebooks"]) and (out >= 0).all()
    ctx.close()


def test_fp16_prefill_needs_the_matrix_core_prefill():
    """fp32 weights prefill position by position: precision 1 is refused there."""
    cfg = synth.config("tiny")
    ctx = _ctx(cfg, synth.make_weights(cfg))
    with pytest.raises(s2ar.S2arError) as e:
        ctx.set_prefill_precision(1)
    assert e.value.code == -1
    ctx.set_prefill_precision(0)
    ctx.close()


@pytest.mark.parametrize("fmt", ["i8", "f8"])
def test_int8_weights_batched_mid_ragged(fmt):
    """8-bit weights through the batched kernels (tiled 8-bit copies, widened to bf16 for the matrix
    cores, row scales on the partial sums) for five ragged streams."""
    cfg = synth.config("mid", max_context=640)
    w = synth.make_weights(cfg)
    ocfg, ow = quant_reference(cfg, w, fmt)
    prompts = _ragged_prompts(cfg, [64, 17, 300, 130, 5], 31)
    per_stream = _oracle_frames_per_stream(ocfg, ow, prompts, 3)
    del ow
    ctx = _ctx(dict(cfg, weight_dtype=fmt), w, max_streams=6)
    ids = [0, 2, 3, 4, 5]
    for s_, p in zip(ids, prompts):
        ctx.prefill(s_, p)
    rep = _compare_batch(ctx, ids, per_stream, cfg, Report()).finish()
    _say(f"[parity] batched mid, {fmt} weights: {rep}")
    ctx.close()


@pytest.mark.timeout(1500)
def test_int8_weights_batched_full_shape():
    """Int8 weights, batched decode at the full S2 shape (three streams, bf16 keys)."""
    cfg = synth.config("multi_stream", max_context=256, kv_dtype="k_bf16")
    w = synth.make_weights(cfg)
    ocfg, ow = quant_reference(cfg, w, "i8")
    prompts = _ragged_prompts(cfg, [41, 9, 70], 32)
    per_stream = _oracle_frames_per_stream(ocfg, ow, prompts, 2)
    del ow
    gc.collect()
    ctx = _ctx(dict(cfg, weight_dtype="i8"), w, max_streams=4)
    del w
    gc.collect()
    ids = [1, 0, 3]
    for s_, p in zip(ids, prompts):
        ctx.prefill(s_, p)
    rep = _compare_batch(ctx, ids, per_stream, cfg, Report()).finish()
    _say(f"[parity] batched full, int8 weights: {rep}")
    ctx.close()


@pytest.mark.parametrize("name,fmt", [("mid", "i8"), ("mid", "f8"), ("full", "i8")])
def test_8bit_weights_graph_frames_equal_the_eager_path(name, fmt):
    """Graph-replayed frames with 8-bit weights, whose Fast steps 2..9 finish the previous Fast pick
    inside their first QKV GEMV, give the eager path's codes (which the teacher-forced tests hold to
    the oracle) bit for bit."""
    cfg = synth.config(name)
    w = synth.make_weights(cfg)
    toks, _, _ = synth.make_prompt(cfg)
    ctx = _ctx(dict(cfg, weight_dtype=fmt), w, max_streams=2)
    del w
    gc.collect()
    ctx.prefill(0, toks)
    ctx.prefill(1, toks)
    n = 4
    graph = ctx.decode_frames([0], n)[:, 0]
    eager = np.stack([ctx.debug_frame(1)["own_codes"] for _ in range(n)])
    assert np.array_equal(graph, eager), "graph replay and the eager path disagree"
    ctx.close()


def test_int8_weights_mid_teacher_forced():
    """Int8 layer matrices and heads with per-row scales (quantised by the library at create) against
    the oracle fed the same quantisation (its own quantiser, dequantised): the bf16 acceptance bar."""
    assert _int8_teacher_forced("mid", 8)["tokens_checked"] > 0


@pytest.mark.timeout(1200)
def test_int8_weights_full_teacher_forced():
    assert _int8_teacher_forced("full", 2)["tokens_checked"] > 0


def test_int8_semantic_slice_head_with_stop_id_mid():
    """The semantic-slice head built from quantised rows (the semantic rows plus the stop row, each
    with its own scale) against the oracle's full head on the same int8 quantisation."""
    cfg = synth.config("mid", head_slice=1, eos_id=7)
    w = synth.make_weights(cfg)
    ocfg, ow = quant_reference(cfg, w, "i8")
    toks, _, _ = synth.make_prompt(cfg)
    frames = oracle_run(ocfg, ow, toks, None, None, 4)
    del ow
    ctx = _ctx(dict(cfg, weight_dtype="i8"), w)
    ctx.prefill(0, toks)
    rep = compare_frames(ctx, 0, frames, cfg).finish()
    _say(f"[parity] mid int8, slice head, stop id 7: {rep}")
    ctx.close()
    assert rep["tokens_checked"] > 0


def test_fp8_weights_mid_teacher_forced():
    """FP8 E4M3 layer matrices and heads with per-row scales, decoded by gfx950's hardware
    conversion, against the oracle fed its own E4M3 quantisation: the bf16 acceptance bar."""
    assert _int8_teacher_forced("mid", 8, "f8")["tokens_checked"] > 0


@pytest.mark.timeout(1200)
def test_fp8_weights_full_teacher_forced():
    assert _int8_teacher_forced("full", 2, "f8")["tokens_checked"] > 0


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


def test_time_frames_per_replay_events():
    """s2ar_time_frames: one positive duration per frame, the stream advances like decode_frames, and
    the next frame's codes equal a decode_frames run over the same frames."""
    cfg = synth.config("tiny")
    w = synth.make_weights(cfg)
    toks, _, _ = synth.make_prompt(cfg)
    ctx = _ctx(cfg, w, max_streams=2)
    ctx.prefill(0, toks)
    ctx.prefill(1, toks)
    ms = ctx.time_frames(0, 3)
    assert ms.shape == (3,) and np.all(ms > 0) and ctx.position(0) == len(toks) + 3
    ctx.decode_frames([1], 3)
    assert np.array_equal(ctx.decode_frames([0], 1), ctx.decode_frames([1], 1))
    with pytest.raises(s2ar.S2arError):
        ctx.time_frames(0, 0)
    ctx.close()


def test_time_kernel_gemv_and_stream_read():
    """The bench's timing entry: the gate/up GEMV and the plain streaming read of the same weights."""
    cfg = synth.config("mid")
    w = synth.make_weights(cfg)
    ctx = _ctx(cfg, w)
    ms0, b0 = ctx.time_kernel(0, 4)
    ms1, b1 = ctx.time_kernel(1, 4)
    s = cfg["slow"]
    assert b1 == 2 * s["ffn"] * s["hidden"] * 2 and b0 > b1
    assert ms0 > 0 and ms1 > 0
    with pytest.raises(s2ar.S2arError) as e:
        ctx.time_kernel(2, 1)
    assert e.value.code == -1
    ctx.close()


# ------------------------------------------------------------------------------ multi-stream

def _oracle_frames_per_stream(cfg, w, prompts, n):
    return [oracle_run(cfg, w, t, None, None, n) for t in prompts]


def _compare_batch(ctx, ids, per_stream, cfg, rep):
    """Drive the batched kernels teacher-forced through every stream's oracle frames."""
    K, Vt = cfg["codebook_size"], cfg["vocab_text"]
    n = len(per_stream[0])
    for t in range(n):
        forced = np.stack([fr[t]["codes"] for fr in per_stream])
        outs = ctx.debug_frame_batch(ids, forced)
        for b, (g, frs) in enumerate(zip(outs, per_stream)):
            f = frs[t]
            tag = f"stream {ids[b]} frame {t}"
            rep.token(f"{tag} c0", int(g["own_codes"][0]), int(f["codes"][0]), f["c0_margin"])
            for j in range(9):
                for l in range(cfg["fast"]["n_layers"]):
                    rep.cos(f"{tag} fast step {j + 1} layer {l}", g["fast_resid"][j, l], f["fast"]["resid"][j, l])
                rep.logits(f"{tag} fast step {j + 1} logits", g["fast_logits"][j], f["fast"]["logits"][j])
                rep.token(f"{tag} c{j + 1}", int(g["own_codes"][j + 1]), int(f["fast"]["codes"][j]), f["fast"]["margins"][j])
                assert int(g["own_codes"][j + 1]) == int(np.argmax(g["fast_logits"][j]))
            for l in range(cfg["slow"]["n_layers"]):
                rep.cos(f"{tag} slow layer {l}", g["slow_resid"][l], f["slow"]["resid"][l])
            rep.cos(f"{tag} slow h", g["slow_h"], f["slow"]["h"])
            rows = slow_rows(cfg)
            rep.logits(f"{tag} slow logits", g["slow_logits"][rows], f["slow"]["logits"][rows])
            rep.token(f"{tag} next c0", int(g["next_c0"]), int(f["slow"]["c0"]), f["slow"]["margin"])
            assert int(g["next_c0"]) == own_slow_pick(g["slow_logits"], cfg)
    return rep


def _ragged_prompts(cfg, lens, seed):
    return [synth.uniform_ints(seed, 900 + i, n, 0, cfg["vocab_text"]) for i, n in enumerate(lens)]


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16"])
def test_batched_multi_stream_teacher_forced_mid_ragged(kv_dtype):
    """Batched decode kernels (matrix-core GEMVs over several streams, ragged paged attention),
    with an fp32 and a bf16 KV cache."""
    cfg = synth.config("mid", max_context=640, kv_dtype=kv_dtype)
    w = synth.make_weights(cfg)
    lens = [64, 17, 300, 130, 5]
    prompts = _ragged_prompts(cfg, lens, 31)
    per_stream = _oracle_frames_per_stream(cfg, w, prompts, 4)
    ctx = _ctx(cfg, w, max_streams=6)
    ids = [0, 2, 3, 4, 5]
    for s_, p in zip(ids, prompts):
        ctx.prefill(s_, p)
    rep = _compare_batch(ctx, ids, per_stream, cfg, Report()).finish()
    _say(f"[parity] batched mid, {kv_dtype} KV: {rep}")
    ctx.close()


def test_batched_sixteen_streams_mid():
    """A full batch of 16 streams (every MFMA column live) with ragged contexts of 5..300 positions."""
    cfg = synth.config("mid", max_context=384)
    lens = [5, 300, 17, 64, 65, 128, 33, 250, 7, 190, 96, 16, 201, 45, 150, 80]
    prompts = _ragged_prompts(cfg, lens, 41)
    w = synth.make_weights(cfg)
    per_stream = _oracle_frames_per_stream(cfg, w, prompts, 2)
    ctx = _ctx(cfg, w, max_streams=16)
    ids = list(range(16))[::-1]
    for s_, p in zip(ids, prompts):
        ctx.prefill(s_, p)
    rep = _compare_batch(ctx, ids, per_stream, cfg, Report()).finish()
    _say(f"[parity] batched 16 streams mid: {rep}")
    ctx.close()


@pytest.mark.parametrize("G,D,kv", [(1, 128, "f32"), (2, 64, "v_bf16")])
def test_batched_slow_attention_split_and_wavefront_boundaries(G, D, kv):
    """The batched Slow attention takes 256-key splits of four 64-key wavefronts.  Twelve streams
    whose two decoded positions fall on every boundary of that layout: the first and second
    positions, the last key of wavefront 0 and the first of wavefront 1, the last key of a split
    and the first of the next, and past them, at 1 and 2 q heads per KV head (the mid and full
    shapes have 4) and head_dim 128 and 64."""
    cfg = synth.micro_config(seed=60 + G, slow_layers=2, fast_layers=1, hidden=512, n_q_heads=512 // D,
                             n_kv_heads=512 // D // G, head_dim=D, ffn=1024, vocab_text=1000,
                             codebook_size=256, weight_dtype="bf16", max_context=704)
    cfg["kv_dtype"] = kv
    w = synth.make_weights(cfg)
    lens = [1, 62, 63, 64, 127, 254, 255, 256, 300, 510, 511, 600]
    prompts = _ragged_prompts(cfg, lens, 70 + G)
    per_stream = _oracle_frames_per_stream(cfg, w, prompts, 2)
    ctx = _ctx(cfg, w, max_streams=12)
    ids = list(range(12))
    for s_, p in zip(ids, prompts):
        ctx.prefill(s_, p)
    rep = _compare_batch(ctx, ids, per_stream, cfg, Report()).finish()
    _say(f"[parity] batched split boundaries, G {G}, D {D}, {kv} KV: {rep}")
    ctx.close()


def test_batched_slow_attention_eight_heads_per_kv_head():
    """Eight q heads per KV head: the batched Slow attention runs the LDS-tiled kernel with
    192-position splits instead of the four-wavefront kernel; positions on its split and chunk
    boundaries."""
    cfg = synth.micro_config(seed=68, slow_layers=2, fast_layers=1, hidden=512, n_q_heads=8, n_kv_heads=1,
                             head_dim=64, ffn=1024, vocab_text=1000, codebook_size=256, weight_dtype="bf16",
                             max_context=512)
    w = synth.make_weights(cfg)
    lens = [1, 63, 127, 190, 191, 192, 383, 384, 450]
    prompts = _ragged_prompts(cfg, lens, 78)
    per_stream = _oracle_frames_per_stream(cfg, w, prompts, 2)
    ctx = _ctx(cfg, w, max_streams=9)
    ids = list(range(9))
    for s_, p in zip(ids, prompts):
        ctx.prefill(s_, p)
    rep = _compare_batch(ctx, ids, per_stream, cfg, Report()).finish()
    _say(f"[parity] batched G 8: {rep}")
    ctx.close()


@pytest.mark.timeout(1500)
def test_batched_multi_stream_teacher_forced_full_shape():
    """Batched decode at the full S2 shape, three streams with different contexts."""
    cfg = synth.config("multi_stream", max_context=256)
    w = synth.make_weights(cfg)
    lens = [41, 9, 70]
    prompts = _ragged_prompts(cfg, lens, 32)
    per_stream = _oracle_frames_per_stream(cfg, w, prompts, 2)
    ctx = _ctx(cfg, w, max_streams=4)
    ids = [1, 0, 3]
    for s_, p in zip(ids, prompts):
        ctx.prefill(s_, p)
    rep = _compare_batch(ctx, ids, per_stream, cfg, Report()).finish()
    _say(f"[parity] batched full: {rep}")
    ctx.close()


@pytest.mark.timeout(900)
def test_batched_kernels_at_the_multi_stream_contexts_match_the_batch1_path():
    """The 16-stream workload at its real shapes and contexts (full S2 shape, 920..3948 positions):
    too long for the fp64 oracle, so the batched kernels are held to the batch-1 path, which the
    oracle pins at the full shape.  Streams 16 and 17 repeat the shortest and the longest prompt;
    one batched frame of streams 0..15 and one batch-1 frame of each repeat, forced with the same
    codes, must agree to the acceptance bar."""
    cfg = synth.config("multi_stream")
    lens = synth.prompt_lengths(cfg)
    w = synth.make_weights(cfg)
    ctx = _ctx(cfg, w, max_streams=18)
    del w
    gc.collect()
    prompts = [synth.make_prompt(cfg, i)[0] for i in range(16)]
    for i, p in enumerate(prompts):
        ctx.prefill(i, p)
    lo, hi = int(np.argmin(lens)), int(np.argmax(lens))
    ctx.prefill(16, prompts[lo])
    ctx.prefill(17, prompts[hi])
    forced = synth.uniform_ints(44, 0, 16 * 10, 0, cfg["codebook_size"]).reshape(16, 10).astype(np.int32)
    outs = ctx.debug_frame_batch(list(range(16)), forced)
    K, Vt = cfg["codebook_size"], cfg["vocab_text"]
    rep = Report()
    for src, rep_id in ((lo, 16), (hi, 17)):
        one = ctx.debug_frame(rep_id, forced=forced[src])
        b = outs[src]
        tag = f"stream {src} ({lens[src]} positions)"
        for l in range(cfg["slow"]["n_layers"]):
            rep.cos(f"{tag} slow layer {l}", b["slow_resid"][l], one["slow_resid"][l].astype(np.float64))
        rep.cos(f"{tag} slow h", b["slow_h"], one["slow_h"].astype(np.float64))
        rep.logits(f"{tag} slow logits", b["slow_logits"], one["slow_logits"].astype(np.float64))
        srt = np.sort(one["slow_logits"][Vt:Vt + K].astype(np.float64))
        rep.token(f"{tag} next c0", int(b["next_c0"]), int(one["next_c0"]), srt[-1] - srt[-2])
        for j in range(9):
            for l in range(cfg["fast"]["n_layers"]):
                rep.cos(f"{tag} fast step {j + 1} layer {l}", b["fast_resid"][j, l], one["fast_resid"][j, l].astype(np.float64))
            fl = one["fast_logits"][j].astype(np.float64)
            rep.logits(f"{tag} fast step {j + 1} logits", b["fast_logits"][j], fl)
            srt = np.sort(fl)
            rep.token(f"{tag} c{j + 1}", int(b["own_codes"][j + 1]), int(one["own_codes"][j + 1]), srt[-1] - srt[-2])
    r = rep.finish()
    _say(f"[parity] batched vs batch-1 at contexts {min(lens)}..{max(lens)}: {r}")
    ctx.close()


def test_batched_graph_equals_eager_batched_frame():
    cfg = synth.config("mid", max_context=256)
    w = synth.make_weights(cfg)
    prompts = _ragged_prompts(cfg, [20, 33, 7], 33)
    ids = [0, 1, 2]
    runs = []
    for eager in (False, True):
        ctx = _ctx(cfg, w, max_streams=3)
        for s_, p in zip(ids, prompts):
            ctx.prefill(s_, p)
        if eager:
            runs.append(np.stack([np.stack([o["own_codes"] for o in ctx.debug_frame_batch(ids)]) for _ in range(6)]))
        else:
            runs.append(ctx.decode_frames(ids, 6))
        ctx.close()
    assert np.array_equal(runs[0], runs[1])


# ----------------------------------------------------- semantic-slice head and the stop id

def _stop_setup(cfg, w, toks, n_frames=6):
    """A stop id (a text id) and the oracle's run with it: the text id with the largest logit at one
    of the oracle's early Slow picks, chosen so that the run stops after at least one frame and the
    stop pick's margin decides it.  Returns (eos, frames, all_margins_decide)."""
    free = oracle_run(cfg, w, toks, None, None, 4)
    Vt = cfg["vocab_text"]
    for at in (2, 1, 3, 0):
        eos = int(np.argmax(free[at]["slow"]["logits"][:Vt]))
        ce = dict(cfg, eos_id=eos)
        pre = {}
        frames = oracle_run(ce, w, toks, None, None, n_frames, prefill_out=pre)
        if pre["c0"] < 0 or not frames or frames[-1]["slow"]["c0"] != -1:
            continue
        if frames[-1]["slow"]["margin"] <= 5e-2:
            continue
        margins = [f["c0_margin"] for f in frames] + [m for f in frames for m in f["fast"]["margins"]]
        return eos, frames, min(margins) > 5e-2
    pytest.skip("no early text id stops this run by a deciding margin")


@pytest.mark.parametrize("head_slice", [0, 1])
def test_stop_id_teacher_forced(head_slice):
    """The Slow pick with a stop id (full head, and the semantic-slice head that keeps only the
    semantic rows plus the stop row): every frame matches the oracle run with the same stop id, and
    the stop pick itself comes out as -1."""
    cfg = synth.config("mid", head_slice=head_slice)
    w = synth.make_weights(cfg)
    toks, _, _ = synth.make_prompt(cfg)
    eos, frames, _ = _stop_setup(cfg, w, toks)
    ce = dict(cfg, eos_id=eos)
    ctx = _ctx(ce, w)
    ctx.prefill(0, toks)
    rep = compare_frames(ctx, 0, frames, ce).finish()
    _say(f"[parity] stop id {eos}, head_slice {head_slice}: {len(frames)} frames then the stop; {rep}")
    # the oracle's stop is the GPU's too: the next frame comes out as the stop, then the stream has ended
    assert np.all(ctx.decode_frames([0], 1) == -1)
    with pytest.raises(s2ar.S2arError):
        ctx.decode_frames([0], 1)
    ctx.close()


def test_semantic_slice_head_batched_teacher_forced():
    """The batched Slow head over the semantic slice plus a stop row, three ragged streams."""
    cfg = synth.config("mid", max_context=640, head_slice=1, eos_id=5)
    w = synth.make_weights(cfg)
    prompts = _ragged_prompts(cfg, [64, 17, 130], 34)
    per_stream = _oracle_frames_per_stream(cfg, w, prompts, 3)
    ctx = _ctx(cfg, w, max_streams=3)
    ids = [2, 0, 1]
    for s_, p in zip(ids, prompts):
        ctx.prefill(s_, p)
    n = min(len(f) for f in per_stream)
    rep = _compare_batch(ctx, ids, [f[:n] for f in per_stream], cfg, Report()).finish()
    _say(f"[parity] batched slice head: {rep}")
    ctx.close()


@pytest.mark.parametrize("batched", [False, True])
def test_stop_id_ends_free_running_stream(batched):
    """decode_frames with a stop id: the stream's frames up to the stop are the oracle's, the stop
    frame and every later frame of the call are -1, a further decode is refused, and a prefill that
    appends to the stream lets it decode again."""
    cfg = synth.config("mid", max_context=640, head_slice=1 if batched else 0)
    w = synth.make_weights(cfg)
    toks, _, _ = synth.make_prompt(cfg)
    eos, frames, decided = _stop_setup(cfg, w, toks)
    ce = dict(cfg, eos_id=eos)
    stop = len(frames)
    ctx = _ctx(ce, w, max_streams=3)
    ctx.prefill(0, toks)
    ids = [0]
    if batched:
        for s_, p in zip((1, 2), _ragged_prompts(cfg, [40, 90], 35)):
            ctx.prefill(s_, p)
        ids = [1, 0, 2]
    out = ctx.decode_frames(ids, stop + 3)
    rows = out[:, ids.index(0)]
    if decided:
        assert np.array_equal(rows[:stop], np.stack([f["codes"] for f in frames]))
        assert np.all(rows[stop:] == -1)
    for s_ in range(len(ids)):  # once a stream's frame is -1, so is every later frame of the call
        r = out[:, s_, 0]
        first = int(np.argmax(r < 0)) if np.any(r < 0) else len(r)
        assert np.all(out[first:, s_] == -1) and np.all(out[:first, s_] >= 0)
    with pytest.raises(s2ar.S2arError):
        ctx.decode_frames([0], 1)
    live = [s_ for i, s_ in enumerate(ids) if s_ != 0 and np.all(out[:, i] >= 0)]
    if live:
        assert ctx.decode_frames(live, 1).shape == (1, len(live), 10)
    ctx.prefill(0, toks[:3])
    assert ctx.decode_frames([0], 1).shape == (1, 1, 10)
    ctx.close()
