"""Batched decode at the 16-stream workload's own contexts against the oracle.

The workload's sixteen contexts (920..3948 positions, drawn by the seed-4 generator) run through
the batched kernels: matrix-core GEMVs over all sixteen streams, ragged paged attention split into
192-position pieces merged in order (up to 21 splits at the longest context), head_dim 128, GQA
32/8.  The oracle decodes four of the streams (the shortest, the longest and two drawn at random
among those of at most 2500 positions), teacher-forced for two frames.

The model has the full S2 layer shape (hidden 2560, 32/8 heads, head_dim 128, FFN 9728, vocabulary
151,680 + 4,096) with 2 Slow layers and 1 Fast layer: every kernel of a layer runs at its real
shape and the real contexts, and the fp64 oracle finishes the four prefills (about 9,000 positions)
in minutes instead of the hours 36 layers would take.  The 36-layer model at these contexts is
held to the batch-1 path in test_gpu_parity.py.  A seventeenth stream repeats the longest prompt
and goes through the batch-1 frame (64-position attention splits, 62 of them), against the same
oracle frames.
"""
import gc
import sys

import numpy as np
import pytest

from dual_ar_codec_amd import s2ar, synth

from parity_util import Report, compare_frames, oracle_run, own_slow_pick, remember_codebook, slow_rows

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _compare_batch(ctx, ids, per_stream, forced_all, cfg, rep):
    """Batched frames of every stream in ids (forced with forced_all[t][i]); the streams with
    oracle frames (per_stream[i] not None) are checked against them."""
    n = len(forced_all)
    for t in range(n):
        outs = ctx.debug_frame_batch(ids, forced_all[t])
        for b, frs in enumerate(per_stream):
            if frs is None:
                continue
            g, f = outs[b], frs[t]
            tag = f"stream {ids[b]} frame {t}"
            rep.token(f"{tag} c0", int(g["own_codes"][0]), int(f["codes"][0]), f["c0_margin"])
            for j in range(9):
                for l in range(cfg["fast"]["n_layers"]):
                    rep.cos(f"{tag} fast step {j + 1} layer {l}", g["fast_resid"][j, l], f["fast"]["resid"][j, l])
                rep.logits(f"{tag} fast step {j + 1} logits", g["fast_logits"][j], f["fast"]["logits"][j])
                rep.token(f"{tag} c{j + 1}", int(g["own_codes"][j + 1]), int(f["fast"]["codes"][j]),
                          f["fast"]["margins"][j])
                assert int(g["own_codes"][j + 1]) == int(np.argmax(g["fast_logits"][j]))
            for l in range(cfg["slow"]["n_layers"]):
                rep.cos(f"{tag} slow layer {l}", g["slow_resid"][l], f["slow"]["resid"][l])
            rep.cos(f"{tag} slow h", g["slow_h"], f["slow"]["h"])
            rows = slow_rows(cfg)
            rep.logits(f"{tag} slow logits", g["slow_logits"][rows], f["slow"]["logits"][rows])
            rep.token(f"{tag} next c0", int(g["next_c0"]), int(f["slow"]["c0"]), f["slow"]["margin"])
            assert int(g["next_c0"]) == own_slow_pick(g["slow_logits"], cfg)
    return rep


@pytest.mark.timeout(1100)
def test_batched_decode_at_the_sixteen_stream_contexts_against_the_oracle():
    import torch

    torch.cuda.set_device(0)
    cfg = synth.config("multi_stream")
    cfg["slow"] = dict(cfg["slow"], n_layers=2)
    cfg["fast"] = dict(cfg["fast"], n_layers=1)
    lens = synth.prompt_lengths(cfg)
    lo, hi = int(np.argmin(lens)), int(np.argmax(lens))
    rest = [i for i in range(16) if i not in (lo, hi) and lens[i] <= 2500]
    pick = synth.uniform_ints(cfg["seed"], 4242, 2, 0, len(rest))
    r1 = rest[int(pick[0])]
    r2 = [i for i in rest if i != r1][int(pick[1]) % (len(rest) - 1)]
    checked = [lo, hi, r1, r2]
    _say(f"[multi] contexts {lens}; oracle on streams {checked} ({[lens[i] for i in checked]} positions)")
    w = synth.make_weights(cfg)
    prompts = [synth.make_prompt(cfg, i)[0] for i in range(16)]
    n_frames = 2
    per_stream = [None] * 16
    for i in checked:
        _say(f"[multi] oracle: stream {i}, {lens[i]} positions + {n_frames} frames")
        per_stream[i] = oracle_run(cfg, w, prompts[i], None, None, n_frames)
    # streams without oracle frames are forced with seeded codes
    other = synth.uniform_ints(cfg["seed"], 4343, n_frames * 16 * 10, 0, cfg["codebook_size"])
    other = other.reshape(n_frames, 16, 10).astype(np.int32)
    forced = [np.stack([per_stream[i][t]["codes"] if per_stream[i] is not None else other[t, i] for i in range(16)])
              for t in range(n_frames)]
    # the fp32 KV cache, and bf16 keys with fp32 values (the 16-stream workload's cache in bench.py)
    for kv in ("f32", "k_bf16"):
        ckv = dict(cfg, kv_dtype=kv)
        _say(f"[multi] GPU, {kv} KV: prefill 16 streams + a repeat of the longest")
        ctx = s2ar.Context(ckv, w, max_streams=17)
        remember_codebook(ctx, ckv, w)
        for i, p in enumerate(prompts):
            ctx.prefill(i, p)
        ctx.prefill(16, prompts[hi])
        ids = list(range(16))
        rep = _compare_batch(ctx, ids, per_stream, forced, ckv, Report()).finish()
        _say(f"[multi] {kv} KV, batched at contexts {min(lens)}..{max(lens)}, oracle on {checked}: {rep}")
        rep1 = compare_frames(ctx, 16, per_stream[hi], ckv).finish()
        _say(f"[multi] {kv} KV, batch-1 at {lens[hi]} positions: {rep1}")
        ctx.close()
        gc.collect()
