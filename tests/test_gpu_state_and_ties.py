"""Stream state across calls, greedy-pick ties and the device-memory hook, on an MI355X.

- A shared prefix followed by a one-position suffix (the position-by-position prefill path) leaves
  both streams equal to the oracle: the suffix is appended at the right position and the shared
  pages are not written.
- A stream that stops is rewound to the positions the model decoded, so a prefill after the stop
  continues exactly like the oracle's context.
- Ties of the greedy pick go to the lowest index ("SGLang Day-0 Support for FishAudio S2",
  Background and Motivation: greedy constrained decoding; argmax indices must be bit-exact): head
  rows are duplicated so that two logits are bit-identical maxima, within one wavefront, across the
  wavefronts of a block, across blocks read by different lanes of the second pass and by the same
  lane, for the Fast head, the full and the semantic-slice Slow head, batch-1 and batched.
- The optional device allocator supplies every block and gets every block back.
"""
import gc
import sys

import numpy as np
import pytest

import oracle
from dual_ar_codec_amd import s2ar, synth

from parity_util import Report, compare_frames, oracle_run, quant_reference, remember_codebook

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


# ------------------------------------------------------------------ shared prefix + short suffix

@pytest.mark.parametrize("name,fmt,n_shared", [("tiny", None, 16), ("tiny", None, 9), ("mid", "i8", 37)])
def test_shared_prefix_then_one_position_suffix(name, fmt, n_shared):
    """fp32 and int8 contexts prefill position by position.  Stream 1 takes the first n_shared
    positions of stream 0 and prefills one position of its own; both streams then match the oracle
    on their full prompts."""
    cfg = synth.config(name)
    w = synth.make_weights(cfg)
    ocfg, ow = (cfg, w) if fmt is None else quant_reference(cfg, w, fmt)
    r = np.random.default_rng(61)
    base = r.integers(0, cfg["vocab_text"], n_shared + 6).astype(np.int32)
    other = np.concatenate([base[:n_shared], r.integers(0, cfg["vocab_text"], 1)]).astype(np.int32)
    refs = [oracle_run(ocfg, ow, t, None, None, 3) for t in (base, other)]
    ctx = _ctx(dict(cfg, weight_dtype=fmt) if fmt else cfg, w, max_streams=2)
    ctx.prefill(0, base)
    ctx.share_prefix(0, 1, n_shared)
    ctx.prefill(1, other[n_shared:])
    assert ctx.position(1) == n_shared + 1
    rep1 = compare_frames(ctx, 1, refs[1], cfg).finish()
    rep0 = compare_frames(ctx, 0, refs[0], cfg).finish()
    _say(f"[state] {name} {fmt} share {n_shared} + 1: {rep0} {rep1}")
    ctx.close()


# ------------------------------------------------------------------ stop, then continue

def _oracle_state_after(cfg, w, toks, frames):
    m = oracle.Model(cfg, w)
    st = m.new_state()
    st.prefill(toks)
    for f in frames:
        st.slow_step(f["codes"])
    return m, st


def _oracle_continue(m, st, toks2, n):
    pre = st.prefill(toks2)
    h, c0, c0m = pre["h"], pre["c0"], pre["margin"]
    out = []
    for _ in range(n):
        fl = m.fast_loop(h, taps=True)
        codes = np.concatenate([[c0], fl["codes"]]).astype(np.int32)
        nxt = st.slow_step(codes, taps=True)
        out.append(dict(codes=codes, c0_margin=c0m, fast=fl, slow=nxt))
        h, c0, c0m = nxt["h"], nxt["c0"], nxt["margin"]
    return out


def _find_stop(cfg, w, toks, n_frames=6):
    """A text id that the oracle picks as the stop after at least one frame, by a deciding margin."""
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


@pytest.mark.parametrize("batched", [False, True])
def test_prefill_after_a_stop_continues_like_the_oracle(batched):
    """decode_frames runs past the stop (frames after it are -1).  The stream is rewound to the
    position after the Slow step that picked the stop, so a prefill of three more text positions
    and the frames after it equal the oracle continuing from exactly the decoded positions."""
    cfg = synth.config("mid", max_context=640)
    w = synth.make_weights(cfg)
    toks, _, _ = synth.make_prompt(cfg)
    eos, frames, decided = _find_stop(cfg, w, toks)
    ce = dict(cfg, eos_id=eos)
    stop = len(frames)
    ctx = _ctx(ce, w, max_streams=3)
    ctx.prefill(0, toks)
    ids = [0]
    if batched:
        for s_, p in zip((1, 2), (toks[:40], toks[:50])):
            ctx.prefill(s_, p)
        ids = [1, 0, 2]
    if decided:  # free-running: the GPU's own frames are the oracle's up to the stop
        out = ctx.decode_frames(ids, stop + 3)[:, ids.index(0)]
        assert np.array_equal(out[:stop], np.stack([f["codes"] for f in frames]))
        assert np.all(out[stop:] == -1)
    else:  # teacher-forced up to the stop, then the stop comes out in the first frame of a call
        compare_frames(ctx, 0, frames, ce).finish()
        out = ctx.decode_frames(ids, 3)[:, ids.index(0)]
        assert np.all(out == -1)
    assert ctx.position(0) == len(toks) + stop
    toks2 = synth.uniform_ints(cfg["seed"], 88, 3, 0, cfg["vocab_text"])
    m, st = _oracle_state_after(ce, w, toks, frames)
    cont = _oracle_continue(m, st, toks2, 3)
    ctx.prefill(0, toks2)
    assert ctx.position(0) == len(toks) + stop + 3
    rep = compare_frames(ctx, 0, cont, ce).finish()
    _say(f"[state] stop at frame {stop} (decided {decided}, batched {batched}), then prefill 3: {rep}")
    ctx.close()


def test_time_frames_refuses_a_context_with_a_stop_id():
    cfg = synth.config("tiny", eos_id=3)
    w = synth.make_weights(cfg)
    ctx = _ctx(cfg, w)
    toks, _, _ = synth.make_prompt(cfg)
    ctx.prefill(0, toks)
    with pytest.raises(s2ar.S2arError) as e:
        ctx.time_frames(0, 2)
    assert e.value.code == -1 and ctx.position(0) == len(toks)
    ctx.close()


# ------------------------------------------------------------------ greedy-pick ties

def _names(cfg):
    return [n for n, _, _ in synth.tensor_specs(cfg)]


def _tie_rows(best, n_rows, kind):
    """Rows whose head row becomes a copy of row `best`, by where the copy sits relative to it in
    the GEMV's pick: 8 rows per block (4 wavefronts x 2 rows), the second pass reading block b in
    lane b % 256."""
    if kind == "wave":        # the other row of the same wavefront
        return [best ^ 1]
    if kind == "block":       # same block of 8 rows, another wavefront
        return [(best // 8) * 8 + ((best % 8) + 4) % 8]
    if kind == "lane":        # another block read by another lane of the second pass
        return [(best + 1000) % n_rows, (best + n_rows - 1000) % n_rows]
    if kind == "same_lane":   # another block read by the same lane (256 blocks apart)
        return [(best + 2048) % n_rows]
    raise ValueError(kind)


def _tie_case(kind, head_slice):
    cfg = synth.config("mid", max_context=256, head_slice=head_slice)
    w = synth.make_weights(cfg)
    names = _names(cfg)
    toks, _, _ = synth.make_prompt(cfg)
    Vt, K = cfg["vocab_text"], cfg["codebook_size"]
    # the frame-1 codes the GPU is forced with (the unmodified model's own), and the rows to copy
    m = oracle.Model(cfg, w)
    st = m.new_state()
    pre = st.prefill(toks)
    fl = m.fast_loop(pre["h"], taps=True)
    forced = np.concatenate([[pre["c0"]], fl["codes"]]).astype(np.int32)
    nxt = st.slow_step(forced, taps=True)
    slow_best = int(np.argmax(nxt["logits"][Vt:Vt + K]))      # semantic code of the Slow pick
    js = int(np.argmax(fl["margins"]))                          # the Fast step with the widest margin
    fast_best = int(np.argmax(fl["logits"][js]))
    s_dups = _tie_rows(slow_best, K, kind)
    f_dups = _tie_rows(fast_best, K, kind)
    del m, st
    w2 = [a.copy() if n in ("slow.head", "fast.head") else a for a, n in zip(w, names)]
    sh, fh = w2[names.index("slow.head")], w2[names.index("fast.head")]
    for d in s_dups:
        sh[Vt + d] = sh[Vt + slow_best]
    for d in f_dups:
        fh[d] = fh[fast_best]
    # the oracle on the modified weights, teacher-forced with the same codes
    m = oracle.Model(cfg, w2)
    st = m.new_state()
    st.prefill(toks)
    ofl = m.fast_loop(pre["h"], forced=forced[1:], taps=True)
    onx = st.slow_step(forced, taps=True)
    return cfg, w2, toks, forced, (slow_best, s_dups, onx), (js, fast_best, f_dups, ofl)


def _check_tie(tag, logits, pick, best, dups, oracle_logits, oracle_pick):
    want = min([best] + dups)
    # the copies give bit-identical logits on the device too
    for d in dups:
        assert logits[d] == logits[best], f"{tag}: row {d} logit {logits[d]!r} != row {best} {logits[best]!r}"
    # the oracle's pick is the lowest tied index (its margin to the rest decides it), so is the GPU's
    assert oracle_pick == want, (tag, oracle_pick, want)
    top = np.sort(np.delete(oracle_logits, [best] + dups))[-1]
    assert oracle_logits[best] - top > 5e-2, f"{tag}: the tied rows do not decide the pick"
    assert pick == want, f"{tag}: GPU picked {pick}, the lowest tied index is {want}"


@pytest.mark.parametrize("kind", ["wave", "block", "lane", "same_lane"])
@pytest.mark.parametrize("head_slice", [0, 1])
def test_argmax_ties_go_to_the_lowest_index(kind, head_slice):
    cfg, w2, toks, forced, slow, fast = _tie_case(kind, head_slice)
    slow_best, s_dups, onx = slow
    js, fast_best, f_dups, ofl = fast
    Vt, K = cfg["vocab_text"], cfg["codebook_size"]
    ctx = _ctx(cfg, w2, max_streams=4)
    for s_ in range(4):
        ctx.prefill(s_, toks)
    # batch-1 (stream 0) and batched (streams 1..3 together)
    g1 = ctx.debug_frame(0, forced=forced)
    gb = ctx.debug_frame_batch([1, 2, 3], np.stack([forced] * 3))
    for tag, g in [("batch-1", g1)] + [(f"batched row {i}", o) for i, o in enumerate(gb)]:
        sl = np.asarray(g["slow_logits"][Vt:Vt + K])
        _check_tie(f"{tag} slow ({kind}, slice {head_slice})", sl, int(g["next_c0"]), slow_best, s_dups,
                   onx["logits"][Vt:Vt + K], int(onx["c0"]))
        _check_tie(f"{tag} fast step {js + 1} ({kind})", np.asarray(g["fast_logits"][js]),
                   int(g["own_codes"][js + 1]), fast_best, f_dups, ofl["logits"][js], int(ofl["codes"][js]))
        # every step's pick is the lowest index among the device's own maxima
        for j in range(9):
            assert int(g["own_codes"][j + 1]) == int(np.argmax(g["fast_logits"][j]))
    _say(f"[ties] {kind}, slice {head_slice}: slow {slow_best} ~ {s_dups}, fast {fast_best} ~ {f_dups}")
    ctx.close()


@pytest.mark.parametrize("kind", ["wave", "block", "lane", "same_lane"])
def test_graph_frames_break_ties_like_the_eager_path(kind):
    """Free-running frames from the frame graph, where the first QKV GEMV of Fast steps 2..9 repeats
    the second pass of the previous Fast head's pick and gathers its own input, on a model whose
    heads hold exact copies of the winning rows: every code equals the eager path's (whose tie rule
    the oracle pins above), and the copies do meet at a Fast step's maximum."""
    cfg, w2, toks, _, _, _ = _tie_case(kind, 0)
    ctx = _ctx(cfg, w2, max_streams=2)
    ctx.prefill(0, toks)
    ctx.prefill(1, toks)
    n = 2
    graph = ctx.decode_frames([0], n)[:, 0]
    eager = [ctx.debug_frame(1) for _ in range(n)]
    assert np.array_equal(graph, np.stack([e["own_codes"] for e in eager])), "graph and eager picks differ"
    ties = 0
    for e in eager:
        for j in range(9):
            lg = np.asarray(e["fast_logits"][j])
            top = np.flatnonzero(lg == lg.max())
            if len(top) > 1:
                ties += 1
                assert int(e["own_codes"][j + 1]) == int(top[0])
    assert ties > 0, "no Fast step met a tie"
    _say(f"[ties] graph frames, {kind}: {ties} tied Fast picks")
    ctx.close()


# ------------------------------------------------------------------ device-memory hook

def _tensor_allocator(log, fail_at=None):
    import torch

    def alloc(nbytes):
        log["calls"] = log.get("calls", 0) + 1
        if fail_at is not None and log["calls"] >= fail_at:
            return 0
        t = torch.empty(int(nbytes), dtype=torch.uint8, device="cuda")
        log.setdefault("live", {})[t.data_ptr()] = (t, int(nbytes))
        log["bytes"] = log.get("bytes", 0) + int(nbytes)
        return t.data_ptr()

    def free(ptr, nbytes):
        t, n = log["live"].pop(ptr)
        assert n == nbytes
        log["freed"] = log.get("freed", 0) + n

    return alloc, free


def test_device_allocator_supplies_and_gets_back_every_block():
    cfg = synth.config("mid", max_context=256)
    w = synth.make_weights(cfg)
    toks, _, _ = synth.make_prompt(cfg)
    outs = []
    for allocator in (None, "log", "torch"):
        log = {}
        ctx = s2ar.Context(cfg, w, max_streams=2,
                           allocator=_tensor_allocator(log) if allocator == "log" else allocator)
        ctx.prefill(0, toks)
        ctx.prefill(1, toks[:30])
        outs.append((ctx.decode_frames([0], 3), ctx.decode_frames([0, 1], 2)))
        ctx.close()
        if allocator == "log":
            assert log["calls"] > 10 and log["bytes"] > 7e8   # the weights came through the hook
            assert not log["live"] and log["freed"] == log["bytes"]
    for o in outs[1:]:
        assert np.array_equal(o[0], outs[0][0]) and np.array_equal(o[1], outs[0][1])


@pytest.mark.parametrize("fail_at", [1, 5, 40])
def test_device_allocator_failure_is_nomem_and_frees_everything(fail_at):
    cfg = synth.config("mid", max_context=256)
    w = synth.make_weights(cfg)
    log = {}
    with pytest.raises(s2ar.S2arError) as e:
        s2ar.Context(cfg, w, max_streams=2, allocator=_tensor_allocator(log, fail_at=fail_at))
    assert e.value.code == -5 and "dev_alloc" in str(e.value)
    assert log["calls"] == fail_at
    assert not log.get("live") and log.get("freed", 0) == log.get("bytes", 0)
    gc.collect()
