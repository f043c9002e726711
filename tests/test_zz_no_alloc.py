"""The allocation-free entry point (s2ar_decode_frames_noalloc) against s2ar_decode_frames.

Twin streams with the same prompt are decoded once through each entry point; the codes must be
equal bit for bit (integer outputs).  Two calls in a row, the second on a shorter context with
fewer frames, so the scratch array holds more of the first call's attention partials than the
second call writes.  A counting device allocator shows that the calls take no device memory from
the library's allocator.
"""
import numpy as np
import pytest

from dual_ar_codec_amd import s2ar, synth

pytestmark = pytest.mark.gpu


def _counting_allocator(log):
    import torch

    def alloc(nbytes):
        t = torch.empty(int(nbytes), dtype=torch.uint8, device="cuda")
        log.setdefault("live", {})[t.data_ptr()] = t
        log["allocs"] = log.get("allocs", 0) + 1
        return t.data_ptr()

    def free(ptr, nbytes):
        del log["live"][ptr]
        log["frees"] = log.get("frees", 0) + 1

    return alloc, free


def test_noalloc_entry_point_matches_decode_frames():
    import torch

    torch.cuda.set_device(0)
    cfg = synth.config("mid", max_context=256)
    w = synth.make_weights(cfg)
    log = {}
    ctx = s2ar.Context(cfg, w, max_streams=4, allocator=_counting_allocator(log))
    long_prompt = synth.uniform_ints(cfg["seed"], 77, 150, 0, cfg["vocab_text"])   # 151.. positions: 3 splits
    short_prompt = synth.uniform_ints(cfg["seed"], 78, 41, 0, cfg["vocab_text"])   # one split
    for sid, p in ((0, long_prompt), (1, long_prompt), (2, short_prompt), (3, short_prompt)):
        ctx.prefill(sid, p)
    n_after_create = log["allocs"]

    # first call: 4 frames at contexts 151..154
    a = ctx.decode_frames_noalloc(0, 4)
    b = ctx.decode_frames([1], 4)[:, 0]
    print("call 1 noalloc", a[:, :3].tolist(), "graph", b[:, :3].tolist(), flush=True)
    assert np.array_equal(a, b)
    # second call, smaller input: 2 frames at contexts 42..43
    a2 = ctx.decode_frames_noalloc(2, 2)
    b2 = ctx.decode_frames([3], 2)[:, 0]
    assert np.array_equal(a2, b2)
    assert ctx.position(0) == ctx.position(1) == 154 and ctx.position(2) == ctx.position(3) == 43
    # and the first streams continue equally after the scratch was reused
    a3 = ctx.decode_frames_noalloc(0, 3)
    b3 = ctx.decode_frames([1], 3)[:, 0]
    assert np.array_equal(a3, b3)
    assert np.all((a >= 0) & (a < cfg["codebook_size"]))
    # the noalloc calls took nothing from the library's allocator (the graph path may have)
    n_graph = log["allocs"]
    ctx.decode_frames_noalloc(2, 1)
    assert log["allocs"] == n_graph
    assert n_after_create >= 1
    ctx.close()
    assert log["allocs"] == log["frees"] and not log["live"]


def test_noalloc_rejects_a_frame_beyond_the_scratch_array():
    import torch

    torch.cuda.set_device(0)
    cfg = synth.config("tiny", max_context=1 << 20)
    w = synth.make_weights(cfg)
    ctx = s2ar.Context(cfg, w)
    ctx.prefill(0, synth.uniform_ints(cfg["seed"], 5, 3, 0, cfg["vocab_text"]))
    with pytest.raises(s2ar.S2arError) as e:
        ctx.decode_frames_noalloc(0, 400000)  # contexts up to 400003: 6251 splits of 4 q heads
    assert e.value.code == -3 and "scratch" in str(e.value)
    assert ctx.position(0) == 3
    out = ctx.decode_frames_noalloc(0, 2)  # still usable
    assert out.shape == (2, 10) and ctx.position(0) == 5
    ctx.close()
