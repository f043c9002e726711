"""Teacher-forced comparison of the HIP path against the CPU oracle.

Acceptance (per frame, same bf16 weights, the GPU forced with the oracle's own
codes so both sides see identical inputs):
  - cosine >= 0.9999 of the residual after every Slow and Fast layer and of the
    final-normed hiddens;
  - max |logit error| <= 2e-2 * max |logit| (Slow over the whole vocabulary,
    Fast per step over the codebook);
  - greedy picks identical wherever the oracle's top-1 minus top-2 margin
    exceeds 5e-2.
"""
import numpy as np

import oracle

COS_MIN = 0.9999
LOGIT_REL = 2e-2
MARGIN = 5e-2


def cosine(a, b):
    a = np.ravel(a).astype(np.float64)
    b = np.ravel(b).astype(np.float64)
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def logit_err(gpu, ref):
    return float(np.max(np.abs(gpu.astype(np.float64) - ref)) / np.max(np.abs(ref)))


class Report:
    def __init__(self):
        self.min_cos = 1.0
        self.max_logit = 0.0
        self.checked = 0
        self.skipped = 0
        self.mismatch = []

    def cos(self, what, a, b):
        c = cosine(a, b)
        self.min_cos = min(self.min_cos, c)
        assert c >= COS_MIN, f"{what}: cosine {c:.7f} < {COS_MIN}"

    def logits(self, what, gpu, ref):
        e = logit_err(gpu, ref)
        self.max_logit = max(self.max_logit, e)
        assert e <= LOGIT_REL, f"{what}: logit error {e:.3e} x max|logit|"

    def token(self, what, gpu, ref, margin):
        if margin > MARGIN:
            self.checked += 1
            if gpu != ref:
                self.mismatch.append((what, gpu, ref, margin))
        else:
            self.skipped += 1

    def finish(self):
        assert not self.mismatch, f"greedy picks differ where the margin exceeds {MARGIN}: {self.mismatch[:5]}"
        return dict(min_cos=self.min_cos, max_logit_rel=self.max_logit, tokens_checked=self.checked,
                    tokens_skipped=self.skipped)


def quant_reference(cfg, weights, fmt="i8"):
    """(cfg, weights) of the oracle's view of an 8-bit-weight context built from bf16 weights: every
    layer matrix and both heads quantised per row by the oracle's own quantiser (int8 or FP8 E4M3)
    and dequantised (value * s in fp32); embeddings, codebooks and gains widened exactly from bf16."""
    from dual_ar_codec_amd import synth
    quant, dequant = ((oracle.quantize_rows_i8, oracle.dequantize_rows_i8) if fmt == "i8"
                      else (oracle.quantize_rows_f8, oracle.dequantize_rows_f8))
    out = []
    for (name, shape, kind), w in zip(synth.tensor_specs(cfg), weights):
        f = (np.ascontiguousarray(w).astype(np.uint32) << 16).view(np.float32).reshape(shape)
        if kind == "matrix" and name not in ("slow.embed", "codebook.embed"):
            q, s = quant(np.ascontiguousarray(w).reshape(shape[0], -1))
            f = dequant(q, s).reshape(shape)
        out.append(np.ascontiguousarray(f, np.float32))
    return dict(cfg, weight_dtype="f32"), out


def int8_reference(cfg, weights):
    return quant_reference(cfg, weights, "i8")


def oracle_run(cfg, weights, tokens, mask, codes, n_frames, prefill_out=None):
    """Oracle free-running decode with every tap; frame t = (fast taps, the Slow
    step that follows frame t).  With a stop id the run ends at the frame whose
    following Slow pick is the stop (its slow["c0"] is -1); a stop at the prefill's
    pick gives no frames (prefill_out, a dict, receives the prefill's outputs)."""
    m = oracle.Model(cfg, weights)
    st = m.new_state()
    pre = st.prefill(tokens, mask, codes)
    if prefill_out is not None:
        prefill_out.update(pre)
    h, c0, c0m = pre["h"], pre["c0"], pre["margin"]
    frames = []
    for _ in range(n_frames):
        if c0 < 0:
            break
        fl = m.fast_loop(h, taps=True)
        codes_t = np.concatenate([[c0], fl["codes"]]).astype(np.int32)
        nxt = st.slow_step(codes_t, taps=True)
        frames.append(dict(codes=codes_t, c0_margin=c0m, fast=fl, slow=nxt))
        h, c0, c0m = nxt["h"], nxt["c0"], nxt["margin"]
    return frames


def slow_rows(cfg):
    """Indices of the Slow logits the GPU computes: all, or the semantic slice plus the stop id."""
    Vt, K, eos = cfg["vocab_text"], cfg["codebook_size"], cfg.get("eos_id", -1)
    if not cfg.get("head_slice", 0):
        return np.arange(Vt + K)
    return np.concatenate([[eos] if eos >= 0 else [], np.arange(Vt, Vt + K)]).astype(np.int64)


def own_slow_pick(logits, cfg):
    """The Slow pick rule applied to the GPU's own logits (the kernel's pick must equal it)."""
    Vt, K, eos = cfg["vocab_text"], cfg["codebook_size"], cfg.get("eos_id", -1)
    b = int(np.argmax(logits[Vt:Vt + K]))
    return -1 if eos >= 0 and logits[eos] >= logits[Vt + b] else b


def compare_frames(ctx, stream, frames, cfg, report=None, gather_check=True):
    """Drive the GPU teacher-forced through the oracle's frames and check each."""
    r = report or Report()
    K, Vt = cfg["codebook_size"], cfg["vocab_text"]
    cb = None
    for t, f in enumerate(frames):
        g = ctx.debug_frame(stream, forced=f["codes"])
        r.token(f"frame {t} c0", int(g["own_codes"][0]), int(f["codes"][0]), f["c0_margin"])
        fl = f["fast"]
        for j in range(9):
            for l in range(cfg["fast"]["n_layers"]):
                r.cos(f"frame {t} fast step {j + 1} layer {l}", g["fast_resid"][j, l], fl["resid"][j, l])
            r.cos(f"frame {t} fast step {j + 1} z", g["fast_z"][j], fl["z"][j])
            r.logits(f"frame {t} fast step {j + 1} logits", g["fast_logits"][j], fl["logits"][j])
            r.token(f"frame {t} c{j + 1}", int(g["own_codes"][j + 1]), int(fl["codes"][j]), fl["margins"][j])
            # the greedy pick is exactly the argmax of the kernel's own logits
            assert int(g["own_codes"][j + 1]) == int(np.argmax(g["fast_logits"][j]))
        s = f["slow"]
        for l in range(cfg["slow"]["n_layers"]):
            r.cos(f"frame {t} slow layer {l}", g["slow_resid"][l], s["resid"][l])
        r.cos(f"frame {t} slow h", g["slow_h"], s["h"])
        rows = slow_rows(cfg)
        r.logits(f"frame {t} slow logits", g["slow_logits"][rows], s["logits"][rows])
        r.token(f"frame {t} next c0", int(g["next_c0"]), int(s["c0"]), s["margin"])
        assert int(g["next_c0"]) == own_slow_pick(g["slow_logits"], cfg)
        if gather_check:
            if cb is None:
                cb = codebook_f32(cfg, ctx)
            want = np.zeros(cfg["slow"]["hidden"], np.float32)
            for k in range(cfg["n_codebooks"]):
                want = want + cb[k, f["codes"][k]]
            assert np.array_equal(g["slow_embed"], want), f"frame {t}: gather-sum is not bit-exact"
    return r


_CB_CACHE = {}


def codebook_f32(cfg, ctx):
    return _CB_CACHE[id(ctx)]


def remember_codebook(ctx, cfg, weights):
    from dual_ar_codec_amd import synth
    names = [n for n, _, _ in synth.tensor_specs(cfg)]
    _CB_CACHE[id(ctx)] = synth.as_f32(weights[names.index("codebook.embed")])
