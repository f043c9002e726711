"""ctypes front of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only users.  The product path never imports it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

c_i32, c_i64, c_dbl, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p


class OrcStack(ctypes.Structure):
    _fields_ = [(n, c_i32) for n in ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn")]


class OrcConfig(ctypes.Structure):
    _fields_ = [("slow", OrcStack), ("fast", OrcStack), ("vocab_text", c_i32), ("n_codebooks", c_i32),
                ("codebook_size", c_i32), ("rope_theta", c_dbl), ("rms_eps", c_dbl), ("weight_dtype", c_i32),
                ("rope_bf16", c_i32), ("max_context", c_i32), ("eos_id", c_i32)]


def build(force: bool = False) -> str:
    src = os.path.join(_HERE, "oracle.c")
    hdr = os.path.join(_HERE, "oracle.h")
    newest = max(os.path.getmtime(src), os.path.getmtime(hdr))
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < newest:
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-Wall",
                               "-o", tmp, src, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        L.orc_model_new.restype = vp
        L.orc_model_new.argtypes = [ctypes.POINTER(OrcConfig), ctypes.POINTER(vp), c_i32]
        L.orc_model_free.argtypes = [vp]
        L.orc_n_tensors.argtypes = [ctypes.POINTER(OrcConfig)]
        L.orc_state_new.restype = vp
        L.orc_state_new.argtypes = [vp]
        L.orc_state_free.argtypes = [vp]
        L.orc_state_pos.argtypes = [vp]
        L.orc_embed_token.argtypes = [vp, c_i32, vp]
        L.orc_embed_codes.argtypes = [vp, vp, vp]
        L.orc_prefill.argtypes = [vp, vp, vp, vp, vp, c_i32, vp, vp, vp, vp]
        L.orc_slow_step_codes.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp]
        L.orc_fast_loop.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp]
        L.orc_generate.argtypes = [vp, vp, vp, c_i32, c_i32, vp]
        L.orc_full_recompute.argtypes = [vp, vp, vp, vp, c_i32, vp]
        L.orc_rmsnorm.argtypes = [vp, vp, c_i32, c_dbl, vp]
        L.orc_rope_row.argtypes = [c_dbl, c_i32, c_i32, c_i32, vp, vp]
        L.orc_rope_apply.argtypes = [vp, c_i32, vp, vp]
        L.orc_attention.argtypes = [vp, vp, vp, c_i32, c_i32, c_i32, c_i32, vp, vp]
        L.orc_silu.restype = c_dbl
        L.orc_silu.argtypes = [c_dbl]
        L.orc_slow_pick.restype = c_i32
        L.orc_slow_pick.argtypes = [vp, c_i32, c_i32, c_i32, vp]
        L.orc_argmax.restype = c_i32
        L.orc_argmax.argtypes = [vp, c_i32, c_i32, vp]
        L.orc_matvec_f32.argtypes = [vp, c_i32, c_i32, vp, c_i32, vp]
        L.orc_bf16_round.restype = c_dbl
        L.orc_bf16_round.argtypes = [c_dbl]
        L.orc_quantize_rows_i8.argtypes = [vp, c_i64, c_i64, vp, vp]
        L.orc_dequantize_rows_i8.argtypes = [vp, vp, c_i64, c_i64, vp]
        L.orc_f8_value.restype = c_dbl
        L.orc_f8_value.argtypes = [ctypes.c_uint8]
        L.orc_quantize_rows_f8.argtypes = [vp, c_i64, c_i64, vp, vp]
        L.orc_dequantize_rows_f8.argtypes = [vp, vp, c_i64, c_i64, vp]
        L.orc_get_counters.argtypes = [vp]
        L.orc_set_threads.argtypes = [c_i32]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def make_config(cfg: dict) -> OrcConfig:
    def st(s):
        return OrcStack(s["n_layers"], s["hidden"], s["n_q_heads"], s["n_kv_heads"], s["head_dim"], s["ffn"])

    return OrcConfig(st(cfg["slow"]), st(cfg["fast"]), cfg["vocab_text"], cfg["n_codebooks"], cfg["codebook_size"],
                     float(cfg["rope_theta"]), float(cfg["rms_eps"]), 1 if cfg["weight_dtype"] == "bf16" else 0,
                     int(cfg["rope_bf16"]), int(cfg["max_context"]), int(cfg.get("eos_id", -1)))


class Model:
    """Oracle model over weights in canonical order (arrays must stay alive)."""

    def __init__(self, cfg: dict, weights: list):
        self.cfg = cfg
        self.weights = [np.ascontiguousarray(w) for w in weights]
        self.ccfg = make_config(cfg)
        arr = (vp * len(self.weights))(*[w.ctypes.data for w in self.weights])
        self.h = lib().orc_model_new(ctypes.byref(self.ccfg), arr, len(self.weights))
        if not self.h:
            raise ValueError("oracle rejected the model shapes")
        self.H = cfg["slow"]["hidden"]
        self.V = cfg["vocab_slow"]
        self.K = cfg["codebook_size"]
        self.NC = cfg["n_codebooks"]

    def __del__(self):
        if getattr(self, "h", None):
            lib().orc_model_free(self.h)
            self.h = None

    def new_state(self):
        return State(self)

    def embed_codes(self, codes):
        x = np.zeros(self.H, np.float64)
        c = np.ascontiguousarray(codes, np.int32)
        if lib().orc_embed_codes(self.h, _p(c), _p(x)):
            raise ValueError("code out of range")
        return x

    def embed_token(self, tok):
        x = np.zeros(self.H, np.float64)
        if lib().orc_embed_token(self.h, int(tok), _p(x)):
            raise ValueError("token out of range")
        return x

    def fast_loop(self, h, forced=None, taps=False):
        nl = self.cfg["fast"]["n_layers"]
        ns = self.NC - 1
        h = np.ascontiguousarray(h, np.float64)
        codes = np.zeros(ns, np.int32)
        margins = np.zeros(ns, np.float64)
        f = None if forced is None else np.ascontiguousarray(forced, np.int32)
        resid = np.zeros((ns, nl, self.H)) if taps else None
        z = np.zeros((ns, self.H)) if taps else None
        logits = np.zeros((ns, self.K)) if taps else None
        rc = lib().orc_fast_loop(self.h, _p(h), _p(f), _p(codes), _p(margins), _p(resid), _p(z), _p(logits))
        if rc:
            raise ValueError(f"orc_fast_loop failed ({rc})")
        out = dict(codes=codes, margins=margins)
        if taps:
            out.update(resid=resid, z=z, logits=logits)
        return out

    def full_recompute(self, tokens, mask=None, codes=None):
        n = len(tokens)
        h = np.zeros((n, self.H))
        t = np.ascontiguousarray(tokens, np.int32)
        m = None if mask is None else np.ascontiguousarray(mask, np.uint8)
        c = None if codes is None else np.ascontiguousarray(codes, np.int32)
        if lib().orc_full_recompute(self.h, _p(t), _p(m), _p(c), n, _p(h)):
            raise ValueError("orc_full_recompute failed")
        return h


class State:
    def __init__(self, model: Model):
        self.m = model
        self.h = lib().orc_state_new(model.h)

    def __del__(self):
        if getattr(self, "h", None):
            lib().orc_state_free(self.h)
            self.h = None

    @property
    def pos(self):
        return lib().orc_state_pos(self.h)

    def prefill(self, tokens, mask=None, codes=None):
        m = self.m
        n = len(tokens)
        t = np.ascontiguousarray(tokens, np.int32)
        mk = None if mask is None else np.ascontiguousarray(mask, np.uint8)
        cd = None if codes is None else np.ascontiguousarray(codes, np.int32)
        h = np.zeros(m.H)
        logits = np.zeros(m.V)
        c0 = np.zeros(1, np.int32)
        mg = np.zeros(1)
        rc = lib().orc_prefill(m.h, self.h, _p(t), _p(mk), _p(cd), n, _p(h), _p(logits), _p(c0), _p(mg))
        if rc:
            raise ValueError(f"orc_prefill failed ({rc})")
        return dict(h=h, logits=logits, c0=int(c0[0]), margin=float(mg[0]))

    def slow_step(self, codes, taps=False):
        m = self.m
        c = np.ascontiguousarray(codes, np.int32)
        resid = np.zeros((m.cfg["slow"]["n_layers"], m.H)) if taps else None
        h = np.zeros(m.H)
        logits = np.zeros(m.V)
        c0 = np.zeros(1, np.int32)
        mg = np.zeros(1)
        rc = lib().orc_slow_step_codes(m.h, self.h, _p(c), _p(resid), _p(h), _p(logits), _p(c0), _p(mg))
        if rc:
            raise ValueError(f"orc_slow_step_codes failed ({rc})")
        out = dict(h=h, logits=logits, c0=int(c0[0]), margin=float(mg[0]))
        if taps:
            out["resid"] = resid
        return out

    def generate(self, h0, c0, n_frames):
        codes = np.zeros((n_frames, self.m.NC), np.int32)
        h0 = np.ascontiguousarray(h0, np.float64)
        if lib().orc_generate(self.m.h, self.h, _p(h0), int(c0), n_frames, _p(codes)):
            raise ValueError("orc_generate failed")
        return codes


def counters():
    out = np.zeros(4, np.int64)
    lib().orc_get_counters(_p(out))
    return dict(slow_steps=int(out[0]), fast_steps=int(out[1]), fast_layer_passes=int(out[2]),
                codes_emitted=int(out[3]))


def reset_counters():
    lib().orc_reset_counters()


def set_threads(n: int):
    lib().orc_set_threads(int(n))


# ---- unit functions ----

def rmsnorm(x, g, eps):
    x = np.ascontiguousarray(x, np.float64)
    g = np.ascontiguousarray(g, np.float64)
    y = np.zeros_like(x)
    lib().orc_rmsnorm(_p(x), _p(g), len(x), float(eps), _p(y))
    return y


def rope_row(theta, head_dim, pos, bf16):
    c = np.zeros(head_dim // 2)
    s = np.zeros(head_dim // 2)
    lib().orc_rope_row(float(theta), head_dim, pos, int(bf16), _p(c), _p(s))
    return c, s


def rope_apply(v, cos_row, sin_row):
    v = np.array(v, np.float64)
    lib().orc_rope_apply(_p(v), len(v), _p(np.ascontiguousarray(cos_row, np.float64)),
                         _p(np.ascontiguousarray(sin_row, np.float64)))
    return v


def attention(q, k_cache, v_cache, n_q_heads, n_kv_heads, head_dim):
    """q: [Hq*D]; caches: [ctx][Hkv*D]. Returns (o [Hq*D], probs [Hq][ctx])."""
    q = np.ascontiguousarray(q, np.float64)
    kc = np.ascontiguousarray(k_cache, np.float64)
    vc = np.ascontiguousarray(v_cache, np.float64)
    ctx = kc.shape[0]
    o = np.zeros(n_q_heads * head_dim)
    probs = np.zeros((n_q_heads, ctx))
    lib().orc_attention(_p(q), _p(kc), _p(vc), n_q_heads, n_kv_heads, head_dim, ctx, _p(o), _p(probs))
    return o, probs


def silu(z):
    return lib().orc_silu(float(z))


def slow_pick(logits, vocab_text, codebook_size, eos_id=-1):
    """(c0, margin): the Slow pick over the semantic ids plus the EOS id (c0 = -1 for EOS)."""
    v = np.ascontiguousarray(logits, np.float64)
    mg = np.zeros(1, np.float64)
    c0 = lib().orc_slow_pick(_p(v), int(vocab_text), int(codebook_size), int(eos_id), _p(mg))
    return int(c0), float(mg[0])


def argmax(v, lo=0, hi=None):
    v = np.ascontiguousarray(v, np.float64)
    hi = len(v) if hi is None else hi
    mg = np.zeros(1)
    i = lib().orc_argmax(_p(v), lo, hi, _p(mg))
    return int(i), float(mg[0])


def matvec_f32(w, x):
    w = np.ascontiguousarray(w, np.float32)
    x = np.ascontiguousarray(x, np.float64)
    P = 1 if x.ndim == 1 else x.shape[0]
    y = np.zeros((P, w.shape[0]))
    lib().orc_matvec_f32(_p(w), w.shape[0], w.shape[1], _p(x), P, _p(y))
    return y[0] if x.ndim == 1 else y


def bf16_round(v):
    return lib().orc_bf16_round(float(v))


def quantize_rows_i8(w_bits):
    """Symmetric per-row int8 of a bf16 matrix (uint16 bit patterns [rows][cols]) -> (q int8, s fp32)."""
    w = np.ascontiguousarray(w_bits, np.uint16)
    rows, cols = w.shape
    q = np.empty((rows, cols), np.int8)
    s = np.empty(rows, np.float32)
    lib().orc_quantize_rows_i8(_p(w), rows, cols, _p(q), _p(s))
    return q, s


def dequantize_rows_i8(q, s):
    q = np.ascontiguousarray(q, np.int8)
    s = np.ascontiguousarray(s, np.float32)
    out = np.empty(q.shape, np.float32)
    lib().orc_dequantize_rows_i8(_p(q), _p(s), q.shape[0], q.shape[1], _p(out))
    return out


def f8_value(b):
    """Value of one OCP FP8 E4M3 byte."""
    return lib().orc_f8_value(int(b) & 0xff)


def quantize_rows_f8(w_bits):
    """Per-row FP8 E4M3 of a bf16 matrix (uint16 bit patterns [rows][cols]) -> (q uint8, s fp32)."""
    w = np.ascontiguousarray(w_bits, np.uint16)
    rows, cols = w.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty(rows, np.float32)
    lib().orc_quantize_rows_f8(_p(w), rows, cols, _p(q), _p(s))
    return q, s


def dequantize_rows_f8(q, s):
    q = np.ascontiguousarray(q, np.uint8)
    s = np.ascontiguousarray(s, np.float32)
    out = np.empty(q.shape, np.float32)
    lib().orc_dequantize_rows_f8(_p(q), _p(s), q.shape[0], q.shape[1], _p(out))
    return out
