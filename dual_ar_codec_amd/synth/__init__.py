"""Seeded synthetic workloads for the Dual-AR decode step.

This module only describes shapes and draws numbers; it holds none of the
model's arithmetic.  The CPU oracle and the HIP library are both fed from it,
so they always see the same bf16 (or fp32) weights, prompt ids and VQ codes.

Shapes follow the architecture the pages describe: a 36-layer Qwen3-style Slow
AR with GQA/RoPE/RMSNorm/SwiGLU, a 4-layer Fast AR over 9 residual codebooks
and a 10-codebook RVQ codec ("SGLang Day-0 Support for FishAudio S2", section
Architecture; "s2pro-native", section What happens to a sentence; "Fish Audio
Abre Codigo do S2", section Arquitetura Dual-AR).  Sizes of the five workloads
(tiny, mid, full, voice_clone, multi_stream) are the synthetic stand-ins for the
pages' measurement settings; the full single stream is the "41-token prompt,
60 frames, greedy" workload of the s2pro-native page (section Where it stands).

Canonical tensor order (shared by the oracle and ``s2ar_create``):
  slow.embed [V_text+K][H]
  per Slow layer: attn_norm[H], wq[Hq*D][H], wk[Hkv*D][H], wv[Hkv*D][H],
                  q_norm[D], k_norm[D], wo[H][Hq*D], mlp_norm[H],
                  w_gate[F][H], w_up[F][H], w_down[H][F]
  slow.final_norm[H], slow.head[V_text+K][H]
  codebook.embed[10][K][H]
  per Fast layer: the same eleven tensors
  fast.final_norm[H], fast.head[K][H]
Matrices are row-major [out][in].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libs2ar_synth.so")
_lib = None

# stream ids of the non-weight inputs (weights use their canonical tensor index)
STREAM_PROMPT = 1 << 20
STREAM_VQ = 2 << 20
STREAM_CTXLEN = 3 << 20
STREAM_PAGES = 4 << 20
STREAM_PROBE = 5 << 20

N_CODEBOOKS = 10
N_FAST_STEPS = N_CODEBOOKS - 1
FRAME_SAMPLES = 2048
SAMPLE_RATE = 44100

LAYER_TENSORS = ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo",
                 "mlp_norm", "w_gate", "w_up", "w_down")


def build_lib(force: bool = False) -> str:
    """Compile the generator with gcc (OpenMP, no host-specific ISA flags)."""
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                               "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_lib()
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.synth_u64.restype = u64
        L.synth_u64.argtypes = [u64, u64, u64]
        for nm in ("synth_normal_f32", "synth_normal_bf16"):
            getattr(L, nm).argtypes = [u64, u64, i64, dbl, vp]
        for nm in ("synth_uniform_f32", "synth_uniform_bf16"):
            getattr(L, nm).argtypes = [u64, u64, i64, dbl, dbl, vp]
        L.synth_uniform_int.argtypes = [u64, u64, i64, ctypes.c_int32, ctypes.c_int32, vp]
        L.synth_permutation.argtypes = [u64, u64, ctypes.c_int32, vp]
        L.synth_fill_f32.argtypes = [i64, ctypes.c_float, vp]
        L.synth_fill_bf16.argtypes = [i64, ctypes.c_float, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# ----------------------------------------------------------------------------------------------
# workloads

def _stack(n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn):
    return dict(n_layers=n_layers, hidden=hidden, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                head_dim=head_dim, ffn=ffn)


def _round_up(v, m):
    return (v + m - 1) // m * m


CONFIGS = {
    # fp32 tiny model: the oracle finishes it in well under a second
    "tiny": dict(seed=0, weight_dtype="f32",
                 slow=_stack(2, 256, 4, 2, 64, 768), fast=_stack(1, 256, 4, 2, 64, 768),
                 vocab_text=4096, codebook_size=1024,
                 prompt=dict(kind="text", n=16), frames=8, n_streams=1),
    "mid": dict(seed=1, weight_dtype="bf16",
                slow=_stack(8, 1024, 16, 4, 64, 3072), fast=_stack(2, 1024, 16, 4, 64, 3072),
                vocab_text=32768, codebook_size=4096,
                prompt=dict(kind="text", n=64), frames=32, n_streams=1),
    # FishAudio S2 shape, one stream: 41-token prompt, 60 frames, greedy
    "full": dict(seed=2, weight_dtype="bf16",
                 slow=_stack(36, 2560, 32, 8, 128, 9728), fast=_stack(4, 2560, 32, 8, 128, 9728),
                 vocab_text=151680, codebook_size=4096,
                 prompt=dict(kind="text", n=41), frames=60, n_streams=1),
    # voice-clone prefix: 1000 VQ positions then 200 text positions
    "voice_clone": dict(seed=3, weight_dtype="bf16",
                        slow=_stack(36, 2560, 32, 8, 128, 9728), fast=_stack(4, 2560, 32, 8, 128, 9728),
                        vocab_text=151680, codebook_size=4096,
                        prompt=dict(kind="voice_clone", n_vq=1000, n_text=200), frames=200, n_streams=1),
    # 16 streams with ragged contexts of 256..4096 positions over pages of 16
    "multi_stream": dict(seed=4, weight_dtype="bf16",
                         slow=_stack(36, 2560, 32, 8, 128, 9728), fast=_stack(4, 2560, 32, 8, 128, 9728),
                         vocab_text=151680, codebook_size=4096,
                         prompt=dict(kind="ragged_text", lo=256, hi=4096), frames=100, n_streams=16),
}

COMMON = dict(n_codebooks=N_CODEBOOKS, rope_theta=1.0e6, rms_eps=1.0e-6, rope_bf16=1, page_size=16)


def config(name: str, **overrides) -> dict:
    """Full description of a workload: shapes, numerics constants and input recipe."""
    c = dict(COMMON)
    c.update({k: (dict(v) if isinstance(v, dict) else v) for k, v in CONFIGS[name].items()})
    c["name"] = name
    c.update(overrides)
    c["vocab_slow"] = c["vocab_text"] + c["codebook_size"]
    if "max_context" not in c:
        longest = max(len_ for len_ in prompt_lengths(c))
        c["max_context"] = _round_up(longest + c["frames"] + 1, 64)
    return c


def micro_config(seed=7, slow_layers=2, fast_layers=1, hidden=64, n_q_heads=4, n_kv_heads=2,
                 head_dim=16, ffn=96, vocab_text=100, codebook_size=32, weight_dtype="f32",
                 n_prompt=6, frames=3, max_context=64, rope_bf16=1):
    """Small model for brute-force oracle checks."""
    c = dict(COMMON)
    c.update(name="micro", seed=seed, weight_dtype=weight_dtype,
             slow=_stack(slow_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn),
             fast=_stack(fast_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn),
             vocab_text=vocab_text, codebook_size=codebook_size,
             prompt=dict(kind="text", n=n_prompt), frames=frames, n_streams=1,
             max_context=max_context, rope_bf16=rope_bf16)
    c["vocab_slow"] = vocab_text + codebook_size
    return c


def prompt_lengths(cfg) -> list:
    p = cfg["prompt"]
    if p["kind"] == "text":
        return [p["n"]] * cfg["n_streams"]
    if p["kind"] == "voice_clone":
        return [p["n_vq"] + p["n_text"]]
    if p["kind"] == "ragged_text":
        out = np.empty(cfg["n_streams"], np.int32)
        lib().synth_uniform_int(cfg["seed"], STREAM_CTXLEN, cfg["n_streams"], p["lo"], p["hi"] + 1, _ptr(out))
        return [int(v) for v in out]
    raise ValueError(p["kind"])


def tensor_specs(cfg) -> list:
    """[(name, shape, kind)] in canonical order; kind is 'matrix' or 'gain'."""
    H, V, K = cfg["slow"]["hidden"], cfg["vocab_slow"], cfg["codebook_size"]
    specs = [("slow.embed", (V, H), "matrix")]

    def layer(prefix, s):
        Hd, Hq, Hkv, D, F = s["hidden"], s["n_q_heads"], s["n_kv_heads"], s["head_dim"], s["ffn"]
        return [(f"{prefix}.attn_norm", (Hd,), "gain"), (f"{prefix}.wq", (Hq * D, Hd), "matrix"),
                (f"{prefix}.wk", (Hkv * D, Hd), "matrix"), (f"{prefix}.wv", (Hkv * D, Hd), "matrix"),
                (f"{prefix}.q_norm", (D,), "gain"), (f"{prefix}.k_norm", (D,), "gain"),
                (f"{prefix}.wo", (Hd, Hq * D), "matrix"), (f"{prefix}.mlp_norm", (Hd,), "gain"),
                (f"{prefix}.w_gate", (F, Hd), "matrix"), (f"{prefix}.w_up", (F, Hd), "matrix"),
                (f"{prefix}.w_down", (Hd, F), "matrix")]

    for i in range(cfg["slow"]["n_layers"]):
        specs += layer(f"slow.layers.{i}", cfg["slow"])
    specs += [("slow.final_norm", (H,), "gain"), ("slow.head", (V, H), "matrix"),
              ("codebook.embed", (cfg["n_codebooks"], K, H), "matrix")]
    for i in range(cfg["fast"]["n_layers"]):
        specs += layer(f"fast.layers.{i}", cfg["fast"])
    specs += [("fast.final_norm", (cfg["fast"]["hidden"],), "gain"), ("fast.head", (K, cfg["fast"]["hidden"]), "matrix")]
    return specs


def weight_bytes(cfg) -> int:
    esz = 4 if cfg["weight_dtype"] == "f32" else 2
    return sum(int(np.prod(s)) * esz for _, s, _ in tensor_specs(cfg))


def make_weights(cfg, gains: str = "unit", std: float = 0.02) -> list:
    """Weights in canonical order: uint16 arrays holding bf16 bits, or float32 arrays.

    Matrices and embeddings are std*N(0,1); norm gains are 1.0 ('unit') or
    U(0.5, 1.5) ('random', used by unit checks so a dropped gain is caught).
    """
    L = lib()
    seed = cfg["seed"]
    bf16 = cfg["weight_dtype"] == "bf16"
    out = []
    for idx, (name, shape, kind) in enumerate(tensor_specs(cfg)):
        n = int(np.prod(shape))
        a = np.empty(shape, np.uint16 if bf16 else np.float32)
        if kind == "matrix":
            (L.synth_normal_bf16 if bf16 else L.synth_normal_f32)(seed, idx, n, std, _ptr(a))
        elif gains == "unit":
            (L.synth_fill_bf16 if bf16 else L.synth_fill_f32)(n, 1.0, _ptr(a))
        else:
            (L.synth_uniform_bf16 if bf16 else L.synth_uniform_f32)(seed, idx, n, 0.5, 1.5, _ptr(a))
        out.append(a)
    return out


def make_prompt(cfg, stream: int = 0):
    """(tokens int32[n], vq_mask uint8[n], vq_codes int32[n][10]) for one stream."""
    L = lib()
    seed, p = cfg["seed"], cfg["prompt"]
    n = prompt_lengths(cfg)[stream]
    tokens = np.zeros(n, np.int32)
    mask = np.zeros(n, np.uint8)
    codes = np.zeros((n, cfg["n_codebooks"]), np.int32)
    if p["kind"] in ("text", "ragged_text"):
        L.synth_uniform_int(seed, STREAM_PROMPT + stream, n, 0, cfg["vocab_text"], _ptr(tokens))
    elif p["kind"] == "voice_clone":
        nvq, nt = p["n_vq"], p["n_text"]
        text = np.empty(nt, np.int32)
        L.synth_uniform_int(seed, STREAM_PROMPT + stream, nt, 0, cfg["vocab_text"], _ptr(text))
        tokens[nvq:] = text
        vq = np.empty((nvq, cfg["n_codebooks"]), np.int32)
        L.synth_uniform_int(seed, STREAM_VQ + stream, vq.size, 0, cfg["codebook_size"], _ptr(vq))
        codes[:nvq] = vq
        mask[:nvq] = 1
        # a masked position carries the semantic id of its codebook-0 code as its token id
        tokens[:nvq] = cfg["vocab_text"] + vq[:, 0]
    else:
        raise ValueError(p["kind"])
    return tokens, mask, codes


def page_permutation(cfg, n_pages: int):
    """Seeded order in which pages of the KV pool are handed to streams."""
    out = np.empty(n_pages, np.int32)
    lib().synth_permutation(cfg["seed"], STREAM_PAGES, n_pages, _ptr(out))
    return out


def uniform_ints(seed, stream, n, lo, hi):
    out = np.empty(n, np.int32)
    lib().synth_uniform_int(seed, stream, n, lo, hi, _ptr(out))
    return out


def normals_f32(seed, stream, n, std=1.0):
    out = np.empty(n, np.float32)
    lib().synth_normal_f32(seed, stream, n, std, _ptr(out))
    return out


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def as_f32(a: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a
