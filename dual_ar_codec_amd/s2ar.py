"""Python binding of libs2ar.so: argument marshalling only.

Every step of the decode path runs in the library's HIP kernels; this module
converts numpy arrays to pointers and return codes to exceptions.  PyTorch, when
present, only supplies the HIP stream the library orders its work after.
There is no CPU fallback: if the library is missing or fails to load, every
entry point raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# S2AR_LIB names another build of the same library (an alternative build to compare against)
LIB_PATH = os.environ.get("S2AR_LIB") or os.path.join(_HERE, "libs2ar.so")

S2AR_OK = 0
ERRORS = {-1: "S2AR_E_ARG", -2: "S2AR_E_RANGE", -3: "S2AR_E_CAPACITY", -4: "S2AR_E_STATE",
          -5: "S2AR_E_NOMEM", -6: "S2AR_E_DEVICE", -7: "S2AR_E_NUMERIC"}

SYMBOLS = ("s2ar_create", "s2ar_prefill", "s2ar_decode_frame", "s2ar_decode_frames", "s2ar_release_stream",
           "s2ar_stream_position", "s2ar_destroy", "s2ar_last_error", "s2ar_error_name", "s2ar_debug_frame",
           "s2ar_time_kernel", "s2ar_debug_frame_batch", "s2ar_share_prefix", "s2ar_time_frames",
           "s2ar_decode_frames_noalloc", "s2ar_set_prefill_precision")

i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p


class S2arError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


class Stack(ctypes.Structure):
    _fields_ = [(n, i32) for n in ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn")]


# device-memory callbacks of s2ar_config: void* dev_alloc(uint64 bytes, void* user),
# void dev_free(void* ptr, uint64 bytes, void* user)
DEV_ALLOC = ctypes.CFUNCTYPE(vp, ctypes.c_uint64, vp)
DEV_FREE = ctypes.CFUNCTYPE(None, vp, ctypes.c_uint64, vp)


class Config(ctypes.Structure):
    _fields_ = [("slow", Stack), ("fast", Stack), ("vocab_text", i32), ("n_codebooks", i32),
                ("codebook_size", i32), ("rope_theta", ctypes.c_double), ("rms_eps", ctypes.c_double),
                ("weight_dtype", i32), ("rope_bf16", i32), ("max_streams", i32), ("max_context", i32),
                ("page_size", i32), ("kv_dtype", i32), ("eos_id", i32), ("head_slice", i32),
                ("dev_alloc", DEV_ALLOC), ("dev_free", DEV_FREE), ("alloc_user", vp)]


class Tensor(ctypes.Structure):
    _fields_ = [("host_ptr", vp), ("nbytes", i64)]


class Taps(ctypes.Structure):
    _fields_ = [(n, vp) for n in ("slow_embed", "slow_resid", "slow_h", "slow_logits", "fast_resid", "fast_z",
                                  "fast_logits", "own_codes", "next_c0")]


_lib = None


def lib():
    """Load libs2ar.so (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.s2ar_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Tensor), i32, vp, ctypes.POINTER(vp)]
        L.s2ar_prefill.argtypes = [vp, i32, vp, vp, vp, i32]
        L.s2ar_decode_frame.argtypes = [vp, vp, i32, vp]
        L.s2ar_decode_frames.argtypes = [vp, vp, i32, i32, vp]
        L.s2ar_release_stream.argtypes = [vp, i32]
        L.s2ar_share_prefix.argtypes = [vp, i32, i32, i32]
        L.s2ar_stream_position.argtypes = [vp, i32, ctypes.POINTER(i32)]
        L.s2ar_destroy.argtypes = [vp]
        L.s2ar_destroy.restype = None
        L.s2ar_last_error.argtypes = [vp]
        L.s2ar_last_error.restype = ctypes.c_char_p
        L.s2ar_error_name.argtypes = [ctypes.c_int]
        L.s2ar_error_name.restype = ctypes.c_char_p
        L.s2ar_debug_frame.argtypes = [vp, i32, vp, ctypes.POINTER(Taps)]
        L.s2ar_time_kernel.argtypes = [vp, i32, i32, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i64)]
        L.s2ar_debug_frame_batch.argtypes = [vp, vp, i32, vp, ctypes.POINTER(Taps)]
        L.s2ar_time_frames.argtypes = [vp, i32, i32, vp]
        L.s2ar_decode_frames_noalloc.argtypes = [vp, i32, i32, vp]
        L.s2ar_set_prefill_precision.argtypes = [vp, i32]
        _lib = L
    return _lib


# "i8" / "f8": bf16 tensors in; the library keeps the layer matrices and heads as int8 / FP8 E4M3
# codes with row scales
WEIGHT_DTYPES = {"f32": 0, "bf16": 1, "i8": 2, "f8": 3}
# KV cache elements: both fp32, both bf16, bf16 keys with fp32 values, fp32 keys with bf16 values
KV_DTYPES = {"f32": 0, "bf16": 1, "k_bf16": 2, "v_bf16": 3}


def make_config(cfg: dict, max_streams: int | None = None) -> Config:
    def st(s):
        return Stack(s["n_layers"], s["hidden"], s["n_q_heads"], s["n_kv_heads"], s["head_dim"], s["ffn"])

    return Config(st(cfg["slow"]), st(cfg["fast"]), cfg["vocab_text"], cfg["n_codebooks"], cfg["codebook_size"],
                  float(cfg["rope_theta"]), float(cfg["rms_eps"]), WEIGHT_DTYPES[cfg["weight_dtype"]],
                  int(cfg["rope_bf16"]), int(max_streams or cfg.get("n_streams", 1)), int(cfg["max_context"]),
                  int(cfg.get("page_size", 16)), KV_DTYPES[cfg.get("kv_dtype", "f32")],
                  int(cfg.get("eos_id", -1)), int(cfg.get("head_slice", 0)))


def _p(a):
    return None if a is None else a.ctypes.data


def current_stream_handle():
    """Handle of torch's current HIP stream on the current device (None without torch/GPU)."""
    try:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
    except ImportError:
        pass
    return None


def s2ar_create(cfg: Config, weights: list, hip_stream=None):
    """Returns (code, ctx_handle)."""
    arr = (Tensor * len(weights))(*[Tensor(w.ctypes.data, w.nbytes) for w in weights])
    out = vp()
    rc = lib().s2ar_create(ctypes.byref(cfg), arr, len(weights), hip_stream, ctypes.byref(out))
    return rc, out.value


def s2ar_last_error(ctx=None) -> str:
    return lib().s2ar_last_error(ctx).decode()


def torch_allocator():
    """(alloc, free) over PyTorch's caching allocator on the current device and stream: the
    context's device memory then belongs to torch's pool."""
    import torch

    dev = torch.cuda.current_device()
    stream = torch.cuda.current_stream()

    def alloc(nbytes):
        return torch.cuda.caching_allocator_alloc(int(nbytes), dev, stream)

    def free(ptr, nbytes):
        torch.cuda.caching_allocator_delete(ptr)

    return alloc, free


class Context:
    """One s2ar context: weights resident in HBM, per-stream KV pages and state.

    allocator: None (the library's hipMalloc), "torch" (PyTorch's caching allocator) or a pair
    (alloc(nbytes) -> device pointer int or 0, free(ptr, nbytes)) of Python callables."""

    def __init__(self, cfg: dict, weights: list, max_streams: int | None = None, hip_stream="torch",
                 allocator=None):
        self.cfg = cfg
        self.NC = cfg["n_codebooks"]
        self.H = cfg["slow"]["hidden"]
        self.V = cfg["vocab_text"] + cfg["codebook_size"]
        self.K = cfg["codebook_size"]
        self._weights = [np.ascontiguousarray(w) for w in weights]
        self.ccfg = make_config(cfg, max_streams)
        if allocator is not None:
            alloc, free = torch_allocator() if allocator == "torch" else allocator
            # the callbacks must outlive the context: the library calls dev_free in s2ar_destroy
            self._cb = (DEV_ALLOC(lambda nbytes, user: alloc(nbytes) or None),
                        DEV_FREE(lambda ptr, nbytes, user: free(ptr, nbytes)))
            self.ccfg.dev_alloc, self.ccfg.dev_free = self._cb
        stream = current_stream_handle() if hip_stream == "torch" else hip_stream
        rc, h = s2ar_create(self.ccfg, self._weights, stream)
        self._weights = None  # uploaded; the library keeps no host pointer
        if rc != S2AR_OK:
            raise S2arError(rc, s2ar_last_error(None))
        self._destroy = lib().s2ar_destroy  # kept: module globals may be gone when __del__ runs at exit
        self.h = h

    def _check(self, rc):
        if rc != S2AR_OK:
            raise S2arError(rc, lib().s2ar_last_error(self.h).decode())

    def close(self):
        if getattr(self, "h", None):
            self._destroy(self.h)
            self.h = None

    def __del__(self):
        self.close()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def prefill(self, stream_id, tokens, mask=None, codes=None):
        t = np.ascontiguousarray(tokens, np.int32)
        m = None if mask is None else np.ascontiguousarray(mask, np.uint8)
        c = None if codes is None else np.ascontiguousarray(codes, np.int32)
        self._check(lib().s2ar_prefill(self.h, int(stream_id), _p(t), _p(m), _p(c), len(t)))

    def set_prefill_precision(self, precision):
        """0: bf16 hi/lo activation split (default); 1: one fp16 activation plane."""
        self._check(lib().s2ar_set_prefill_precision(self.h, int(precision)))

    def decode_frame(self, stream_ids):
        ids = np.ascontiguousarray(np.atleast_1d(stream_ids), np.int32)
        out = np.zeros((len(ids), self.NC), np.int32)
        self._check(lib().s2ar_decode_frame(self.h, _p(ids), len(ids), _p(out)))
        return out

    def decode_frames(self, stream_ids, n_frames):
        ids = np.ascontiguousarray(np.atleast_1d(stream_ids), np.int32)
        out = np.zeros((n_frames, len(ids), self.NC), np.int32)
        self._check(lib().s2ar_decode_frames(self.h, _p(ids), len(ids), int(n_frames), _p(out)))
        return out

    def decode_frames_noalloc(self, stream_id, n_frames):
        """n_frames frames of one stream through the allocation-free entry point."""
        out = np.zeros((int(n_frames), self.NC), np.int32)
        self._check(lib().s2ar_decode_frames_noalloc(self.h, int(stream_id), int(n_frames), _p(out)))
        return out

    def release(self, stream_id):
        self._check(lib().s2ar_release_stream(self.h, int(stream_id)))

    def share_prefix(self, src_id, dst_id, n_positions):
        self._check(lib().s2ar_share_prefix(self.h, int(src_id), int(dst_id), int(n_positions)))

    def position(self, stream_id):
        p = i32()
        self._check(lib().s2ar_stream_position(self.h, int(stream_id), ctypes.byref(p)))
        return p.value

    def debug_frame(self, stream_id, forced=None):
        cfg = self.cfg
        Ls, Lf, H, K, NC = cfg["slow"]["n_layers"], cfg["fast"]["n_layers"], self.H, self.K, self.NC
        out = dict(slow_embed=np.zeros(H, np.float32), slow_resid=np.zeros((Ls, H), np.float32),
                   slow_h=np.zeros(H, np.float32), slow_logits=np.zeros(self.V, np.float32),
                   fast_resid=np.zeros((NC - 1, Lf, H), np.float32), fast_z=np.zeros((NC - 1, H), np.float32),
                   fast_logits=np.zeros((NC - 1, K), np.float32), own_codes=np.zeros(NC, np.int32),
                   next_c0=np.zeros(1, np.int32))
        taps = Taps(*[out[n].ctypes.data for n, _ in Taps._fields_])
        f = None if forced is None else np.ascontiguousarray(forced, np.int32)
        self._check(lib().s2ar_debug_frame(self.h, int(stream_id), _p(f), ctypes.byref(taps)))
        out["next_c0"] = int(out["next_c0"][0])
        return out

    def _tap_buffers(self):
        cfg = self.cfg
        Ls, Lf, H, K, NC = cfg["slow"]["n_layers"], cfg["fast"]["n_layers"], self.H, self.K, self.NC
        return dict(slow_embed=np.zeros(H, np.float32), slow_resid=np.zeros((Ls, H), np.float32),
                    slow_h=np.zeros(H, np.float32), slow_logits=np.zeros(self.V, np.float32),
                    fast_resid=np.zeros((NC - 1, Lf, H), np.float32), fast_z=np.zeros((NC - 1, H), np.float32),
                    fast_logits=np.zeros((NC - 1, K), np.float32), own_codes=np.zeros(NC, np.int32),
                    next_c0=np.zeros(1, np.int32))

    def debug_frame_batch(self, stream_ids, forced=None):
        """Eager batched frame of several streams (the batched decode kernels) with taps."""
        ids = np.ascontiguousarray(np.atleast_1d(stream_ids), np.int32)
        outs = [self._tap_buffers() for _ in ids]
        taps = (Taps * len(ids))(*[Taps(*[o[n].ctypes.data for n, _ in Taps._fields_]) for o in outs])
        f = None if forced is None else np.ascontiguousarray(forced, np.int32)
        self._check(lib().s2ar_debug_frame_batch(self.h, _p(ids), len(ids), _p(f), taps))
        for o in outs:
            o["next_c0"] = int(o["next_c0"][0])
        return outs

    def time_frames(self, stream_id, n_frames):
        """Per-frame graph-replay durations (ms) of n_frames frames of one stream, from HIP events."""
        out = np.zeros(int(n_frames), np.float32)
        self._check(lib().s2ar_time_frames(self.h, int(stream_id), int(n_frames), _p(out)))
        return out

    def time_kernel(self, which=0, iters=100):
        ms = ctypes.c_float()
        nb = i64()
        self._check(lib().s2ar_time_kernel(self.h, int(which), int(iters), ctypes.byref(ms), ctypes.byref(nb)))
        return ms.value, nb.value
