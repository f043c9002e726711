"""The C-ABI library loads, exports every declared symbol and validates its
arguments before touching a device (no compute call needs a GPU here)."""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

from dual_ar_codec_amd import s2ar, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(s2ar.LIB_PATH):
        from dual_ar_codec_amd import build
        build.build_hip()
    return s2ar.lib()


def _declared():
    txt = open(os.path.join(ROOT, "include", "s2ar.h")).read()
    return sorted(set(re.findall(r"\b(s2ar_[a-z_]+)\s*\(", txt)))


def test_every_declared_symbol_is_exported(L):
    decl = _declared()
    assert "s2ar_create" in decl and "s2ar_decode_frame" in decl
    out = subprocess.check_output(["nm", "-D", "--defined-only", s2ar.LIB_PATH]).decode()
    exported = set(re.findall(r" T (s2ar_\w+)", out))
    missing = [d for d in decl if d not in exported]
    assert not missing, missing
    for d in decl:
        getattr(L, d)
    assert set(s2ar.SYMBOLS) <= exported


def test_error_names(L):
    assert L.s2ar_error_name(0) == b"S2AR_OK"
    for code, name in s2ar.ERRORS.items():
        assert L.s2ar_error_name(code).decode() == name


def test_null_and_noop_calls(L):
    L.s2ar_destroy(None)
    assert L.s2ar_prefill(None, 0, None, None, None, 1) == -1
    assert L.s2ar_decode_frame(None, None, 1, None) == -1
    assert L.s2ar_debug_frame(None, 0, None, None) == -1
    assert L.s2ar_time_frames(None, 0, 1, None) == -1
    assert L.s2ar_share_prefix(None, 0, 1, 1) == -1
    out = ctypes.c_void_p()
    assert L.s2ar_create(None, None, 0, None, ctypes.byref(out)) == -1
    assert out.value is None
    assert "non-null" in s2ar.s2ar_last_error(None)


def _cfg(**over):
    c = synth.config("tiny")
    for k, v in over.items():
        if "." in k:
            a, b = k.split(".")
            c[a] = dict(c[a], **{b: v})
        else:
            c[k] = v
    return c


@pytest.mark.parametrize("over,needle", [
    ({"slow.n_kv_heads": 3}, "multiple of n_kv_heads"),
    ({"slow.head_dim": 96}, "head_dim"),
    ({"fast.hidden": 512}, "fast.hidden"),
    ({"page_size": 32}, "page_size"),
    ({"n_codebooks": 1}, "n_codebooks"),
    ({"max_context": 0}, "max_context"),
    ({"slow.ffn": 770}, "multiples of 4"),
    ({"rope_theta": -1.0}, "rope_theta"),
    ({"eos_id": 4096}, "eos_id"),        # a semantic id (tiny: 4096 text ids) cannot be the stop id
    ({"eos_id": -2}, "eos_id"),
    ({"head_slice": 2}, "head_slice"),
])
def test_config_validation(L, over, needle):
    cfg = _cfg(**over)
    w = [np.zeros(1, np.float32)]
    rc, h = s2ar.s2ar_create(s2ar.make_config(cfg), w, None)
    assert rc == -1 and h is None
    assert needle in s2ar.s2ar_last_error(None)


@pytest.mark.parametrize("field,value,needle", [("weight_dtype", 4, "weight_dtype"), ("kv_dtype", 4, "kv_dtype"),
                                               ("kv_dtype", -1, "kv_dtype")])
def test_raw_config_fields_out_of_range(L, field, value, needle):
    c = s2ar.make_config(_cfg())
    setattr(c, field, value)
    rc, h = s2ar.s2ar_create(c, [np.zeros(1, np.float32)], None)
    assert rc == -1 and h is None and needle in s2ar.s2ar_last_error(None)


def test_tensor_validation(L):
    cfg = _cfg()
    w = synth.make_weights(cfg)
    c = s2ar.make_config(cfg)
    rc, _ = s2ar.s2ar_create(c, w[:-1], None)
    assert rc == -1 and "n_tensors" in s2ar.s2ar_last_error(None)
    bad = list(w)
    bad[3] = bad[3][:-1]
    rc, _ = s2ar.s2ar_create(c, bad, None)
    assert rc == -1 and "tensor 3" in s2ar.s2ar_last_error(None)


def test_valid_config_reaches_the_device_check(L):
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except ImportError:
        pass
    cfg = _cfg()
    w = synth.make_weights(cfg)
    rc, h = s2ar.s2ar_create(s2ar.make_config(cfg), w, None)
    assert rc == -6 and h is None
    assert "device" in s2ar.s2ar_last_error(None)


def test_product_path_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "dual_ar_codec_amd")
    pat = re.compile(r"(import\s+oracle|from\s+oracle|liboracle|orc_[a-z])")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".c", ".cpp")):
                assert not pat.search(open(os.path.join(dirpath, f)).read()), f


def test_a_missing_library_is_an_error_not_a_fallback(tmp_path):
    """With no built libs2ar.so the binding raises on first use; nothing runs in its place."""
    code = ("from dual_ar_codec_amd import s2ar\n"
            "try:\n    s2ar.lib()\nexcept RuntimeError as e:\n    print('raised:', e)\n")
    env = dict(os.environ, S2AR_LIB=str(tmp_path / "libs2ar.so"))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    assert "raised:" in r.stdout and "not built" in r.stdout


def test_allocator_callbacks_must_come_in_pairs(L):
    """dev_alloc without dev_free (or the reverse) is rejected before any device work, and no
    callback runs."""
    calls = []
    alloc = s2ar.DEV_ALLOC(lambda nbytes, user: calls.append(nbytes) or None)
    free = s2ar.DEV_FREE(lambda ptr, nbytes, user: calls.append(-1))
    for set_alloc, set_free in ((True, False), (False, True)):
        c = s2ar.make_config(_cfg())
        if set_alloc:
            c.dev_alloc = alloc
        if set_free:
            c.dev_free = free
        rc, h = s2ar.s2ar_create(c, [np.zeros(1, np.float32)], None)
        assert rc == -1 and h is None and "dev_alloc and dev_free" in s2ar.s2ar_last_error(None)
    assert calls == []


def test_config_struct_matches_the_header():
    """The binding's Config mirrors s2ar_config field for field (names in header order)."""
    txt = open(os.path.join(ROOT, "include", "s2ar.h")).read()
    body = txt[txt.index("typedef struct {\n  s2ar_stack slow, fast;"):txt.index("} s2ar_config;")]
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    names = []
    for decl in body.split(";"):
        decl = decl.strip()
        if not decl or decl.startswith("typedef"):
            if decl.startswith("typedef struct {"):
                decl = decl[len("typedef struct {"):].strip()
            else:
                continue
        m = re.search(r"\(\*\s*(\w+)\)", decl)
        if m:
            names.append(m.group(1))
            continue
        names += [n.strip().lstrip("*") for n in decl.split(None, 1)[1].split(",")]
    assert names == [n for n, _ in s2ar.Config._fields_]
