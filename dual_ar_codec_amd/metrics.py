"""Frame accounting for the Dual-AR decode step: audio time per frame, RTF and
algorithmic bytes per frame.

- A frame is one semantic code plus nine residual codes, and the codec turns it
  into 2048 samples at 44.1 kHz ("s2pro-native", What happens to a sentence).
- RTF is compute time divided by audio time ("s2pro-native", Where it stands).
- At batch 1 each frame streams every weight of the Slow stack and its head
  once, and the Fast stack and its head nine times ("s2pro-native", Where it
  stands, counts about 7.75 billion parameters per frame).
"""
from __future__ import annotations

N_CODEBOOKS = 10
N_FAST_STEPS = N_CODEBOOKS - 1
FRAME_SAMPLES = 2048
SAMPLE_RATE = 44100


def frame_seconds() -> float:
    """Audio time covered by one frame."""
    return FRAME_SAMPLES / SAMPLE_RATE


def rtf(frames_per_s: float) -> float:
    """Real-time factor: seconds of compute per second of audio."""
    return 1.0 / (frames_per_s * frame_seconds())


def codebook_tokens_per_s(frames_per_s: float) -> float:
    return N_CODEBOOKS * frames_per_s


def _esz(cfg) -> int:
    return 4 if cfg["weight_dtype"] == "f32" else 2


def layer_matrix_params(s: dict) -> int:
    H, Hq, Hkv, D, F = s["hidden"], s["n_q_heads"], s["n_kv_heads"], s["head_dim"], s["ffn"]
    return H * Hq * D + 2 * H * Hkv * D + Hq * D * H + 3 * H * F


def layer_gain_params(s: dict) -> int:
    return 2 * s["hidden"] + 2 * s["head_dim"]


def params_per_frame(cfg, head_rows: int | None = None) -> int:
    """Weight parameters one batch-1 frame streams (matrices only).

    head_rows defaults to the full Slow vocabulary (text + semantic ids)."""
    rows = cfg["vocab_slow"] if head_rows is None else head_rows
    s, f = cfg["slow"], cfg["fast"]
    slow = s["n_layers"] * layer_matrix_params(s) + rows * s["hidden"]
    fast = f["n_layers"] * layer_matrix_params(f) + cfg["codebook_size"] * f["hidden"]
    return slow + N_FAST_STEPS * fast


def kv_bytes_per_position(cfg) -> int:
    """K and V of one Slow position over all layers: fp32 by default; "bf16" both halves, "k_bf16"
    bf16 keys with fp32 values, "v_bf16" fp32 keys with bf16 values."""
    s = cfg["slow"]
    kv = cfg.get("kv_dtype", "f32")
    k_esz = 2 if kv in ("bf16", "k_bf16") else 4
    v_esz = 2 if kv in ("bf16", "v_bf16") else 4
    return s["n_layers"] * s["n_kv_heads"] * s["head_dim"] * (k_esz + v_esz)


GAIN_BYTES = 4  # norm gains are held in fp32 on the device, whatever the weights' dtype


def frame_bytes(cfg, context_len: int) -> dict:
    """Algorithmic HBM bytes of one batch-1 frame at a Slow context of context_len.

    weights: every matrix and gain the frame reads (Fast stack and head x9);
    kv: Slow keys/values read by attention (plus the new position's write);
    embed: codebook rows gathered for the Slow input (10) and Fast inputs (8).
    """
    esz = _esz(cfg)
    s, f = cfg["slow"], cfg["fast"]
    w = params_per_frame(cfg) * esz
    w += (s["n_layers"] * layer_gain_params(s) + s["hidden"]) * GAIN_BYTES
    w += N_FAST_STEPS * (f["n_layers"] * layer_gain_params(f) + f["hidden"]) * GAIN_BYTES
    kv = kv_bytes_per_position(cfg) * (context_len + 1)
    embed = (N_CODEBOOKS + N_FAST_STEPS - 1) * s["hidden"] * esz
    return dict(weights=w, kv=kv, embed=embed, total=w + kv + embed)


def int8_frame_bytes(cfg, context_len: int) -> dict:
    """frame_bytes with the layer matrices and both heads stored as 8-bit codes (int8 or FP8) plus one fp32 scale per
    row (embeddings, codebooks and gains as in frame_bytes)."""
    fb = frame_bytes(cfg, context_len)
    s, f = cfg["slow"], cfg["fast"]

    def rows(st):
        H, D = st["hidden"], st["head_dim"]
        return (st["n_q_heads"] + 2 * st["n_kv_heads"]) * D + H + 2 * st["ffn"] + H

    p = params_per_frame(cfg)
    scale_rows = s["n_layers"] * rows(s) + cfg["vocab_slow"] + N_FAST_STEPS * (f["n_layers"] * rows(f) + cfg["codebook_size"])
    w = fb["weights"] - p * _esz(cfg) + p + 4 * scale_rows
    return dict(fb, weights=w, total=w + fb["kv"] + fb["embed"])


def gate_up_launch_bytes(cfg, stack: str = "slow") -> int:
    """Algorithmic bytes of one fused RMSNorm + gate/up + SwiGLU launch:
    both weight matrices, the gain, the fp32 input and the fp32 output."""
    s = cfg[stack]
    esz = _esz(cfg)
    return 2 * s["ffn"] * s["hidden"] * esz + s["hidden"] * GAIN_BYTES + s["hidden"] * 4 + s["ffn"] * 4
