"""The QKV projection and what its epilogue emits, float64 reference (oracle; test infrastructure only).

The explainer's section 1.1 obtains Q, K and V from the input X by three linear projections; the
rotary position embedding (rotate-half pairs (c, c + d/2), the tables supplied by the caller) acts
on Q and K.  The products are rounded to bf16, the storage precision of the path.  The same step
also emits, for the later stages:
  * the mean of every block of b rounded queries / keys (the pooled vectors of Flex-Prefill's
    pattern test and query-aware rows, explainer section 1.2);
  * the symmetric per-(head, token) int8 codes of the rounded values (W8A8, explainer sections 3.3
    and 4.2): s = max|x| / 127 in float32 (1 for an all-zero row), codes rint(x / s) (half to even)
    clamped to [-127, 127], computed in float32.
"""
from __future__ import annotations

import numpy as np
import torch


def as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def bf16_round(x) -> np.ndarray:
    """Nearest bf16 (ties to even) of float64 values, returned as float64."""
    return torch.from_numpy(as64(x)).to(torch.bfloat16).to(torch.float64).numpy()


def rope(x, cos, sin) -> np.ndarray:
    """Rotary embedding of rows x [S, d]: pairs (c, c + d/2) rotated by the angle whose cos / sin
    (tables [S, d/2]) are given for each position and frequency."""
    x = as64(x)
    half = x.shape[1] // 2
    a, b = x[:, :half], x[:, half:]
    c, s = as64(cos), as64(sin)
    return np.concatenate([a * c - b * s, b * c + a * s], axis=1)


def quantize(x):
    """Symmetric per-row int8 over the last axis, float32 arithmetic: (codes int8, scales float32)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    s = np.where(amax > 0, amax / np.float32(127.0), np.float32(1.0)).astype(np.float32)
    codes = np.clip(np.rint(x / s[..., None]), -127, 127).astype(np.int8)
    return codes, s


def block_means(x, b: int) -> np.ndarray:
    x = as64(x)
    return x.reshape(x.shape[0] // b, b, x.shape[1]).mean(axis=1)


def project(X, W, Hq: int, Hkv: int, b: int, cos=None, sin=None, d: int = 128) -> dict:
    """X [S, D], W [(Hq + 2 Hkv) d, D] (rows: Q heads, K heads, V heads).  Returns the bf16-rounded
    head-major q [Hq, S, d], k, v [Hkv, S, d] (float64), their block means qbar, kbar, and the int8
    codes / scales q8, sq, k8, sk, v8, sv."""
    Y = as64(X) @ as64(W).T
    out = {}
    for name, h0, nh, rot in (("q", 0, Hq, True), ("k", Hq, Hkv, True), ("v", Hq + Hkv, Hkv, False)):
        heads = []
        for h in range(nh):
            y = Y[:, (h0 + h) * d:(h0 + h + 1) * d]
            if rot and cos is not None:
                y = rope(y, cos, sin)
            heads.append(bf16_round(y))
        out[name] = np.stack(heads)
        q8, s = quantize(out[name])
        out[name + "8"], out["s" + name] = q8, s
    out["qbar"] = np.stack([block_means(x, b) for x in out["q"]])
    out["kbar"] = np.stack([block_means(x, b) for x in out["k"]])
    return out
