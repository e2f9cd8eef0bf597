"""Generator "planted-v1": seeded synthetic long-context attention layers.

The layer shapes follow the workloads the FAST-Prefill write-ups talk about
(Llama-3-family layers, contexts up to 128K tokens, blocks of b = 128 or 256
tokens, grouped-query attention).  No trained weights exist here, so Q, K and V
are Gaussian and the two sparsity structures the method distinguishes are
planted on purpose:

* vertical-slash (VS) KV groups: all queries of the group share a common offset
  direction, a few "sink" key positions are pushed along the mean query, and
  every key gets half of the mean query at its own position (a local band);
* query-aware (QA) KV groups: keys of each block sit around a per-block
  centroid, and the queries of block i sit near the sum of the centroids of up
  to three earlier blocks chosen at random per head.

Draw order (all from one numpy PCG64 stream, seed given by the caller):
  1. Zq [Hq,S,d], Zk [Hkv,S,d], V [Hkv,S,d]  ~ N(0,1) float32
  2. rotary embedding (base 500000, rotate-half pairs (i, i+d/2)) on Zq and Zk
  3. per KV group g = 0..Hkv-1 in order:
       VS group: unit direction u_g (d normals), then 8 distinct spike positions
       QA group: centroids c_g [N,d], then for each head of the group and each
                 block i >= 1, min(3, i) distinct earlier blocks
  4. round Q, K, V to bf16 (round-half-to-even); both paths consume these bits
  5. (W8A8 only) per-(head, token) symmetric int8 quantisation, fp32 arithmetic

Groups 0..ceil(f*Hkv)-1 are VS and the rest QA (f = 1/2, or 3/4 for the 8B
shape).  The amplitudes (query offset 8, spike 4 x mean query, band 0.5,
unit-variance centroids) are conventions of this generator.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import numpy as np
import torch

VS_QUERY_OFFSET = 8.0   # shared query offset along u_g for VS groups
VS_SPIKE_GAIN = 4.0     # sink keys get += 4 * mean query of the group
VS_BAND_GAIN = 0.5      # every key gets += 0.5 * mean over heads of Q at its position
VS_N_SINKS = 4          # positions 0..3
VS_N_RANDOM = 8         # plus 8 distinct random positions in [4, S)
QA_SOURCES = 3          # a query block sits near the sum of 3 earlier centroids


@dataclass(frozen=True)
class LayerConfig:
    name: str
    S: int
    b: int
    Hq: int
    Hkv: int
    d: int = 128
    gamma: float = 0.9
    tau: float = 0.1
    vs_frac: float = 0.5
    int8: bool = False
    rope_base: float = 500000.0

    @property
    def N(self) -> int:
        return self.S // self.b

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


CONFIGS: Dict[str, LayerConfig] = {
    # one attention layer, S=2048, b=128, 4 query heads over 2 KV heads
    "tiny": LayerConfig("tiny", S=2048, b=128, Hq=4, Hkv=2),
    # Llama-3.2-3B attention shape (24 query heads, 8 KV heads, d=128)
    "3b-32k": LayerConfig("3b-32k", S=32768, b=128, Hq=24, Hkv=8),
    "3b-128k": LayerConfig("3b-128k", S=131072, b=128, Hq=24, Hkv=8),
    # Llama-3-8B attention shape (32 query heads, 8 KV heads), b=256
    "8b-64k": LayerConfig("8b-64k", S=65536, b=256, Hq=32, Hkv=8, gamma=0.95, vs_frac=0.75),
    # W8A8 variant of the 128K 3B layer
    "w8a8-128k": LayerConfig("w8a8-128k", S=131072, b=128, Hq=24, Hkv=8, int8=True),
    # the 128K 3B layer with 64-token blocks (N = 2048)
    "3b-128k-b64": LayerConfig("3b-128k-b64", S=131072, b=64, Hq=24, Hkv=8),
}


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-half-to-even), returned as uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _bf16_bits_fast(x: np.ndarray) -> np.ndarray:
    """Same rounding as bf16_bits_from_f32 (round-half-to-even), multi-threaded through torch's
    float32 -> bfloat16 cast; used for the large tensors of a layer."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_from_bf16_bits(u16: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize_rows(x: np.ndarray):
    """Symmetric per-row int8 quantisation over the last axis, float32 arithmetic.

    s = max|x| / 127 (s = 1 for an all-zero row); x8 = clamp(rint_half_even(x / s), -127, 127).
    Returns (int8 array, float32 scales with the last axis dropped).
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    s = np.where(amax > 0, s, np.float32(1.0)).astype(np.float32)
    q = np.rint(x / s[..., None]).astype(np.float32)
    q = np.clip(q, -127, 127).astype(np.int8)
    return q, s


def _rope_tables(S: int, d: int, base: float):
    half = d // 2
    inv = base ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.arange(S, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _apply_rope_inplace(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> None:
    """x: [H, S, d] float32, rotate-half pairs (i, i + d/2)."""
    half = x.shape[-1] // 2
    for h in range(x.shape[0]):
        a = x[h, :, :half].copy()
        c = x[h, :, half:]
        x[h, :, :half] = a * cos - c * sin
        x[h, :, half:] = c * cos + a * sin


@dataclass
class Layer:
    cfg: LayerConfig
    seed: int
    q: np.ndarray              # uint16 bf16 bits [Hq, S, d]
    k: np.ndarray              # uint16 bf16 bits [Hkv, S, d]
    v: np.ndarray              # uint16 bf16 bits [Hkv, S, d]
    planted: np.ndarray        # uint8 [Hq]: 0 = planted vertical-slash, 1 = planted query-aware
    spikes: Dict[int, np.ndarray] = field(default_factory=dict)  # VS group -> spike token positions
    _i8: Optional[dict] = None

    def f32(self, name: str) -> np.ndarray:
        return f32_from_bf16_bits(getattr(self, name))

    def int8(self) -> dict:
        """Per-(head, token) int8 copies of Q, K, V with float32 scales [H, S]."""
        if self._i8 is None:
            out = {}
            for name in ("q", "k", "v"):
                q8, s = quantize_rows(self.f32(name))
                out[name + "8"] = q8
                out["s" + name] = s
            self._i8 = out
        return self._i8


def make(cfg, seed: int = 0) -> Layer:
    """Draw one layer of the given config (a LayerConfig or a name in CONFIGS)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    S, b, Hq, Hkv, d = cfg.S, cfg.b, cfg.Hq, cfg.Hkv, cfg.d
    if S % b or Hq % Hkv or d % 2:
        raise ValueError("generator needs S % b == 0, Hq % Hkv == 0 and even d")
    N, G = S // b, Hq // Hkv
    rng = np.random.Generator(np.random.PCG64(seed))

    q = rng.standard_normal((Hq, S, d), dtype=np.float32)
    k = rng.standard_normal((Hkv, S, d), dtype=np.float32)
    v = rng.standard_normal((Hkv, S, d), dtype=np.float32)

    cos, sin = _rope_tables(S, d, cfg.rope_base)
    _apply_rope_inplace(q, cos, sin)
    _apply_rope_inplace(k, cos, sin)
    del cos, sin

    n_vs = int(math.ceil(cfg.vs_frac * Hkv - 1e-9))
    planted = np.zeros(Hq, dtype=np.uint8)
    spikes: Dict[int, np.ndarray] = {}
    for g in range(Hkv):
        heads = range(g * G, (g + 1) * G)
        if g < n_vs:
            u = rng.standard_normal(d)
            u = (u / np.linalg.norm(u)).astype(np.float32)
            for h in heads:
                q[h] += np.float32(VS_QUERY_OFFSET) * u
            m_g = np.zeros(d, dtype=np.float64)
            for h in heads:
                m_g += q[h].sum(axis=0, dtype=np.float64)
            m_g = (m_g / (G * S)).astype(np.float32)
            n_sink = min(VS_N_SINKS, S)
            n_rand = min(VS_N_RANDOM, max(S - VS_N_SINKS, 0))
            pos = list(range(n_sink))
            if n_rand > 0:
                pos += list(rng.choice(S - VS_N_SINKS, size=n_rand, replace=False) + VS_N_SINKS)
            pos = np.array(sorted(pos), dtype=np.int64)
            spikes[g] = pos
            k[g, pos] += np.float32(VS_SPIKE_GAIN) * m_g
            qmean = q[g * G].copy()
            for h in list(heads)[1:]:
                qmean += q[h]
            qmean *= np.float32(1.0 / G)
            k[g] += np.float32(VS_BAND_GAIN) * qmean
            del qmean
        else:
            for h in heads:
                planted[h] = 1
            c = rng.standard_normal((N, d), dtype=np.float32)
            k[g] += np.repeat(c, b, axis=0)
            for h in heads:
                for i in range(1, N):
                    src = rng.choice(i, size=min(QA_SOURCES, i), replace=False)
                    q[h, i * b:(i + 1) * b] += c[src].sum(axis=0)

    qb = _bf16_bits_fast(q)
    del q
    kb = _bf16_bits_fast(k)
    vb = _bf16_bits_fast(v)
    return Layer(cfg=cfg, seed=seed, q=qb, k=kb, v=vb, planted=planted, spikes=spikes)


def rope_tables(S: int, d: int = 128, base: float = 500000.0):
    """The rotary embedding's cos / sin tables [S, d/2] (float32) for positions 0..S-1."""
    return _rope_tables(S, d, base)


def projection_inputs(S: int, D: int, Hq: int, Hkv: int, seed: int = 0, d: int = 128):
    """Seeded inputs of a QKV projection: X [S, D] ~ N(0, 1) and W [(Hq + 2 Hkv) * d, D] ~ N(0, 1/D)
    (so every projected value is about N(0, 1)), both rounded to bf16 (uint16 bit patterns), and the
    rotary tables [S, d/2] (float32, base 500000)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    X = rng.standard_normal((S, D), dtype=np.float32)
    W = rng.standard_normal(((Hq + 2 * Hkv) * d, D), dtype=np.float32) * np.float32(1.0 / math.sqrt(D))
    cos, sin = _rope_tables(S, d, 500000.0)
    return {"x": _bf16_bits_fast(X), "w": _bf16_bits_fast(W), "cos": cos, "sin": sin}
