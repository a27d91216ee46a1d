"""Workload definitions and seeded input draws.

Six workloads, named by what they model:

* ``dit_tiny_f32``    fp32, B=1, H=2,  N=1024,   d=64,  block 64, non-causal,
                      clustered keys (centre + 0.1 noise), alpha=0.5, tail on.
* ``dit_image_8k``    bf16, B=1, H=24, N=8192,   d=128, block 64, non-causal,
                      clustered keys (centre + 0.3 noise), density 0.15, tail on.
* ``dit_video_32k``   bf16, B=1, H=40, N=32760,  d=128, block 64, non-causal,
                      key centres drifting smoothly from block to block
                      (stand-in for a 3D-contiguous token order), ragged last
                      block of 56 tokens, density 0.15, tail on.
* ``llm_prefill_128k`` bf16, B=1, 32 Q / 8 KV heads, N=131072, d=128, block 128,
                      causal, attention-sink + local-diagonal structure,
                      alpha=0.5, no tail.
* ``llm_prefill_256k`` bf16, B=1, H=8, N=262144, d=128, block 128, causal, same
                      generator as the 128K prefill, alpha=0.5, no tail.
* ``llm_prefill_128k_tail`` the 128K prefill with the 0th-order tail on: the
                      diagonal block is always exact, the tail covers the
                      unselected blocks left of it.

Every tensor is drawn in float32 from a numpy ``Generator`` seeded by
``SeedSequence([seed, workload tag, batch, kv group, stream])``, so one KV
group (its K, V and the Q heads that share it) can be drawn alone.  bf16
workloads are rounded once to bf16 (round-to-nearest-even) and returned as
float32 arrays holding exactly representable bf16 values.
"""

from __future__ import annotations

import dataclasses
import math
import zlib
from typing import Dict, List, Optional, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    block: int
    causal: bool
    select: str         # "alpha" or "density"
    alpha: float
    density: float
    approx: bool
    kind: str           # "cluster", "drift" or "sink"
    noise: float = 0.3  # key noise around the block centre (cluster/drift)

    @property
    def M(self) -> int:
        return -(-self.N // self.block)

    @property
    def tag(self) -> int:
        return zlib.crc32(self.name.encode()) & 0x7FFFFFFF

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


CONFIGS: List[Workload] = [
    Workload("dit_tiny_f32", "f32", 1, 2, 2, 1024, 64, 64, False, "alpha", 0.5, 0.0,
             True, "cluster", noise=0.1),
    Workload("dit_image_8k", "bf16", 1, 24, 24, 8192, 128, 64, False, "density", 0.0, 0.15,
             True, "cluster", noise=0.3),
    Workload("dit_video_32k", "bf16", 1, 40, 40, 32760, 128, 64, False, "density", 0.0, 0.15,
             True, "drift", noise=0.3),
    Workload("llm_prefill_128k", "bf16", 1, 32, 8, 131072, 128, 128, True, "alpha", 0.5, 0.0,
             False, "sink"),
    Workload("llm_prefill_256k", "bf16", 1, 8, 8, 262144, 128, 128, True, "alpha", 0.5, 0.0,
             False, "sink"),
    Workload("llm_prefill_128k_tail", "bf16", 1, 32, 8, 131072, 128, 128, True, "alpha", 0.5, 0.0,
             True, "sink"),
]


def get_config(name: str) -> Workload:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(f"unknown workload {name!r}; known: {[c.name for c in CONFIGS]}")


# --------------------------------------------------------------------------
# bf16 rounding (input preparation only)
# --------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bf16 (ties to even), kept as float32."""
    return (bf16_bits(x).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# seeded streams
# --------------------------------------------------------------------------

_S_STRUCT, _S_KNOISE, _S_V, _S_Q0, _S_DOUT = 0, 1, 2, 16, 64


def _rng(seed: int, tag: int, b: int, g: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tag, b, g, stream]))


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def _block_index(N: int, block: int) -> np.ndarray:
    return np.arange(N) // block


def _keys_cluster(rng_s, rng_n, N, d, block, noise):
    M = -(-N // block)
    centres = _normal(rng_s, (M, d))
    k = centres[_block_index(N, block)]
    k += np.float32(noise) * _normal(rng_n, (N, d))
    return k


def _keys_drift(rng_s, rng_n, N, d, block, noise):
    M = -(-N // block)
    xi = _normal(rng_s, (M, d))
    centres = np.empty((M, d), np.float32)
    centres[0] = xi[0]
    c = np.float32(0.9)
    s = np.float32(math.sqrt(1.0 - 0.81))
    for J in range(1, M):
        centres[J] = c * centres[J - 1] + s * xi[J]
    k = centres[_block_index(N, block)]
    k += np.float32(noise) * _normal(rng_n, (N, d))
    return k


_SINK_ANCHOR_EVERY = 64      # tokens between positional anchors
_SINK_TOKENS = 64            # keys carrying the large-norm sink offset
_SINK_CORR_TOKENS = 2048     # anchor correlation falls to 0.5 over this many tokens


def _sink_structure(rng_s, N, d):
    """Unit sink direction u and per-token positional anchor p(t) (AR(1) over anchors)."""
    u = _normal(rng_s, (d,))
    u /= np.linalg.norm(u)
    n_anchor = -(-N // _SINK_ANCHOR_EVERY)
    rho = 0.5 ** (_SINK_ANCHOR_EVERY / _SINK_CORR_TOKENS)
    xi = _normal(rng_s, (n_anchor, d)) * np.float32(1.0 / math.sqrt(d))
    a = np.empty((n_anchor, d), np.float32)
    a[0] = xi[0]
    c = np.float32(rho)
    s = np.float32(math.sqrt(1.0 - rho * rho))
    for n in range(1, n_anchor):
        a[n] = c * a[n - 1] + s * xi[n]
    return u.astype(np.float32), a


def make_group(wl: Workload, seed: int, b: int, g: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Draw KV group ``g`` of batch ``b``.

    Returns ``(q, k, v)`` with ``q`` of shape [Hq/Hkv, N, d] (the Q heads
    ``g*G .. g*G+G-1``) and ``k``, ``v`` of shape [N, d]; float32 arrays, bf16
    rounded for bf16 workloads.
    """
    N, d, G = wl.N, wl.d, wl.Hq // wl.Hkv
    rs = _rng(seed, wl.tag, b, g, _S_STRUCT)
    rn = _rng(seed, wl.tag, b, g, _S_KNOISE)
    if wl.kind == "cluster":
        k = _keys_cluster(rs, rn, N, d, wl.block, wl.noise)
        q = np.stack([_normal(_rng(seed, wl.tag, b, g, _S_Q0 + h), (N, d)) for h in range(G)])
    elif wl.kind == "drift":
        k = _keys_drift(rs, rn, N, d, wl.block, wl.noise)
        q = np.stack([_normal(_rng(seed, wl.tag, b, g, _S_Q0 + h), (N, d)) for h in range(G)])
    elif wl.kind == "sink":
        u, a = _sink_structure(rs, N, d)
        p = np.repeat(a, _SINK_ANCHOR_EVERY, axis=0)[:N] * np.float32(5.0)
        k = _normal(rn, (N, d))
        k += p
        k[: min(N, _SINK_TOKENS)] += np.float32(20.0) * u
        q = np.empty((G, N, d), np.float32)
        for h in range(G):
            qh = _normal(_rng(seed, wl.tag, b, g, _S_Q0 + h), (N, d))
            qh += p
            qh += np.float32(2.0) * u
            q[h] = qh
    else:
        raise ValueError(f"unknown generator kind {wl.kind!r}")
    v = _normal(_rng(seed, wl.tag, b, g, _S_V), (N, d))
    if wl.dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    return q, k, v


def make_inputs(wl: Workload, seed: int = 0, groups: Optional[List[int]] = None
                ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Full BHND inputs: q [B,Hq,N,d], k/v [B,Hkv,N,d] (float32, bf16-exact for bf16).

    ``groups`` restricts the draw to some KV groups (the other heads stay zero);
    heads are independent, so a subset is an exact sample of the full input.
    """
    G = wl.Hq // wl.Hkv
    q = np.zeros((wl.B, wl.Hq, wl.N, wl.d), np.float32)
    k = np.zeros((wl.B, wl.Hkv, wl.N, wl.d), np.float32)
    v = np.zeros((wl.B, wl.Hkv, wl.N, wl.d), np.float32)
    for b in range(wl.B):
        for g in (range(wl.Hkv) if groups is None else groups):
            qg, kg, vg = make_group(wl, seed, b, g)
            q[b, g * G:(g + 1) * G] = qg
            k[b, g] = kg
            v[b, g] = vg
    return q, k, v


def output_gradient(wl: Workload, seed: int = 0) -> np.ndarray:
    """Seeded dL/d(out) [B,Hq,N,d] for gradient tests: iid N(0,1) per (batch,
    query head) from its own stream (bf16-exact for bf16 workloads)."""
    g = np.empty((wl.B, wl.Hq, wl.N, wl.d), np.float32)
    for b in range(wl.B):
        for h in range(wl.Hq):
            g[b, h] = _normal(_rng(seed, wl.tag, b, h, _S_DOUT), (wl.N, wl.d))
    return bf16_round(g) if wl.dtype == "bf16" else g


def random_qkv(B: int, Hq: int, Hkv: int, N: int, d: int, *, seed: int, block: int = 64,
               kind: str = "cluster", noise: float = 0.3, dtype: str = "f32",
               scale_q: float = 1.0) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Small arbitrary-shape inputs for parity and edge-case tests.

    ``kind``: "iid" (all N(0,1)), "cluster" (keys = per-block centre + noise),
    "drift", or "sink".  Returns float32 arrays (bf16-exact if dtype="bf16").
    """
    wl = Workload("adhoc", dtype, B, Hq, Hkv, N, d, block, False, "alpha", 0.5, 0.0, True,
                  "cluster" if kind == "iid" else kind, noise=noise)
    tag = zlib.crc32(f"adhoc-{kind}-{B}-{Hq}-{Hkv}-{N}-{d}-{block}".encode()) & 0x7FFFFFFF
    wl = dataclasses.replace(wl, name=f"adhoc{tag}")
    q, k, v = make_inputs(wl, seed)
    if kind == "iid":
        rng = np.random.default_rng(np.random.SeedSequence([seed, tag, 99]))
        k = _normal(rng, k.shape)
        if dtype == "bf16":
            k = bf16_round(k)
    if scale_q != 1.0:
        q = q * np.float32(scale_q)
        if dtype == "bf16":
            q = bf16_round(q)
    return q, k, v


def describe(wl: Workload) -> Dict:
    """JSON-able description of a workload (for bench lines)."""
    d = dataclasses.asdict(wl)
    d["M"] = wl.M
    return d
