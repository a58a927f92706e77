"""Seeded synthetic workloads for hash-scored top-k sparse decode attention.

This module only draws random numbers and lays them out; it computes none of
the method's arithmetic (no hashing, no scores, no selection, no attention).
Both the CPU oracle and the GPU path read the bytes it produces.

The workloads stand in for the long-context decode settings the pages evaluate
on (SOCKET page, "Experimental results": Llama-3.1-8B / Qwen3 models,
RULER-32K at 50x sparsity, 100K-140K-token contexts at 33x sparsity; HGA page:
needle-in-a-haystack at 64K).  No public suite is used: planted "needle" keys
play the role of the relevant tokens.

Recipe (every draw is from numpy's PCG64 through ``default_rng`` with a list
seed, so any (batch, kv-head) slab can be generated on its own):

* keys   K[j, c] = f_c * g[j, c]; g ~ N(0, 1); f_c = exp(0.5 * n_c), n_c ~ N(0, 1)
  drawn once per (kv head, channel) and shared over batch and tokens
  (log-normal(0, 0.5) channel scales);
* values V[j, c] ~ N(0, 1);
* needles: a random unit direction c_dir per slab; m needle directions
  u_i = 0.8 * c_dir + 0.6 * e_i with e_i a random unit vector orthogonal to
  c_dir (so cos(u_i, c_dir) = 0.8 exactly); m distinct positions uniform in
  [0, N_b); the key at each position is replaced by ||K_pos|| * u_i;
* queries: q_h = sum_i u_i + eps_h, eps_h ~ N(0, 0.5^2 I), independently per
  query head of the group;
* hyperplanes W[h] ~ N(0, I) of shape [L*P, d] and HATA-style projections
  R[h] ~ N(0, I) of shape [128, d], per kv head;
* ragged context lengths N_b ~ U{lo..hi} (inclusive), drawn first.

Normals are drawn in float32 (numpy's ziggurat), needle geometry is done in
float64, and everything is rounded to the storage dtype at the end: float32
as is, bf16 by round-to-nearest-even from the float32 value.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Dict, List, Optional, Tuple

import numpy as np

# Stream tags mixed into the seed list, so every kind of draw has its own
# independent stream.
_TAG_SLAB = 0
_TAG_CHANNEL_SCALE = 1
_TAG_PLANES = 2
_TAG_PROJ = 3
_TAG_LENS = 4


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    scheme: str            # "softlsh" or "hamming"
    B: int
    Hq: int
    Hkv: int
    d: int
    N: int                 # Nmax: cache capacity per sequence
    kv_dtype: str          # "f32" or "bf16"
    norm_dtype: str        # "f32" or "f16" (soft-LSH value-norm storage)
    L: int = 0             # hash tables (soft-LSH)
    P: int = 0             # hyperplanes per table (soft-LSH)
    tau: float = 0.0       # soft-assignment temperature (soft-LSH)
    code_bits: int = 128   # binary code length (hamming)
    k: int = 0             # fixed top-k, 0 if k derives from sparsity
    sparsity: float = 0.0  # k_b = ceil(N_b / sparsity) when k == 0
    needles: int = 0       # planted needle keys per (b, kv head)
    ragged: Optional[Tuple[int, int]] = None  # inclusive range of N_b
    seed: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def seq_lens(self) -> np.ndarray:
        """Context length of every sequence (int32 [B])."""
        if self.ragged is None:
            return np.full(self.B, self.N, dtype=np.int32)
        lo, hi = self.ragged
        rng = np.random.default_rng([self.seed, _TAG_LENS])
        return rng.integers(lo, hi, size=self.B, endpoint=True).astype(np.int32)

    def k_per_seq(self) -> np.ndarray:
        """Number of keys selected per sequence (int32 [B])."""
        lens = self.seq_lens()
        if self.k > 0:
            return np.minimum(lens, self.k).astype(np.int32)
        return np.array([math.ceil(int(n) / self.sparsity) for n in lens],
                        dtype=np.int32)

    def k_max(self) -> int:
        return int(self.k_per_seq().max())


WORKLOADS: Dict[str, Workload] = {
    # Tiny parity case: fp32 everything, GQA 4:1, d=64, N=4096, 8 tables of
    # 4 hyperplanes (16 buckets), tau=0.5, k=128, 8 needles.
    "tiny_softlsh_fp32": Workload(
        name="tiny_softlsh_fp32", scheme="softlsh", B=1, Hq=4, Hkv=1, d=64,
        N=4096, kv_dtype="f32", norm_dtype="f32", L=8, P=4, tau=0.5, k=128,
        needles=8, seed=20260000),
    # Llama-3.1-8B-shaped decode step: B=8, 32/8 heads, d=128, bf16, N=32768,
    # 64 tables x 8 hyperplanes, fp16 value norms, tau=0.3, k=ceil(N/33)=993.
    "llama8b_softlsh_b8_n32k": Workload(
        name="llama8b_softlsh_b8_n32k", scheme="softlsh", B=8, Hq=32, Hkv=8,
        d=128, N=32768, kv_dtype="bf16", norm_dtype="f16", L=64, P=8,
        tau=0.3, sparsity=33.0, needles=16, seed=20260001),
    # Long-context single sequence: B=1, 32/8 heads, N=131072, k=3972 (33x).
    "longctx_softlsh_b1_n128k": Workload(
        name="longctx_softlsh_b1_n128k", scheme="softlsh", B=1, Hq=32, Hkv=8,
        d=128, N=131072, kv_dtype="bf16", norm_dtype="f16", L=64, P=8,
        tau=0.3, sparsity=33.0, needles=16, seed=20260002),
    # Binary-code (HATA-style) top-k: B=16, 32/8, N=65536, 128-bit codes,
    # k=ceil(N/20)=3277.
    "hata_hamming_b16_n64k": Workload(
        name="hata_hamming_b16_n64k", scheme="hamming", B=16, Hq=32, Hkv=8,
        d=128, N=65536, kv_dtype="bf16", norm_dtype="f16", code_bits=128,
        sparsity=20.0, needles=16, seed=20260003),
    # Qwen3-30B-A3B attention shape, ragged batch: B=32, 32/4 heads,
    # N_b ~ U{8192..65536}, k_b = ceil(N_b/50), 32 needles.
    "qwen30b_ragged_softlsh_b32": Workload(
        name="qwen30b_ragged_softlsh_b32", scheme="softlsh", B=32, Hq=32,
        Hkv=4, d=128, N=65536, kv_dtype="bf16", norm_dtype="f16", L=64, P=8,
        tau=0.3, sparsity=50.0, needles=32, ragged=(8192, 65536),
        seed=20260004),
}


# ---------------------------------------------------------------------------
# storage rounding helpers (data plumbing, not the method)

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round to the storage dtype; returns float32 (f32) or uint16 bits (bf16)."""
    x32 = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return np.ascontiguousarray(x32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def storage_to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# draws

def channel_scales(w: Workload, kvh: int) -> np.ndarray:
    rng = np.random.default_rng([w.seed, _TAG_CHANNEL_SCALE, kvh])
    n = rng.standard_normal(w.d)
    return np.exp(0.5 * n)


def make_slab(w: Workload, b: int, kvh: int, n_b: Optional[int] = None) -> dict:
    """Keys, values and the G queries of one (batch, kv head) slab.

    Returns storage-typed arrays ``K`` [n_b, d], ``V`` [n_b, d], ``q`` [G, d]
    (float32, or uint16 bf16 bits) and ``needle_pos`` (sorted int64).
    """
    if n_b is None:
        n_b = int(w.seq_lens()[b])
    rng = np.random.default_rng([w.seed, _TAG_SLAB, b, kvh])
    f = channel_scales(w, kvh).astype(np.float32)
    K = rng.standard_normal((n_b, w.d), dtype=np.float32)
    K *= f[None, :]
    V = rng.standard_normal((n_b, w.d), dtype=np.float32)

    m = min(w.needles, n_b)
    c_dir = rng.standard_normal(w.d)
    c_dir /= np.linalg.norm(c_dir)
    us = []
    for _ in range(m):
        e = rng.standard_normal(w.d)
        e -= np.dot(e, c_dir) * c_dir
        e /= np.linalg.norm(e)
        us.append(0.8 * c_dir + 0.6 * e)
    pos = (np.sort(rng.choice(n_b, size=m, replace=False)) if m > 0
           else np.zeros(0, dtype=np.int64))
    for i, p in enumerate(pos):
        K[p] = (np.linalg.norm(K[p].astype(np.float64)) * us[i]).astype(np.float32)
    u_sum = np.sum(us, axis=0) if m > 0 else np.zeros(w.d)
    q = u_sum[None, :] + 0.5 * rng.standard_normal((w.G, w.d))
    return {
        "K": to_storage(K, w.kv_dtype),
        "V": to_storage(V, w.kv_dtype),
        "q": to_storage(q, w.kv_dtype),
        "needle_pos": pos.astype(np.int64),
        "needle_dirs": np.array(us).reshape(m, w.d),
        "needle_center": c_dir,
    }


def make_planes(w: Workload, kvh: int) -> np.ndarray:
    """Random hyperplanes for one kv head: [L*P, d], row l*P + p."""
    rng = np.random.default_rng([w.seed, _TAG_PLANES, kvh])
    x = rng.standard_normal((w.L * w.P, w.d), dtype=np.float32)
    return to_storage(x, w.kv_dtype)


def make_projection(w: Workload, kvh: int) -> np.ndarray:
    """Random projection for binary codes of one kv head: [code_bits, d]."""
    rng = np.random.default_rng([w.seed, _TAG_PROJ, kvh])
    x = rng.standard_normal((w.code_bits, w.d), dtype=np.float32)
    return to_storage(x, w.kv_dtype)


def storage_np_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


def make_full(w: Workload, slabs: Optional[List[Tuple[int, int]]] = None,
              workers: Optional[int] = None) -> dict:
    """Whole-batch arrays in the library layout.

    K, V: [B, Hkv, Nmax, d]; q: [B, Hq, d]; W: [Hkv, L*P, d] (soft-LSH) or
    R: [Hkv, 128, d] (hamming).  Rows j >= N_b are zero.  ``slabs`` limits
    generation to the listed (b, kvh) pairs (other slabs stay zero), which is
    how large workloads are sampled on the host.
    """
    lens = w.seq_lens()
    dt = storage_np_dtype(w.kv_dtype)
    K = np.zeros((w.B, w.Hkv, w.N, w.d), dtype=dt)
    V = np.zeros((w.B, w.Hkv, w.N, w.d), dtype=dt)
    q = np.zeros((w.B, w.Hq, w.d), dtype=dt)
    needles = {}
    todo = slabs if slabs is not None else [(b, h) for b in range(w.B)
                                            for h in range(w.Hkv)]

    def fill(bh):
        b, h = bh
        s = make_slab(w, b, h, int(lens[b]))
        n = int(lens[b])
        K[b, h, :n] = s["K"]
        V[b, h, :n] = s["V"]
        q[b, h * w.G:(h + 1) * w.G] = s["q"]
        return bh, s["needle_pos"]

    # every slab has its own seed and its own rows, so slabs can be drawn on
    # worker threads (numpy's samplers release the GIL) with the same result
    if workers is None:
        workers = min(16, os.cpu_count() or 1)
    if workers > 1 and len(todo) > 1:
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            for bh, pos in ex.map(fill, todo):
                needles[bh] = pos
    else:
        for bh in todo:
            needles[bh] = fill(bh)[1]
    out = {"K": K, "V": V, "q": q, "seq_lens": lens,
           "k_per_seq": w.k_per_seq(), "needles": needles}
    if w.scheme == "softlsh":
        out["W"] = np.stack([make_planes(w, h) for h in range(w.Hkv)])
    else:
        out["R"] = np.stack([make_projection(w, h) for h in range(w.Hkv)])
    return out
