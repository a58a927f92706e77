"""Plain float64 CPU oracle of the hash-scored top-k sparse decode step.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.  It
shares no code with the HIP library.

Sources (the pages are cited by title and section):

* SOCKET overview page ("SOCKET - SOft Collision Kernel EsTimator",
  gist.science), section "Core mechanism: soft LSH" (中核メカニズム：ソフト LSH),
  items 1-4: keys hashed into L tables by random projections with one bucket
  per table plus a cached value norm (1); the query induces a probability over
  all buckets of each table through a temperature softmax of a soft hash score
  built from its projections on the random hyperplanes (2); each key's score is
  the probability mass on its own buckets summed over the L tables, weighted by
  its value norm (3); the top-k keys are chosen deterministically and exact
  attention runs over that subset (4).
* Same page, section "Theoretical foundations" (理論的基盤): the soft
  bucketization bias vanishes as tau -> 0 (Theorem 3), and attention with
  soft-LSH scores approximates an angular kernel.
* HATA explainer page ("HATA: Hash-Aware Top-k Attention", aibr.jp),
  section 3 (中核となる技術的要素): queries and keys are mapped to binary hash
  codes and ranked by comparing codes rather than by exact q.k scores.  The
  learned hash is out of scope; a seeded Gaussian projection followed by the
  sign stands in for it.

Readings where the pages are silent (each listed with its reason in the
design notes):

* the query is normalised before projection (q_hat = q / ||q||; zero q gives
  uniform bucket probabilities);
* the bucket logit of table l is <s(b), z_l> / tau, where s_p(b) = +1 if bit p
  of bucket b is set and -1 otherwise, and z_l are the query's projections on
  the table's P hyperplanes;
* hyperplane p of a table is bit p of the bucket id, and a projection equal
  to zero (either sign) sets the bit;
* the value norm is the L2 norm rounded to its storage dtype, and the score
  uses the stored value;
* with grouped-query attention, the scores of a kv head sum the bucket
  probabilities (soft) or the code similarities (binary) of its query heads;
* ties in the top-k go to the lower index, the result is returned in
  ascending index order, and k >= N selects everything;
* attention uses scale 1/sqrt(d), only the selected cached keys, no extra
  sink or window tokens.

All arithmetic is float64 on the exact values of the stored inputs (bf16 and
fp16 widen exactly).  The sign decisions of the hashes are exact: products of
two stored values are exact in float64, and any projection whose float64 sum
is within the rounding bound of zero is summed again with ``math.fsum``
(correctly rounded), so the bit is the sign of the true real sum.
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np

__all__ = [
    "exact_projection_signs", "hash_keys_softlsh", "value_norms",
    "binary_codes", "query_tables", "score_softlsh", "score_hamming",
    "select_topk", "attend", "decode_slab_softlsh", "decode_slab_hamming",
    "append_tokens", "select_mass", "chunk_card_keys", "chunk_cards_softlsh",
    "route_slab_softlsh", "decode_shared_prefix_softlsh",
]

_U64 = 2.0 ** -53


def exact_projection_signs(X: np.ndarray, Wp: np.ndarray) -> np.ndarray:
    """bits[i, r] = [ sum_c Wp[r, c] * X[i, c] >= 0 ] for the exact real sum.

    X [n, d] and Wp [R, d] hold exactly-representable stored values (float32
    or bf16 widened to float64), so every product is exact in float64.  The
    float64 dot products carry at most gamma_d * sum|products| of error for any
    summation order; entries inside twice that bound are re-summed with
    math.fsum, whose correctly rounded result has the sign of the true sum.
    """
    X = np.asarray(X, dtype=np.float64)
    Wp = np.asarray(Wp, dtype=np.float64)
    d = X.shape[1]
    Y = X @ Wp.T
    S = np.abs(X) @ np.abs(Wp).T
    gamma = d * _U64 / (1.0 - d * _U64)
    unsure = np.abs(Y) <= 2.0 * gamma * S
    for i, r in zip(*np.nonzero(unsure)):
        Y[i, r] = math.fsum((X[i] * Wp[r]).tolist())
    return Y >= 0.0


def hash_keys_softlsh(K: np.ndarray, W: np.ndarray, L: int, P: int) -> np.ndarray:
    """Soft-LSH bucket ids of keys (SOCKET page, core mechanism, item 1).

    K [n, d] keys, W [L*P, d] hyperplanes (row l*P + p).  Bucket id of table l
    is sum_p bit_{l,p} * 2^p with bit_{l,p} = [W[l*P+p] . k >= 0].
    Returns uint8 [n, L] (P <= 8).
    """
    bits = exact_projection_signs(K, W).reshape(K.shape[0], L, P)
    weights = (1 << np.arange(P)).astype(np.int64)
    ids = (bits.astype(np.int64) * weights[None, None, :]).sum(axis=2)
    return ids.astype(np.uint8)


def value_norms(V: np.ndarray, norm_dtype: str) -> np.ndarray:
    """Cached value norms (SOCKET page, core mechanism, item 1).

    L2 norm of each value row, rounded (nearest-even) to the storage dtype
    ("f16" or "f32"); returned as the float64 value of the stored number.
    """
    n = np.sqrt(np.sum(np.asarray(V, dtype=np.float64) ** 2, axis=1))
    if norm_dtype == "f16":
        return n.astype(np.float16).astype(np.float64)
    if norm_dtype == "f32":
        return n.astype(np.float32).astype(np.float64)
    raise ValueError(norm_dtype)


def binary_codes(X: np.ndarray, R: np.ndarray) -> np.ndarray:
    """Binary hash codes (HATA page, section 3; random-projection stand-in).

    bit i = [R[i] . x >= 0]; bit i is stored in word i // 32 at position
    i % 32.  X [n, d], R [nbits, d] with nbits a multiple of 32.
    Returns uint32 [n, nbits // 32].
    """
    bits = exact_projection_signs(X, R).astype(np.uint64)
    n, nbits = bits.shape
    words = np.zeros((n, nbits // 32), dtype=np.uint64)
    for i in range(nbits):
        words[:, i // 32] |= bits[:, i] << np.uint64(i % 32)
    return words.astype(np.uint32)


def query_tables(qg: np.ndarray, W: np.ndarray, L: int, P: int,
                 tau: float) -> np.ndarray:
    """Soft bucket assignment of the query heads of one kv head.

    SOCKET page, core mechanism, item 2.  For each query head g:
    q_hat = q_g / ||q_g||, z_{l,p} = W[l*P+p] . q_hat, the logit of bucket b
    in table l is sum_p s_p(b) z_{l,p} / tau, and pi_{g,l} is the softmax of
    these logits over all 2^P buckets.  The kv head's table is
    T[l, b] = sum_g pi_{g,l}(b).  Returns float64 [L, 2^P].
    """
    qg = np.asarray(qg, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    nb = 1 << P
    # s[b, p] = +1 if bit p of b is set, else -1
    s = np.array([[1.0 if (b >> p) & 1 else -1.0 for p in range(P)]
                  for b in range(nb)])
    T = np.zeros((L, nb))
    for g in range(qg.shape[0]):
        nrm = np.linalg.norm(qg[g])
        q_hat = qg[g] / nrm if nrm > 0 else np.zeros_like(qg[g])
        z = (W @ q_hat).reshape(L, P)
        logits = (z @ s.T) / tau                      # [L, nb]
        top = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - top)
        T += e / e.sum(axis=1, keepdims=True)
    return T


def score_softlsh(T: np.ndarray, ids: np.ndarray, vnorm: np.ndarray) -> np.ndarray:
    """Soft-collision score of every key (SOCKET page, core mechanism, item 3).

    score_j = vnorm_j * sum_l T[l, ids[j, l]].  Returns float64 [n].
    """
    L = T.shape[0]
    ids = np.asarray(ids, dtype=np.int64)
    mass = np.zeros(ids.shape[0])
    for l in range(L):
        mass += T[l, ids[:, l]]
    return np.asarray(vnorm, dtype=np.float64) * mass


def score_hamming(qcodes: np.ndarray, kcodes: np.ndarray, nbits: int = 128) -> np.ndarray:
    """Code-similarity score of every key (HATA page, section 3).

    score_j = sum_g (nbits - popcount(qcodes[g] XOR kcodes[j])) over the query
    heads g of the kv head.  Returns int64 [n].
    """
    q = np.asarray(qcodes, dtype=np.uint32)
    k = np.asarray(kcodes, dtype=np.uint32)
    total = np.zeros(k.shape[0], dtype=np.int64)
    for g in range(q.shape[0]):
        x = np.bitwise_xor(k, q[g][None, :])
        ham = np.bitwise_count(x).astype(np.int64).sum(axis=1)
        total += nbits - ham
    return total


def select_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """Deterministic top-k (SOCKET page, core mechanism, item 4).

    Orders keys by (score descending, index ascending), keeps the first
    min(k, n), and returns their indices in ascending order (int64).
    """
    scores = np.asarray(scores)
    n = scores.shape[0]
    kk = max(0, min(int(k), n))
    order = np.lexsort((np.arange(n), -scores))
    return np.sort(order[:kk])


def attend(qg: np.ndarray, K: np.ndarray, V: np.ndarray, idx: np.ndarray,
           scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Exact softmax attention over the selected keys (SOCKET page, item 4).

    For each query head g: a_j = scale * q_g . K_j for j in idx,
    out_g = sum_j softmax(a)_j V_j, lse_g = log sum_j exp(a_j).
    Returns (out [G, d], lse [G]) in float64; an empty idx gives zeros and
    -inf.
    """
    qg = np.asarray(qg, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    G, d = qg.shape
    if idx.size == 0:
        return np.zeros((G, d)), np.full(G, -np.inf)
    Ks = np.asarray(K, dtype=np.float64)[idx]
    Vs = np.asarray(V, dtype=np.float64)[idx]
    a = scale * (qg @ Ks.T)                          # [G, k]
    m = a.max(axis=1, keepdims=True)
    p = np.exp(a - m)
    l = p.sum(axis=1, keepdims=True)
    out = (p @ Vs) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


def decode_slab_softlsh(qg, K, V, W, L, P, tau, k, norm_dtype, scale=None,
                        ids=None, vnorm=None) -> dict:
    """Whole soft-LSH decode step for one (batch, kv head) slab.

    Hash keys (unless ``ids``/``vnorm`` are given), build the query tables,
    score all keys, select the top-k and attend.  Every array is float64 or
    integer.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(K.shape[1])
    if ids is None:
        ids = hash_keys_softlsh(K, W, L, P)
    if vnorm is None:
        vnorm = value_norms(V, norm_dtype)
    T = query_tables(qg, W, L, P, tau)
    s = score_softlsh(T, ids, vnorm)
    idx = select_topk(s, k)
    out, lse = attend(qg, K, V, idx, scale)
    return {"ids": ids, "vnorm": vnorm, "T": T, "scores": s, "idx": idx,
            "out": out, "lse": lse}


def decode_slab_hamming(qg, K, V, R, k, scale=None, kcodes=None) -> dict:
    """Whole binary-code decode step for one (batch, kv head) slab."""
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(K.shape[1])
    if kcodes is None:
        kcodes = binary_codes(K, R)
    qcodes = binary_codes(qg, R)
    nbits = np.asarray(R).shape[0]
    s = score_hamming(qcodes, kcodes, nbits)
    idx = select_topk(s, k)
    out, lse = attend(qg, K, V, idx, scale)
    return {"kcodes": kcodes, "qcodes": qcodes, "scores": s, "idx": idx,
            "out": out, "lse": lse}


def append_tokens(K, V, lens, k_new, v_new, *, W=None, L=0, P=0, norm_dtype="f16",
                  ids=None, vnorm=None, R=None, codes=None) -> None:
    """Decode-time append of one token per sequence, in place.

    SOCKET page, core mechanism, item 1: a key's bucket ids and its value norm
    are computed once, when it enters the cache; HATA page, section 3: a key's
    binary code likewise.  For each sequence b with n = max(lens[b], 0) < Nmax
    the token k_new[b, h] / v_new[b, h] becomes row n of every kv head h, its
    metadata is hashed (``W`` [Hkv, L*P, d] with ``ids``/``vnorm``, or ``R``
    [Hkv, nbits, d] with ``codes``), and lens[b] becomes n + 1.  A sequence
    whose cache is full is left as it is.
    """
    B, Hkv, Nmax, _ = K.shape
    for b in range(B):
        n = max(int(lens[b]), 0)
        if n >= Nmax:
            continue
        for h in range(Hkv):
            K[b, h, n] = k_new[b, h]
            V[b, h, n] = v_new[b, h]
            key = np.asarray(k_new[b, h], dtype=np.float64)[None]
            if W is not None:
                ids[b, h, n] = hash_keys_softlsh(key, W[h], L, P)[0]
                vnorm[b, h, n] = value_norms(np.asarray(v_new[b, h])[None], norm_dtype)[0]
            if R is not None:
                codes[b, h, n] = binary_codes(key, R[h])[0]
        lens[b] = n + 1


def select_mass(qg: np.ndarray, K: np.ndarray, cand: np.ndarray, p: float,
                scale: float) -> np.ndarray:
    """Cumulative-mass selection over a candidate set (Tactic page, sections 1
    and 3: keep adding tokens until the summed normalised attention score of
    the chosen set reaches a target, so the count adapts per head and query).

    cand: candidate key indices (entries outside [0, len(K)) are padding,
    as the selection pads with -1).  For the G query
    heads of the KV head, a_gj = scale * q_g . K_j over the candidates, the
    softmax pi_gj = exp(a_gj) / sum_i exp(a_gi) per head, and the mass of
    key j is m_j = (1/G) sum_g pi_gj (the masses sum to 1).  Keys are taken
    in the order (m_j descending, index ascending) until the running sum is
    >= p * sum_j m_j; at least one key is taken when there is a candidate.
    Returns the chosen indices in ascending order.
    """
    cand = np.asarray(cand, dtype=np.int64)
    cand = cand[(cand >= 0) & (cand < np.asarray(K).shape[0])]
    if cand.size == 0:
        return cand
    qg = np.asarray(qg, dtype=np.float64)
    a = scale * (qg @ np.asarray(K, dtype=np.float64)[cand].T)       # [G, c]
    e = np.exp(a - a.max(axis=1, keepdims=True))
    m = (e / e.sum(axis=1, keepdims=True)).mean(axis=0)              # [c]
    order = np.lexsort((cand, -m))
    csum = np.cumsum(m[order])
    total = csum[-1]
    count = int(np.searchsorted(csum >= p * total, True)) + 1
    return np.sort(cand[order[:max(1, min(count, cand.size))]])


CHUNK = 64  # tokens per chunk (HGA page, step 1)


def chunk_card_keys(K: np.ndarray, storage: str) -> np.ndarray:
    """Card keys of 64-token chunks (HGA explainer page, section 2, step 1:
    the context is cut into 64-token chunks, each summarised on a small
    card that the query scans before it goes back to the exact tokens).

    The card key of chunk c is the sum of its keys (64c .. min(64c + 64,
    n) - 1), accumulated in float64 in index order and rounded to the key
    storage type ("f32": float32; "bf16": float32, then bf16, both to
    nearest even), so that a card is itself a stored key.  Returns float64
    [nc, d] holding the stored values.
    """
    K = np.asarray(K, dtype=np.float64)
    n, d = K.shape
    nc = (n + CHUNK - 1) // CHUNK
    out = np.zeros((nc, d))
    for c in range(nc):
        acc = np.zeros(d)
        for j in range(c * CHUNK, min(n, (c + 1) * CHUNK)):
            acc = acc + K[j]
        x32 = acc.astype(np.float32)
        if storage == "bf16":
            b = x32.view(np.uint32).astype(np.uint64)
            b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16          # nearest even
            x32 = (b.astype(np.uint32) << 16).view(np.float32)
        elif storage != "f32":
            raise ValueError(storage)
        out[c] = x32.astype(np.float64)
    return out


def chunk_cards_softlsh(K: np.ndarray, vnorm: np.ndarray, W: np.ndarray, L: int, P: int,
                        storage: str) -> Tuple[np.ndarray, np.ndarray]:
    """Index cards: the soft-LSH bucket ids of each chunk's card key (hashed
    like any key, exact signs) and, as its weight, the largest stored value
    norm in the chunk.  Returns (ids uint8 [nc, L], weights [nc])."""
    keys = chunk_card_keys(K, storage)
    ids = hash_keys_softlsh(keys, W, L, P)
    n = np.asarray(K).shape[0]
    wts = np.array([np.max(vnorm[c * CHUNK:min(n, (c + 1) * CHUNK)])
                    for c in range(keys.shape[0])])
    return ids, wts


def route_slab_softlsh(qg, K, V, W, L, P, tau, k, C, norm_dtype, storage, scale=None,
                       ids=None, vnorm=None, cards=None) -> dict:
    """Two-level routed decode step for one (sequence, kv head) slab (HGA
    page, section 2: chunk routing on the cards, then token routing inside
    the chosen chunks, and exact attention over the original tokens).

    The cards are scored like keys (card weight times the summed table
    probability of the card's buckets), the C chunks first in the order
    (score descending, chunk index ascending) are kept, every key of those
    chunks is scored, and the k keys first in the order (score descending,
    index ascending) among them are attended.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n = K.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(K.shape[1])
    if ids is None:
        ids = hash_keys_softlsh(K, W, L, P)
    if vnorm is None:
        vnorm = value_norms(V, norm_dtype)
    if cards is None:
        cards = chunk_cards_softlsh(K, vnorm, W, L, P, storage)
    T = query_tables(qg, W, L, P, tau)
    cscore = score_softlsh(T, cards[0], cards[1])
    chunks = select_topk(cscore, C)
    keys = np.concatenate([np.arange(c * CHUNK, min(n, (c + 1) * CHUNK)) for c in chunks]) \
        if chunks.size else np.zeros(0, dtype=np.int64)
    s = score_softlsh(T, ids[keys], vnorm[keys])
    idx = np.sort(keys[select_topk(s, k)])
    out, lse = attend(qg, K, V, idx, scale)
    return {"cards": cards, "T": T, "chunk_scores": cscore, "chunks": chunks, "keys": keys,
            "scores": s, "idx": idx, "out": out, "lse": lse}


def decode_shared_prefix_softlsh(qg, Kp, Vp, Ks, Vs, W, L, P, tau, k, norm_dtype,
                                 scale=None) -> dict:
    """Decode step of one sequence whose context is a prefix shared by the
    batch followed by its own suffix (bifurcated-attention page, sections 1
    and 3: the shared context and each sample's incremental part are kept
    apart so the shared part is read once for the whole batch).

    The result is the plain step over the concatenated context: key j < Np
    is prefix key j, key Np + j is suffix key j.
    """
    K = np.concatenate([np.asarray(Kp, dtype=np.float64), np.asarray(Ks, dtype=np.float64)])
    V = np.concatenate([np.asarray(Vp, dtype=np.float64), np.asarray(Vs, dtype=np.float64)])
    return decode_slab_softlsh(qg, K, V, W, L, P, tau, k, norm_dtype, scale=scale)
