"""Pins of the CPU oracle against facts fixed outside it.

Each test checks the oracle against something other than its own formula:
hand-derived golden values (tests/golden, each file citing its passage),
closed forms, limits the pages state, textbook identities, exact rational
brute force on tiny inputs, library routines, and invariants.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle as O
import workloads as WL


def _read_golden(golden_dir, name):
    rows = []
    with open(os.path.join(golden_dir, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([part.strip() for part in line.split("|")])
    return rows


# ---------------------------------------------------------------- hashing

def test_hash_axes_golden(golden_dir):
    rows = _read_golden(golden_dir, "hash_axes.txt")
    assert len(rows) >= 8
    for lpd, wrows, key, ids in rows:
        L, P, d = (int(x) for x in lpd.split())
        W = np.array([[float(x) for x in r.split()] for r in wrows.split(";")])
        assert W.shape == (L * P, d)
        k = np.array([[float(x) for x in key.split()]])
        want = [int(x) for x in ids.split()]
        got = O.hash_keys_softlsh(k, W, L, P)
        assert got.dtype == np.uint8
        assert got[0].tolist() == want, (lpd, wrows, key)


def test_hash_sign_is_exact_under_cancellation():
    # Products 2^60, -1, -2^60: the true projection is -1 (bit 0) although a
    # left-to-right float64 sum gives 0 (bit 1).  All values are exact float32.
    k = np.array([[2.0 ** 30, -1.0, -(2.0 ** 30)]], dtype=np.float32)
    W = np.array([[2.0 ** 30, 1.0, 2.0 ** 30]], dtype=np.float32)
    naive = (float(W[0, 0]) * float(k[0, 0]) + float(W[0, 1]) * float(k[0, 1])) \
        + float(W[0, 2]) * float(k[0, 2])
    assert naive == 0.0  # the trap is real
    assert O.hash_keys_softlsh(k.astype(np.float64), W.astype(np.float64), 1, 1)[0, 0] == 0
    # and the mirrored case sets the bit
    assert O.hash_keys_softlsh(-k.astype(np.float64), W.astype(np.float64), 1, 1)[0, 0] == 1


def _brute_ids(K, W, L, P):
    """Exact rational projections, one key/table/plane at a time."""
    out = []
    for key in K:
        row = []
        for l in range(L):
            bid = 0
            for p in range(P):
                y = sum(Fraction(float(w)) * Fraction(float(x))
                        for w, x in zip(W[l * P + p], key))
                if y >= 0:
                    bid |= 1 << p
            row.append(bid)
        out.append(row)
    return np.array(out)


def test_hash_bruteforce_rational():
    rng = np.random.default_rng(7)
    L, P, d, n = 3, 4, 6, 40
    K = rng.standard_normal((n, d)).astype(np.float32).astype(np.float64)
    W = rng.standard_normal((L * P, d)).astype(np.float32).astype(np.float64)
    K[3] = 0.0  # every projection is zero: all bits set
    np.testing.assert_array_equal(O.hash_keys_softlsh(K, W, L, P), _brute_ids(K, W, L, P))
    assert (O.hash_keys_softlsh(K, W, L, P)[3] == (1 << P) - 1).all()


def test_hash_scale_and_negation_invariants():
    rng = np.random.default_rng(11)
    L, P, d, n = 8, 8, 32, 200
    K = rng.standard_normal((n, d)).astype(np.float32).astype(np.float64)
    W = rng.standard_normal((L * P, d)).astype(np.float32).astype(np.float64)
    ids = O.hash_keys_softlsh(K, W, L, P)
    for a in (0.25, 2.0, 1024.0):
        np.testing.assert_array_equal(O.hash_keys_softlsh(a * K, W, L, P), ids)
    neg = O.hash_keys_softlsh(-K, W, L, P)
    np.testing.assert_array_equal(neg.astype(int), (1 << P) - 1 - ids.astype(int))


def test_simhash_collision_law():
    # Random-hyperplane signs collide with probability 1 - theta/pi per plane
    # (the angular kernel the SOCKET page names in "Theoretical foundations").
    rng = np.random.default_rng(5)
    d = 16
    x = np.zeros(d); x[0] = 1.0
    for theta in (math.pi / 6, math.pi / 3, math.pi / 2, 2 * math.pi / 3):
        y = np.zeros(d); y[0] = math.cos(theta); y[1] = math.sin(theta)
        for P in (1, 4):
            L = 20000
            W = rng.standard_normal((L * P, d))
            ids = O.hash_keys_softlsh(np.stack([x, y]), W, L, P)
            frac = float(np.mean(ids[0] == ids[1]))
            p = (1 - theta / math.pi) ** P
            sigma = math.sqrt(p * (1 - p) / L)
            assert abs(frac - p) < 4 * sigma + 1e-9, (theta, P, frac, p)


def test_value_norms_golden():
    V = np.array([[3.0, 4.0], [1.0, 1.0], [0.0, 0.0]])
    np.testing.assert_array_equal(O.value_norms(V, "f32"),
                                  [5.0, float(np.float32(math.sqrt(2))), 0.0])
    # fp16 nearest-even of sqrt(2): 1 + 424/1024
    np.testing.assert_array_equal(O.value_norms(V, "f16"), [5.0, 1.0 + 424 / 1024, 0.0])
    assert float(np.float32(math.sqrt(2))) == float.fromhex("0x1.6a09e6p0")


def test_append_tokens_rows_lengths_and_metadata():
    # Decode-time append (SOCKET page, core mechanism, item 1; HATA page,
    # section 3): each token lands at row max(lens[b], 0), hashed exactly, and
    # the length advances; a full sequence is left untouched.
    rng = np.random.default_rng(21)
    B, Hkv, Nmax, d, L, P = 4, 2, 5, 4, 2, 3
    lens0 = np.array([-2, 0, 3, 5], dtype=np.int64)
    K = rng.standard_normal((B, Hkv, Nmax, d))
    V = rng.standard_normal((B, Hkv, Nmax, d))
    ids = rng.integers(0, 8, (B, Hkv, Nmax, L)).astype(np.uint8)
    vnorm = rng.standard_normal((B, Hkv, Nmax))
    codes = rng.integers(0, 2**32, (B, Hkv, Nmax, 4), dtype=np.uint64).astype(np.uint32)
    W = rng.standard_normal((Hkv, L * P, d)).astype(np.float32).astype(np.float64)
    R = rng.standard_normal((Hkv, 128, d)).astype(np.float32).astype(np.float64)
    toks = [(rng.standard_normal((B, Hkv, d)).astype(np.float32).astype(np.float64),
             rng.integers(-8, 9, (B, Hkv, d)) / 4.0) for _ in range(3)]
    toks[1][0][0, 0] = 0.0                      # a zero key: every bit set
    init = [a.copy() for a in (K, V, ids, vnorm, codes)]
    lens = lens0.copy()
    for kn, vn in toks:
        O.append_tokens(K, V, lens, kn, vn, W=W, L=L, P=P, norm_dtype="f16", ids=ids,
                        vnorm=vnorm, R=R, codes=codes)
    np.testing.assert_array_equal(lens, [3, 3, 5, 5])
    for b in range(B):
        start = max(int(lens0[b]), 0)
        rows = {start + t: t for t in range(3) if start + t < Nmax}
        for h in range(Hkv):
            for j in range(Nmax):
                if j not in rows:        # untouched
                    np.testing.assert_array_equal(K[b, h, j], init[0][b, h, j])
                    np.testing.assert_array_equal(ids[b, h, j], init[2][b, h, j])
                    np.testing.assert_array_equal(codes[b, h, j], init[4][b, h, j])
                    assert vnorm[b, h, j] == init[3][b, h, j]
                    continue
                kn, vn = toks[rows[j]][0][b, h], toks[rows[j]][1][b, h]
                np.testing.assert_array_equal(K[b, h, j], kn)
                np.testing.assert_array_equal(V[b, h, j], vn)
                np.testing.assert_array_equal(ids[b, h, j], _brute_ids(kn[None], W[h], L, P)[0])
                # squares of quarter-integers sum exactly; sqrt then fp16 rounding
                exact = math.sqrt(float(sum(Fraction(float(x)) ** 2 for x in vn)))
                assert vnorm[b, h, j] == float(np.float16(exact))
                want = [0, 0, 0, 0]
                for i in range(128):
                    y = sum(Fraction(float(w)) * Fraction(float(x)) for w, x in zip(R[h, i], kn))
                    if y >= 0:
                        want[i // 32] |= 1 << (i % 32)
                np.testing.assert_array_equal(codes[b, h, j].astype(np.int64), want)
    assert ids[0, 0, 1].tolist() == [(1 << P) - 1] * L
    assert codes[0, 0, 1].tolist() == [0xFFFFFFFF] * 4


# ---------------------------------------------------------------- codes

def test_codes_axes_golden(golden_dir):
    rows = _read_golden(golden_dir, "codes_axes.txt")
    assert len(rows) >= 5
    for d, x, words in rows:
        d = int(d)
        R = np.zeros((128, d))
        for i in range(128):
            R[i, i % d] = 1.0
        xs = np.array([[float(v) for v in x.split()]])
        want = [int(w, 16) for w in words.split()]
        got = O.binary_codes(xs, R)
        assert got.dtype == np.uint32
        assert got[0].tolist() == want


def test_hamming_bruteforce_bits():
    rng = np.random.default_rng(3)
    d, n, G = 16, 60, 4
    X = rng.standard_normal((n, d))
    Q = rng.standard_normal((G, d))
    R = rng.standard_normal((128, d))
    kc = O.binary_codes(X, R)
    qc = O.binary_codes(Q, R)

    def bits(words):
        return "".join(format(int(w), "032b")[::-1] for w in words)

    # the packed bits equal the projection signs, bit by bit
    for j in range(n):
        s = bits(kc[j])
        for i in range(128):
            assert s[i] == ("1" if float(np.dot(R[i], X[j])) >= 0 else "0")
    got = O.score_hamming(qc, kc)
    for j in range(n):
        want = sum(sum(1 for a, b in zip(bits(qc[g]), bits(kc[j])) if a == b)
                   for g in range(G))
        assert got[j] == want
    assert ((got >= 0) & (got <= 128 * G)).all()
    # a key equal to a query head agrees on all 128 bits for that head
    self_score = O.score_hamming(qc[:1], qc[:1])
    assert self_score[0] == 128


def test_hamming_angle_law():
    rng = np.random.default_rng(9)
    d = 32
    x = np.zeros(d); x[0] = 1
    theta = 1.0
    y = np.zeros(d); y[0] = math.cos(theta); y[1] = math.sin(theta)
    trials = 400
    hams = []
    for _ in range(trials):
        R = rng.standard_normal((128, d))
        c = O.binary_codes(np.stack([x, y]), R)
        hams.append(128 - int(O.score_hamming(c[:1], c[1:2])[0]))
    mean = np.mean(hams)
    p = theta / math.pi
    sigma = math.sqrt(128 * p * (1 - p) / trials)
    assert abs(mean - 128 * p) < 4 * sigma


# ---------------------------------------------------------------- tables

def _logistic(x):
    return 1.0 / (1.0 + math.exp(-x))


def test_tables_single_plane_closed_form():
    # P=1, w=(1,0), q=(3,4): q_hat=(0.6,0.8), z=0.6; buckets {0,1} have logits
    # -+z/tau, so the set bucket has probability logistic(2 z / tau).
    W = np.array([[1.0, 0.0]])
    T = O.query_tables(np.array([[3.0, 4.0]]), W, 1, 1, 0.5)
    assert abs(T[0, 1] - _logistic(2.4)) < 1e-15
    assert abs(T[0, 0] - _logistic(-2.4)) < 1e-15
    assert abs(T[0, 1] - 0.916827303506) < 1e-11


def test_tables_factorise_into_logistics():
    # softmax over all sign patterns of a linear logit = product of logistics
    rng = np.random.default_rng(21)
    L, P, d, G, tau = 5, 6, 12, 3, 0.3
    W = rng.standard_normal((L * P, d))
    qg = rng.standard_normal((G, d))
    T = O.query_tables(qg, W, L, P, tau)
    want = np.zeros((L, 1 << P))
    for g in range(G):
        qh = qg[g] / math.sqrt(sum(v * v for v in qg[g]))
        for l in range(L):
            z = [sum(W[l * P + p, c] * qh[c] for c in range(d)) for p in range(P)]
            for b in range(1 << P):
                prob = 1.0
                for p in range(P):
                    sgn = 1.0 if (b >> p) & 1 else -1.0
                    prob *= _logistic(2.0 * sgn * z[p] / tau)
                want[l, b] += prob
    np.testing.assert_allclose(T, want, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(T.sum(axis=1), G, rtol=1e-13)


def test_tables_limits_and_invariants():
    rng = np.random.default_rng(2)
    L, P, d, G = 6, 4, 10, 2
    W = rng.standard_normal((L * P, d))
    qg = rng.standard_normal((G, d))
    T = O.query_tables(qg, W, L, P, 0.5)
    # the query is normalised first: any positive scale gives the same table
    np.testing.assert_allclose(O.query_tables(7.5 * qg, W, L, P, 0.5), T, rtol=1e-12)
    # tau -> infinity: uniform over 2^P buckets
    np.testing.assert_allclose(O.query_tables(qg, W, L, P, 1e9), G / (1 << P), rtol=1e-7)
    # zero query: uniform
    np.testing.assert_allclose(O.query_tables(np.zeros((1, d)), W, L, P, 0.5),
                               1.0 / (1 << P), rtol=1e-14)
    # tau -> 0: one-hot on the query's own hard bucket (its hash id)
    hard = O.hash_keys_softlsh(qg, W, L, P)
    T0 = O.query_tables(qg, W, L, P, 1e-6)
    want = np.zeros((L, 1 << P))
    for g in range(G):
        for l in range(L):
            want[l, hard[g, l]] += 1.0
    np.testing.assert_allclose(T0, want, atol=1e-6)


# ---------------------------------------------------------------- scores

def _random_softlsh_case(rng, n=300, L=8, P=4, d=16, G=4):
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    W = rng.standard_normal((L * P, d))
    qg = rng.standard_normal((G, d))
    ids = O.hash_keys_softlsh(K, W, L, P)
    vn = O.value_norms(V, "f32")
    return K, V, W, qg, ids, vn


def test_scores_bruteforce_without_tables():
    rng = np.random.default_rng(4)
    L, P, d, G, tau = 8, 4, 16, 4, 0.5
    K, V, W, qg, ids, vn = _random_softlsh_case(rng, L=L, P=P, d=d, G=G)
    s = O.score_softlsh(O.query_tables(qg, W, L, P, tau), ids, vn)
    for j in range(0, K.shape[0], 7):
        tot = 0.0
        for g in range(G):
            qh = qg[g] / np.linalg.norm(qg[g])
            for l in range(L):
                prob = 1.0
                for p in range(P):
                    z = float(np.dot(W[l * P + p], qh))
                    sgn = 1.0 if (int(ids[j, l]) >> p) & 1 else -1.0
                    prob *= _logistic(2 * sgn * z / tau)
                tot += prob
        assert abs(s[j] - vn[j] * tot) <= 1e-12 * abs(vn[j] * tot)


def test_scores_tau_to_zero_is_hard_collision_count():
    # Theorem 3 of the SOCKET page: the soft-bucketization bias vanishes as
    # tau -> 0, leaving the hard collision count weighted by the value norm.
    rng = np.random.default_rng(6)
    L, P, d, G = 8, 4, 16, 4
    K, V, W, qg, ids, vn = _random_softlsh_case(rng, L=L, P=P, d=d, G=G)
    qh = qg / np.linalg.norm(qg, axis=1, keepdims=True)
    zmin = np.abs(qh @ W.T).min()
    tau = zmin / 20.0
    s = O.score_softlsh(O.query_tables(qg, W, L, P, tau), ids, vn)
    hard_q = O.hash_keys_softlsh(qg, W, L, P)
    counts = np.zeros(K.shape[0])
    for g in range(G):
        counts += (ids == hard_q[g][None, :]).sum(axis=1)
    np.testing.assert_allclose(s, vn * counts, rtol=1e-6, atol=1e-12)
    assert counts.max() > 0


def test_scores_bounds_and_tau_infinity():
    rng = np.random.default_rng(8)
    L, P, d, G = 8, 4, 16, 4
    K, V, W, qg, ids, vn = _random_softlsh_case(rng, L=L, P=P, d=d, G=G)
    s = O.score_softlsh(O.query_tables(qg, W, L, P, 0.3), ids, vn)
    assert (s >= 0).all() and (s <= G * L * vn * (1 + 1e-12)).all()
    s_inf = O.score_softlsh(O.query_tables(qg, W, L, P, 1e12), ids, vn)
    np.testing.assert_allclose(s_inf, vn * G * L / (1 << P), rtol=1e-9)
    # so the top-k at tau -> infinity is the top-k by value norm
    np.testing.assert_array_equal(O.select_topk(s_inf, 17), O.select_topk(vn, 17))


def test_metadata_overhead_matches_page():
    # SOCKET page, "Experimental results": about 15% memory over the KV cache
    # for the bucket ids plus value norms.  64 one-byte ids + a 2-byte norm per
    # key against 2 x 128 bf16 elements of K and V: 66 / 512 = 12.9%.
    frac = (64 * 1 + 2) / (2 * 128 * 2)
    assert 0.10 < frac < 0.17


# ---------------------------------------------------------------- select

def test_select_golden(golden_dir):
    rows = _read_golden(golden_dir, "select_small.txt")
    assert len(rows) >= 10
    for scores, k, want in rows:
        s = np.array([float(x) for x in scores.split()])
        got = O.select_topk(s, int(k))
        exp = [] if want == "-" else [int(x) for x in want.split()]
        assert got.tolist() == exp, (scores, k)


def _select_brute(scores, k):
    left = list(range(len(scores)))
    chosen = []
    for _ in range(min(k, len(scores))):
        best = left[0]
        for j in left:
            if scores[j] > scores[best]:
                best = j
        chosen.append(best)
        left.remove(best)
    return sorted(chosen)


@settings(max_examples=300, deadline=None)
@given(st.lists(st.integers(min_value=0, max_value=5), min_size=0, max_size=60),
       st.integers(min_value=0, max_value=70))
def test_select_matches_bruteforce_with_ties(vals, k):
    s = np.array(vals, dtype=np.float64)
    got = O.select_topk(s, k).tolist()
    assert got == _select_brute(vals, k)
    if 0 < k < len(vals):
        inside = s[got]
        outside = np.delete(s, got)
        assert inside.min() >= outside.max()


@settings(max_examples=100, deadline=None)
@given(st.lists(st.integers(min_value=0, max_value=512), min_size=1, max_size=80),
       st.integers(min_value=1, max_value=90))
def test_select_integer_scores(vals, k):
    s = np.array(vals, dtype=np.int64)
    assert O.select_topk(s, k).tolist() == _select_brute(vals, k)


# ---------------------------------------------------------------- mass selection

def _masses(qg, K, cand, scale):
    """Per-candidate mass, head by head with math.exp (no numpy reductions)."""
    G = len(qg)
    out = [0.0] * len(cand)
    for g in range(G):
        a = [scale * sum(float(x) * float(y) for x, y in zip(qg[g], K[j])) for j in cand]
        mx = max(a)
        e = [math.exp(v - mx) for v in a]
        z = math.fsum(e)
        for i, v in enumerate(e):
            out[i] += v / z / G
    return out


def test_select_mass_is_the_smallest_set_reaching_the_target():
    # Tactic page, section 3: tokens are added until the cumulative normalised
    # score reaches the target; by brute force over all subsets, no smaller
    # set reaches it, and the chosen set does.
    rng = np.random.default_rng(17)
    import itertools
    for trial in range(30):
        G, d, c = int(rng.integers(1, 4)), 6, int(rng.integers(1, 9))
        qg = rng.standard_normal((G, d)) * 2.0
        K = rng.standard_normal((20, d))
        cand = np.sort(rng.choice(20, c, replace=False))
        p = float(rng.choice([0.3, 0.5, 0.8, 0.95, 1.0]))
        got = O.select_mass(qg, K, cand, p, 0.5)
        m = dict(zip(cand.tolist(), _masses(qg, K, cand.tolist(), 0.5)))
        total = math.fsum(m.values())
        need = min(r for r in range(1, c + 1)
                   for sub in itertools.combinations(cand.tolist(), r)
                   if math.fsum(m[j] for j in sub) >= p * total * (1 - 1e-12))
        assert len(got) == need, (trial, len(got), need)
        assert math.fsum(m[j] for j in got) >= p * total * (1 - 1e-12)
        assert set(got.tolist()) <= set(cand.tolist())
        assert (np.diff(got) > 0).all()


def test_select_mass_ties_uniform_and_padding():
    d = 8
    K = np.tile(np.arange(1.0, d + 1.0), (12, 1))        # identical keys: equal masses
    qg = np.ones((2, d))
    cand = np.array([11, 2, 7, 5, -1, 9, 0, -1])
    # 6 equal masses of 1/6: half the mass takes the 3 lowest indices
    np.testing.assert_array_equal(O.select_mass(qg, K, cand, 0.5, 0.1), [0, 2, 5])
    np.testing.assert_array_equal(O.select_mass(qg, K, cand, 1.0, 0.1), [0, 2, 5, 7, 9, 11])
    # a target just above k/6 needs k + 1 keys
    np.testing.assert_array_equal(O.select_mass(qg, K, cand, 2 / 6 + 1e-9, 0.1), [0, 2, 5])
    assert O.select_mass(qg, K, np.array([-1, -1]), 0.5, 0.1).size == 0
    # indices past the context are padding too
    np.testing.assert_array_equal(O.select_mass(qg, K, np.array([0, 2, 12, 40]), 1.0, 0.1), [0, 2])
    # the smallest target still takes one key
    np.testing.assert_array_equal(O.select_mass(qg, K, cand, 1e-300, 0.1), [0])


def test_select_mass_dominant_keys_and_head_average():
    d = 16
    K = np.zeros((10, d))
    K[3, 0] = 1.0
    K[8, 1] = 1.0
    q1 = np.zeros((1, d)); q1[0, 0] = 100.0
    # one head whose softmax sits on key 3
    np.testing.assert_array_equal(O.select_mass(q1, K, np.arange(10), 0.99, 1.0), [3])
    # two heads, one on key 3 and one on key 8: each holds half of the mass
    q2 = np.zeros((2, d)); q2[0, 0] = 100.0; q2[1, 1] = 100.0
    np.testing.assert_array_equal(O.select_mass(q2, K, np.arange(10), 0.4, 1.0), [3])
    np.testing.assert_array_equal(O.select_mass(q2, K, np.arange(10), 0.6, 1.0), [3, 8])
    # the count never falls as the target rises
    rng = np.random.default_rng(4)
    qg = rng.standard_normal((4, d)) * 3
    Kr = rng.standard_normal((300, d))
    counts = [O.select_mass(qg, Kr, np.arange(300), p, 0.25).size
              for p in np.linspace(0.05, 1.0, 40)]
    assert all(a <= b for a, b in zip(counts, counts[1:]))
    assert counts[-1] == 300


# ---------------------------------------------------------------- chunk routing

def test_chunk_cards_bruteforce_rational_and_weights():
    # HGA page, section 2, step 1: one card per 64-token chunk.  The card key
    # is the chunk's key sum rounded to the storage type (checked against an
    # exact rational sum and the rounding rule), its bits are exact signs
    # (rational brute force), its weight the largest stored value norm; the
    # last chunk may be short.
    rng = np.random.default_rng(31)
    L, P, d, n = 3, 4, 5, 150
    K = WL.bf16_bits_to_f32(WL.f32_to_bf16_bits(
        rng.standard_normal((n, d)).astype(np.float32))).astype(np.float64)
    K[96:128] = -K[64:96]                     # chunk 1 sums to exactly zero: all bits set
    W = rng.standard_normal((L * P, d)).astype(np.float32).astype(np.float64)
    vn = rng.random(n)
    for storage in ("f32", "bf16"):
        keys = O.chunk_card_keys(K, storage)
        assert keys.shape == (3, d)
        for c in range(3):
            exact = [sum(Fraction(float(x)) for x in K[c * 64:min(n, c * 64 + 64), i])
                     for i in range(d)]
            want = np.array([float(v) for v in exact], dtype=np.float64).astype(np.float32)
            if storage == "bf16":
                want = WL.bf16_bits_to_f32(WL.f32_to_bf16_bits(want))
            np.testing.assert_array_equal(keys[c], want.astype(np.float64))
        ids, wts = O.chunk_cards_softlsh(K, vn, W, L, P, storage)
        np.testing.assert_array_equal(ids, _brute_ids(keys, W, L, P))
        assert (ids[1] == (1 << P) - 1).all()
        for c in range(3):
            assert wts[c] == vn[c * 64:min(n, c * 64 + 64)].max()
    # a chunk of one key is that key's own bucket ids
    one = O.chunk_cards_softlsh(K[:1], vn[:1], W, L, P, "bf16")[0]
    np.testing.assert_array_equal(one, O.hash_keys_softlsh(K[:1], W, L, P))


def test_routing_reduces_to_plain_topk_and_keeps_chosen_chunks():
    rng = np.random.default_rng(8)
    L, P, d, n, G, k, tau = 8, 4, 16, 700, 2, 40, 0.4
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    W = rng.standard_normal((L * P, d))
    qg = rng.standard_normal((G, d))
    nc = (n + 63) // 64
    full = O.decode_slab_softlsh(qg, K, V, W, L, P, tau, k, "f16")
    # every chunk kept: the plain top-k step
    r = O.route_slab_softlsh(qg, K, V, W, L, P, tau, k, nc, "f16", "f32")
    np.testing.assert_array_equal(r["idx"], full["idx"])
    np.testing.assert_allclose(r["out"], full["out"], rtol=0, atol=0)
    # one chunk kept: the best card (lower index on ties) and keys inside it
    r1 = O.route_slab_softlsh(qg, K, V, W, L, P, tau, k, 1, "f16", "f32")
    cs = r1["chunk_scores"]
    best = min(range(nc), key=lambda c: (-cs[c], c))
    assert r1["chunks"].tolist() == [best]
    assert ((r1["idx"] >= 64 * best) & (r1["idx"] < 64 * best + 64)).all()
    assert r1["idx"].size == min(k, 64, n - 64 * best)
    # the card score is the card weight times the table mass of its buckets
    T = r1["T"]
    cid, cw = r1["cards"]
    for c in range(nc):
        assert abs(cs[c] - cw[c] * sum(T[l, cid[c, l]] for l in range(L))) <= 1e-12 * cs[c]


def test_shared_prefix_is_the_step_over_the_concatenated_context():
    # The prefix comes first: a planted key at suffix position j is index
    # Np + j, and a batch of sequences sharing a prefix gives, sequence by
    # sequence, the plain step over prefix + own suffix.
    rng = np.random.default_rng(12)
    L, P, d, G, tau = 8, 4, 16, 2, 0.3
    Np, Ns = 150, 40
    W = rng.standard_normal((L * P, d))
    Kp, Vp = rng.standard_normal((Np, d)), rng.standard_normal((Np, d))
    qg = np.repeat(rng.standard_normal((1, d)) * 3.0, G, axis=0)
    Ks, Vs = rng.standard_normal((Ns, d)), rng.standard_normal((Ns, d))
    Ks[7] = 4.0 * qg[0] / np.linalg.norm(qg[0])   # in every query bucket
    Vs[7] *= 10.0                                  # and the largest value norm
    r = O.decode_shared_prefix_softlsh(qg, Kp, Vp, Ks, Vs, W, L, P, tau, 1, "f32")
    np.testing.assert_array_equal(r["idx"], [Np + 7])
    r2 = O.decode_shared_prefix_softlsh(qg, Kp, Vp, Ks, Vs, W, L, P, tau, 12, "f32")
    full = O.decode_slab_softlsh(qg, np.concatenate([Kp, Ks]), np.concatenate([Vp, Vs]), W, L,
                                 P, tau, 12, "f32")
    np.testing.assert_array_equal(r2["idx"], full["idx"])
    # no suffix: the step over the prefix alone
    r3 = O.decode_shared_prefix_softlsh(qg, Kp, Vp, Ks[:0], Vs[:0], W, L, P, tau, 12, "f32")
    alone = O.decode_slab_softlsh(qg, Kp, Vp, W, L, P, tau, 12, "f32")
    np.testing.assert_array_equal(r3["idx"], alone["idx"])
    np.testing.assert_allclose(r3["out"], alone["out"], rtol=0, atol=0)


# ---------------------------------------------------------------- attention

def test_attend_all_keys_equals_dense_sdpa():
    rng = np.random.default_rng(12)
    n, d, G = 257, 32, 4
    K = rng.standard_normal((n, d)); V = rng.standard_normal((n, d))
    qg = rng.standard_normal((G, d))
    out, lse = O.attend(qg, K, V, np.arange(n), 1 / math.sqrt(d))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qg)[None, :, None, :],
        torch.from_numpy(K)[None, None].expand(1, G, n, d),
        torch.from_numpy(V)[None, None].expand(1, G, n, d))[0, :, 0, :].numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    ref_lse = torch.logsumexp(torch.from_numpy(qg @ K.T / math.sqrt(d)), dim=1).numpy()
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-13)


def test_attend_invariants():
    rng = np.random.default_rng(13)
    n, d, G = 100, 16, 2
    K = rng.standard_normal((n, d)); V = rng.standard_normal((n, d))
    qg = rng.standard_normal((G, d))
    # one key: the output is that value row
    out1, lse1 = O.attend(qg, K, V, np.array([42]), 0.25)
    np.testing.assert_allclose(out1, np.stack([V[42]] * G), rtol=1e-14)
    np.testing.assert_allclose(lse1, 0.25 * (qg @ K[42]), rtol=1e-14)
    # the result does not depend on the order of the selected set
    S = np.array([3, 17, 40, 41, 77, 90])
    o_a, l_a = O.attend(qg, K, V, S, 0.3)
    o_b, l_b = O.attend(qg, K, V, S[::-1].copy(), 0.3)
    np.testing.assert_allclose(o_a, o_b, rtol=1e-13)
    # merging two halves through their log-sum-exp equals one pass
    o1, l1 = O.attend(qg, K, V, S[:2], 0.3)
    o2, l2 = O.attend(qg, K, V, S[2:], 0.3)
    m = np.maximum(l1, l2)
    w1, w2 = np.exp(l1 - m), np.exp(l2 - m)
    merged = (o1 * w1[:, None] + o2 * w2[:, None]) / (w1 + w2)[:, None]
    np.testing.assert_allclose(merged, o_a, rtol=1e-12)
    np.testing.assert_allclose(m + np.log(w1 + w2), l_a, rtol=1e-13)
    # empty selection
    o0, l0 = O.attend(qg, K, V, np.zeros(0, dtype=np.int64), 0.3)
    assert (o0 == 0).all() and np.isneginf(l0).all()


def test_decode_slab_with_all_keys_is_dense_attention():
    rng = np.random.default_rng(14)
    n, d, G, L, P = 64, 16, 2, 4, 3
    K = rng.standard_normal((n, d)); V = rng.standard_normal((n, d))
    W = rng.standard_normal((L * P, d)); qg = rng.standard_normal((G, d))
    r = O.decode_slab_softlsh(qg, K, V, W, L, P, 0.5, n, "f32")
    assert r["idx"].tolist() == list(range(n))
    dense, _ = O.attend(qg, K, V, np.arange(n), 1 / math.sqrt(d))
    np.testing.assert_allclose(r["out"], dense, rtol=1e-13)


# ---------------------------------------------------------------- binary-code decode slab

_AX_KEYS = np.array([[-1, -1, 1, 1], [1, 1, 1, 1], [1, -1, 1, 1], [1, 1, -1, 1],
                     [-1, -1, -1, -1], [-1, 1, 1, 1]], dtype=np.float64)
_AX_Q = np.array([[1, 1, 1, 1], [-1, 1, 1, 1]], dtype=np.float64)
_AX_R = np.array([np.eye(4)[i % 4] for i in range(128)])


def test_decode_slab_hamming_hand_derived_selection(golden_dir):
    rows = _read_golden(golden_dir, "hamming_step_axes.txt")
    assert len(rows) == 6
    V = np.arange(24, dtype=np.float64).reshape(6, 4)
    for kk, sel in rows:
        r = O.decode_slab_hamming(_AX_Q, _AX_KEYS, V, _AX_R, int(kk))
        assert r["idx"].tolist() == [int(x) for x in sel.split()]
    r = O.decode_slab_hamming(_AX_Q, _AX_KEYS, V, _AX_R, 3)
    assert r["scores"].tolist() == [160, 224, 160, 160, 32, 224]
    assert r["kcodes"][1].tolist() == [0xFFFFFFFF] * 4
    assert r["kcodes"][4].tolist() == [0] * 4


def test_decode_slab_hamming_hand_derived_attention():
    # k = 3 keeps keys 0, 1, 5 (golden file above).  With scale 1/sqrt(4) the
    # logits are q1: (0, 2, 1) and q2: (1, 1, 2); one-hot values make the
    # output the softmax weights themselves.
    V = np.zeros((6, 4))
    V[0, 0] = V[1, 1] = V[5, 3] = 1.0
    V[2] = V[3] = V[4] = 7.0  # never selected
    r = O.decode_slab_hamming(_AX_Q, _AX_KEYS, V, _AX_R, 3)
    e = math.e
    z1, z2 = 1 + e * e + e, 2 * e + e * e
    want = np.array([[1 / z1, e * e / z1, 0, e / z1], [e / z2, e / z2, 0, e * e / z2]])
    np.testing.assert_allclose(r["out"], want, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(r["lse"], [math.log(z1), math.log(z2)], rtol=1e-14)
    # an explicit scale replaces 1/sqrt(d)
    r2 = O.decode_slab_hamming(_AX_Q, _AX_KEYS, V, _AX_R, 3, scale=1.0)
    z1b = 1 + e ** 4 + e ** 2
    np.testing.assert_allclose(r2["out"][0], [1 / z1b, e ** 4 / z1b, 0, e ** 2 / z1b], rtol=1e-14)


def test_decode_slab_hamming_all_keys_is_dense_attention():
    rng = np.random.default_rng(15)
    n, d, G = 48, 32, 3
    K = rng.standard_normal((n, d)); V = rng.standard_normal((n, d))
    R = rng.standard_normal((64, d)); qg = rng.standard_normal((G, d))
    r = O.decode_slab_hamming(qg, K, V, R, n)
    assert r["idx"].tolist() == list(range(n))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qg)[None, :, None, :], torch.from_numpy(K)[None, None].expand(1, G, n, d),
        torch.from_numpy(V)[None, None].expand(1, G, n, d))[0, :, 0].numpy()
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-13)
    # and for soft-LSH, the same library reference
    W = rng.standard_normal((4 * 3, d))
    rs = O.decode_slab_softlsh(qg, K, V, W, 4, 3, 0.5, n, "f32")
    np.testing.assert_allclose(rs["out"], ref, rtol=1e-12, atol=1e-13)
