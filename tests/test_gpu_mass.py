"""Cumulative-mass selection through the C ABI against the oracle (Tactic
page, sections 1 and 3).

* hst_select_mass on given candidate lists: ragged, empty and padded lists,
  lists up to the 8192 maximum, grouped query heads, ties between identical
  keys, targets from 0.3 to 1.  The kept set and its count equal the
  oracle's.  Both sides decide in float64, but exp and the summation order
  differ in the last bits, so a cut whose running sum lies within 1e-12
  relative of the target may land on either side: such a result is
  accepted when it equals the oracle's selection at a target moved by that
  much.
* hst_decode_step_softlsh_mass end to end, stage by stage: its candidates
  are the exact top-k of the GPU's hash scores; the kept set is the
  oracle's selection over those candidates; the attention over the kept set
  matches the oracle within the bf16 tolerance.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from tests.gpu_helpers import norm_torch_dtype, to_dev

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
EPS = 1e-12


def _store(x64, dt):
    x32 = np.asarray(x64, dtype=np.float32)
    return WL.f32_to_bf16_bits(x32) if dt == "bf16" else x32


def _accept(qg, K, cand, p, scale, got):
    for pp in (p, p * (1 - EPS), min(1.0, p * (1 + EPS))):
        if np.array_equal(O.select_mass(qg, K, cand, pp, scale), got):
            return True
    return False


CASES = [
    ("f32", 64, 1, 1, 0.9, False),
    ("bf16", 128, 4, 300, 0.9, False),
    ("bf16", 128, 8, 4096, 0.5, False),
    ("f32", 128, 4, 8192, 0.99, False),
    ("bf16", 64, 2, 1000, 1.0, False),
    ("bf16", 128, 4, 777, 0.3, False),
    ("bf16", 128, 4, 3000, 0.5, True),    # every key equal: one mass, cut by index
    ("f32", 64, 2, 5000, 0.999, False),
]


@pytest.mark.parametrize("dt,d,G,kcap,p,flat", CASES)
def test_select_mass_matches_oracle(dt, d, G, kcap, p, flat):
    import hash_scored_top_amd as hst

    print(f"[mass] {dt} d={d} G={G} k={kcap} p={p} flat={flat}", flush=True)
    rng = np.random.default_rng(kcap + 13 * G + d)
    B, Hkv, Nmax = 3, 2, 9000
    Hq = G * Hkv
    lens = np.array([Nmax, 2000, 0], dtype=np.int32)
    K = rng.standard_normal((B, Hkv, Nmax, d))
    # identical keys in every head: equal masses, decided by the index
    K[:, :, 10:20] = K[:, :, 5:6]
    if flat:
        K[:] = K[:, :, :1]
    q = rng.standard_normal((B, Hq, d)) * 2.0
    K, q = _store(K, dt), _store(q, dt)
    cand = np.full((B, Hkv, kcap), -1, dtype=np.int32)
    for b in range(B):
        for h in range(Hkv):
            n = int(lens[b])
            c = min(kcap, n)
            if c == 0:
                continue
            # the identical keys 5..14 first, then a random draw
            forced = np.arange(5, 15)
            pool = rng.permutation(n)
            pool = pool[~np.isin(pool, forced)]
            cand[b, h, :c] = np.sort(np.concatenate([forced, pool])[:c])
            if c < kcap:                  # an index past the context is padding
                cand[b, h, c] = n + 3
    scale = d ** -0.5
    Kd, qd = to_dev(K, dt, DEV), to_dev(q, dt, DEV)
    sl = torch.from_numpy(lens).to(DEV)
    idx, counts = hst.hst_select_mass(qd, Kd, torch.from_numpy(cand).to(DEV), p, scale,
                                      seq_lens=sl)
    torch.cuda.synchronize()
    idx, counts = idx.cpu().numpy(), counts.cpu().numpy()
    K64, q64 = WL.storage_to_f64(K, dt), WL.storage_to_f64(q, dt)
    edge = 0
    for b in range(B):
        n = int(lens[b])
        for h in range(Hkv):
            c = int(counts[b, h])
            got = idx[b, h, :c]
            assert (idx[b, h, c:] == -1).all(), (b, h)
            qg = q64[b, h * G:(h + 1) * G]
            want = O.select_mass(qg, K64[b, h, :n], cand[b, h], p, scale)
            if not np.array_equal(got, want):
                assert _accept(qg, K64[b, h, :n], cand[b, h], p, scale, got), (b, h, c, want.size)
                edge += 1
    assert edge <= 1


def test_decode_step_mass_matches_oracle_stage_by_stage():
    import hash_scored_top_amd as hst

    base = WL.WORKLOADS["llama8b_softlsh_b8_n32k"]
    w = dataclasses.replace(base, name="mass_small", B=2, N=4096, ragged=(2500, 4096))
    print(f"[mass-decode] {w.name}", flush=True)
    x = WL.make_full(w)
    lens, ks = x["seq_lens"], x["k_per_seq"]
    kmax = int(ks.max())
    p = 0.9
    K, V, q, Wp = (to_dev(x[n], w.kv_dtype, DEV) for n in ("K", "V", "q", "W"))
    sl = torch.from_numpy(lens).to(DEV)
    kp = torch.from_numpy(ks).to(DEV)
    nd = norm_torch_dtype(w.norm_dtype)
    ids, vn = hst.hst_hash_keys_softlsh(K, V, Wp, w.L, w.P, nd, seq_lens=sl)
    step = hst.DecodeSoftLSHMass(K, w.Hq, w.L, w.P, w.tau, kmax, p, nd, seq_lens=sl,
                                 k_per_seq=kp)
    idx, counts, out, lse = step(q, K, V, Wp, ids, vn)
    scores = hst.hst_score_keys_softlsh(q, Wp, w.L, w.P, w.tau, ids, vn, K, seq_lens=sl)
    cand = hst.hst_select_topk(scores, kmax, w.Hq, w.d, K.dtype, k_per_seq=kp, seq_lens=sl)
    torch.cuda.synchronize()
    idx, counts, out, lse = (t.cpu().numpy() for t in (idx, counts, out, lse))
    cand = cand.cpu().numpy()
    f64 = lambda a: WL.storage_to_f64(a, w.kv_dtype)
    scale = w.d ** -0.5
    G = w.G
    for b in range(w.B):
        n = int(lens[b])
        for h in range(w.Hkv):
            qg = f64(x["q"][b, h * G:(h + 1) * G])
            K64, V64 = f64(x["K"][b, h, :n]), f64(x["V"][b, h, :n])
            c = int(counts[b, h])
            got = idx[b, h, :c]
            assert 1 <= c <= int(ks[b]) and (idx[b, h, c:] == -1).all()
            want = O.select_mass(qg, K64, cand[b, h], p, scale)
            if not np.array_equal(got, want):
                assert _accept(qg, K64, cand[b, h], p, scale, got), (b, h)
            o_ref, l_ref = O.attend(qg, K64, V64, got, scale)
            assert np.abs(out[b, h * G:(h + 1) * G] - o_ref).max() <= 2e-2, (b, h)
            np.testing.assert_allclose(lse[b, h * G:(h + 1) * G], l_ref, rtol=1e-4, atol=1e-4)
            print(f"[mass-decode] slab {(b, h)}: kept {c} of {int(ks[b])} candidates",
                  flush=True)
