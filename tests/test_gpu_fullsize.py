"""Parity at the full workload sizes, in the configuration the benchmark times.

Each large workload is generated whole, hashed on the GPU and run through the
pre-sized decode step (the same objects and launches the benchmark replays).
The float64 oracle recomputes a sample of (batch, kv head) slabs end to end
from the generated inputs, and every slab is checked against properties that
hold at any size:

* sampled slabs: bucket ids, value norms and binary codes bit-exact; soft
  scores within 1e-5 relative, Hamming scores exact; the selected set equal
  to the oracle's (soft-LSH: keys outside the intersection must sit within
  the float32 rounding band of the k-th score); attention over the GPU's own
  selected set within 2e-2 absolute of the oracle's attention over that set,
  and the log-sum-exp within 1e-4;
* sampled slabs: the candidates the step's own filtering scan kept, read back
  from its workspace, carry their oracle scores (soft-LSH within 1e-5
  relative, binary codes exactly) and include every key clearly above the
  head's threshold;
* every slab: indices ascending, in [0, N_b), exactly k_b of them, -1 after;
  and the set is exactly the first k_b keys in the order (score descending,
  index ascending) of the scores the GPU scorer produces.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

LARGE = ["llama8b_softlsh_b8_n32k", "longctx_softlsh_b1_n128k", "hata_hamming_b16_n64k",
         "qwen30b_ragged_softlsh_b32"]


def _sample_slabs(w, lens, count):
    """Seeded slab sample; ragged batches include the shortest and longest sequence."""
    every = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    if len(every) <= count:
        return every
    rng = np.random.default_rng(7)
    pick = {(0, 0), (w.B - 1, w.Hkv - 1)}
    if w.ragged is not None:
        pick.add((int(np.argmin(lens)), 0))
        pick.add((int(np.argmax(lens)), w.Hkv - 1))
    while len(pick) < count:
        pick.add(every[int(rng.integers(len(every)))])
    return sorted(pick)


def _topk_of(scores, k):
    """First k keys by (score descending, index ascending), ascending."""
    n = scores.shape[0]
    order = np.lexsort((np.arange(n), -scores.astype(np.float64)))
    return np.sort(order[:k])


CAND_CAP = 16384  # candidates read back per head (the step's own filtering-scan scores)


def _check_candidates(scheme, s, keys, index, count, theta, kk, where):
    """The candidates the step's filtering scan kept for one head, against the
    oracle's scores s: in index order, each with its own score (soft-LSH:
    within 1e-5 relative; binary codes: exact), and every key clearly above
    the threshold among them (binary codes: exactly the keys >= it)."""
    c = min(count, CAND_CAP)
    assert count >= kk, where
    ix = index[:c]
    assert (np.diff(ix) > 0).all() and ix[0] >= 0 and ix[-1] < s.shape[0], where
    u = keys[:c].astype(np.uint32)
    th = np.uint32(theta & 0xFFFFFFFF)
    if scheme == "softlsh":
        assert (u & np.uint32(0x80000000)).all(), where
        got = (u & np.uint32(0x7FFFFFFF)).view(np.float32).astype(np.float64)
        rel = np.abs(got - s[ix]) / s[ix]
        assert rel.max() <= 1e-5, (where, rel.max())
        thf = float(np.array([th & np.uint32(0x7FFFFFFF)], np.uint32).view(np.float32)[0]) \
            if th & np.uint32(0x80000000) else 0.0
        must = np.nonzero(s >= thf * (1 + 2e-5))[0]
        must = must[must <= ix[-1]] if count > c else must
        assert np.isin(must, ix).all(), where
    else:
        got = (u ^ np.uint32(0x80000000)).view(np.int32)
        np.testing.assert_array_equal(got, s[ix], err_msg=str(where))
        thi = int(np.array([th ^ np.uint32(0x80000000)], np.uint32).view(np.int32)[0])
        want = np.nonzero(s >= thi)[0]
        np.testing.assert_array_equal(ix, want[:c], err_msg=str(where))


@pytest.mark.parametrize("name", LARGE)
def test_fullsize_decode_step(name):
    import hash_scored_top_amd as hst
    from workloads.device import norm_torch_dtype, to_dev

    w = WL.WORKLOADS[name]
    print(f"[fullsize] {name}: generating", flush=True)
    x = WL.make_full(w)
    lens, ks = x["seq_lens"], x["k_per_seq"]
    kmax = int(ks.max())
    ragged = w.ragged is not None
    K = to_dev(x["K"], w.kv_dtype, DEV)
    V = to_dev(x["V"], w.kv_dtype, DEV)
    q = to_dev(x["q"], w.kv_dtype, DEV)
    sl = torch.from_numpy(lens).to(DEV) if ragged else None
    kp = torch.from_numpy(ks).to(DEV) if ragged else None

    print(f"[fullsize] {name}: hashing + decode step on the GPU", flush=True)
    if w.scheme == "softlsh":
        Wd = to_dev(x["W"], w.kv_dtype, DEV)
        ids, vn = hst.hst_hash_keys_softlsh(K, V, Wd, w.L, w.P, norm_torch_dtype(w.norm_dtype),
                                            seq_lens=sl)
        step = hst.DecodeSoftLSH(K, w.Hq, w.L, w.P, w.tau, kmax, vn.dtype, seq_lens=sl,
                                 k_per_seq=kp)
        idx, out, lse = step(q, K, V, Wd, ids, vn)
        cand = step.candidates(CAND_CAP)
        scores = hst.hst_score_keys_softlsh(q, Wd, w.L, w.P, w.tau, ids, vn, K, seq_lens=sl)
        meta = (ids.cpu().numpy(), vn.cpu().numpy().astype(np.float64))
    else:
        Rd = to_dev(x["R"], w.kv_dtype, DEV)
        codes = hst.hst_hash_keys_binary(K, Rd, seq_lens=sl)
        step = hst.DecodeHamming(K, w.Hq, kmax, seq_lens=sl, k_per_seq=kp)
        idx, out, lse = step(q, K, V, Rd, codes)
        cand = step.candidates(CAND_CAP)
        scores = hst.hst_score_keys_hamming(q, Rd, codes, K, seq_lens=sl)
        meta = (codes.cpu().numpy().view(np.uint32),)
    torch.cuda.synchronize()
    idx, out, lse = idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()
    scores = scores.cpu().numpy()
    ckeys, cidx, ccount, ctheta = (t.cpu().numpy() for t in cand)
    paths = np.frombuffer(step.ws[:64 * w.B * w.Hkv].cpu().numpy().tobytes(),
                          dtype=np.uint32).reshape(-1, 16)[:, 4]
    print(f"[fullsize] {name}: selection paths {np.bincount(paths, minlength=3).tolist()}",
          flush=True)
    del K, V, q, step
    torch.cuda.empty_cache()

    # properties of every slab
    for b in range(w.B):
        n, kb = int(lens[b]), int(ks[b])
        kk = min(kb, n)
        for h in range(w.Hkv):
            got = idx[b, h]
            assert (got[kk:] == -1).all(), (b, h)
            sel = got[:kk]
            assert (np.diff(sel) > 0).all() and sel[0] >= 0 and sel[-1] < n, (b, h)
            np.testing.assert_array_equal(sel, _topk_of(scores[b, h, :n], kk),
                                          err_msg=f"slab {(b, h)}")
            assert np.isfinite(out[b, h * w.G:(h + 1) * w.G]).all()

    # oracle on sampled slabs
    f64 = lambda a: WL.storage_to_f64(a, w.kv_dtype)
    sample = _sample_slabs(w, lens, 8 if w.scheme == "hamming" else 4)
    if w.B * w.Hkv <= 8:
        sample = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    print(f"[fullsize] {name}: oracle on slabs {sample}", flush=True)
    G = w.G
    from tests.gpu_helpers import check_attention
    for (b, h) in sample:
        n, kb = int(lens[b]), int(ks[b])
        q64 = f64(x["q"][b, h * G:(h + 1) * G])
        K64, V64 = f64(x["K"][b, h, :n]), f64(x["V"][b, h, :n])
        if w.scheme == "softlsh":
            r = O.decode_slab_softlsh(q64, K64, V64, f64(x["W"][h]), w.L, w.P, w.tau, kb,
                                      w.norm_dtype)
            np.testing.assert_array_equal(meta[0][b, h, :n], r["ids"])
            np.testing.assert_array_equal(meta[1][b, h, :n], r["vnorm"])
            rel = np.abs(scores[b, h, :n] - r["scores"]) / np.abs(r["scores"])
            assert rel.max() <= 1e-5, (b, h, rel.max())
        else:
            r = O.decode_slab_hamming(q64, K64, V64, f64(x["R"][h]), kb)
            np.testing.assert_array_equal(meta[0][b, h, :n], r["kcodes"])
            np.testing.assert_array_equal(scores[b, h, :n], r["scores"])
        _check_candidates(w.scheme, r["scores"], ckeys[b, h], cidx[b, h], int(ccount[b, h]),
                          int(ctheta[b, h]), min(kb, n), (b, h))
        got = idx[b, h, :min(kb, n)]
        diff = set(got.tolist()) ^ set(r["idx"].tolist())
        if w.scheme == "hamming":
            assert not diff, (b, h)
        if diff:
            kth = np.sort(r["scores"])[::-1][kb - 1]
            for j in diff:
                assert abs(r["scores"][j] - kth) <= 2e-5 * kth, (b, h, j)
        # attention over the GPU's own selection, on every sampled slab
        check_attention(out[b, h * G:(h + 1) * G], lse[b, h * G:(h + 1) * G], q64, K64, V64,
                        got, w.kv_dtype, where=(b, h))
        if not diff:
            assert np.abs(out[b, h * G:(h + 1) * G] - r["out"]).max() <= 2e-2, (b, h)
