"""The decode step's stages, its candidate filter and its selection paths.

* The three stage calls (prepare, filter, finish) give exactly the fused
  step's indices, outputs and log-sum-exp.
* The filter stage's candidates, read back through hst_decode_candidates,
  are checked against the oracle's scores: each candidate's own score within
  1e-5 relative (soft-LSH; exact for binary codes), in index order, and every
  key scoring clearly above the threshold is a candidate.
* Inputs crafted so that fewer than k keys pass the sample threshold force
  the selection over every key, rescored from the metadata (path 2); the
  result must equal the oracle's exactly.
* Score distributions that drive each way the head's candidate histogram is
  resolved (a bin taken whole, one-value bins of integer scores, a ranked
  boundary bin, an overflowing or over-full bin that falls back to radix
  passes) give exactly the oracle's top-k.
"""
import ctypes
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from tests.gpu_helpers import check_attention, norm_torch_dtype, to_dev
from tests.test_gpu_parity import MED_HAM, MED_SOFT, _sample_positions, _select_raw, inputs, slab64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _hst():
    import hash_scored_top_amd as hst
    return hst


def _paths(ws, B, Hkv):
    head = ws[:B * Hkv * 64].cpu().numpy().view(np.uint32).reshape(B * Hkv, 16)
    return head[:, 4].copy()


def _key_to_f32(keys):
    """Order keys of non-negative float32 scores back to the scores."""
    k = np.asarray(keys).astype(np.uint32)
    assert (k & 0x80000000).all()
    return (k & 0x7FFFFFFF).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("scheme", ["softlsh", "hamming"])
def test_staged_step_equals_fused(scheme):
    hst = _hst()
    w = MED_SOFT if scheme == "softlsh" else MED_HAM
    x, d = inputs(w)
    sl, kp = d["seq_lens"], d["k_per_seq"]
    if scheme == "softlsh":
        ids, vn = hst.hst_hash_keys_softlsh(d["K"], d["V"], d["W"], w.L, w.P,
                                            norm_torch_dtype(w.norm_dtype), seq_lens=sl)
        step = hst.DecodeSoftLSH(d["K"], w.Hq, w.L, w.P, w.tau, w.k_max(), vn.dtype, seq_lens=sl,
                                 k_per_seq=kp)
        ref = [t.clone() for t in step(d["q"], d["K"], d["V"], d["W"], ids, vn)]
        step.prepare(d["q"], d["W"], ids, vn)
        step.filter(ids, vn)
        got = step.finish(d["q"], d["K"], d["V"], ids, vn)
    else:
        codes = hst.hst_hash_keys_binary(d["K"], d["R"], seq_lens=sl)
        step = hst.DecodeHamming(d["K"], w.Hq, w.k_max(), seq_lens=sl, k_per_seq=kp)
        ref = [t.clone() for t in step(d["q"], d["K"], d["V"], d["R"], codes)]
        step.prepare(d["q"], d["R"], codes)
        step.filter(codes)
        got = step.finish(d["q"], d["K"], d["V"], codes)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


@pytest.mark.parametrize("scheme", ["softlsh", "hamming"])
def test_filter_candidates_against_oracle(scheme):
    hst = _hst()
    w = MED_SOFT if scheme == "softlsh" else MED_HAM
    x, d = inputs(w)
    sl, kp = d["seq_lens"], d["k_per_seq"]
    if scheme == "softlsh":
        ids, vn = hst.hst_hash_keys_softlsh(d["K"], d["V"], d["W"], w.L, w.P,
                                            norm_torch_dtype(w.norm_dtype), seq_lens=sl)
        step = hst.DecodeSoftLSH(d["K"], w.Hq, w.L, w.P, w.tau, w.k_max(), vn.dtype, seq_lens=sl,
                                 k_per_seq=kp)
        step(d["q"], d["K"], d["V"], d["W"], ids, vn)
    else:
        codes = hst.hst_hash_keys_binary(d["K"], d["R"], seq_lens=sl)
        step = hst.DecodeHamming(d["K"], w.Hq, w.k_max(), seq_lens=sl, k_per_seq=kp)
        step(d["q"], d["K"], d["V"], d["R"], codes)
    keys, index, count, theta = (t.cpu().numpy() for t in step.candidates(w.N))
    torch.cuda.synchronize()
    theta = theta.view(np.uint32)
    for b in range(w.B):
        n, kb = int(x["seq_lens"][b]), int(x["k_per_seq"][b])
        for h in range(w.Hkv):
            q64, K64, V64 = slab64(w, x, b, h)
            c = int(count[b, h])
            assert kb <= c <= n, (b, h, c)
            ix = index[b, h, :c]
            assert (np.diff(ix) > 0).all() and ix[0] >= 0 and ix[-1] < n
            if scheme == "softlsh":
                r = O.decode_slab_softlsh(q64, K64, V64, WL.storage_to_f64(x["W"][h], w.kv_dtype),
                                          w.L, w.P, w.tau, kb, w.norm_dtype)
                s = r["scores"]
                got = _key_to_f32(keys[b, h, :c])
                rel = np.abs(got - s[ix]) / s[ix]
                assert rel.max() <= 1e-5, (b, h, rel.max())
                th = float(_key_to_f32([theta[b, h]])[0]) if theta[b, h] & np.uint32(0x80000000) else 0.0
                assert (s[ix] >= th * (1 - 2e-5)).all()
                must = np.nonzero(s >= th * (1 + 2e-5))[0]
                assert np.isin(must, ix).all(), (b, h)
            else:
                r = O.decode_slab_hamming(q64, K64, V64, WL.storage_to_f64(x["R"][h], w.kv_dtype), kb)
                s = r["scores"]
                got = (keys[b, h, :c].astype(np.uint32) ^ np.uint32(0x80000000)).view(np.int32)
                np.testing.assert_array_equal(got, s[ix])
                th = int(np.array([theta[b, h] ^ np.uint32(0x80000000)], np.uint32).view(np.int32)[0])
                np.testing.assert_array_equal(ix, np.nonzero(s >= th)[0])


def test_decode_rescoring_path_softlsh():
    """Sampled keys get large value norms, every other key a small one and
    the same bucket ids: the threshold from the sample passes fewer keys than
    k, so the step selects over every key rescored from the metadata."""
    hst = _hst()
    B, Hq, Hkv, d, n, L, P, tau, k = 1, 4, 1, 64, 20000, 16, 4, 0.5, 3000
    rng = np.random.default_rng(31)
    K = rng.standard_normal((B, Hkv, n, d)).astype(np.float32)
    V = rng.standard_normal((B, Hkv, n, d)).astype(np.float32)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    W = rng.standard_normal((Hkv, L * P, d)).astype(np.float32)
    ids = np.zeros((B, Hkv, n, L), np.uint8)
    vn = np.ones((B, Hkv, n), np.float32)
    samp = _sample_positions(n)
    vn[0, 0, samp] = 100.0 + np.arange(len(samp), dtype=np.float32)
    Kd, Vd, qd, Wd = (to_dev(a, "f32", DEV) for a in (K, V, q, W))
    idd, vnd = torch.from_numpy(ids).to(DEV), torch.from_numpy(vn).to(DEV)
    step = hst.DecodeSoftLSH(Kd, Hq, L, P, tau, k, torch.float32)
    idx, out, lse = step(qd, Kd, Vd, Wd, idd, vnd)
    torch.cuda.synchronize()
    assert _paths(step.ws, B, Hkv)[0] == 2
    T = O.query_tables(q[0].astype(np.float64), W[0].astype(np.float64), L, P, tau)
    s = O.score_softlsh(T, ids[0, 0], vn[0, 0].astype(np.float64))
    want = O.select_topk(s, k)
    got = idx.cpu().numpy()[0, 0]
    np.testing.assert_array_equal(got, want)
    check_attention(out.cpu().numpy()[0], lse.cpu().numpy()[0], q[0].astype(np.float64),
                    K[0, 0].astype(np.float64), V[0, 0].astype(np.float64), got, "f32")


def test_decode_rescoring_path_hamming():
    """Sampled keys carry the first query head's code, every other key its
    complement: the sample threshold passes 2048 keys for k = 3000, so the
    step selects over every key rescored from the codes."""
    hst = _hst()
    B, Hq, Hkv, d, n, k = 1, 4, 1, 64, 20000, 3000
    rng = np.random.default_rng(32)
    K = rng.standard_normal((B, Hkv, n, d)).astype(np.float32)
    V = rng.standard_normal((B, Hkv, n, d)).astype(np.float32)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    R = rng.standard_normal((Hkv, 128, d)).astype(np.float32)
    qc = O.binary_codes(q[0].astype(np.float64), R[0].astype(np.float64))
    codes = np.broadcast_to(~qc[0], (B, Hkv, n, 4)).copy()
    samp = _sample_positions(n)
    codes[0, 0, samp] = qc[0]
    Kd, Vd, qd, Rd = (to_dev(a, "f32", DEV) for a in (K, V, q, R))
    cd = torch.from_numpy(codes.view(np.int32)).to(DEV)
    step = hst.DecodeHamming(Kd, Hq, k)
    idx, out, lse = step(qd, Kd, Vd, Rd, cd)
    torch.cuda.synchronize()
    assert _paths(step.ws, B, Hkv)[0] == 2
    r = O.decode_slab_hamming(q[0].astype(np.float64), K[0, 0].astype(np.float64),
                              V[0, 0].astype(np.float64), R[0].astype(np.float64), k,
                              kcodes=codes[0, 0])
    np.testing.assert_array_equal(idx.cpu().numpy()[0, 0], r["idx"])
    assert np.abs(out.cpu().numpy()[0] - r["out"]).max() <= 1e-5 * np.abs(r["out"]).max()


def _hist_cases():
    n = 50000
    rng = np.random.default_rng(41)
    samp = np.array(_sample_positions(n))
    other = np.setdiff1d(np.arange(n), samp)
    cases = []
    # float scores, spread: the boundary bin is ranked (or taken whole)
    cases.append(("uniform", rng.random(n).astype(np.float32), [1, 700, 1515, 4000]))
    # integer scores over a small range: every bin is one value
    cases.append(("int_small", rng.integers(0, 40, n).astype(np.int32), [1, 1000, 3333]))
    # a wide spread plus a large block of equal scores just above the
    # threshold: the boundary bin is too full to rank and falls back to radix
    s = rng.random(n).astype(np.float32)
    blk = other[rng.permutation(other.size)[:3000]]
    s[blk] = np.float32(0.97)
    cases.append(("equal_block", s, [1200, 1500, 2000]))
    # the top keys lie far above the sample's range: they all fall into the
    # overflow bin, whose entries are ranked or sorted out by radix passes
    s = rng.random(n).astype(np.float32)
    top = other[rng.permutation(other.size)[:3000]]
    s[top] = (1000.0 + 1000.0 * rng.random(top.size)).astype(np.float32)
    cases.append(("overflow", s, [100, 2000, 2990]))
    small = other[rng.permutation(other.size)[:200]]
    s2 = rng.random(n).astype(np.float32)
    s2[small] = (1000.0 + rng.random(small.size)).astype(np.float32)
    cases.append(("overflow_small", s2, [150, 600]))
    # negative and positive zero, subnormals and ties at the boundary
    s = np.zeros(n, np.float32)
    s[rng.permutation(n)[:5000]] = np.float32(1e-40)
    s[rng.permutation(n)[:3000]] = np.float32(-0.0)
    s[rng.permutation(n)[:1500]] = np.float32(2.0)
    cases.append(("zeros_subnormal", s, [1000, 1500, 3000, 7000]))
    return cases


@pytest.mark.parametrize("case", range(6))
def test_select_histogram_resolutions(case):
    name, s, ks = _hist_cases()[case]
    print(f"[hist] {name}", flush=True)
    for k in ks:
        idx, path = _select_raw(s[None, None, :], k)
        ref = O.select_topk(s.astype(np.float64) if s.dtype == np.float32 else s.astype(np.int64), k)
        np.testing.assert_array_equal(idx[0, 0], ref, err_msg=f"{name} k={k} path {path}")
