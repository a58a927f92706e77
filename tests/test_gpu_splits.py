"""The decode step across attention split regimes, against the CPU oracle.

The attention splits of a kv head each select the head's rows, gather their
part of the index row, and the last one to finish merges the others (SOCKET
overview page, "Core mechanism: soft LSH", item 4: exact attention over the
selected subset, split-K with a log-sum-exp merge).  The split count follows
the rows per head: a single split (k = 40), the usual many splits, splits
of more than 1024 rows each when the heads are many (so that one round of
workgroups holds them all), and more than 128 splits of one head.  Each case checks every slab: the index row
(ascending, -1 padded, equal to the oracle's up to near-ties for soft-LSH,
bit-exact for binary codes) and the attention over the GPU's own selected set.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from tests.gpu_helpers import check_attention, norm_torch_dtype, to_dev

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

ONE_SPLIT = dataclasses.replace(WL.WORKLOADS["llama8b_softlsh_b8_n32k"], name="one_split", B=2, Hq=8,
                                Hkv=2, N=6000, needles=4, ragged=(3000, 6000), sparsity=150.0, seed=211)
WIDE_SOFT = dataclasses.replace(WL.WORKLOADS["llama8b_softlsh_b8_n32k"], name="wide_soft", B=8, Hq=32,
                                Hkv=8, N=8400, needles=4, ragged=None, sparsity=2.0, seed=212)
# one kv head, half its keys selected: about 157 splits of 64 rows, more
# than the 128 whose (m, l) pairs the merging split loads in one round trip
MANY_SPLITS = dataclasses.replace(WL.WORKLOADS["llama8b_softlsh_b8_n32k"], name="many_splits", B=1, Hq=4,
                                  Hkv=1, N=20000, needles=4, ragged=None, sparsity=2.0, seed=214)
WIDE_HAM = dataclasses.replace(WL.WORKLOADS["hata_hamming_b16_n64k"], name="wide_ham", B=16, Hq=16,
                               Hkv=8, N=6000, needles=4, ragged=None, sparsity=2.0, seed=213)


def _slab(w, x, b, h):
    G = w.Hq // w.Hkv
    n = int(x["seq_lens"][b])
    f = lambda a: WL.storage_to_f64(a, w.kv_dtype)  # noqa: E731
    return f(x["q"][b, h * G:(h + 1) * G]), f(x["K"][b, h, :n]), f(x["V"][b, h, :n])


def _check_rows(idx, kb, n):
    got = idx[:kb]
    assert (idx[kb:] == -1).all()
    assert (np.diff(got) > 0).all() and got[0] >= 0 and got[-1] < n
    return got


@pytest.mark.parametrize("w", [ONE_SPLIT, WIDE_SOFT, MANY_SPLITS], ids=lambda w: w.name)
def test_softlsh_step_split_regimes(w):
    import hash_scored_top_amd as hst
    x = WL.make_full(w)
    K, V, q, W = (to_dev(x[n], w.kv_dtype, DEV) for n in ("K", "V", "q", "W"))
    ragged = w.ragged is not None
    sl = torch.from_numpy(x["seq_lens"]).to(DEV) if ragged else None
    kp = torch.from_numpy(x["k_per_seq"]).to(DEV) if ragged else None
    ids, vn = hst.hst_hash_keys_softlsh(K, V, W, w.L, w.P, norm_torch_dtype(w.norm_dtype), seq_lens=sl)
    print(f"[splits] {w.name}: B={w.B} Hkv={w.Hkv} N={w.N} k={w.k_max()}", flush=True)
    idx, out, lse = hst.hst_decode_step_softlsh(q, K, V, W, ids, vn, w.L, w.P, w.tau, w.k_max(),
                                                seq_lens=sl, k_per_seq=kp)
    idx, out, lse = idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()
    G = w.Hq // w.Hkv
    slabs = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    oracle_slabs = set(slabs[:: max(1, len(slabs) // 6)])  # the oracle's full step on a sample
    for b, h in slabs:
        kb = int(x["k_per_seq"][b])
        q64, K64, V64 = _slab(w, x, b, h)
        got = _check_rows(idx[b, h], kb, K64.shape[0])
        sl_ = slice(h * G, (h + 1) * G)
        check_attention(out[b, sl_], lse[b, sl_], q64, K64, V64, got, w.kv_dtype, where=(w.name, b, h))
        if (b, h) in oracle_slabs:
            r = O.decode_slab_softlsh(q64, K64, V64, WL.storage_to_f64(x["W"][h], w.kv_dtype), w.L, w.P,
                                      w.tau, kb, w.norm_dtype)
            kth = np.sort(r["scores"])[::-1][kb - 1]
            for j in set(got.tolist()) ^ set(r["idx"].tolist()):
                assert abs(r["scores"][j] - kth) <= 2e-5 * kth, (w.name, b, h, j)


def test_hamming_step_wide_splits():
    import hash_scored_top_amd as hst
    w = WIDE_HAM
    x = WL.make_full(w)
    K, V, q, R = (to_dev(x[n], w.kv_dtype, DEV) for n in ("K", "V", "q", "R"))
    codes = hst.hst_hash_keys_binary(K, R)
    k = w.k_max()
    print(f"[splits] {w.name}: B={w.B} Hkv={w.Hkv} N={w.N} k={k}", flush=True)
    idx, out, lse = hst.hst_decode_step_hamming(q, K, V, R, codes, k)
    idx, out, lse = idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()
    G = w.Hq // w.Hkv
    slabs = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    for b, h in slabs[:: max(1, len(slabs) // 8)]:
        q64, K64, V64 = _slab(w, x, b, h)
        r = O.decode_slab_hamming(q64, K64, V64, WL.storage_to_f64(x["R"][h], w.kv_dtype), k)
        np.testing.assert_array_equal(idx[b, h], r["idx"])
        sl_ = slice(h * G, (h + 1) * G)
        check_attention(out[b, sl_], lse[b, sl_], q64, K64, V64, r["idx"], w.kv_dtype, where=(w.name, b, h))
    for b, h in slabs:  # every slab: a well-formed row and the attention over it
        q64, K64, V64 = _slab(w, x, b, h)
        got = _check_rows(idx[b, h], k, K64.shape[0])
        sl_ = slice(h * G, (h + 1) * G)
        check_attention(out[b, sl_], lse[b, sl_], q64, K64, V64, got, w.kv_dtype, where=(w.name, b, h))
    assert math.isfinite(float(np.abs(out).max()))
