"""The no-allocation soft-LSH decode step against the workspace entry point.

hst_decode_step_softlsh_noalloc runs the same kernels as
hst_decode_step_softlsh on the library's fixed per-GPU workspace.  Two calls
in a row, the second on a smaller batch (fewer sequences, heads and keys),
must each give exactly the workspace entry point's indices, outputs and
log-sum-exp; the first is also checked against the oracle on its slabs.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from tests.gpu_helpers import check_attention, norm_torch_dtype, to_dev

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

BIG = dataclasses.replace(WL.WORKLOADS["llama8b_softlsh_b8_n32k"], name="noalloc_big", B=3, Hq=8,
                          Hkv=2, N=7000, needles=8, ragged=(2500, 7000), seed=91)
SMALL = dataclasses.replace(WL.WORKLOADS["llama8b_softlsh_b8_n32k"], name="noalloc_small", B=1,
                            Hq=4, Hkv=1, N=2600, needles=4, ragged=None, seed=92)


def _run(w):
    import hash_scored_top_amd as hst
    x = WL.make_full(w)
    K, V, q, W = (to_dev(x[n], w.kv_dtype, DEV) for n in ("K", "V", "q", "W"))
    ragged = w.ragged is not None
    sl = torch.from_numpy(x["seq_lens"]).to(DEV) if ragged else None
    kp = torch.from_numpy(x["k_per_seq"]).to(DEV) if ragged else None
    ids, vn = hst.hst_hash_keys_softlsh(K, V, W, w.L, w.P, norm_torch_dtype(w.norm_dtype),
                                        seq_lens=sl)
    k = w.k_max()
    print(f"[noalloc] {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} k={k}", flush=True)
    ref = [t.clone() for t in hst.hst_decode_step_softlsh(q, K, V, W, ids, vn, w.L, w.P, w.tau, k,
                                                          seq_lens=sl, k_per_seq=kp)]
    got = hst.hst_decode_step_softlsh_noalloc(q, K, V, W, ids, vn, w.L, w.P, w.tau, k,
                                              seq_lens=sl, k_per_seq=kp)
    torch.cuda.synchronize()
    return x, ref, [t.cpu() for t in got]


def test_noalloc_matches_workspace_step_twice():
    x, ref, got = _run(BIG)
    for a, b in zip(ref, got):
        assert torch.equal(a.cpu(), b)
    # the first call against the oracle on every slab
    w = BIG
    idx, out, lse = (t.numpy() for t in got)
    f64 = lambda a: WL.storage_to_f64(a, w.kv_dtype)
    for b in range(w.B):
        n, kb = int(x["seq_lens"][b]), int(x["k_per_seq"][b])
        for h in range(w.Hkv):
            qg = f64(x["q"][b, h * w.G:(h + 1) * w.G])
            K64, V64 = f64(x["K"][b, h, :n]), f64(x["V"][b, h, :n])
            r = O.decode_slab_softlsh(qg, K64, V64, f64(x["W"][h]), w.L, w.P, w.tau, kb,
                                      w.norm_dtype)
            sel = idx[b, h, :kb]
            kth = np.sort(r["scores"])[::-1][kb - 1]
            for j in set(sel.tolist()) ^ set(r["idx"].tolist()):
                assert abs(r["scores"][j] - kth) <= 2e-5 * kth, (b, h, j)
            check_attention(out[b, h * w.G:(h + 1) * w.G], lse[b, h * w.G:(h + 1) * w.G], qg,
                            K64, V64, sel, w.kv_dtype, where=(b, h))
    # a second call right after, on a smaller input: the array still holds the
    # first call's contents
    _, ref2, got2 = _run(SMALL)
    for a, b in zip(ref2, got2):
        assert torch.equal(a.cpu(), b)
