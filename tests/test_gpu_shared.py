"""Shared-prefix decode through the C ABI (bifurcated-attention page,
sections 1 and 3) against the oracle's step over the concatenated context
and against the plain GPU step on a materialised concatenation.

The prefix spans two scan tiles plus a ragged tail.  Suffixes are ragged,
one key long and empty.  Selections may differ from the oracle's only at
keys whose scores lie within float32 rounding of the k-th.  Where the
selection matches, attention is within the bf16 / float32 tolerances.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from tests.gpu_helpers import norm_torch_dtype, to_dev

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _store(x64, dt):
    x32 = np.asarray(x64, dtype=np.float32)
    return WL.f32_to_bf16_bits(x32) if dt == "bf16" else x32


@pytest.mark.parametrize("dt,d,L,P,nd,G", [("bf16", 128, 64, 8, "f16", 4),
                                           ("f32", 64, 16, 4, "f32", 2)])
def test_shared_prefix_step_matches_oracle(dt, d, L, P, nd, G):
    import hash_scored_top_amd as hst

    print(f"[shared] {dt} d={d} L={L} P={P} G={G}", flush=True)
    rng = np.random.default_rng(d + L)
    B, Hkv, Np, Ns, k, tau = 4, 2, 9000, 700, 64, 0.3
    Hq = G * Hkv
    slens = np.array([700, 1, 350, 0], dtype=np.int32)
    kps = np.array([64, 5, 40, 64], dtype=np.int32)
    Kp = _store(rng.standard_normal((1, Hkv, Np, d)), dt)
    Vp = _store(rng.standard_normal((1, Hkv, Np, d)), dt)
    Ks = _store(rng.standard_normal((B, Hkv, Ns, d)), dt)
    Vs = _store(rng.standard_normal((B, Hkv, Ns, d)), dt)
    W = _store(rng.standard_normal((Hkv, L * P, d)), dt)
    q = _store(rng.standard_normal((B, Hq, d)) * 2.0, dt)
    Kpd, Vpd, Ksd, Vsd, Wd, qd = (to_dev(a, dt, DEV) for a in (Kp, Vp, Ks, Vs, W, q))
    sl = torch.from_numpy(slens).to(DEV)
    kp = torch.from_numpy(kps).to(DEV)
    ntd = norm_torch_dtype(nd)
    ids_p, vn_p = hst.hst_hash_keys_softlsh(Kpd, Vpd, Wd, L, P, ntd)
    ids_s, vn_s = hst.hst_hash_keys_softlsh(Ksd, Vsd, Wd, L, P, ntd, seq_lens=sl)
    step = hst.DecodeSoftLSHShared(Ksd, Np, Hq, L, P, tau, k, ntd, seq_lens=sl, k_per_seq=kp)
    idx, out, lse = step(qd, Kpd, Vpd, ids_p, vn_p, Ksd, Vsd, ids_s, vn_s, Wd)
    # the plain step on the materialised concatenation
    Kc = torch.cat([Kpd.expand(B, -1, -1, -1), Ksd], dim=2).contiguous()
    Vc = torch.cat([Vpd.expand(B, -1, -1, -1), Vsd], dim=2).contiguous()
    cl = torch.from_numpy(Np + slens).to(DEV)
    ids_c, vn_c = hst.hst_hash_keys_softlsh(Kc, Vc, Wd, L, P, ntd, seq_lens=cl)
    plain = hst.DecodeSoftLSH(Kc, Hq, L, P, tau, k, ntd, seq_lens=cl, k_per_seq=kp)
    pidx, pout, _ = plain(qd, Kc, Vc, Wd, ids_c, vn_c)
    torch.cuda.synchronize()
    idx, out, lse = idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()
    pidx, pout = pidx.cpu().numpy(), pout.cpu().numpy()
    f64 = lambda a: WL.storage_to_f64(a, dt)
    from tests.gpu_helpers import check_attention
    for b in range(B):
        n = Np + int(slens[b])
        kb = min(int(kps[b]), n)
        for h in range(Hkv):
            qg = f64(q[b, h * G:(h + 1) * G])
            r = O.decode_shared_prefix_softlsh(qg, f64(Kp[0, h]), f64(Vp[0, h]),
                                               f64(Ks[b, h, :slens[b]]), f64(Vs[b, h, :slens[b]]),
                                               f64(W[h]), L, P, tau, int(kps[b]), nd)
            got = idx[b, h, :kb]
            assert (idx[b, h, kb:] == -1).all() and (np.diff(got) > 0).all(), (b, h)
            assert got[0] >= 0 and got[-1] < n
            kth = np.sort(r["scores"])[::-1][kb - 1]
            for ref in (r["idx"], pidx[b, h, :kb]):
                for j in set(got.tolist()) ^ set(np.asarray(ref).tolist()):
                    assert abs(r["scores"][j] - kth) <= 2e-5 * kth, (b, h, j)
            # attention over the GPU's own selection, on every slab
            Kc64 = np.concatenate([f64(Kp[0, h]), f64(Ks[b, h, :slens[b]])])
            Vc64 = np.concatenate([f64(Vp[0, h]), f64(Vs[b, h, :slens[b]])])
            check_attention(out[b, h * G:(h + 1) * G], lse[b, h * G:(h + 1) * G], qg, Kc64, Vc64,
                            got, dt, where=(b, h))
            if np.array_equal(got, pidx[b, h, :kb]):
                np.testing.assert_allclose(out[b, h * G:(h + 1) * G], pout[b, h * G:(h + 1) * G],
                                           rtol=1e-5, atol=1e-5)
