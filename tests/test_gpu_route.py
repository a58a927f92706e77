"""Two-level chunk routing through the C ABI against the oracle (HGA page,
section 2).

* hst_build_cards_softlsh: card keys (bit for bit in the KV storage type),
  card bucket ids, card weights and card counts equal the oracle's, over
  ragged, one-key and exactly cancelling chunks.
* hst_decode_step_softlsh_routed, stage by stage:
  - the chunks it keeps are the exact top-C of the card scores, which the
    public scan computes from the same tables.  Against the oracle they
    differ only where card scores lie within float32 rounding of the C-th.
  - every selected key lies in a kept chunk, and the selection is the
    oracle's top-k over those chunks' keys (near-ties aside).
  - attention matches the oracle within the bf16 tolerance.
  Keeping every chunk reduces to the plain top-k step.
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


def _store(x64, dt):
    x32 = np.asarray(x64, dtype=np.float32)
    return WL.f32_to_bf16_bits(x32) if dt == "bf16" else x32


def _host(t, dt):
    if dt == "bf16":
        return t.cpu().view(torch.int16).numpy().view(np.uint16)
    return t.cpu().numpy()


@pytest.mark.parametrize("dt,d,L,P,nd", [("bf16", 128, 64, 8, "f16"), ("f32", 64, 16, 4, "f32"),
                                         ("bf16", 64, 32, 8, "f32")])
def test_cards_match_oracle(dt, d, L, P, nd):
    import hash_scored_top_amd as hst

    print(f"[cards] {dt} d={d} L={L} P={P}", flush=True)
    rng = np.random.default_rng(d + L + P)
    B, Hkv, Nmax = 3, 2, 1000
    lens = np.array([1000, 130, 1], dtype=np.int32)
    K = rng.standard_normal((B, Hkv, Nmax, d))
    K[:, :, 96:128] = -K[:, :, 64:96]           # chunk 1 of the long sequence sums to zero
    K = _store(K, dt)
    V = _store(rng.standard_normal((B, Hkv, Nmax, d)), dt)
    W = _store(rng.standard_normal((Hkv, L * P, d)), dt)
    Kd, Vd, Wd = (to_dev(a, dt, DEV) for a in (K, V, W))
    sl = torch.from_numpy(lens).to(DEV)
    ids, vn = hst.hst_hash_keys_softlsh(Kd, Vd, Wd, L, P, norm_torch_dtype(nd), seq_lens=sl)
    ckeys, cids, cw, clens = hst.hst_build_cards_softlsh(Kd, vn, Wd, L, P, seq_lens=sl)
    torch.cuda.synchronize()
    ckeys, cids = _host(ckeys, dt), cids.cpu().numpy()
    cw, clens, vnh = cw.cpu().numpy(), clens.cpu().numpy(), vn.cpu().numpy()
    np.testing.assert_array_equal(clens, (lens + 63) // 64)
    f64 = lambda a: WL.storage_to_f64(a, dt)
    for b in range(B):
        n = int(lens[b])
        nc = (n + 63) // 64
        for h in range(Hkv):
            keys = O.chunk_card_keys(f64(K[b, h, :n]), dt)
            np.testing.assert_array_equal(f64(ckeys[b, h, :nc]), keys)
            cid, cwt = O.chunk_cards_softlsh(f64(K[b, h, :n]), vnh[b, h, :n].astype(np.float64),
                                             f64(W[h]), L, P, dt)
            np.testing.assert_array_equal(cids[b, h, :nc], cid)
            np.testing.assert_array_equal(cw[b, h, :nc].astype(np.float64), cwt)
    assert (cids[0, :, 1] == (1 << P) - 1).all()


def _band(scores, chosen_a, chosen_b, kth_rank):
    """Items in exactly one of two selections must score within float32
    rounding of the selection boundary."""
    diff = set(np.asarray(chosen_a).tolist()) ^ set(np.asarray(chosen_b).tolist())
    if not diff:
        return 0
    kth = np.sort(scores)[::-1][kth_rank - 1]
    for j in diff:
        assert abs(scores[j] - kth) <= 2e-5 * kth, (j, scores[j], kth)
    return len(diff)


@pytest.mark.parametrize("C", [8, 64])
def test_routed_step_matches_oracle_stage_by_stage(C):
    import hash_scored_top_amd as hst

    base = WL.WORKLOADS["llama8b_softlsh_b8_n32k"]
    w = dataclasses.replace(base, name="route_small", B=2, N=4096, ragged=(2500, 4096))
    print(f"[route] {w.name} C={C}", flush=True)
    x = WL.make_full(w)
    lens, ks = x["seq_lens"], x["k_per_seq"]
    kmax = int(ks.max())
    K, V, q, Wp = (to_dev(x[n], w.kv_dtype, DEV) for n in ("K", "V", "q", "W"))
    sl = torch.from_numpy(lens).to(DEV)
    kp = torch.from_numpy(ks).to(DEV)
    nd = norm_torch_dtype(w.norm_dtype)
    ids, vn = hst.hst_hash_keys_softlsh(K, V, Wp, w.L, w.P, nd, seq_lens=sl)
    _, cids, cw, clens = hst.hst_build_cards_softlsh(K, vn, Wp, w.L, w.P, seq_lens=sl)
    step = hst.DecodeSoftLSHRouted(K, w.Hq, w.L, w.P, w.tau, kmax, C, nd, seq_lens=sl,
                                   k_per_seq=kp)
    idx, out, lse = step(q, K, V, Wp, ids, vn, cids, cw)
    # the card scores and the kept chunks through the public entry points
    Nc = cids.shape[2]
    tables = hst.hst_query_tables_softlsh(q, Wp, w.L, w.P, w.tau, K, seq_lens=sl)
    cdummy = torch.empty((w.B, w.Hkv, Nc, w.d), dtype=K.dtype, device=DEV)  # shape carrier
    cscore = hst.hst_score_scan_softlsh(tables, cids, cw, cdummy, w.Hq, seq_lens=clens)
    kept = hst.hst_select_topk(cscore, C, w.Hq, w.d, K.dtype, seq_lens=clens)
    plain = hst.DecodeSoftLSH(K, w.Hq, w.L, w.P, w.tau, kmax, nd, seq_lens=sl, k_per_seq=kp)
    pidx, _, _ = plain(q, K, V, Wp, ids, vn)
    torch.cuda.synchronize()
    idx, out, lse, kept = idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy(), kept.cpu().numpy()
    pidx = pidx.cpu().numpy()
    f64 = lambda a: WL.storage_to_f64(a, w.kv_dtype)
    G = w.G
    for b in range(w.B):
        n, kb = int(lens[b]), int(ks[b])
        nc = (n + 63) // 64
        for h in range(w.Hkv):
            qg = f64(x["q"][b, h * G:(h + 1) * G])
            K64, V64 = f64(x["K"][b, h, :n]), f64(x["V"][b, h, :n])
            r = O.route_slab_softlsh(qg, K64, V64, f64(x["W"][h]), w.L, w.P, w.tau, kb, C,
                                     w.norm_dtype, w.kv_dtype)
            chunks = kept[b, h][kept[b, h] >= 0]
            assert chunks.size == min(C, nc)
            _band(r["chunk_scores"], chunks, r["chunks"], min(C, nc))
            keys = np.concatenate([np.arange(c * 64, min(n, c * 64 + 64)) for c in chunks])
            kk = min(kb, keys.size)
            got = idx[b, h, :kk]
            assert (idx[b, h, kk:] == -1).all() and (np.diff(got) > 0).all()
            assert np.isin(got, keys).all()
            # token routing inside the kept chunks, with the oracle's scores
            T = r["T"]
            ids64 = O.hash_keys_softlsh(K64, f64(x["W"][h]), w.L, w.P)
            vn64 = O.value_norms(V64, w.norm_dtype)
            s_keys = O.score_softlsh(T, ids64[keys], vn64[keys])
            want = keys[O.select_topk(s_keys, kb)]
            pos = {j: i for i, j in enumerate(keys)}
            _band(s_keys, [pos[j] for j in got], [pos[j] for j in want], kk)
            if C >= nc:   # every chunk kept: the plain top-k step
                _band(s_keys, got, pidx[b, h, :kk], kk)
            # attention over the GPU's own selection, on every slab
            check_attention(out[b, h * G:(h + 1) * G], lse[b, h * G:(h + 1) * G], qg, K64, V64,
                            got, w.kv_dtype, where=(b, h))
