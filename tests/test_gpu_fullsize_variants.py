"""Parity of the variant steps at the sizes the benchmark times them.

* cumulative-mass step at the 128K workload (B1, 32/8 heads, k 3972 candidates,
  p = 0.9): for every slab the kept set is the oracle's selection over the
  step's candidates (the exact top-k of the GPU's hash scores), and the
  attention over it matches the oracle;
* routed step at the 128K workload (252 chunks kept): cards bit-exact on
  sampled slabs; kept chunks and selected keys equal the oracle's up to
  float32 near-ties; attention within the bf16 tolerance; and past 2048
  cards per head (140000 keys), where the card cut changes method;
* shared-prefix step on a batch of 8 sharing a 32768-key prefix with ragged
  suffixes: sampled slabs against the oracle over the concatenated context;
* 64- and 256-bit codes at the binary-code workload's shape (B16, 64K):
  codes, scores and selections bit-exact on sampled slabs.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from tests.gpu_helpers import check_attention, norm_torch_dtype, to_dev

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _accept_mass(qg, K, cand, p, scale, got):
    for pp in (p, p * (1 - 1e-12), min(1.0, p * (1 + 1e-12))):
        if np.array_equal(O.select_mass(qg, K, cand, pp, scale), got):
            return True
    return False


def _band(scores, a, b, rank):
    diff = set(np.asarray(a).tolist()) ^ set(np.asarray(b).tolist())
    if diff:
        kth = np.sort(scores)[::-1][rank - 1]
        for j in diff:
            assert abs(scores[j] - kth) <= 2e-5 * kth, (j, scores[j], kth)
    return len(diff)


@pytest.fixture(scope="module")
def longctx():
    import hash_scored_top_amd as hst
    w = WL.WORKLOADS["longctx_softlsh_b1_n128k"]
    print("[fullsize-variants] generating the 128K workload", flush=True)
    x = WL.make_full(w)
    K, V, q, Wp = (to_dev(x[n], w.kv_dtype, DEV) for n in ("K", "V", "q", "W"))
    nd = norm_torch_dtype(w.norm_dtype)
    ids, vn = hst.hst_hash_keys_softlsh(K, V, Wp, w.L, w.P, nd)
    return w, x, (K, V, q, Wp, ids, vn, nd)


def test_mass_step_at_128k(longctx):
    import hash_scored_top_amd as hst
    w, x, (K, V, q, Wp, ids, vn, nd) = longctx
    kmax, p = int(x["k_per_seq"].max()), 0.9
    print("[fullsize-variants] mass step", flush=True)
    step = hst.DecodeSoftLSHMass(K, w.Hq, w.L, w.P, w.tau, kmax, p, nd)
    idx, counts, out, lse = step(q, K, V, Wp, ids, vn)
    scores = hst.hst_score_keys_softlsh(q, Wp, w.L, w.P, w.tau, ids, vn, K)
    cand = hst.hst_select_topk(scores, kmax, w.Hq, w.d, K.dtype)
    torch.cuda.synchronize()
    idx, counts, out, lse = (t.cpu().numpy() for t in (idx, counts, out, lse))
    cand = cand.cpu().numpy()
    f64 = lambda a: WL.storage_to_f64(a, w.kv_dtype)
    G, scale = w.G, w.d ** -0.5
    for h in range(w.Hkv):
        qg = f64(x["q"][0, h * G:(h + 1) * G])
        K64, V64 = f64(x["K"][0, h]), f64(x["V"][0, h])
        c = int(counts[0, h])
        got = idx[0, h, :c]
        assert (idx[0, h, c:] == -1).all()
        want = O.select_mass(qg, K64, cand[0, h], p, scale)
        if not np.array_equal(got, want):
            assert _accept_mass(qg, K64, cand[0, h], p, scale, got), h
        o_ref, l_ref = O.attend(qg, K64, V64, got, scale)
        assert np.abs(out[0, h * G:(h + 1) * G] - o_ref).max() <= 2e-2, h
        np.testing.assert_allclose(lse[0, h * G:(h + 1) * G], l_ref, rtol=1e-4, atol=1e-4)


def test_routed_step_at_128k(longctx):
    import hash_scored_top_amd as hst
    w, x, (K, V, q, Wp, ids, vn, nd) = longctx
    kmax = int(x["k_per_seq"].max())
    C = min(256, 4 * math.ceil(kmax / 64))
    print(f"[fullsize-variants] routed step C={C}", flush=True)
    _, cids, cw, clens = hst.hst_build_cards_softlsh(K, vn, Wp, w.L, w.P)
    step = hst.DecodeSoftLSHRouted(K, w.Hq, w.L, w.P, w.tau, kmax, C, nd)
    idx, out, lse = step(q, K, V, Wp, ids, vn, cids, cw)
    # the kept chunks through the public entry points (same tables, same cut)
    Nc = cids.shape[2]
    tables = hst.hst_query_tables_softlsh(q, Wp, w.L, w.P, w.tau, K)
    carrier = torch.empty((w.B, w.Hkv, Nc, w.d), dtype=K.dtype, device=DEV)
    cscore = hst.hst_score_scan_softlsh(tables, cids, cw, carrier, w.Hq, seq_lens=clens)
    kept = hst.hst_select_topk(cscore, C, w.Hq, w.d, K.dtype, seq_lens=clens)
    torch.cuda.synchronize()
    idx, out, lse = idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()
    cids, cw = cids.cpu().numpy(), cw.cpu().numpy().astype(np.float64)
    kept = kept.cpu().numpy()
    f64 = lambda a: WL.storage_to_f64(a, w.kv_dtype)
    G = w.G
    for h in (0, w.Hkv - 1):
        qg = f64(x["q"][0, h * G:(h + 1) * G])
        K64, V64 = f64(x["K"][0, h]), f64(x["V"][0, h])
        r = O.route_slab_softlsh(qg, K64, V64, f64(x["W"][h]), w.L, w.P, w.tau, kmax, C,
                                 w.norm_dtype, w.kv_dtype)
        np.testing.assert_array_equal(cids[0, h], r["cards"][0])
        np.testing.assert_array_equal(cw[0, h], r["cards"][1])
        got = idx[0, h, :kmax]
        assert (np.diff(got) > 0).all() and (idx[0, h, kmax:] == -1).all()
        chunks = kept[0, h][kept[0, h] >= 0]
        assert np.isin(got // 64, chunks).all()
        if _band(r["chunk_scores"], chunks, r["chunks"], C) == 0:
            pos = lambda a: np.searchsorted(r["keys"], a)
            _band(r["scores"], pos(got), pos(r["idx"]), kmax)
        check_attention(out[0, h * G:(h + 1) * G], lse[0, h * G:(h + 1) * G], qg, K64, V64, got,
                        w.kv_dtype, where=h)
        if np.array_equal(got, r["idx"]):
            assert np.abs(out[0, h * G:(h + 1) * G] - r["out"]).max() <= 2e-2, h


def test_routed_step_past_2048_cards():
    # 140000 keys: 2188 cards per head, so the card cut takes the
    # count-histogram path (the register-held selection takes up to 2048)
    import dataclasses
    import hash_scored_top_amd as hst
    base = WL.WORKLOADS["longctx_softlsh_b1_n128k"]
    w = dataclasses.replace(base, name="route_many_cards", N=140000)
    x = WL.make_full(w)
    kmax = int(x["k_per_seq"].max())
    C = min(256, 4 * math.ceil(kmax / 64))
    print(f"[fullsize-variants] routed step N={w.N} C={C}", flush=True)
    K, V, q, Wp = (to_dev(x[n], w.kv_dtype, DEV) for n in ("K", "V", "q", "W"))
    nd = norm_torch_dtype(w.norm_dtype)
    ids, vn = hst.hst_hash_keys_softlsh(K, V, Wp, w.L, w.P, nd)
    _, cids, cw, clens = hst.hst_build_cards_softlsh(K, vn, Wp, w.L, w.P)
    assert cids.shape[2] > 2048
    step = hst.DecodeSoftLSHRouted(K, w.Hq, w.L, w.P, w.tau, kmax, C, nd)
    idx, out, lse = step(q, K, V, Wp, ids, vn, cids, cw)
    torch.cuda.synchronize()
    idx, out = idx.cpu().numpy(), out.cpu().numpy()
    f64 = lambda a: WL.storage_to_f64(a, w.kv_dtype)
    G = w.G
    for h in (0, w.Hkv - 1):
        qg = f64(x["q"][0, h * G:(h + 1) * G])
        K64, V64 = f64(x["K"][0, h]), f64(x["V"][0, h])
        r = O.route_slab_softlsh(qg, K64, V64, f64(x["W"][h]), w.L, w.P, w.tau, kmax, C,
                                 w.norm_dtype, w.kv_dtype)
        got = idx[0, h, :kmax]
        assert (np.diff(got) > 0).all() and (idx[0, h, kmax:] == -1).all()
        # every selected key in one of the oracle's kept chunks, up to near-ties
        # of the C-th card score
        outside = set((got // 64).tolist()) - set(np.asarray(r["chunks"]).tolist())
        kth = np.sort(r["chunk_scores"])[::-1][C - 1]
        for c in outside:
            assert abs(r["chunk_scores"][c] - kth) <= 2e-5 * kth, (h, c)
        if not outside:
            pos = lambda a: np.searchsorted(r["keys"], a)
            if _band(r["scores"], pos(got), pos(r["idx"]), kmax) == 0:
                assert np.abs(out[0, h * G:(h + 1) * G] - r["out"]).max() <= 2e-2, h


def test_shared_prefix_step_at_bench_size():
    import hash_scored_top_amd as hst
    print("[fullsize-variants] shared prefix B8 Np32768 Ns2048", flush=True)
    rng = np.random.default_rng(41)
    B, Hq, Hkv, d, Np, Ns, L, P, tau = 8, 32, 8, 128, 32768, 2048, 64, 8, 0.3
    G = Hq // Hkv
    bf = lambda a: WL.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))
    slens = rng.integers(Ns // 4, Ns + 1, B).astype(np.int32)
    kps = ((Np + slens + 32) // 33).astype(np.int32)
    kmax = int(kps.max())
    Kp, Vp = bf(rng.standard_normal((1, Hkv, Np, d))), bf(rng.standard_normal((1, Hkv, Np, d)))
    Ks, Vs = bf(rng.standard_normal((B, Hkv, Ns, d))), bf(rng.standard_normal((B, Hkv, Ns, d)))
    W, q = bf(rng.standard_normal((Hkv, L * P, d))), bf(rng.standard_normal((B, Hq, d)))
    Kpd, Vpd, Ksd, Vsd, Wd, qd = (to_dev(a, "bf16", DEV) for a in (Kp, Vp, Ks, Vs, W, q))
    sl, kp = torch.from_numpy(slens).to(DEV), torch.from_numpy(kps).to(DEV)
    ids_p, vn_p = hst.hst_hash_keys_softlsh(Kpd, Vpd, Wd, L, P, torch.float16)
    ids_s, vn_s = hst.hst_hash_keys_softlsh(Ksd, Vsd, Wd, L, P, torch.float16, seq_lens=sl)
    step = hst.DecodeSoftLSHShared(Ksd, Np, Hq, L, P, tau, kmax, torch.float16, seq_lens=sl,
                                   k_per_seq=kp)
    idx, out, lse = step(qd, Kpd, Vpd, ids_p, vn_p, Ksd, Vsd, ids_s, vn_s, Wd)
    torch.cuda.synchronize()
    idx, out, lse = idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()
    f64 = lambda a: WL.storage_to_f64(a, "bf16")
    for b, h in ((0, 0), (B - 1, Hkv - 1), (3, 5)):
        n, kb = Np + int(slens[b]), int(kps[b])
        qg = f64(q[b, h * G:(h + 1) * G])
        r = O.decode_shared_prefix_softlsh(qg, f64(Kp[0, h]), f64(Vp[0, h]),
                                           f64(Ks[b, h, :slens[b]]), f64(Vs[b, h, :slens[b]]),
                                           f64(W[h]), L, P, tau, kb, "f16")
        got = idx[b, h, :kb]
        assert (idx[b, h, kb:] == -1).all() and (np.diff(got) > 0).all() and got[-1] < n
        Kc64 = np.concatenate([f64(Kp[0, h]), f64(Ks[b, h, :slens[b]])])
        Vc64 = np.concatenate([f64(Vp[0, h]), f64(Vs[b, h, :slens[b]])])
        check_attention(out[b, h * G:(h + 1) * G], lse[b, h * G:(h + 1) * G], qg, Kc64, Vc64,
                        got, "bf16", where=(b, h))
        if _band(r["scores"], got, r["idx"], kb) == 0:
            assert np.abs(out[b, h * G:(h + 1) * G] - r["out"]).max() <= 2e-2, (b, h)


@pytest.mark.parametrize("bits", [64, 256])
def test_code_lengths_at_bench_shape(bits):
    import hash_scored_top_amd as hst
    w = WL.WORKLOADS["hata_hamming_b16_n64k"]
    print(f"[fullsize-variants] {bits}-bit codes at {w.name}", flush=True)
    x = WL.make_full(w)
    K, V, q = (to_dev(x[n], w.kv_dtype, DEV) for n in ("K", "V", "q"))
    kmax = int(x["k_per_seq"].max())
    rng = np.random.default_rng(bits)
    Rb = WL.f32_to_bf16_bits(rng.standard_normal((w.Hkv, bits, w.d)).astype(np.float32))
    Rd = to_dev(Rb, "bf16", DEV)
    codes = hst.hst_hash_keys_binary(K, Rd, code_bits=bits)
    scores = hst.hst_score_keys_hamming(q, Rd, codes, K, code_bits=bits)
    step = hst.DecodeHamming(K, w.Hq, kmax, code_bits=bits)
    idx, out, lse = step(q, K, V, Rd, codes)
    torch.cuda.synchronize()
    codes, scores = codes.cpu().numpy().view(np.uint32), scores.cpu().numpy()
    idx, out = idx.cpu().numpy(), out.cpu().numpy()
    f64 = lambda a: WL.storage_to_f64(a, w.kv_dtype)
    G = w.G
    for b, h in ((0, 0), (w.B - 1, w.Hkv - 1)):
        qg = f64(x["q"][b, h * G:(h + 1) * G])
        r = O.decode_slab_hamming(qg, f64(x["K"][b, h]), f64(x["V"][b, h]), f64(Rb[h]), kmax)
        np.testing.assert_array_equal(codes[b, h], r["kcodes"])
        np.testing.assert_array_equal(scores[b, h], r["scores"])
        np.testing.assert_array_equal(idx[b, h], r["idx"])
        assert np.abs(out[b, h * G:(h + 1) * G] - r["out"]).max() <= 2e-2, (b, h)
