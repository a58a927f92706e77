"""Decode-time append with incremental hashing, through the C ABI, against the
oracle's append (SOCKET page, core mechanism, item 1; HATA page, section 3).

* Several appends in a row over ragged, empty, negative-length and full
  sequences: K/V rows, bucket ids, value norms, binary codes and lengths equal
  the oracle's bit for bit, and every other row is left as it was.  Keys mix
  Gaussian rows with rows whose projections cancel exactly or nearly.
* After appending, the metadata equals the prefill hashing of the final cache,
  and a decode step over it matches the oracle.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from tests.gpu_helpers import cancel_case, to_dev

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _store(x64, dt):
    """float64 values -> storage array (float32, or bf16 bits) after rounding."""
    x32 = np.asarray(x64, dtype=np.float32)
    return WL.f32_to_bf16_bits(x32) if dt == "bf16" else x32


def _keys(rng, d, nplanes, shape, dt):
    """Gaussian keys with one in two replaced by a cancellation row."""
    n = int(np.prod(shape))
    g = rng.standard_normal((n, d))
    c = cancel_case(rng, d, nplanes, n)[1]
    pick = rng.random(n) < 0.5
    g[pick] = c[pick]
    return _store(g.reshape(*shape, d), dt)


CASES = [
    ("softlsh", "bf16", 128, 16, 8, "f16"),
    ("softlsh", "f32", 64, 128, 8, "f32"),
    ("softlsh", "bf16", 64, 7, 3, "f32"),
    ("softlsh", "bf16", 128, 301, 5, "f16"),  # 26 groups of 12 tables, the last one short
    ("hamming", "bf16", 128, 0, 0, None),
    ("hamming", "f32", 64, 0, 0, None),
]


@pytest.mark.parametrize("scheme,dt,d,L,P,nd", CASES)
def test_append_matches_oracle(scheme, dt, d, L, P, nd):
    import hash_scored_top_amd as hst

    print(f"[append] {scheme} {dt} d={d} L={L} P={P}", flush=True)
    rng = np.random.default_rng(d + 7 * L + P)
    B, Hkv, Nmax, steps = 5, 2, 24, 4
    lens0 = np.array([-1, 0, 11, 22, 24], dtype=np.int32)
    nplanes = L * P if scheme == "softlsh" else 128
    K = _store(rng.standard_normal((B, Hkv, Nmax, d)), dt)
    V = _store(rng.standard_normal((B, Hkv, Nmax, d)), dt)
    planes = np.stack([cancel_case(rng, d, nplanes, 1)[0] for _ in range(Hkv)])
    Wst = _store(planes, dt)
    toks = [(_keys(rng, d, nplanes, (B, Hkv), dt), _store(rng.standard_normal((B, Hkv, d)), dt))
            for _ in range(steps)]
    f64 = lambda a: WL.storage_to_f64(a, dt)

    Kd, Vd, Wd = to_dev(K, dt, DEV), to_dev(V, dt, DEV), to_dev(Wst, dt, DEV)
    sl = torch.from_numpy(lens0.copy()).to(DEV)
    K64, V64, lens = f64(K), f64(V), lens0.astype(np.int64)
    if scheme == "softlsh":
        ids0 = rng.integers(0, 1 << P, (B, Hkv, Nmax, L)).astype(np.uint8)
        vn0 = rng.random((B, Hkv, Nmax)).astype(np.float16 if nd == "f16" else np.float32)
        idsd, vnd = torch.from_numpy(ids0.copy()).to(DEV), torch.from_numpy(vn0.copy()).to(DEV)
        ids64, vn64 = ids0.copy(), vn0.astype(np.float64)
    else:
        c0 = rng.integers(-2**31, 2**31, (B, Hkv, Nmax, 4), dtype=np.int64).astype(np.int32)
        cd = torch.from_numpy(c0.copy()).to(DEV)
        c64 = c0.view(np.uint32).copy()
    for kn, vn in toks:
        knd, vnd_ = to_dev(kn, dt, DEV), to_dev(vn, dt, DEV)
        if scheme == "softlsh":
            hst.hst_append_kv_softlsh(knd, vnd_, Wd, L, P, Kd, Vd, idsd, vnd, sl)
            O.append_tokens(K64, V64, lens, f64(kn), f64(vn), W=f64(Wst), L=L, P=P,
                            norm_dtype=nd, ids=ids64, vnorm=vn64)
        else:
            hst.hst_append_kv_binary(knd, vnd_, Wd, Kd, Vd, cd, sl)
            O.append_tokens(K64, V64, lens, f64(kn), f64(vn), R=f64(Wst), codes=c64)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sl.cpu().numpy(), lens)
    np.testing.assert_array_equal(lens, [4, 4, 15, 24, 24])
    to_np = lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16) if dt == "bf16" \
        else t.cpu().numpy()
    np.testing.assert_array_equal(f64(to_np(Kd)), K64)
    np.testing.assert_array_equal(f64(to_np(Vd)), V64)
    if scheme == "softlsh":
        np.testing.assert_array_equal(idsd.cpu().numpy(), ids64)
        np.testing.assert_array_equal(vnd.cpu().numpy().astype(np.float64), vn64)
    else:
        np.testing.assert_array_equal(cd.cpu().numpy().view(np.uint32), c64)


@pytest.mark.parametrize("scheme", ["softlsh", "hamming"])
def test_append_then_decode(scheme):
    import hash_scored_top_amd as hst

    print(f"[append-decode] {scheme}", flush=True)
    rng = np.random.default_rng(3 if scheme == "softlsh" else 4)
    dt, d, Hq, Hkv, B, Nmax, k = "bf16", 128, 8, 2, 3, 300, 32
    L, P, tau, nd = 16, 8, 0.3, "f16"
    G = Hq // Hkv
    lens0 = np.array([5, 150, 297], dtype=np.int32)
    K = _store(rng.standard_normal((B, Hkv, Nmax, d)), dt)
    V = _store(rng.standard_normal((B, Hkv, Nmax, d)), dt)
    planes = _store(rng.standard_normal((Hkv, L * P if scheme == "softlsh" else 128, d)), dt)
    q = _store(rng.standard_normal((B, Hq, d)), dt)
    Kd, Vd, Wd, qd = (to_dev(a, dt, DEV) for a in (K, V, planes, q))
    sl = torch.from_numpy(lens0.copy()).to(DEV)
    if scheme == "softlsh":
        ids, vn = hst.hst_hash_keys_softlsh(Kd, Vd, Wd, L, P, torch.float16, seq_lens=sl)
    else:
        codes = hst.hst_hash_keys_binary(Kd, Wd, seq_lens=sl)
    for _ in range(4):
        kn = to_dev(_store(rng.standard_normal((B, Hkv, d)), dt), dt, DEV)
        vv = to_dev(_store(rng.standard_normal((B, Hkv, d)), dt), dt, DEV)
        if scheme == "softlsh":
            hst.hst_append_kv_softlsh(kn, vv, Wd, L, P, Kd, Vd, ids, vn, sl)
        else:
            hst.hst_append_kv_binary(kn, vv, Wd, Kd, Vd, codes, sl)
    torch.cuda.synchronize()
    lens = sl.cpu().numpy()
    np.testing.assert_array_equal(lens, [9, 154, 300])

    # the appended metadata equals hashing the final cache from scratch
    if scheme == "softlsh":
        ids2, vn2 = hst.hst_hash_keys_softlsh(Kd, Vd, Wd, L, P, torch.float16, seq_lens=sl)
        step = hst.DecodeSoftLSH(Kd, Hq, L, P, tau, k, torch.float16, seq_lens=sl)
        idx, out, lse = step(qd, Kd, Vd, Wd, ids, vn)
        meta = (ids.cpu().numpy(), vn.cpu().numpy().astype(np.float64))
        fresh = (ids2.cpu().numpy(), vn2.cpu().numpy().astype(np.float64))
    else:
        codes2 = hst.hst_hash_keys_binary(Kd, Wd, seq_lens=sl)
        step = hst.DecodeHamming(Kd, Hq, k, seq_lens=sl)
        idx, out, lse = step(qd, Kd, Vd, Wd, codes)
        meta = (codes.cpu().numpy(),)
        fresh = (codes2.cpu().numpy(),)
    torch.cuda.synchronize()
    for b in range(B):
        for a, f in zip(meta, fresh):
            np.testing.assert_array_equal(a[b, :, :lens[b]], f[b, :, :lens[b]])
    idx, out, lse = idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()
    Kf = WL.storage_to_f64(Kd.cpu().view(torch.int16).numpy().view(np.uint16), dt)
    Vf = WL.storage_to_f64(Vd.cpu().view(torch.int16).numpy().view(np.uint16), dt)
    q64, W64 = WL.storage_to_f64(q, dt), WL.storage_to_f64(planes, dt)
    for b in range(B):
        n = int(lens[b])
        for h in range(Hkv):
            qg = q64[b, h * G:(h + 1) * G]
            if scheme == "softlsh":
                r = O.decode_slab_softlsh(qg, Kf[b, h, :n], Vf[b, h, :n], W64[h], L, P, tau, k, nd)
                np.testing.assert_array_equal(meta[0][b, h, :n], r["ids"])
                np.testing.assert_array_equal(meta[1][b, h, :n], r["vnorm"])
            else:
                r = O.decode_slab_hamming(qg, Kf[b, h, :n], Vf[b, h, :n], W64[h], k)
                np.testing.assert_array_equal(meta[0][b, h, :n].view(np.uint32), r["kcodes"])
            kk = min(k, n)
            got = idx[b, h, :kk]
            assert (idx[b, h, kk:] == -1).all()
            diff = set(got.tolist()) ^ set(r["idx"].tolist())
            if scheme == "hamming":
                assert not diff, (b, h)
            if diff:   # only keys within the float32 rounding band of the k-th score
                kth = np.sort(r["scores"])[::-1][k - 1]
                for j in diff:
                    assert abs(r["scores"][j] - kth) <= 2e-5 * kth, (b, h, j)
            # attention over the GPU's own selection, on every slab
            from tests.gpu_helpers import check_attention
            check_attention(out[b, h * G:(h + 1) * G], lse[b, h * G:(h + 1) * G], qg,
                            Kf[b, h, :n], Vf[b, h, :n], got, dt, where=(b, h))
            if not diff:
                assert np.abs(out[b, h * G:(h + 1) * G] - r["out"]).max() <= 2e-2, (b, h)
