"""Binary codes of 64, 128 and 256 bits (HATA page, section 3, and the
code-length trade-off of section 1) through the C ABI against the oracle.

Codes are bit-exact, including keys whose projections cancel exactly or
nearly.  Hamming scores are exact.  The decode step's selection is exact
(integer scores) and its attention lies within the bf16 / float32
tolerances.  The 128-bit codes take the fused decode path; 64 and 256 bits
take the composed one.
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
    x32 = np.asarray(x64, dtype=np.float32)
    return WL.f32_to_bf16_bits(x32) if dt == "bf16" else x32


@pytest.mark.parametrize("bits,dt,d", [(64, "bf16", 128), (256, "bf16", 128), (64, "f32", 64),
                                       (256, "f32", 64), (128, "bf16", 128)])
def test_code_lengths_match_oracle(bits, dt, d):
    import hash_scored_top_amd as hst

    print(f"[codes] {bits} bits {dt} d={d}", flush=True)
    rng = np.random.default_rng(bits + d)
    B, Hkv, G, N, k = 3, 2, 4, 3000, 50
    Hq = G * Hkv
    lens = np.array([3000, 1, 1717], dtype=np.int32)
    kps = np.array([50, 3, 17], dtype=np.int32)
    R = np.stack([cancel_case(rng, d, bits, 1)[0] for _ in range(Hkv)])
    Kraw = rng.standard_normal((B, Hkv, N, d))
    canc = cancel_case(rng, d, bits, N)[1]
    Kraw[0, 0] = canc                                 # one slab of cancelling keys
    K, V = _store(Kraw, dt), _store(rng.standard_normal((B, Hkv, N, d)), dt)
    q = _store(rng.standard_normal((B, Hq, d)), dt)
    Rs = _store(R, dt)
    Kd, Vd, qd, Rd = (to_dev(a, dt, DEV) for a in (K, V, q, Rs))
    sl, kp = torch.from_numpy(lens).to(DEV), torch.from_numpy(kps).to(DEV)
    codes = hst.hst_hash_keys_binary(Kd, Rd, code_bits=bits, seq_lens=sl)
    scores = hst.hst_score_keys_hamming(qd, Rd, codes, Kd, code_bits=bits, seq_lens=sl)
    step = hst.DecodeHamming(Kd, Hq, k, code_bits=bits, seq_lens=sl, k_per_seq=kp)
    idx, out, lse = step(qd, Kd, Vd, Rd, codes)
    torch.cuda.synchronize()
    codes = codes.cpu().numpy().view(np.uint32)
    scores, idx = scores.cpu().numpy(), idx.cpu().numpy()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    f64 = lambda a: WL.storage_to_f64(a, dt)
    for b in range(B):
        n = int(lens[b])
        for h in range(Hkv):
            qg = f64(q[b, h * G:(h + 1) * G])
            r = O.decode_slab_hamming(qg, f64(K[b, h, :n]), f64(V[b, h, :n]), f64(Rs[h]),
                                      int(kps[b]))
            np.testing.assert_array_equal(codes[b, h, :n], r["kcodes"], err_msg=f"{(b, h)}")
            np.testing.assert_array_equal(scores[b, h, :n], r["scores"])
            kk = min(int(kps[b]), n)
            np.testing.assert_array_equal(idx[b, h, :kk], r["idx"])
            assert (idx[b, h, kk:] == -1).all()
            tol = 2e-2 if dt == "bf16" else 1e-4
            assert np.abs(out[b, h * G:(h + 1) * G] - r["out"]).max() <= tol, (b, h)
            np.testing.assert_allclose(lse[b, h * G:(h + 1) * G], r["lse"], rtol=1e-4,
                                       atol=1e-4)
