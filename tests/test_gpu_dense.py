"""Attention over every cached key (k = N) through hst_sparse_decode_attention,
the dense reference point of the benchmark, against the oracle's attention
(SOCKET page, core mechanism, item 4, with the whole context selected).
Indices past a sequence's length are padding and are skipped."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from tests.gpu_helpers import to_dev

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def test_dense_attention_all_keys():
    import hash_scored_top_amd as hst

    print("[dense] B2 Hq8 Hkv2 d128 bf16 N65536", flush=True)
    rng = np.random.default_rng(99)
    B, Hq, Hkv, d, N = 2, 8, 2, 128, 65536
    G = Hq // Hkv
    lens = np.array([N, 50001], dtype=np.int32)
    K = WL.f32_to_bf16_bits(rng.standard_normal((B, Hkv, N, d)).astype(np.float32))
    V = WL.f32_to_bf16_bits(rng.standard_normal((B, Hkv, N, d)).astype(np.float32))
    q = WL.f32_to_bf16_bits((rng.standard_normal((B, Hq, d)) * 3).astype(np.float32))
    idx = torch.arange(N, dtype=torch.int32, device=DEV).repeat(B, Hkv, 1).contiguous()
    sl = torch.from_numpy(lens).to(DEV)
    out, lse = hst.hst_sparse_decode_attention(to_dev(q, "bf16", DEV), to_dev(K, "bf16", DEV),
                                               to_dev(V, "bf16", DEV), idx, seq_lens=sl)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    f64 = lambda a: WL.storage_to_f64(a, "bf16")
    for b in range(B):
        n = int(lens[b])
        for h in range(Hkv):
            qg = f64(q[b, h * G:(h + 1) * G])
            o_ref, l_ref = O.attend(qg, f64(K[b, h, :n]), f64(V[b, h, :n]), np.arange(n),
                                    d ** -0.5)
            assert np.abs(out[b, h * G:(h + 1) * G] - o_ref).max() <= 2e-2, (b, h)
            np.testing.assert_allclose(lse[b, h * G:(h + 1) * G], l_ref, rtol=1e-4, atol=1e-4)
