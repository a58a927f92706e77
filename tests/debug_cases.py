"""Decode-path cases run by both the release and the bounds-checked debug
library (tests/test_gpu_debug_build.py).  Run as a module with
HST_LIBRARY=debug it writes its results and the debug check word to the npz
file named by its argument."""
import dataclasses
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as WL  # noqa: E402
from workloads.device import norm_torch_dtype, to_dev  # noqa: E402

DEV = torch.device("cuda:0")

SOFT = dataclasses.replace(WL.WORKLOADS["llama8b_softlsh_b8_n32k"], name="dbg_soft", B=3, Hq=8, Hkv=2,
                           N=7000, needles=8, ragged=(2500, 7000), seed=301)
HAM = dataclasses.replace(WL.WORKLOADS["hata_hamming_b16_n64k"], name="dbg_ham", B=2, Hq=8, Hkv=2,
                          N=5000, needles=8, seed=302)
TINY = WL.WORKLOADS["tiny_softlsh_fp32"]


def run_cases(hst):
    res = {}
    for w in (SOFT, TINY):
        x = WL.make_full(w)
        K, V, q, W = (to_dev(x[n], w.kv_dtype, DEV) for n in ("K", "V", "q", "W"))
        ragged = w.ragged is not None
        sl = torch.from_numpy(x["seq_lens"]).to(DEV) if ragged else None
        kp = torch.from_numpy(x["k_per_seq"]).to(DEV) if ragged else None
        ids, vn = hst.hst_hash_keys_softlsh(K, V, W, w.L, w.P, norm_torch_dtype(w.norm_dtype), seq_lens=sl)
        idx, out, lse = hst.hst_decode_step_softlsh(q, K, V, W, ids, vn, w.L, w.P, w.tau, w.k_max(),
                                                    seq_lens=sl, k_per_seq=kp)
        o2, l2 = hst.hst_sparse_decode_attention(q, K, V, idx, seq_lens=sl)
        res[f"{w.name}_ids"] = ids.cpu().numpy()
        res[f"{w.name}_vn"] = vn.float().cpu().numpy()
        res[f"{w.name}_idx"] = idx.cpu().numpy()
        res[f"{w.name}_out"] = out.cpu().numpy()
        res[f"{w.name}_lse"] = lse.cpu().numpy()
        res[f"{w.name}_out_given"] = o2.cpu().numpy()
        if w is SOFT:  # the routed step: index cards scored by the prepare kernel, card and token cuts
            k = w.k_max()
            C = min(256, 4 * -(-k // 64))
            cards = hst.hst_build_cards_softlsh(K, vn, W, w.L, w.P, seq_lens=sl)
            rstep = hst.DecodeSoftLSHRouted(K, w.Hq, w.L, w.P, w.tau, k, C, vn.dtype, seq_lens=sl, k_per_seq=kp)
            ridx, rout, rlse = rstep(q, K, V, W, ids, vn, cards[1], cards[2])
            res["routed_idx"] = ridx.cpu().numpy()
            res["routed_out"] = rout.cpu().numpy()
            res["routed_lse"] = rlse.cpu().numpy()
    w = HAM
    x = WL.make_full(w)
    K, V, q, R = (to_dev(x[n], w.kv_dtype, DEV) for n in ("K", "V", "q", "R"))
    codes = hst.hst_hash_keys_binary(K, R)
    idx, out, lse = hst.hst_decode_step_hamming(q, K, V, R, codes, w.k_max())
    res["ham_codes"] = codes.cpu().numpy()
    res["ham_idx"] = idx.cpu().numpy()
    res["ham_out"] = out.cpu().numpy()
    # stand-alone top-k over scores with ties
    g = torch.Generator().manual_seed(303)
    sc = torch.randint(0, 50, (2, 2, 6000), generator=g).float().to(DEV)
    res["topk"] = hst.hst_select_topk(sc, 700, 8, 128).cpu().numpy()
    torch.cuda.synchronize()
    return res


if __name__ == "__main__":
    import hash_scored_top_amd as hst
    assert hst.LIB_PATH.endswith("libhst_debug.so"), hst.LIB_PATH
    out = run_cases(hst)
    out["debug_word"] = np.array([hst.debug_status()], dtype=np.int64)
    np.savez(sys.argv[1], **out)
    print(f"[debug-build] cases done, check word {int(out['debug_word'][0])}", flush=True)
