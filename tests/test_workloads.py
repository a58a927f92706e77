"""The seeded synthetic workloads: determinism, shapes and planted structure."""
import math

import numpy as np

import workloads as WL


def test_k_from_sparsity():
    assert WL.WORKLOADS["llama8b_softlsh_b8_n32k"].k_max() == 993
    assert WL.WORKLOADS["longctx_softlsh_b1_n128k"].k_max() == 3972
    assert WL.WORKLOADS["hata_hamming_b16_n64k"].k_max() == 3277
    assert WL.WORKLOADS["tiny_softlsh_fp32"].k_max() == 128
    w = WL.WORKLOADS["qwen30b_ragged_softlsh_b32"]
    lens = w.seq_lens()
    assert lens.shape == (32,) and lens.min() >= 8192 and lens.max() <= 65536
    assert len(set(lens.tolist())) > 20
    np.testing.assert_array_equal(w.k_per_seq(), [math.ceil(n / 50) for n in lens])


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9],
                 dtype=np.float32)
    back = WL.bf16_bits_to_f32(WL.f32_to_bf16_bits(x))
    # 1+2^-8 is a tie between 1 and 1+2^-7: goes to even (1); 1+3*2^-8 -> 1+2^-6
    np.testing.assert_array_equal(back, [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0])


def test_slab_determinism_and_needles():
    w = WL.WORKLOADS["tiny_softlsh_fp32"]
    a = WL.make_slab(w, 0, 0)
    b = WL.make_slab(w, 0, 0)
    for key in ("K", "V", "q", "needle_pos"):
        np.testing.assert_array_equal(a[key], b[key])
    assert a["K"].shape == (4096, 64) and a["q"].shape == (4, 64)
    assert len(a["needle_pos"]) == 8 and len(set(a["needle_pos"].tolist())) == 8
    c = a["needle_center"]
    for u in a["needle_dirs"]:
        assert abs(np.dot(u, c) / np.linalg.norm(u) - 0.8) < 1e-12
    # needle keys point along their needle direction
    for i, p in enumerate(a["needle_pos"]):
        k = a["K"][p].astype(np.float64)
        cosv = np.dot(k, a["needle_dirs"][i]) / np.linalg.norm(k)
        assert cosv > 0.999999


def test_bf16_slab_and_full_layout():
    w = WL.WORKLOADS["llama8b_softlsh_b8_n32k"]
    full = WL.make_full(w, slabs=[(3, 5)])
    assert full["K"].dtype == np.uint16 and full["K"].shape == (8, 8, 32768, 128)
    s = WL.make_slab(w, 3, 5)
    np.testing.assert_array_equal(full["K"][3, 5], s["K"])
    np.testing.assert_array_equal(full["q"][3, 5 * 4:6 * 4], s["q"])
    assert not full["K"][0, 0].any()
    assert full["W"].shape == (8, 512, 128)
