"""Device plumbing and shared input builders for the GPU tests."""
import numpy as np

import workloads as WL
from workloads.device import norm_torch_dtype, norms_to_dev, to_dev  # noqa: F401


def cancel_case(rng, d, nplanes, n):
    """bf16-exact planes and keys whose projections are often exactly zero or
    a tiny residue of large cancelling terms (the float32 sum of such a
    projection can have either sign)."""
    h = d // 2

    def bf(x):  # round to bf16 (values are chosen representable or close)
        return WL.bf16_bits_to_f32(WL.f32_to_bf16_bits(np.asarray(x, np.float32)))

    W = bf(rng.standard_normal((nplanes, d)) * 2.0 ** rng.integers(-2, 3, (nplanes, 1)))
    dup = rng.random(nplanes) < 0.5          # planes with w[c + d/2] = w[c]
    W[dup, h:] = W[dup, :h]
    big = dup & (rng.random(nplanes) < 0.5)  # large entries, one tiny one
    W[big, :] = bf(np.sign(W[big, :]) * 2.0 ** 10)
    W[big, h - 1] = W[big, d - 1] = 2.0 ** -6
    K = bf(rng.standard_normal((n, d)))
    kind = rng.integers(0, 5, n)
    anti = kind >= 2                         # k[c + d/2] = -k[c]: zero on duplicated planes
    K[anti, h:] = -K[anti, :h]
    K[kind == 1] = 0.0
    huge = kind == 3                         # large cancelling products
    K[huge] = bf(np.sign(K[huge]) * 2.0 ** 10)
    K[huge, h:] = -K[huge, :h]
    pert = kind == 4                         # antisymmetric but one channel nudged by an ulp
    K[pert, d - 1] = bf(K[pert, d - 1] * (1.0 + 2.0 ** -7))
    return W.astype(np.float32), K.astype(np.float32)


def check_attention(out_g, lse_g, qg, K64, V64, sel, kv_dtype, scale=None, where=""):
    """The GPU's attention rows (out_g [G, d], lse_g [G] or None) against the
    oracle's exact attention over the GPU's own selected set `sel` (context
    indices of K64/V64): 1e-5 of the output scale for fp32 K/V, 2e-2 absolute
    for bf16; the log-sum-exp within 1e-4.  Used on every checked slab, so a
    selection that differs from the oracle's at a near-tie still has its
    attention checked."""
    import math
    import oracle as O
    if scale is None:
        scale = 1.0 / math.sqrt(K64.shape[1])
    ro, rl = O.attend(qg, K64, V64, np.asarray(sel, dtype=np.int64), scale)
    if kv_dtype == "f32":
        tol = 1e-5 * max(np.abs(ro).max(), 1e-30)
    else:
        tol = 2e-2
    err = np.abs(np.asarray(out_g, dtype=np.float64) - ro).max()
    assert err <= tol, (where, "out", err, tol)
    if lse_g is not None:
        np.testing.assert_allclose(np.asarray(lse_g, dtype=np.float64), rl, rtol=1e-4, atol=1e-4,
                                   err_msg=f"{where} lse")
