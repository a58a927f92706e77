"""The C-ABI library loads, exports what include/hst.h declares, and rejects
invalid arguments before anything is enqueued (host logic only; no GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from hash_scored_top_amd import _lib
    return _lib


def test_header_symbols_exported():
    L = _lib()
    with open(os.path.join(ROOT, "include", "hst.h")) as f:
        text = f.read()
    declared = set(re.findall(r"\b(hst_[a-z_]+)\s*\(", text))
    assert declared, "no declarations found"
    lib = ctypes.CDLL(L.LIB_PATH)
    for name in sorted(declared):
        assert hasattr(lib, name), name
    assert declared == set(L.EXPORTED)


def _shape(L, **kw):
    base = dict(B=2, Hq=8, Hkv=2, d=128, Nmax=1024, kv_dtype=L.HST_BF16, seq_lens=None)
    base.update(kw)
    return L.HstShape(**base)


def test_status_strings_and_version():
    L = _lib()
    C = L._C
    assert C.hst_version() >= 100
    for s in (0, -1, -2, -3, -4):
        assert C.hst_status_string(s).startswith(b"HST_")
    assert C.hst_last_hip_error() == 0


@pytest.mark.parametrize("kw,want", [
    (dict(B=0), -1), (dict(Hq=7), -1), (dict(d=96), -2), (dict(kv_dtype=2), -2),
    (dict(Nmax=0), -1), (dict(Hkv=0), -1),
])
def test_workspace_size_rejects_bad_shapes(kw, want):
    L = _lib()
    out = ctypes.c_size_t(0)
    sh = _shape(L, **kw)
    st = L._C.hst_workspace_size(L.HST_OP_DECODE_SOFTLSH, ctypes.byref(sh), 64, 8, 128, 10,
                                 ctypes.byref(out))
    assert st == want


def test_workspace_sizes_monotone():
    L = _lib()
    sh = _shape(L)
    a = L.workspace_size(L.HST_OP_DECODE_SOFTLSH, sh, 64, 8, k=10)
    b = L.workspace_size(L.HST_OP_DECODE_SOFTLSH, sh, 64, 8, k=1000)
    assert 0 < a <= b
    assert L.workspace_size(L.HST_OP_HASH_SOFTLSH, sh, 64, 8) == 0
    with pytest.raises(L.HstError):
        L.workspace_size(L.HST_OP_DECODE_SOFTLSH, sh, 64, 9)   # P > 8
    with pytest.raises(L.HstError):
        L.workspace_size(L.HST_OP_SELECT_TOPK, sh, k=0)


FAKE = 1 << 20  # aligned non-null "device" address; never dereferenced on these paths


def test_entry_points_validate_before_launch():
    L = _lib()
    C = L._C
    sh = _shape(L)
    by = ctypes.byref(sh)
    # null pointers
    assert C.hst_hash_keys_softlsh(by, None, FAKE, FAKE, 64, 8, L.HST_F16, FAKE, FAKE, None) == -1
    # misaligned pointer
    assert C.hst_hash_keys_softlsh(by, FAKE + 2, FAKE, FAKE, 64, 8, L.HST_F16, FAKE, FAKE,
                                   None) == -1
    # unsupported P / norm dtype / code bits
    assert C.hst_hash_keys_softlsh(by, FAKE, FAKE, FAKE, 64, 9, L.HST_F16, FAKE, FAKE, None) == -2
    assert C.hst_hash_keys_softlsh(by, FAKE, FAKE, FAKE, 64, 8, L.HST_BF16, FAKE, FAKE, None) == -2
    assert C.hst_hash_keys_binary(by, FAKE, FAKE, 96, FAKE, None) == -2
    # tau must be positive and finite
    for tau in (0.0, -1.0, float("inf"), float("nan")):
        assert C.hst_score_keys_softlsh(by, FAKE, FAKE, 64, 8, tau, FAKE, FAKE, L.HST_F16, FAKE,
                                        FAKE, 1 << 30, None) == -1
    # workspace too small
    assert C.hst_score_keys_softlsh(by, FAKE, FAKE, 64, 8, 0.3, FAKE, FAKE, L.HST_F16, FAKE,
                                    FAKE, 16, None) == -3
    # k < 1, bad score dtype
    assert C.hst_select_topk(by, L.HST_F32, FAKE, 0, None, FAKE, FAKE, 1 << 30, None) == -1
    assert C.hst_select_topk(by, L.HST_F16, FAKE, 5, None, FAKE, FAKE, 1 << 30, None) == -2
    # attention: group too large, non-finite scale
    big = _shape(L, Hq=32, Hkv=2)
    assert C.hst_sparse_decode_attention(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, 8, 0.1, FAKE,
                                         None, FAKE, 1 << 30, None) == -2
    assert C.hst_sparse_decode_attention(by, FAKE, FAKE, FAKE, FAKE, 8, float("nan"), FAKE, None,
                                         FAKE, 1 << 30, None) == -1
    # decode step: workspace too small
    assert C.hst_decode_step_softlsh(by, FAKE, FAKE, FAKE, FAKE, 64, 8, 0.3, FAKE, FAKE,
                                     L.HST_F16, 10, None, 0.1, FAKE, FAKE, None, FAKE, 100,
                                     None) == -3
    assert C.hst_decode_step_hamming(by, FAKE, FAKE, FAKE, FAKE, 128, FAKE, 10, None, 0.1, FAKE,
                                     FAKE, None, FAKE, 100, None) == -3
    assert C.hst_last_hip_error() == 0


def test_append_entry_points_validate_before_launch():
    L = _lib()
    C = L._C
    sh = _shape(L)                              # no seq_lens: the lengths must advance
    by = ctypes.byref(sh)
    assert C.hst_append_kv_softlsh(by, FAKE, FAKE, FAKE, 16, 8, L.HST_F16, FAKE, FAKE, FAKE,
                                   FAKE, None) == -1
    assert C.hst_append_kv_binary(by, FAKE, FAKE, FAKE, 128, FAKE, FAKE, FAKE, None) == -1
    shl = _shape(L, seq_lens=FAKE)
    byl = ctypes.byref(shl)
    # L > 1024, P > 8, L < 1, bad norm dtype, misaligned or null pointers
    assert C.hst_append_kv_softlsh(byl, FAKE, FAKE, FAKE, 1025, 8, L.HST_F16, FAKE, FAKE, FAKE,
                                   FAKE, None) == -2
    assert C.hst_append_kv_softlsh(byl, FAKE, FAKE, FAKE, 16, 9, L.HST_F16, FAKE, FAKE, FAKE,
                                   FAKE, None) == -2
    assert C.hst_append_kv_softlsh(byl, FAKE, FAKE, FAKE, 0, 8, L.HST_F16, FAKE, FAKE, FAKE,
                                   FAKE, None) == -1
    assert C.hst_append_kv_softlsh(byl, FAKE, FAKE, FAKE, 16, 8, L.HST_BF16, FAKE, FAKE, FAKE,
                                   FAKE, None) == -2
    assert C.hst_append_kv_softlsh(byl, FAKE + 2, FAKE, FAKE, 16, 8, L.HST_F16, FAKE, FAKE,
                                   FAKE, FAKE, None) == -1
    assert C.hst_append_kv_binary(byl, FAKE, FAKE, FAKE, 64, FAKE, FAKE, FAKE, None) == -2
    assert C.hst_append_kv_binary(byl, FAKE, None, FAKE, 128, FAKE, FAKE, FAKE, None) == -1
    assert C.hst_last_hip_error() == 0


def test_mass_entry_points_validate_before_launch():
    L = _lib()
    C = L._C
    sh = _shape(L)
    by = ctypes.byref(sh)
    big = 1 << 30
    # p outside (0, 1], NaN, k beyond 8192, idx aliasing cand, workspace too small
    for p in (0.0, -0.5, 1.5, float("nan")):
        assert C.hst_select_mass(by, FAKE, FAKE, FAKE, 16, p, 0.1, FAKE + 256, FAKE, FAKE, big,
                                 None) == -1
    assert C.hst_select_mass(by, FAKE, FAKE, FAKE, 8193, 0.9, 0.1, FAKE + 256, FAKE, FAKE, big,
                             None) == -2
    assert C.hst_select_mass(by, FAKE, FAKE, FAKE, 16, 0.9, 0.1, FAKE, FAKE, FAKE, big,
                             None) == -1
    assert C.hst_select_mass(by, FAKE, FAKE, FAKE, 16, 0.9, 0.1, FAKE + 256, FAKE, FAKE, 16,
                             None) == -3
    need = L.workspace_size(L.HST_OP_SELECT_MASS, sh, k=100)
    assert need >= 2 * 8 * 100 * 8          # B * Hq * k float64 logits
    a = L.workspace_size(L.HST_OP_DECODE_SOFTLSH_MASS, sh, 64, 8, k=100)
    assert a > L.workspace_size(L.HST_OP_DECODE_SOFTLSH, sh, 64, 8, k=100)
    assert C.hst_decode_step_softlsh_mass(by, FAKE, FAKE, FAKE, FAKE, 64, 8, 0.3, FAKE, FAKE,
                                          L.HST_F16, 100, None, 2.0, 0.1, FAKE, FAKE, FAKE, None,
                                          FAKE, big, None) == -1
    assert C.hst_decode_step_softlsh_mass(by, FAKE, FAKE, FAKE, FAKE, 64, 8, 0.3, FAKE, FAKE,
                                          L.HST_F16, 100, None, 0.9, 0.1, FAKE, FAKE, FAKE, None,
                                          FAKE, 100, None) == -3
    assert C.hst_last_hip_error() == 0


def test_routing_entry_points_validate_before_launch():
    L = _lib()
    C = L._C
    sh = _shape(L)
    by = ctypes.byref(sh)
    big = 1 << 30
    args = lambda Lt, Cc, ws: (by, FAKE, FAKE, FAKE, FAKE, Lt, 8, 0.3, FAKE, FAKE, L.HST_F16,
                               FAKE, FAKE, Cc, 100, None, 0.1, FAKE, FAKE, None, FAKE, ws, None)
    assert C.hst_decode_step_softlsh_routed(*args(64, 0, big)) == -1      # C < 1
    assert C.hst_decode_step_softlsh_routed(*args(64, 257, big)) == -2    # C > 256
    assert C.hst_decode_step_softlsh_routed(*args(48, 8, big)) == -2      # L not 16/32/64/128
    assert C.hst_decode_step_softlsh_routed(*args(64, 8, 100)) == -3      # workspace
    need = L.workspace_size(L.HST_OP_DECODE_SOFTLSH_ROUTED, sh, 64, 8, k=100)
    assert need > 2 * 2 * 256 * 64 * 4                                    # key scores of 256 chunks
    # cards: null output, bad norm dtype, P > 8
    assert C.hst_build_cards_softlsh(by, FAKE, FAKE, L.HST_F16, FAKE, 64, 8, FAKE, FAKE, FAKE,
                                     None, None) == -1
    assert C.hst_build_cards_softlsh(by, FAKE, FAKE, L.HST_BF16, FAKE, 64, 8, FAKE, FAKE, FAKE,
                                     FAKE, None) == -2
    assert C.hst_build_cards_softlsh(by, FAKE, FAKE, L.HST_F16, FAKE, 64, 9, FAKE, FAKE, FAKE,
                                     FAKE, None) == -2
    assert C.hst_last_hip_error() == 0


def test_shared_prefix_entry_points_validate_before_launch():
    L = _lib()
    C = L._C
    sh = _shape(L)
    by = ctypes.byref(sh)
    out = ctypes.c_size_t(0)
    assert C.hst_workspace_size_shared(by, 4096, 64, 8, 100, ctypes.byref(out)) == 0
    assert out.value > 2 * 2 * (4096 + 1024) * 4          # the context scores alone
    assert C.hst_workspace_size_shared(by, -1, 64, 8, 100, ctypes.byref(out)) == -1
    assert C.hst_workspace_size_shared(by, 4096, 48, 8, 100, ctypes.byref(out)) == -2
    assert C.hst_workspace_size_shared(by, 4096, 64, 8, 0, ctypes.byref(out)) == -1
    assert C.hst_workspace_size_shared(by, 4096, 64, 8, 100, None) == -1
    call = lambda Np, ws: C.hst_decode_step_softlsh_shared(
        by, Np, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 8, 0.3,
        L.HST_F16, 100, None, 0.1, FAKE, FAKE, None, FAKE, ws, None)
    assert call(4096, 100) == -3                           # workspace too small
    assert call(1 << 30, 1 << 40) == -2                    # context too long
    assert C.hst_last_hip_error() == 0


def test_sizing_and_validation_from_many_threads():
    """The host-side calls are reentrant: workspace sizing (which reads the
    device's compute-unit count through its atomic cache on a GPU host) and
    argument validation give the same answers from several threads at once."""
    import threading
    L = _lib()
    C = L._C
    shapes = [_shape(L, B=b, Nmax=n) for b in (1, 3, 8) for n in (1000, 40000, 131072)]
    want = [L.workspace_size(L.HST_OP_DECODE_SOFTLSH, sh, 64, 8, k=100) for sh in shapes]
    errors = []

    def worker(tid):
        try:
            for rep in range(200):
                i = (tid + rep) % len(shapes)
                out = ctypes.c_size_t(0)
                st = C.hst_workspace_size(L.HST_OP_DECODE_SOFTLSH, ctypes.byref(shapes[i]), 64, 8,
                                          128, 100, ctypes.byref(out))
                assert st == 0 and out.value == want[i]
                bad = _shape(L, d=96)
                st = C.hst_workspace_size(L.HST_OP_DECODE_SOFTLSH, ctypes.byref(bad), 64, 8, 128,
                                          100, ctypes.byref(out))
                assert st == -2
                # validation before launch: a null query is rejected, nothing enqueued
                st = C.hst_decode_step_softlsh(ctypes.byref(shapes[i]), None, None, None, None, 64,
                                               8, 0.3, None, None, L.HST_F16, 100, None, 0.1, None,
                                               None, None, None, 0, None)
                assert st == -1
        except Exception as e:  # pragma: no cover - reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]


def test_noalloc_rejects_before_launch():
    """The no-allocation step validates like the workspace step, and rejects a
    shape whose workspace exceeds its fixed array with HST_ERR_WORKSPACE,
    before any device call (the pointers below are never dereferenced)."""
    L = _lib()
    C = L._C
    cap = C.hst_noalloc_scratch_bytes()
    assert cap == 64 << 20
    fake = 0x10000  # aligned, never touched: validation ends before any launch
    big = _shape(L, B=32, Hq=32, Hkv=4, Nmax=65536)
    assert L.workspace_size(L.HST_OP_DECODE_SOFTLSH, big, 64, 8, k=1311) > cap
    args = lambda sh, q: (ctypes.byref(sh), q, fake, fake, fake, 64, 8, 0.3, fake, fake, L.HST_F16,
                          1311, None, 0.088, fake, fake, fake, None)
    assert C.hst_decode_step_softlsh_noalloc(*args(big, fake)) == -3
    small = _shape(L)
    assert L.workspace_size(L.HST_OP_DECODE_SOFTLSH, small, 64, 8, k=1311) <= cap
    assert C.hst_decode_step_softlsh_noalloc(*args(small, None)) == -1
    assert C.hst_decode_step_softlsh_noalloc(*args(_shape(L, d=96), fake)) == -2
