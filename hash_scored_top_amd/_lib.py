"""ctypes binding of libhst (the C ABI declared in include/hst.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libhst.so.  PyTorch supplies device memory (outputs and
workspace) and the current stream.  If the library is missing this module
raises at import time; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# HST_LIBRARY=debug loads the bounds-checked debug build (libhst_debug.so)
LIB_PATH = os.path.join(_PKG, "libhst_debug.so" if os.environ.get("HST_LIBRARY") == "debug" else "libhst.so")

HST_OK, HST_ERR_INVALID_ARG, HST_ERR_UNSUPPORTED, HST_ERR_WORKSPACE, HST_ERR_HIP = 0, -1, -2, -3, -4
HST_F32, HST_BF16, HST_F16, HST_I32 = 0, 1, 2, 3
(HST_OP_HASH_SOFTLSH, HST_OP_HASH_BINARY, HST_OP_SCORE_SOFTLSH, HST_OP_SCORE_HAMMING,
 HST_OP_SELECT_TOPK, HST_OP_SPARSE_ATTENTION, HST_OP_DECODE_SOFTLSH,
 HST_OP_DECODE_HAMMING, HST_OP_SELECT_MASS, HST_OP_DECODE_SOFTLSH_MASS,
 HST_OP_DECODE_SOFTLSH_ROUTED) = range(11)
CHUNK = 64  # tokens per routing chunk

EXPORTED = (
    "hst_version", "hst_status_string", "hst_last_hip_error", "hst_debug_status", "hst_workspace_size",
    "hst_hash_keys_softlsh", "hst_hash_keys_binary", "hst_score_keys_softlsh",
    "hst_score_keys_hamming", "hst_select_topk", "hst_sparse_decode_attention",
    "hst_decode_step_softlsh", "hst_decode_step_hamming", "hst_query_tables_softlsh",
    "hst_score_scan_softlsh", "hst_append_kv_softlsh", "hst_append_kv_binary",
    "hst_select_mass", "hst_decode_step_softlsh_mass", "hst_build_cards_softlsh",
    "hst_decode_step_softlsh_routed", "hst_decode_step_softlsh_shared", "hst_workspace_size_shared",
    "hst_noalloc_scratch_bytes", "hst_decode_step_softlsh_noalloc",
    "hst_decode_prepare_softlsh", "hst_decode_filter_softlsh", "hst_decode_finish_softlsh",
    "hst_decode_prepare_hamming", "hst_decode_filter_hamming", "hst_decode_finish_hamming",
    "hst_decode_candidates",
)


class HstShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("Nmax", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("seq_lens", ctypes.c_void_p)]


class HstError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _C.hst_status_string(status).decode()
        if status == HST_ERR_HIP:
            msg += f" (hipError {_C.hst_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, D, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_double, ctypes.c_size_t
    SH = ctypes.POINTER(HstShape)
    sig = {
        "hst_version": ([], I),
        "hst_status_string": ([I], ctypes.c_char_p),
        "hst_last_hip_error": ([], I),
        "hst_debug_status": ([ctypes.POINTER(ctypes.c_uint32)], I),
        "hst_workspace_size": ([I, SH, I, I, I, I, ctypes.POINTER(SZ)], I),
        "hst_hash_keys_softlsh": ([SH, P, P, P, I, I, I, P, P, P], I),
        "hst_hash_keys_binary": ([SH, P, P, I, P, P], I),
        "hst_append_kv_softlsh": ([SH, P, P, P, I, I, I, P, P, P, P, P], I),
        "hst_append_kv_binary": ([SH, P, P, P, I, P, P, P, P], I),
        "hst_score_keys_softlsh": ([SH, P, P, I, I, D, P, P, I, P, P, SZ, P], I),
        "hst_score_keys_hamming": ([SH, P, P, I, P, P, P, SZ, P], I),
        "hst_query_tables_softlsh": ([SH, P, P, I, I, D, P, P], I),
        "hst_score_scan_softlsh": ([SH, P, I, I, P, P, I, P, P], I),
        "hst_select_topk": ([SH, I, P, I, P, P, P, SZ, P], I),
        "hst_sparse_decode_attention": ([SH, P, P, P, P, I, F, P, P, P, SZ, P], I),
        "hst_decode_step_softlsh": ([SH, P, P, P, P, I, I, D, P, P, I, I, P, F, P, P, P, P, SZ, P], I),
        "hst_decode_step_hamming": ([SH, P, P, P, P, I, P, I, P, F, P, P, P, P, SZ, P], I),
        "hst_select_mass": ([SH, P, P, P, I, D, F, P, P, P, SZ, P], I),
        "hst_build_cards_softlsh": ([SH, P, P, I, P, I, I, P, P, P, P, P], I),
        "hst_decode_step_softlsh_shared": ([SH, I, P, P, P, P, P, P, P, P, P, P, I, I, D, I, I, P,
                                            F, P, P, P, P, SZ, P], I),
        "hst_workspace_size_shared": ([SH, I, I, I, I, ctypes.POINTER(SZ)], I),
        "hst_decode_step_softlsh_routed": ([SH, P, P, P, P, I, I, D, P, P, I, P, P, I, I, P, F, P,
                                            P, P, P, SZ, P], I),
        "hst_decode_step_softlsh_mass": ([SH, P, P, P, P, I, I, D, P, P, I, I, P, D, F, P, P, P,
                                          P, P, SZ, P], I),
        "hst_noalloc_scratch_bytes": ([], SZ),
        "hst_decode_prepare_softlsh": ([SH, P, P, I, I, D, P, P, I, I, P, P, SZ, P], I),
        "hst_decode_filter_softlsh": ([SH, I, I, P, P, I, I, P, P, SZ, P], I),
        "hst_decode_finish_softlsh": ([SH, P, P, P, I, I, P, P, I, I, F, P, P, P, P, SZ, P], I),
        "hst_decode_prepare_hamming": ([SH, P, P, P, I, P, P, SZ, P], I),
        "hst_decode_filter_hamming": ([SH, P, I, P, P, SZ, P], I),
        "hst_decode_finish_hamming": ([SH, P, P, P, P, I, F, P, P, P, P, SZ, P], I),
        "hst_decode_candidates": ([SH, I, I, I, I, P, SZ, I, P, P, P, P, P], I),
        "hst_decode_step_softlsh_noalloc": ([SH, P, P, P, P, I, I, D, P, P, I, I, P, F, P, P, P, P],
                                            I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_C = _load()


# --------------------------------------------------------------------- helpers

def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libhst must be contiguous")
    return t.data_ptr()


def _stream(device: torch.device) -> Optional[int]:
    if device.type != "cuda":
        return None
    return torch.cuda.current_stream(device).cuda_stream


def _kv_code(dtype: torch.dtype) -> int:
    if dtype == torch.float32:
        return HST_F32
    if dtype == torch.bfloat16:
        return HST_BF16
    raise ValueError(f"unsupported K/V dtype {dtype}")


def _norm_code(dtype: torch.dtype) -> int:
    if dtype == torch.float16:
        return HST_F16
    if dtype == torch.float32:
        return HST_F32
    raise ValueError(f"unsupported value-norm dtype {dtype}")


def make_shape(K: torch.Tensor, Hq: int, seq_lens: Optional[torch.Tensor] = None) -> HstShape:
    """Shape descriptor from a [B, Hkv, Nmax, d] key cache."""
    B, Hkv, Nmax, d = K.shape
    if seq_lens is not None and seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be int32")
    return HstShape(B, Hq, Hkv, d, Nmax, _kv_code(K.dtype), _ptr(seq_lens))


def _check(status: int, where: str) -> None:
    if status != HST_OK:
        raise HstError(status, where)


def debug_status() -> int:
    """The first failed bounds check since the last call (0: none), from the
    debug build (HST_LIBRARY=debug); synchronises the device.  Raises
    HstError(HST_ERR_UNSUPPORTED) with the release library."""
    code = ctypes.c_uint32(0)
    _check(_C.hst_debug_status(ctypes.byref(code)), "hst_debug_status")
    return int(code.value)


def workspace_size(op: int, shape: HstShape, L: int = 0, P: int = 0, code_bits: int = 128,
                   k: int = 1) -> int:
    out = ctypes.c_size_t(0)
    _check(_C.hst_workspace_size(op, ctypes.byref(shape), L, P, code_bits, k, ctypes.byref(out)),
           "hst_workspace_size")
    return out.value


def _workspace(nbytes: int, device: torch.device) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


# --------------------------------------------------------------------- entry points

def hst_hash_keys_softlsh(K, V, W, L: int, P: int, norm_dtype=torch.float16,
                          seq_lens=None, ids=None, vnorm=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Bucket ids [B,Hkv,Nmax,L] uint8 and value norms [B,Hkv,Nmax].

    ``ids`` / ``vnorm`` may be passed in (rows past N_b are left as they are);
    new ones start zeroed."""
    B, Hkv, Nmax, d = K.shape
    shape = make_shape(K, Hkv, seq_lens)
    if ids is None:
        ids = torch.zeros((B, Hkv, Nmax, L), dtype=torch.uint8, device=K.device)
    if vnorm is None:
        vnorm = torch.zeros((B, Hkv, Nmax), dtype=norm_dtype, device=K.device)
    if ids.shape != (B, Hkv, Nmax, L) or ids.dtype != torch.uint8 or vnorm.dtype != norm_dtype:
        raise ValueError("ids / vnorm do not match the shape and dtypes")
    _check(_C.hst_hash_keys_softlsh(ctypes.byref(shape), _ptr(K), _ptr(V), _ptr(W), L, P,
                                    _norm_code(norm_dtype), _ptr(ids), _ptr(vnorm),
                                    _stream(K.device)), "hst_hash_keys_softlsh")
    return ids, vnorm


def hst_hash_keys_binary(K, R, code_bits: int = 128, seq_lens=None, codes=None) -> torch.Tensor:
    """Binary codes [B,Hkv,Nmax,code_bits/32] int32 (uint32 bit patterns).

    ``codes`` may be passed in (rows past N_b are left as they are)."""
    B, Hkv, Nmax, d = K.shape
    shape = make_shape(K, Hkv, seq_lens)
    if codes is None:
        codes = torch.zeros((B, Hkv, Nmax, code_bits // 32), dtype=torch.int32, device=K.device)
    if codes.shape != (B, Hkv, Nmax, code_bits // 32) or codes.dtype != torch.int32:
        raise ValueError("codes do not match the shape and dtype")
    _check(_C.hst_hash_keys_binary(ctypes.byref(shape), _ptr(K), _ptr(R), code_bits,
                                   _ptr(codes), _stream(K.device)), "hst_hash_keys_binary")
    return codes


def _append_checks(K, V, k_new, v_new, seq_lens):
    B, Hkv, Nmax, d = K.shape
    if seq_lens is None or seq_lens.shape != (B,) or seq_lens.device != K.device:
        raise ValueError("seq_lens [B] int32 on the cache's device is required (it advances)")
    for t in (V, k_new, v_new):
        if t.dtype != K.dtype or t.device != K.device:
            raise ValueError("K, V, k_new and v_new must share dtype and device")
    if V.shape != K.shape or k_new.shape != (B, Hkv, d) or v_new.shape != (B, Hkv, d):
        raise ValueError("k_new / v_new must be [B, Hkv, d] and V the shape of K")


def hst_append_kv_softlsh(k_new, v_new, W, L: int, P: int, K, V, ids, vnorm, seq_lens) -> None:
    """Writes one token per sequence at row seq_lens[b] of K, V, ids and vnorm
    (hashed on the way in) and advances seq_lens; full sequences are left as
    they are.  Everything is updated in place."""
    _append_checks(K, V, k_new, v_new, seq_lens)
    B, Hkv, Nmax, d = K.shape
    if ids.shape != (B, Hkv, Nmax, L) or ids.dtype != torch.uint8 or vnorm.shape != (B, Hkv, Nmax):
        raise ValueError("ids / vnorm do not match the cache")
    shape = make_shape(K, Hkv, seq_lens)
    _check(_C.hst_append_kv_softlsh(ctypes.byref(shape), _ptr(k_new), _ptr(v_new), _ptr(W), L, P,
                                    _norm_code(vnorm.dtype), _ptr(K), _ptr(V), _ptr(ids),
                                    _ptr(vnorm), _stream(K.device)), "hst_append_kv_softlsh")


def hst_append_kv_binary(k_new, v_new, R, K, V, codes, seq_lens, code_bits: int = 128) -> None:
    """Writes one token per sequence at row seq_lens[b] of K, V and codes
    (hashed on the way in) and advances seq_lens; full sequences are left as
    they are.  Everything is updated in place."""
    _append_checks(K, V, k_new, v_new, seq_lens)
    B, Hkv, Nmax, d = K.shape
    if codes.shape != (B, Hkv, Nmax, code_bits // 32) or codes.dtype != torch.int32:
        raise ValueError("codes do not match the cache")
    shape = make_shape(K, Hkv, seq_lens)
    _check(_C.hst_append_kv_binary(ctypes.byref(shape), _ptr(k_new), _ptr(v_new), _ptr(R),
                                   code_bits, _ptr(K), _ptr(V), _ptr(codes), _stream(K.device)),
           "hst_append_kv_binary")


def hst_score_keys_softlsh(q, W, L: int, P: int, tau: float, ids, vnorm, Nmax_like,
                           seq_lens=None) -> torch.Tensor:
    """Soft-collision scores [B,Hkv,Nmax] float32; Nmax_like is the K cache."""
    B, Hq, d = q.shape
    shape = make_shape(Nmax_like, Hq, seq_lens)
    scores = torch.zeros((shape.B, shape.Hkv, shape.Nmax), dtype=torch.float32, device=q.device)
    ws = _workspace(workspace_size(HST_OP_SCORE_SOFTLSH, shape, L, P), q.device)
    _check(_C.hst_score_keys_softlsh(ctypes.byref(shape), _ptr(q), _ptr(W), L, P, float(tau),
                                     _ptr(ids), _ptr(vnorm), _norm_code(vnorm.dtype),
                                     _ptr(scores), _ptr(ws), ws.numel(), _stream(q.device)),
           "hst_score_keys_softlsh")
    return scores


def hst_query_tables_softlsh(q, W, L: int, P: int, tau: float, Nmax_like,
                             seq_lens=None) -> torch.Tensor:
    """Bucket-probability tables, bucket-major: [B,Hkv,2^P,L] float32."""
    B, Hq, d = q.shape
    shape = make_shape(Nmax_like, Hq, seq_lens)
    tables = torch.empty((shape.B, shape.Hkv, 1 << P, L), dtype=torch.float32, device=q.device)
    _check(_C.hst_query_tables_softlsh(ctypes.byref(shape), _ptr(q), _ptr(W), L, P, float(tau),
                                       _ptr(tables), _stream(q.device)),
           "hst_query_tables_softlsh")
    return tables


def hst_score_scan_softlsh(tables, ids, vnorm, Nmax_like, Hq: int, seq_lens=None,
                           scores=None, stream=None) -> torch.Tensor:
    """Score scan over precomputed tables: [B,Hkv,Nmax] float32."""
    B, Hkv, nb, L = tables.shape
    shape = make_shape(Nmax_like, Hq, seq_lens)
    if scores is None:
        scores = torch.zeros((shape.B, shape.Hkv, shape.Nmax), dtype=torch.float32,
                             device=tables.device)
    st = _stream(tables.device) if stream is None else stream
    _check(_C.hst_score_scan_softlsh(ctypes.byref(shape), _ptr(tables), L, nb.bit_length() - 1,
                                     _ptr(ids), _ptr(vnorm), _norm_code(vnorm.dtype),
                                     _ptr(scores), st), "hst_score_scan_softlsh")
    return scores


def hst_score_keys_hamming(q, R, codes, Nmax_like, code_bits: int = 128,
                           seq_lens=None) -> torch.Tensor:
    """Code-similarity scores [B,Hkv,Nmax] int32."""
    B, Hq, d = q.shape
    shape = make_shape(Nmax_like, Hq, seq_lens)
    scores = torch.zeros((shape.B, shape.Hkv, shape.Nmax), dtype=torch.int32, device=q.device)
    ws = _workspace(workspace_size(HST_OP_SCORE_HAMMING, shape, code_bits=code_bits), q.device)
    _check(_C.hst_score_keys_hamming(ctypes.byref(shape), _ptr(q), _ptr(R), code_bits,
                                     _ptr(codes), _ptr(scores), _ptr(ws), ws.numel(),
                                     _stream(q.device)), "hst_score_keys_hamming")
    return scores


def hst_select_topk(scores, k: int, Hq: int, d: int, kv_dtype=torch.bfloat16,
                    k_per_seq=None, seq_lens=None) -> torch.Tensor:
    """Top-k indices [B,Hkv,k] int32, ascending, -1 padded."""
    B, Hkv, Nmax = scores.shape
    shape = HstShape(B, Hq, Hkv, d, Nmax, _kv_code(kv_dtype), _ptr(seq_lens))
    sd = HST_F32 if scores.dtype == torch.float32 else HST_I32
    if scores.dtype not in (torch.float32, torch.int32):
        raise ValueError("scores must be float32 or int32")
    idx = torch.empty((B, Hkv, k), dtype=torch.int32, device=scores.device)
    ws = _workspace(workspace_size(HST_OP_SELECT_TOPK, shape, k=k), scores.device)
    _check(_C.hst_select_topk(ctypes.byref(shape), sd, _ptr(scores), k, _ptr(k_per_seq),
                              _ptr(idx), _ptr(ws), ws.numel(), _stream(scores.device)),
           "hst_select_topk")
    return idx


def hst_sparse_decode_attention(q, K, V, idx, scale: Optional[float] = None, seq_lens=None,
                                want_lse: bool = True):
    """Attention over selected rows: out [B,Hq,d] float32, lse [B,Hq] float32."""
    B, Hq, d = q.shape
    shape = make_shape(K, Hq, seq_lens)
    k = idx.shape[-1]
    if scale is None:
        scale = d ** -0.5
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if want_lse else None
    ws = _workspace(workspace_size(HST_OP_SPARSE_ATTENTION, shape, k=k), q.device)
    _check(_C.hst_sparse_decode_attention(ctypes.byref(shape), _ptr(q), _ptr(K), _ptr(V),
                                          _ptr(idx), k, float(scale), _ptr(out), _ptr(lse),
                                          _ptr(ws), ws.numel(), _stream(q.device)),
           "hst_sparse_decode_attention")
    return out, lse


def hst_select_mass(q, K, cand, p: float, scale: Optional[float] = None, seq_lens=None):
    """Cumulative-mass selection over candidates cand [B,Hkv,k] int32 (as
    hst_select_topk writes them): idx [B,Hkv,k] int32 (-1 padded) and
    counts [B,Hkv] int32."""
    B, Hq, d = q.shape
    shape = make_shape(K, Hq, seq_lens)
    k = cand.shape[-1]
    if cand.dtype != torch.int32 or cand.shape != (B, K.shape[1], k):
        raise ValueError("cand must be int32 [B, Hkv, k]")
    if scale is None:
        scale = d ** -0.5
    idx = torch.empty_like(cand)
    counts = torch.empty((B, K.shape[1]), dtype=torch.int32, device=q.device)
    ws = _workspace(workspace_size(HST_OP_SELECT_MASS, shape, k=k), q.device)
    _check(_C.hst_select_mass(ctypes.byref(shape), _ptr(q), _ptr(K), _ptr(cand), k, float(p),
                              float(scale), _ptr(idx), _ptr(counts), _ptr(ws), ws.numel(),
                              _stream(q.device)), "hst_select_mass")
    return idx, counts


class DecodeSoftLSH:
    """Pre-sized soft-LSH decode step: outputs and workspace allocated once."""

    def __init__(self, K, Hq: int, L: int, P: int, tau: float, k: int, norm_dtype,
                 seq_lens=None, k_per_seq=None, scale: Optional[float] = None):
        B, Hkv, Nmax, d = K.shape
        self.shape = make_shape(K, Hq, seq_lens)
        self._keep = (seq_lens, k_per_seq)
        self.L, self.P, self.tau, self.k = L, P, float(tau), k
        self.norm_code = _norm_code(norm_dtype)
        self.scale = float(d ** -0.5 if scale is None else scale)
        dev = K.device
        self.idx = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        self.ws = _workspace(workspace_size(HST_OP_DECODE_SOFTLSH, self.shape, L, P, k=k), dev)
        self.k_per_seq = k_per_seq

    def __call__(self, q, K, V, W, ids, vnorm, stream: Optional[int] = None):
        st = _stream(q.device) if stream is None else stream
        _check(_C.hst_decode_step_softlsh(
            ctypes.byref(self.shape), _ptr(q), _ptr(K), _ptr(V), _ptr(W), self.L, self.P,
            self.tau, _ptr(ids), _ptr(vnorm), self.norm_code, self.k, _ptr(self.k_per_seq),
            self.scale, _ptr(self.idx), _ptr(self.out), _ptr(self.lse), _ptr(self.ws),
            self.ws.numel(), st), "hst_decode_step_softlsh")
        return self.idx, self.out, self.lse

    # the step's three stages (the call above runs them in order)
    def prepare(self, q, W, ids, vnorm, stream: Optional[int] = None):
        st = _stream(q.device) if stream is None else stream
        _check(_C.hst_decode_prepare_softlsh(
            ctypes.byref(self.shape), _ptr(q), _ptr(W), self.L, self.P, self.tau, _ptr(ids),
            _ptr(vnorm), self.norm_code, self.k, _ptr(self.k_per_seq), _ptr(self.ws),
            self.ws.numel(), st), "hst_decode_prepare_softlsh")

    def filter(self, ids, vnorm, stream: Optional[int] = None):
        st = _stream(ids.device) if stream is None else stream
        _check(_C.hst_decode_filter_softlsh(
            ctypes.byref(self.shape), self.L, self.P, _ptr(ids), _ptr(vnorm), self.norm_code,
            self.k, _ptr(self.k_per_seq), _ptr(self.ws), self.ws.numel(), st),
            "hst_decode_filter_softlsh")

    def finish(self, q, K, V, ids, vnorm, stream: Optional[int] = None):
        st = _stream(q.device) if stream is None else stream
        _check(_C.hst_decode_finish_softlsh(
            ctypes.byref(self.shape), _ptr(q), _ptr(K), _ptr(V), self.L, self.P, _ptr(ids),
            _ptr(vnorm), self.norm_code, self.k, self.scale, _ptr(self.idx), _ptr(self.out),
            _ptr(self.lse), _ptr(self.ws), self.ws.numel(), st), "hst_decode_finish_softlsh")
        return self.idx, self.out, self.lse

    def candidates(self, cap: int):
        return _candidates(self.shape, HST_OP_DECODE_SOFTLSH, self.L, self.P, self.k, self.ws, cap)


def _candidates(shape, op, L, P, k, ws, cap):
    """The filter stage's candidates per (sequence, kv head): order keys
    [B,Hkv,cap] (int32 bit patterns of the uint32 keys), indices [B,Hkv,cap],
    counts [B,Hkv] and thresholds [B,Hkv] (order keys as int32 bits)."""
    B, Hkv, dev = shape.B, shape.Hkv, ws.device
    keys = torch.zeros((B, Hkv, cap), dtype=torch.int32, device=dev)
    index = torch.full((B, Hkv, cap), -1, dtype=torch.int32, device=dev)
    count = torch.zeros((B, Hkv), dtype=torch.int32, device=dev)
    theta = torch.zeros((B, Hkv), dtype=torch.int32, device=dev)
    _check(_C.hst_decode_candidates(ctypes.byref(shape), op, L, P, k, _ptr(ws), ws.numel(), cap,
                                    _ptr(keys), _ptr(index), _ptr(count), _ptr(theta),
                                    _stream(dev)), "hst_decode_candidates")
    return keys, index, count, theta


class DecodeHamming:
    """Pre-sized binary-code decode step."""

    def __init__(self, K, Hq: int, k: int, code_bits: int = 128, seq_lens=None, k_per_seq=None,
                 scale: Optional[float] = None):
        B, Hkv, Nmax, d = K.shape
        self.shape = make_shape(K, Hq, seq_lens)
        self._keep = (seq_lens, k_per_seq)
        self.k, self.code_bits = k, code_bits
        self.scale = float(d ** -0.5 if scale is None else scale)
        dev = K.device
        self.idx = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        self.ws = _workspace(workspace_size(HST_OP_DECODE_HAMMING, self.shape, code_bits=code_bits,
                                            k=k), dev)
        self.k_per_seq = k_per_seq

    def __call__(self, q, K, V, R, codes, stream: Optional[int] = None):
        st = _stream(q.device) if stream is None else stream
        _check(_C.hst_decode_step_hamming(
            ctypes.byref(self.shape), _ptr(q), _ptr(K), _ptr(V), _ptr(R), self.code_bits,
            _ptr(codes), self.k, _ptr(self.k_per_seq), self.scale, _ptr(self.idx),
            _ptr(self.out), _ptr(self.lse), _ptr(self.ws), self.ws.numel(), st),
            "hst_decode_step_hamming")
        return self.idx, self.out, self.lse

    # the step's three stages (128-bit codes; the call above runs them in order)
    def prepare(self, q, R, codes, stream: Optional[int] = None):
        st = _stream(q.device) if stream is None else stream
        _check(_C.hst_decode_prepare_hamming(
            ctypes.byref(self.shape), _ptr(q), _ptr(R), _ptr(codes), self.k, _ptr(self.k_per_seq),
            _ptr(self.ws), self.ws.numel(), st), "hst_decode_prepare_hamming")

    def filter(self, codes, stream: Optional[int] = None):
        st = _stream(codes.device) if stream is None else stream
        _check(_C.hst_decode_filter_hamming(
            ctypes.byref(self.shape), _ptr(codes), self.k, _ptr(self.k_per_seq), _ptr(self.ws),
            self.ws.numel(), st), "hst_decode_filter_hamming")

    def finish(self, q, K, V, codes, stream: Optional[int] = None):
        st = _stream(q.device) if stream is None else stream
        _check(_C.hst_decode_finish_hamming(
            ctypes.byref(self.shape), _ptr(q), _ptr(K), _ptr(V), _ptr(codes), self.k, self.scale,
            _ptr(self.idx), _ptr(self.out), _ptr(self.lse), _ptr(self.ws), self.ws.numel(), st),
            "hst_decode_finish_hamming")
        return self.idx, self.out, self.lse

    def candidates(self, cap: int):
        return _candidates(self.shape, HST_OP_DECODE_HAMMING, 0, 0, self.k, self.ws, cap)


def hst_decode_step_softlsh_noalloc(q, K, V, W, ids, vnorm, L: int, P: int, tau: float, k: int,
                                    seq_lens=None, k_per_seq=None, scale=None, idx=None, out=None,
                                    lse=None):
    """The soft-LSH decode step on the library's fixed per-GPU workspace (no
    workspace allocation; outputs may be passed in)."""
    B, Hq, d = q.shape
    Hkv = K.shape[1]
    shape = make_shape(K, Hq, seq_lens)
    if idx is None:
        idx = torch.empty((B, Hkv, k), dtype=torch.int32, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    sc = float(d ** -0.5 if scale is None else scale)
    _check(_C.hst_decode_step_softlsh_noalloc(
        ctypes.byref(shape), _ptr(q), _ptr(K), _ptr(V), _ptr(W), L, P, float(tau), _ptr(ids),
        _ptr(vnorm), _norm_code(vnorm.dtype), k, _ptr(k_per_seq), sc, _ptr(idx), _ptr(out),
        _ptr(lse), _stream(q.device)), "hst_decode_step_softlsh_noalloc")
    return idx, out, lse


def hst_decode_step_softlsh(q, K, V, W, ids, vnorm, L: int, P: int, tau: float, k: int,
                            seq_lens=None, k_per_seq=None, scale=None):
    step = DecodeSoftLSH(K, q.shape[1], L, P, tau, k, vnorm.dtype, seq_lens, k_per_seq, scale)
    return step(q, K, V, W, ids, vnorm)


def hst_decode_step_hamming(q, K, V, R, codes, k: int, seq_lens=None, k_per_seq=None,
                            scale=None):
    step = DecodeHamming(K, q.shape[1], k, 128, seq_lens, k_per_seq, scale)
    return step(q, K, V, R, codes)


class DecodeSoftLSHMass:
    """Pre-sized soft-LSH decode step with a cumulative-mass budget: the k
    keys of highest hash score are the candidates, the kept set reaches mass
    p of their softmax."""

    def __init__(self, K, Hq: int, L: int, P: int, tau: float, k: int, p: float, norm_dtype,
                 seq_lens=None, k_per_seq=None, scale: Optional[float] = None):
        B, Hkv, Nmax, d = K.shape
        self.shape = make_shape(K, Hq, seq_lens)
        self._keep = (seq_lens, k_per_seq)
        self.L, self.P, self.tau, self.k, self.p = L, P, float(tau), k, float(p)
        self.norm_code = _norm_code(norm_dtype)
        self.scale = float(d ** -0.5 if scale is None else scale)
        dev = K.device
        self.idx = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
        self.counts = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        self.ws = _workspace(workspace_size(HST_OP_DECODE_SOFTLSH_MASS, self.shape, L, P, k=k),
                             dev)
        self.k_per_seq = k_per_seq

    def __call__(self, q, K, V, W, ids, vnorm, stream: Optional[int] = None):
        st = _stream(q.device) if stream is None else stream
        _check(_C.hst_decode_step_softlsh_mass(
            ctypes.byref(self.shape), _ptr(q), _ptr(K), _ptr(V), _ptr(W), self.L, self.P,
            self.tau, _ptr(ids), _ptr(vnorm), self.norm_code, self.k, _ptr(self.k_per_seq),
            self.p, self.scale, _ptr(self.idx), _ptr(self.counts), _ptr(self.out),
            _ptr(self.lse), _ptr(self.ws), self.ws.numel(), st), "hst_decode_step_softlsh_mass")
        return self.idx, self.counts, self.out, self.lse


def hst_build_cards_softlsh(K, vnorm, W, L: int, P: int, seq_lens=None):
    """Index cards of 64-token chunks: card keys [B,Hkv,Nc,d] (KV dtype),
    card ids [B,Hkv,Nc,L] uint8, card weights [B,Hkv,Nc] (vnorm dtype) and
    card counts [B] int32, with Nc = ceil(Nmax / 64)."""
    B, Hkv, Nmax, d = K.shape
    Nc = (Nmax + CHUNK - 1) // CHUNK
    shape = make_shape(K, Hkv, seq_lens)
    ckeys = torch.zeros((B, Hkv, Nc, d), dtype=K.dtype, device=K.device)
    cids = torch.zeros((B, Hkv, Nc, L), dtype=torch.uint8, device=K.device)
    cw = torch.zeros((B, Hkv, Nc), dtype=vnorm.dtype, device=K.device)
    clens = torch.zeros((B,), dtype=torch.int32, device=K.device)
    _check(_C.hst_build_cards_softlsh(ctypes.byref(shape), _ptr(K), _ptr(vnorm),
                                      _norm_code(vnorm.dtype), _ptr(W), L, P, _ptr(ckeys),
                                      _ptr(cids), _ptr(cw), _ptr(clens), _stream(K.device)),
           "hst_build_cards_softlsh")
    return ckeys, cids, cw, clens


class DecodeSoftLSHRouted:
    """Pre-sized soft-LSH decode step with two-level routing: C chunks by
    their cards, then the k best keys inside them."""

    def __init__(self, K, Hq: int, L: int, P: int, tau: float, k: int, C: int, norm_dtype,
                 seq_lens=None, k_per_seq=None, scale: Optional[float] = None):
        B, Hkv, Nmax, d = K.shape
        self.shape = make_shape(K, Hq, seq_lens)
        self._keep = (seq_lens, k_per_seq)
        self.L, self.P, self.tau, self.k, self.C = L, P, float(tau), k, C
        self.norm_code = _norm_code(norm_dtype)
        self.scale = float(d ** -0.5 if scale is None else scale)
        dev = K.device
        self.idx = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        self.ws = _workspace(workspace_size(HST_OP_DECODE_SOFTLSH_ROUTED, self.shape, L, P, k=k),
                             dev)
        self.k_per_seq = k_per_seq

    def __call__(self, q, K, V, W, ids, vnorm, card_ids, card_w, stream: Optional[int] = None):
        st = _stream(q.device) if stream is None else stream
        _check(_C.hst_decode_step_softlsh_routed(
            ctypes.byref(self.shape), _ptr(q), _ptr(K), _ptr(V), _ptr(W), self.L, self.P,
            self.tau, _ptr(ids), _ptr(vnorm), self.norm_code, _ptr(card_ids), _ptr(card_w),
            self.C, self.k, _ptr(self.k_per_seq), self.scale, _ptr(self.idx), _ptr(self.out),
            _ptr(self.lse), _ptr(self.ws), self.ws.numel(), st), "hst_decode_step_softlsh_routed")
        return self.idx, self.out, self.lse


class DecodeSoftLSHShared:
    """Pre-sized soft-LSH decode step for a batch sharing a prefix: K / V /
    ids / vnorm of the suffixes [B,Hkv,Ns,...] plus the prefix cache
    [Hkv,Np,...] (a batch of one); indices are into prefix + suffix."""

    def __init__(self, Ks, Np: int, Hq: int, L: int, P: int, tau: float, k: int, norm_dtype,
                 seq_lens=None, k_per_seq=None, scale: Optional[float] = None):
        B, Hkv, Ns, d = Ks.shape
        self.shape = make_shape(Ks, Hq, seq_lens)
        self._keep = (seq_lens, k_per_seq)
        self.Np, self.L, self.P, self.tau, self.k = Np, L, P, float(tau), k
        self.norm_code = _norm_code(norm_dtype)
        self.scale = float(d ** -0.5 if scale is None else scale)
        dev = Ks.device
        self.idx = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        nbytes = ctypes.c_size_t(0)
        _check(_C.hst_workspace_size_shared(ctypes.byref(self.shape), Np, L, P, k,
                                            ctypes.byref(nbytes)), "hst_workspace_size_shared")
        self.ws = _workspace(nbytes.value, dev)
        self.k_per_seq = k_per_seq

    def __call__(self, q, Kp, Vp, ids_p, vn_p, Ks, Vs, ids_s, vn_s, W,
                 stream: Optional[int] = None):
        st = _stream(q.device) if stream is None else stream
        _check(_C.hst_decode_step_softlsh_shared(
            ctypes.byref(self.shape), self.Np, _ptr(q), _ptr(Kp), _ptr(Vp), _ptr(ids_p),
            _ptr(vn_p), _ptr(Ks), _ptr(Vs), _ptr(ids_s), _ptr(vn_s), _ptr(W), self.L, self.P,
            self.tau, self.norm_code, self.k, _ptr(self.k_per_seq), self.scale, _ptr(self.idx),
            _ptr(self.out), _ptr(self.lse), _ptr(self.ws), self.ws.numel(), st),
            "hst_decode_step_softlsh_shared")
        return self.idx, self.out, self.lse
