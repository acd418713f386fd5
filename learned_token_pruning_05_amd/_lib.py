"""ctypes binding of libtokengate: the C-ABI entry points under the same names.

Argument marshalling only: shapes, strides, data pointers and the current
stream are read from torch tensors and passed through; every step of the path
runs in the library's HIP kernels.  Output tensors the caller does not pass are
allocated with torch on the input's device.  A non-zero status raises
TokenGateError.  There is no fallback: if the library is missing, load() raises.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtokengate.so")

TG_OK, TG_ERR_INVALID_ARG, TG_ERR_UNSUPPORTED, TG_ERR_WORKSPACE, TG_ERR_HIP = range(5)
TG_F32, TG_BF16 = 0, 1

# symbol -> (restype, argtypes)
_P, _I32, _I64, _F, _D, _SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                               ctypes.c_double, ctypes.c_size_t)
SIGNATURES = {
    "tg_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "tg_kept_counts": (ctypes.c_int, [_I32, _P, _P, _P, _P, _P]),
    "tg_random_budgets": (ctypes.c_int, [ctypes.c_uint64, _I32, _P, _P, _P]),
    "tg_gate_score": (ctypes.c_int, [_P, _I32, _I64, _I32, _I64, _P, _P, _P, _F, _I32, _P, _P]),
    "tg_topk_workspace_bytes": (_SZ, [_I32, _I64, _I32]),
    "tg_topk_select": (ctypes.c_int, [_P, _I32, _I64, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "tg_gather_kept": (ctypes.c_int, [_P, _I32, _I32, _I64, _P, _P, _I64, _I32, _P, _P, _P, _P, _P, _P]),
    "tg_gated_select": (ctypes.c_int, [_P, _I32, _I64, _I32, _I64, _P, _P, _P, _F, _I32, _I32, _I32, _P, _P, _P, _P,
                                       _P, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "tg_attn_workspace_bytes": (_SZ, [_I32, _I64, _I32, _I32]),
    "tg_keybias_attn_prefill": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P, _P, _F, _P, _P, _I32, _I64,
                                               _I32, _I32, _I32, _I32, _D, _P, _P, _P, _SZ, _P]),
    "tg_attn_prepare": (ctypes.c_int, [_P, _P, _I64, _P, _P, _P, _I32, _I64, _I32, _I32, _D, _P, _SZ, _P]),
    "tg_attn_forward": (ctypes.c_int, [_P, _I64, _P, _F, _P, _I32, _I64, _I32, _I32, _I32, _I32, _D, _P, _P,
                                       _P, _SZ, _P]),
    "tg_topk_noalloc_max_bytes": (_SZ, []),
    "tg_topk_select_noalloc": (ctypes.c_int, [_P, _I32, _I64, _I32, _P, _P, _P, _P, _P, _P, _P]),
    "tg_random_k_workspace_bytes": (_SZ, [_I32, _I64, _I32]),
    "tg_random_k_select": (ctypes.c_int, [ctypes.c_uint64, _I32, _I64, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "tg_attn_decode_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "tg_attn_decode": (ctypes.c_int, [_P, _I64, _P, _P, _F, _P, _P, _I32, _I64, _I32, _I32, _I32, _I32, _D, _P,
                                      _SZ, _P, _P, _P, _SZ, _P]),
    "tg_attn_gate_grads_workspace_bytes": (_SZ, [_I32, _I64, _I32, _I32, _I32]),
    "tg_attn_gate_grads": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _P, _F, _P, _I32, _I64, _I32, _I32, _I32, _I32,
                                          _D, _P, _P, _P, _I64, _P, _SZ, _P, _P, _P, _P, _SZ, _P]),
}


class TokenGateError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


_lib = None


def load():
    """Load the in-tree libtokengate.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(lib, name)
            f.restype, f.argtypes = res, args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().tg_status_string(status).decode()


def _check(fn, status):
    if status != TG_OK:
        raise TokenGateError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return TG_BF16
    if t.dtype == torch.float32:
        return TG_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _rows(t):
    """(n_rows, row_len, row_stride) of a 2-D tensor with unit inner stride."""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with contiguous rows")
    return t.shape[0], t.shape[1], t.stride(0)


def _i32_host(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _req(t, name, dtype=None, dim=None, numel=None, dense=True, device=None, optional=False):
    """Check a tensor argument before its pointer reaches a kernel: a torch
    tensor on a GPU device (the same one as `device` if given), of the given
    dtype(s) and rank, dense when the kernels read it as one flat array.
    Raises TypeError / ValueError; a wrong tensor never becomes a bad device
    address inside a kernel."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if dtype is not None:
        dts = dtype if isinstance(dtype, tuple) else (dtype,)
        if t.dtype not in dts:
            raise TypeError(f"{name} must be {' or '.join(str(d) for d in dts)}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dimensions, got shape {tuple(t.shape)}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, not {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other tensors on {device}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    if dense and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_I32T, _F32T, _BF16T, _U8T = torch.int32, torch.float32, torch.bfloat16, torch.uint8


# ------------------------------------------------------------------ entries --
def tg_kept_counts(cu_seqlens, doc_begin, doc_end, k_doc) -> np.ndarray:
    """Host-side kept counts -> cu_kept (int32 numpy, S+1)."""
    cu, b, e, k = (_i32_host(a) for a in (cu_seqlens, doc_begin, doc_end, k_doc))
    s = len(cu) - 1
    out = np.zeros(s + 1, dtype=np.int32)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    _check("tg_kept_counts", load().tg_kept_counts(s, p(cu), p(b), p(e), p(k), p(out)))
    return out


def _check_gate(x, w1, b1, w2, scores):
    _req(x, "x", (_BF16T, _F32T), dim=2, dense=False)
    n, d_model, stride = _rows(x)
    _req(w1, "w1", x.dtype, dim=2, device=x.device)
    if w1.shape[1] != d_model:
        raise ValueError(f"w1 must be [d_hid, {d_model}], got {tuple(w1.shape)}")
    d_hid = w1.shape[0]
    _req(b1, "b1", _F32T, dim=1, numel=d_hid, device=x.device, optional=True)
    _req(w2, "w2", _F32T, dim=1, numel=d_hid, device=x.device)
    _req(scores, "scores", _F32T, dim=1, numel=n, device=x.device, optional=True)
    return n, d_model, stride, d_hid


def _check_meta(dev, n_seqs, **meta):
    for name, t in meta.items():
        _req(t, name, _I32T, dim=1, numel=n_seqs + (1 if name.startswith("cu_") else 0), device=dev)


def tg_gate_score(x, w1, b1, w2, b2: float, scores=None):
    n, d_model, stride, d_hid = _check_gate(x, w1, b1, w2, scores)
    if scores is None:
        scores = torch.empty(n, dtype=torch.float32, device=x.device)
    st = load().tg_gate_score(_ptr(x), _dtype_code(x), n, d_model, stride, _ptr(w1), _ptr(b1), _ptr(w2),
                              float(b2), d_hid, _ptr(scores), _stream(x))
    _check("tg_gate_score", st)
    return scores


def tg_topk_workspace_bytes(n_seqs, n_tokens_total, max_seqlen) -> int:
    return load().tg_topk_workspace_bytes(n_seqs, n_tokens_total, max_seqlen)


def tg_topk_select(scores, cu_seqlens, doc_begin, doc_end, k_doc, cu_kept, n_kept_total: int,
                   max_seqlen: int, kept_idx=None, workspace=None):
    """Device metadata tensors (int32); n_kept_total = cu_kept[-1] known on the host."""
    _req(scores, "scores", _F32T, dim=1)
    _req(cu_seqlens, "cu_seqlens", _I32T, dim=1, device=scores.device)
    n_seqs = cu_seqlens.shape[0] - 1
    _check_meta(scores.device, n_seqs, doc_begin=doc_begin, doc_end=doc_end, k_doc=k_doc, cu_kept=cu_kept)
    _req(kept_idx, "kept_idx", _I32T, dim=1, numel=int(n_kept_total), device=scores.device, optional=True)
    _req(workspace, "workspace", _U8T, device=scores.device, optional=True)
    if kept_idx is None:
        kept_idx = torch.empty(n_kept_total, dtype=torch.int32, device=scores.device)
    lib = load()
    if workspace is None:
        need = lib.tg_topk_workspace_bytes(n_seqs, scores.shape[0], max_seqlen)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=scores.device)
    st = lib.tg_topk_select(_ptr(scores), n_seqs, scores.shape[0], max_seqlen, _ptr(cu_seqlens), _ptr(doc_begin),
                            _ptr(doc_end), _ptr(k_doc), _ptr(cu_kept), _ptr(kept_idx), _ptr(workspace),
                            workspace.numel(), _stream(scores))
    _check("tg_topk_select", st)
    return kept_idx


def tg_topk_select_noalloc(scores, cu_seqlens, doc_begin, doc_end, k_doc, cu_kept, n_kept_total: int,
                           max_seqlen: int, kept_idx=None):
    """tg_topk_select with the library's own scratch array (no workspace; the C
    call allocates nothing).  kept_idx is allocated here only if not given."""
    _req(scores, "scores", _F32T, dim=1)
    _req(cu_seqlens, "cu_seqlens", _I32T, dim=1, device=scores.device)
    n_seqs = cu_seqlens.shape[0] - 1
    _check_meta(scores.device, n_seqs, doc_begin=doc_begin, doc_end=doc_end, k_doc=k_doc, cu_kept=cu_kept)
    _req(kept_idx, "kept_idx", _I32T, dim=1, numel=int(n_kept_total), device=scores.device, optional=True)
    if kept_idx is None:
        kept_idx = torch.empty(n_kept_total, dtype=torch.int32, device=scores.device)
    st = load().tg_topk_select_noalloc(_ptr(scores), n_seqs, scores.shape[0], max_seqlen, _ptr(cu_seqlens),
                                       _ptr(doc_begin), _ptr(doc_end), _ptr(k_doc), _ptr(cu_kept), _ptr(kept_idx),
                                       _stream(scores))
    _check("tg_topk_select_noalloc", st)
    return kept_idx


def tg_random_k_workspace_bytes(n_seqs, n_tokens_total, max_seqlen) -> int:
    return load().tg_random_k_workspace_bytes(n_seqs, n_tokens_total, max_seqlen)


def tg_random_k_select(seed: int, cu_seqlens, doc_begin, doc_end, k_doc, cu_kept, n_tokens: int, n_kept_total: int,
                       max_seqlen: int, kept_idx=None, workspace=None):
    """Random-K selector mode: as tg_topk_select over seeded SplitMix64 scores."""
    _req(cu_seqlens, "cu_seqlens", _I32T, dim=1)
    n_seqs = cu_seqlens.shape[0] - 1
    dev = cu_seqlens.device
    _check_meta(dev, n_seqs, doc_begin=doc_begin, doc_end=doc_end, k_doc=k_doc, cu_kept=cu_kept)
    _req(kept_idx, "kept_idx", _I32T, dim=1, numel=int(n_kept_total), device=dev, optional=True)
    _req(workspace, "workspace", _U8T, device=dev, optional=True)
    if kept_idx is None:
        kept_idx = torch.empty(n_kept_total, dtype=torch.int32, device=dev)
    lib = load()
    if workspace is None:
        need = tg_random_k_workspace_bytes(n_seqs, n_tokens, max_seqlen)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib.tg_random_k_select(int(seed) % (1 << 64), n_seqs, n_tokens, max_seqlen, _ptr(cu_seqlens),
                                _ptr(doc_begin), _ptr(doc_end), _ptr(k_doc), _ptr(cu_kept), _ptr(kept_idx),
                                _ptr(workspace), workspace.numel(), _stream(cu_seqlens))
    _check("tg_random_k_select", st)
    return kept_idx


def tg_gather_kept(x, scores, kept_idx, cu_seqlens, cu_kept, x_kept=None, scores_kept=None,
                   pos_kept=None):
    _req(x, "x", (_BF16T, _F32T), dim=2, dense=False)
    n, d_model, stride = _rows(x)
    dev = x.device
    _req(kept_idx, "kept_idx", _I32T, dim=1, device=dev)
    m = kept_idx.shape[0]
    _req(scores, "scores", _F32T, dim=1, numel=n, device=dev, optional=True)
    _req(cu_seqlens, "cu_seqlens", _I32T, dim=1, device=dev)
    _req(cu_kept, "cu_kept", _I32T, dim=1, numel=cu_seqlens.shape[0], device=dev)
    _req(x_kept, "x_kept", x.dtype, dim=2, numel=m * d_model, device=dev, optional=True)
    _req(scores_kept, "scores_kept", _F32T, dim=1, numel=m, device=dev, optional=True)
    _req(pos_kept, "pos_kept", _I32T, dim=1, numel=m, device=dev, optional=True)
    if x_kept is None:
        x_kept = torch.empty((m, d_model), dtype=x.dtype, device=dev)
    if scores_kept is None and scores is not None:
        scores_kept = torch.empty(m, dtype=torch.float32, device=dev)
    if pos_kept is None:
        pos_kept = torch.empty(m, dtype=torch.int32, device=dev)
    st = load().tg_gather_kept(_ptr(x), _dtype_code(x), d_model, stride, _ptr(scores), _ptr(kept_idx), m,
                               cu_seqlens.shape[0] - 1, _ptr(cu_seqlens), _ptr(cu_kept), _ptr(x_kept),
                               _ptr(scores_kept), _ptr(pos_kept), _stream(x))
    _check("tg_gather_kept", st)
    return x_kept, scores_kept, pos_kept


def tg_gated_select(x, w1, b1, w2, b2: float, cu_seqlens, doc_begin, doc_end, k_doc, cu_kept, n_kept_total: int,
                    max_seqlen: int, scores=None, kept_idx=None, x_kept=None, scores_kept=None, pos_kept=None,
                    workspace=None):
    """gate -> top-K -> gather in one call.  Returns (scores, kept_idx, x_kept, scores_kept, pos_kept)."""
    n, d_model, stride, d_hid = _check_gate(x, w1, b1, w2, scores)
    dev = x.device
    _req(cu_seqlens, "cu_seqlens", _I32T, dim=1, device=dev)
    n_seqs = cu_seqlens.shape[0] - 1
    _check_meta(dev, n_seqs, doc_begin=doc_begin, doc_end=doc_end, k_doc=k_doc, cu_kept=cu_kept)
    m = int(n_kept_total)
    _req(kept_idx, "kept_idx", _I32T, dim=1, numel=m, device=dev, optional=True)
    _req(x_kept, "x_kept", x.dtype, dim=2, numel=m * d_model, device=dev, optional=True)
    _req(scores_kept, "scores_kept", _F32T, dim=1, numel=m, device=dev, optional=True)
    _req(pos_kept, "pos_kept", _I32T, dim=1, numel=m, device=dev, optional=True)
    _req(workspace, "workspace", _U8T, device=dev, optional=True)
    if scores is None:
        scores = torch.empty(n, dtype=torch.float32, device=dev)
    if kept_idx is None:
        kept_idx = torch.empty(m, dtype=torch.int32, device=dev)
    if x_kept is None:
        x_kept = torch.empty((m, d_model), dtype=x.dtype, device=dev)
    if scores_kept is None:
        scores_kept = torch.empty(m, dtype=torch.float32, device=dev)
    if pos_kept is None:
        pos_kept = torch.empty(m, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(1, tg_topk_workspace_bytes(n_seqs, n, max_seqlen)), dtype=torch.uint8,
                                device=dev)
    st = load().tg_gated_select(_ptr(x), _dtype_code(x), n, d_model, stride, _ptr(w1), _ptr(b1), _ptr(w2),
                                float(b2), d_hid, n_seqs, int(max_seqlen), _ptr(cu_seqlens), _ptr(doc_begin),
                                _ptr(doc_end), _ptr(k_doc), _ptr(cu_kept), m, _ptr(scores), _ptr(kept_idx),
                                _ptr(x_kept), _ptr(scores_kept), _ptr(pos_kept), _ptr(workspace),
                                workspace.numel(), _stream(x))
    _check("tg_gated_select", st)
    return scores, kept_idx, x_kept, scores_kept, pos_kept


def tg_attn_workspace_bytes(n_seqs, n_kept_total, n_kv_heads, head_dim) -> int:
    return load().tg_attn_workspace_bytes(n_seqs, n_kept_total, n_kv_heads, head_dim)


def _check_kv(k, v):
    _req(k, "k", _BF16T, dim=3, dense=False)
    _req(v, "v", _BF16T, dim=3, dense=False, device=k.device)
    if v.shape != k.shape:
        raise ValueError(f"k and v must have one shape, got {tuple(k.shape)} and {tuple(v.shape)}")
    if k.stride(2) != 1 or k.stride(1) != k.shape[2] or v.stride() != k.stride():
        raise ValueError("heads must be contiguous within a token row; k and v must share strides")


def _check_q(q, name="q"):
    _req(q, name, _BF16T, dim=3, dense=False)
    if q.stride(2) != 1 or q.stride(1) != q.shape[2]:
        raise ValueError("heads must be contiguous within a token row")


def _check_attn_meta(dev, m, hq, key_score=None, head_gain=None, pos=None, cu_kept=None):
    _req(key_score, "key_score", _F32T, dim=1, numel=m, device=dev, optional=key_score is None)
    _req(head_gain, "head_gain", _F32T, dim=1, numel=hq, device=dev, optional=hq is None)
    _req(pos, "pos", _I32T, dim=1, numel=m, device=dev, optional=pos is None)
    _req(cu_kept, "cu_kept", _I32T, dim=1, device=dev)


def tg_attn_prepare(k, v, key_score, pos, cu_kept, rope_base: float = 1e6, workspace=None):
    """Kept-only key/value cache for tg_attn_forward; returns the workspace."""
    _check_kv(k, v)
    m, hkv, d = k.shape
    _check_attn_meta(k.device, m, None, key_score=key_score, pos=pos, cu_kept=cu_kept)
    _req(workspace, "workspace", _U8T, device=k.device, optional=True)
    n_seqs = cu_kept.shape[0] - 1
    need = tg_attn_workspace_bytes(n_seqs, m, hkv, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=k.device)
    st = load().tg_attn_prepare(_ptr(k), _ptr(v), k.stride(0), _ptr(key_score), _ptr(pos), _ptr(cu_kept), n_seqs, m,
                                hkv, d, float(rope_base), _ptr(workspace), workspace.numel(), _stream(k))
    _check("tg_attn_prepare", st)
    return workspace


def tg_attn_forward(q, head_gain, tau: float, cu_kept, max_kept_seqlen: int, n_kv_heads: int, workspace,
                    rope_base: float = 1e6, out=None, lse=None, want_lse: bool = True):
    """q: [M, Hq, D] bf16 over a workspace filled by tg_attn_prepare with the same metadata."""
    _check_q(q)
    m, hq, d = q.shape
    dev = q.device
    _check_attn_meta(dev, m, hq, head_gain=head_gain, cu_kept=cu_kept)
    _req(workspace, "workspace", _U8T, device=dev)
    _req(out, "out", _BF16T, numel=m * hq * d, device=dev, optional=True)
    _req(lse, "lse", _F32T, numel=m * hq, device=dev, optional=True)
    if out is None:
        out = torch.empty((m, hq, d), dtype=torch.bfloat16, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((hq, m), dtype=torch.float32, device=dev)
    st = load().tg_attn_forward(_ptr(q), q.stride(0), _ptr(head_gain), float(tau), _ptr(cu_kept),
                                cu_kept.shape[0] - 1, m, int(max_kept_seqlen), hq, int(n_kv_heads), d,
                                float(rope_base), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                _stream(q))
    _check("tg_attn_forward", st)
    return out, lse


def tg_keybias_attn_prefill(q, k, v, key_score, head_gain, tau: float, pos, cu_kept,
                            max_kept_seqlen: int, rope_base: float = 1e6, out=None, lse=None,
                            workspace=None, want_lse: bool = True):
    """q: [M, Hq, D] (token rows may be strided), k/v: [M, Hkv, D] bf16."""
    _check_q(q)
    _check_kv(k, v)
    m, hq, d = q.shape
    hkv = k.shape[1]
    dev = q.device
    if k.device != dev or k.shape[0] != m or k.shape[2] != d:
        raise ValueError("q, k and v must share the device, the token count and head_dim")
    _check_attn_meta(dev, m, hq, key_score=key_score, head_gain=head_gain, pos=pos, cu_kept=cu_kept)
    _req(workspace, "workspace", _U8T, device=dev, optional=True)
    _req(out, "out", _BF16T, numel=m * hq * d, device=dev, optional=True)
    _req(lse, "lse", _F32T, numel=m * hq, device=dev, optional=True)
    n_seqs = cu_kept.shape[0] - 1
    if out is None:
        out = torch.empty((m, hq, d), dtype=torch.bfloat16, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((hq, m), dtype=torch.float32, device=dev)
    need = tg_attn_workspace_bytes(n_seqs, m, hkv, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = load().tg_keybias_attn_prefill(_ptr(q), _ptr(k), _ptr(v), q.stride(0), k.stride(0), _ptr(key_score),
                                        _ptr(head_gain), float(tau), _ptr(pos), _ptr(cu_kept), n_seqs, m,
                                        int(max_kept_seqlen), hq, hkv, d, float(rope_base), _ptr(out),
                                        _ptr(lse), _ptr(workspace), workspace.numel(), _stream(q))
    _check("tg_keybias_attn_prefill", st)
    return out, lse


def tg_attn_decode_workspace_bytes(n_seqs, max_kept_seqlen, n_q_heads, head_dim) -> int:
    return int(load().tg_attn_decode_workspace_bytes(n_seqs, max_kept_seqlen, n_q_heads, head_dim))


def tg_attn_decode(q, q_pos, head_gain, tau: float, pos, cu_kept, max_kept_seqlen: int, n_kv_heads: int, cache,
                   rope_base: float = 1e6, out=None, lse=None, want_lse: bool = True, workspace=None):
    """One new query per sequence over a cache filled by tg_attn_prepare.

    q: [S, Hq, D] bf16 (row stride between sequences allowed); q_pos: [S] int32;
    pos, cu_kept: the kept positions and offsets the cache was prepared with.
    Returns (out [S, Hq, D] bf16, lse [Hq, S] fp32 or None).
    """
    _check_q(q)
    n_seqs, hq, d = q.shape
    dev = q.device
    _req(pos, "pos", _I32T, dim=1, device=dev)
    m = int(pos.shape[0])
    _req(q_pos, "q_pos", _I32T, dim=1, numel=n_seqs, device=dev)
    _check_attn_meta(dev, m, hq, head_gain=head_gain, cu_kept=cu_kept)
    _req(cache, "cache", _U8T, device=dev)
    _req(out, "out", _BF16T, numel=n_seqs * hq * d, device=dev, optional=True)
    _req(lse, "lse", _F32T, numel=n_seqs * hq, device=dev, optional=True)
    _req(workspace, "workspace", _U8T, device=dev, optional=True)
    if out is None:
        out = torch.empty((n_seqs, hq, d), dtype=torch.bfloat16, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((hq, n_seqs), dtype=torch.float32, device=dev)
    need = tg_attn_decode_workspace_bytes(n_seqs, int(max_kept_seqlen), hq, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = load().tg_attn_decode(_ptr(q), q.stride(0), _ptr(q_pos), _ptr(head_gain), float(tau), _ptr(pos),
                               _ptr(cu_kept), n_seqs, m, int(max_kept_seqlen), hq, int(n_kv_heads), d,
                               float(rope_base), _ptr(cache), cache.numel(), _ptr(out), _ptr(lse), _ptr(workspace),
                               workspace.numel(), _stream(q))
    _check("tg_attn_decode", st)
    return out, lse



def tg_attn_gate_grads_workspace_bytes(n_seqs, n_kept_total, max_kept_seqlen, n_q_heads, head_dim) -> int:
    return int(load().tg_attn_gate_grads_workspace_bytes(n_seqs, n_kept_total, max_kept_seqlen, n_q_heads,
                                                         head_dim))


def tg_attn_gate_grads(q, v, key_score, head_gain, tau: float, cu_kept, max_kept_seqlen: int, out, lse, d_out,
                       cache, rope_base: float = 1e6, d_score=None, d_gain=None, d_tau=None, workspace=None):
    """dL/dscore, dL/dgain, dL/dtau of a forward run over `cache` (tg_attn_prepare).

    q: [M, Hq, D], v: [M, Hkv, D], out: [M, Hq, D] (the forward's, dense),
    lse: [Hq, M] (the forward's), d_out: [M, Hq, D] bf16.
    Returns (d_score [M], d_gain [Hq], d_tau [1]) fp32.
    """
    _check_q(q)
    _check_q(d_out, "d_out")
    _req(v, "v", _BF16T, dim=3, dense=False, device=q.device)
    if v.stride(2) != 1 or v.stride(1) != v.shape[2]:
        raise ValueError("heads must be contiguous within a token row")
    m, hq, d = q.shape
    hkv = v.shape[1]
    dev = q.device
    if d_out.shape != q.shape or d_out.device != dev or v.shape[0] != m or v.shape[2] != d:
        raise ValueError("q, v and d_out must share the device, the token count and head_dim")
    _req(out, "out", _BF16T, dim=3, numel=m * hq * d, device=dev)
    _req(lse, "lse", _F32T, numel=m * hq, device=dev)
    _check_attn_meta(dev, m, hq, key_score=key_score, head_gain=head_gain, cu_kept=cu_kept)
    _req(cache, "cache", _U8T, device=dev)
    _req(d_score, "d_score", _F32T, dim=1, numel=m, device=dev, optional=True)
    _req(d_gain, "d_gain", _F32T, dim=1, numel=hq, device=dev, optional=True)
    _req(d_tau, "d_tau", _F32T, dim=1, numel=1, device=dev, optional=True)
    _req(workspace, "workspace", _U8T, device=dev, optional=True)
    n_seqs = cu_kept.shape[0] - 1
    if d_score is None:
        d_score = torch.empty(m, dtype=torch.float32, device=dev)
    if d_gain is None:
        d_gain = torch.empty(hq, dtype=torch.float32, device=dev)
    if d_tau is None:
        d_tau = torch.empty(1, dtype=torch.float32, device=dev)
    need = tg_attn_gate_grads_workspace_bytes(n_seqs, m, int(max_kept_seqlen), hq, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = load().tg_attn_gate_grads(_ptr(q), q.stride(0), _ptr(v), v.stride(0), _ptr(key_score), _ptr(head_gain),
                                   float(tau), _ptr(cu_kept), n_seqs, m, int(max_kept_seqlen), hq, hkv, d,
                                   float(rope_base), _ptr(out), _ptr(lse), _ptr(d_out), d_out.stride(0),
                                   _ptr(cache), cache.numel(), _ptr(d_score), _ptr(d_gain), _ptr(d_tau),
                                   _ptr(workspace), workspace.numel(), _stream(q))
    _check("tg_attn_gate_grads", st)
    return d_score, d_gain, d_tau


def tg_random_budgets(seed: int, doc_begin, doc_end):
    """Host call: a uniform random document budget per sequence (int32 numpy array)."""
    db = np.ascontiguousarray(doc_begin, dtype=np.int32)
    de = np.ascontiguousarray(doc_end, dtype=np.int32)
    if db.shape != de.shape or db.ndim != 1:
        raise ValueError("doc_begin and doc_end must be 1-D of one length")
    out = np.empty(len(db), dtype=np.int32)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    st = load().tg_random_budgets(int(seed) % (1 << 64), len(db), p(db), p(de), p(out))
    _check("tg_random_budgets", st)
    return out
