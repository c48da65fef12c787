"""Thin Python binding of librva (argument marshalling only).

Every function has the name of its C entry point without the ``rva_`` prefix, takes
``torch.Tensor`` arguments that live on the GPU (their ``data_ptr()`` is passed as the
device pointer) and plain Python scalars, and enqueues work on the current torch stream
(``torch.cuda.current_stream()``) unless ``stream`` is given.  Nothing is computed here:
every step runs in the HIP kernels of librva.so.  A missing library raises at import of
the first call -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

from .build import LIB_PATH

F32, BF16 = 0, 1
COMPACT, STATIC = 0, 1

DEV_BAD_WINDOW = 0x01
DEV_BAD_TOKEN = 0x02
DEV_BAD_CONF = 0x04
DEV_BAD_COST = 0x08
DEV_BAD_CONTEXT = 0x10
DEV_BAD_PAGE = 0x20
DEV_BAD_ROWS = 0x40

_STATUS = {0: "RVA_OK", 1: "RVA_ERR_INVALID_ARGUMENT", 2: "RVA_ERR_UNSUPPORTED",
           3: "RVA_ERR_WORKSPACE_TOO_SMALL", 4: "RVA_ERR_HIP"}

EXPORTED = [
    "rva_schedule_windows", "rva_pack_ragged", "rva_schedule_and_pack", "rva_verify_attention",
    "rva_verify_attention_workspace_size", "rva_verify_attention_noalloc", "rva_accept_and_commit",
    "rva_accept_workspace_size", "rva_confidence_labels", "rva_accept_capped", "rva_sts_fit",
    "rva_sts_fit_workspace_size", "rva_calibration_ece", "rva_calibration_ece_workspace_size",
    "rva_markov_sample", "rva_markov_workspace_size", "rva_last_error", "rva_version",
]


class RvaError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None

_i, _f, _p, _z = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

_SIGS = {
    "rva_schedule_windows": [_i, _i, _i, _p, _i, _i, _p, _f, _p, _p, _f, _p, _i, _p, _i,
                             _p, _p, _p, _p, _p, _p, _p],
    "rva_pack_ragged": [_i, _i, _p, _p, _p, _i, _p, _z, _p, _i, _p, _p, _p, _p, _p, _p],
    "rva_schedule_and_pack": [_i, _i, _i, _p, _i, _i, _p, _f, _p, _p, _f, _p, _i, _p, _i, _p, _p, _p,
                              _p, _p, _p, _p, _i, _p, _z, _p, _i, _p, _p, _p, _p, _p, _p],
    "rva_verify_attention": [_i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p,
                             _p, _p, _f, _p, _p, _p, _z, _p],
    "rva_verify_attention_workspace_size": [_i, _i, _i, _i, _i, _i, _i, _i],
    "rva_verify_attention_noalloc": [_i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p,
                                     _p, _p, _p, _p, _f, _p, _p, _p],
    "rva_accept_and_commit": [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                              _p, _p, _p, _z, _p],
    "rva_accept_workspace_size": [_i, _i, _i, _i],
    "rva_confidence_labels": [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _z, _p],
    "rva_accept_capped": [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                          _p, _p, _p, _z, _p],
    "rva_sts_fit": [_i, _i, _p, _p, _p, _f, _f, _p, _p, _p, _z, _p],
    "rva_sts_fit_workspace_size": [_i],
    "rva_calibration_ece": [_i, _i, _p, _p, _p, _p, _i, _p, _p, _p, _z, _p],
    "rva_calibration_ece_workspace_size": [_i, _i, _i],
    "rva_markov_sample": [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _z, _p],
    "rva_markov_workspace_size": [_i, _i],
    "rva_last_error": [],
    "rva_version": [],
}
_RESTYPES = {"rva_verify_attention_workspace_size": _z, "rva_accept_workspace_size": _z,
             "rva_sts_fit_workspace_size": _z, "rva_calibration_ece_workspace_size": _z,
             "rva_markov_workspace_size": _z,
             "rva_last_error": ctypes.c_char_p}


def lib(path: str | None = None):
    """Load librva.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    # RVA_LIBRARY: another build of the same library (the host-sanitizer build of the tests)
    path = path or os.environ.get("RVA_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"librva.so not found at {path}: build it first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(path)
    for name, args in _SIGS.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = _RESTYPES.get(name, ctypes.c_int)
    _lib = L
    return L


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor or None")
    if not t.is_cuda:
        raise ValueError("device tensors are required")
    if not t.is_contiguous():
        raise ValueError("contiguous tensors are required")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, status):
    if status != 0:
        raise RvaError(fn, status, lib().rva_last_error().decode())


def version() -> int:
    return lib().rva_version()


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def schedule_windows(B, gamma, mode, hidden, H, head_w, head_b, conf_in, sts_T, bias_ms,
                     alpha_ms, theta_ms, conf_out, surv_out, windows, K_out, ratio_out,
                     device_status=None, stream=None):
    hd = dtype_code(hidden) if hidden is not None else BF16
    _check("rva_schedule_windows", lib().rva_schedule_windows(
        B, gamma, mode, _ptr(hidden), hd, H, _ptr(head_w), float(head_b), _ptr(conf_in),
        _ptr(sts_T), float(bias_ms), _ptr(alpha_ms), alpha_ms.numel(), _ptr(theta_ms),
        theta_ms.numel(), _ptr(conf_out), _ptr(surv_out), _ptr(windows), _ptr(K_out),
        _ptr(ratio_out), _ptr(device_status), _stream(stream)))


def pack_ragged(B, gamma, windows, context_lens, tiers, src, dst, max_rows, cu_seqlens,
                row_req, row_pos, total_tier, device_status=None, stream=None):
    t = (ctypes.c_int32 * len(tiers))(*[int(x) for x in tiers])
    row_bytes = _pack_row_bytes(B, gamma, src, dst)
    _check("rva_pack_ragged", lib().rva_pack_ragged(
        B, gamma, _ptr(windows), _ptr(context_lens), ctypes.cast(t, ctypes.c_void_p), len(tiers),
        _ptr(src), row_bytes, _ptr(dst), max_rows, _ptr(cu_seqlens), _ptr(row_req),
        _ptr(row_pos), _ptr(total_tier), _ptr(device_status), _stream(stream)))


def _pack_row_bytes(B, gamma, src, dst):
    if src is None:
        return 0
    # src is [>= B, gamma, ...] (only the first B blocks are read); a row is one block
    # position's trailing elements
    if src.dim() < 2 or src.shape[0] < B or src.shape[1] != gamma or not src.is_contiguous():
        raise ValueError(f"pack source must be contiguous [>= {B}, {gamma}, ...], "
                         f"got {tuple(src.shape)}")
    row_bytes = src.element_size() * (src.numel() // (src.shape[0] * gamma))
    if dst is None or dst.element_size() * (dst.numel() // max(1, dst.shape[0])) != row_bytes:
        raise ValueError("pack destination rows must have the source's row size")
    return row_bytes


def schedule_and_pack(B, gamma, mode, hidden, H, head_w, head_b, conf_in, sts_T, bias_ms,
                      alpha_ms, theta_ms, conf_out, surv_out, windows, K_out, ratio_out,
                      context_lens, tiers, src, dst, max_rows, cu_seqlens, row_req, row_pos,
                      total_tier, device_status=None, stream=None):
    hd = dtype_code(hidden) if hidden is not None else BF16
    t = (ctypes.c_int32 * len(tiers))(*[int(x) for x in tiers])
    row_bytes = _pack_row_bytes(B, gamma, src, dst)
    _check("rva_schedule_and_pack", lib().rva_schedule_and_pack(
        B, gamma, mode, _ptr(hidden), hd, H, _ptr(head_w), float(head_b), _ptr(conf_in),
        _ptr(sts_T), float(bias_ms), _ptr(alpha_ms), alpha_ms.numel(), _ptr(theta_ms),
        theta_ms.numel(), _ptr(conf_out), _ptr(surv_out), _ptr(windows), _ptr(K_out),
        _ptr(ratio_out), _ptr(context_lens), ctypes.cast(t, ctypes.c_void_p), len(tiers),
        _ptr(src), row_bytes, _ptr(dst), max_rows, _ptr(cu_seqlens), _ptr(row_req),
        _ptr(row_pos), _ptr(total_tier), _ptr(device_status), _stream(stream)))


def verify_attention_workspace_size(B, max_window, Hq, Hkv, D, page_size, max_pages, kv_dtype):
    return lib().rva_verify_attention_workspace_size(B, max_window, Hq, Hkv, D, page_size,
                                                     max_pages, kv_dtype)


def verify_attention(B, max_window, max_rows, Hq, Hkv, D, page_size, num_pages, max_pages, q,
                     k_new, v_new, k_cache, v_cache, block_table, context_lens, cu_seqlens,
                     total_tier, softmax_scale, out, workspace, device_status=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("rva_verify_attention", lib().rva_verify_attention(
        B, max_window, max_rows, Hq, Hkv, D, page_size, num_pages, max_pages, dtype_code(q),
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(context_lens), _ptr(cu_seqlens), _ptr(total_tier), float(softmax_scale), _ptr(out),
        _ptr(device_status), _ptr(workspace), ws_bytes, _stream(stream)))


def verify_attention_noalloc(B, max_window, max_rows, Hq, Hkv, D, page_size, num_pages, max_pages,
                             q, k_new, v_new, k_cache, v_cache, block_table, context_lens,
                             cu_seqlens, total_tier, softmax_scale, out, device_status=None,
                             stream=None):
    _check("rva_verify_attention_noalloc", lib().rva_verify_attention_noalloc(
        B, max_window, max_rows, Hq, Hkv, D, page_size, num_pages, max_pages, dtype_code(q),
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(context_lens), _ptr(cu_seqlens), _ptr(total_tier), float(softmax_scale), _ptr(out),
        _ptr(device_status), _stream(stream)))


def accept_workspace_size(B, gamma, V, max_rows):
    return lib().rva_accept_workspace_size(B, gamma, V, max_rows)


def accept_and_commit(B, gamma, V, max_rows, target_logits, draft_logits, draft_tokens,
                      u_accept, u_resample, cu_seqlens, accept_len, committed, context_lens,
                      p_t_at_draft, p_d_at_draft, labels, workspace, device_status=None,
                      stream=None):
    _check("rva_accept_and_commit", lib().rva_accept_and_commit(
        B, gamma, V, dtype_code(target_logits), max_rows, _ptr(target_logits),
        _ptr(draft_logits), _ptr(draft_tokens), _ptr(u_accept), _ptr(u_resample),
        _ptr(cu_seqlens), _ptr(accept_len), _ptr(committed), _ptr(context_lens),
        _ptr(p_t_at_draft), _ptr(p_d_at_draft), _ptr(labels), _ptr(device_status),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def confidence_labels(B, gamma, V, max_rows, target_logits, draft_logits, cu_seqlens, labels,
                      workspace, device_status=None, stream=None):
    _check("rva_confidence_labels", lib().rva_confidence_labels(
        B, gamma, V, dtype_code(target_logits), max_rows, _ptr(target_logits),
        _ptr(draft_logits), _ptr(cu_seqlens), _ptr(labels), _ptr(device_status),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def accept_capped(B, gamma, V, max_rows, target_logits, draft_logits, draft_tokens, u_accept,
                  u_resample, cu_seqlens, cap_windows, accept_len, accept_len_full, committed,
                  context_lens, p_t_at_draft, p_d_at_draft, labels, workspace,
                  device_status=None, stream=None):
    _check("rva_accept_capped", lib().rva_accept_capped(
        B, gamma, V, dtype_code(target_logits), max_rows, _ptr(target_logits),
        _ptr(draft_logits), _ptr(draft_tokens), _ptr(u_accept), _ptr(u_resample),
        _ptr(cu_seqlens), _ptr(cap_windows), _ptr(accept_len), _ptr(accept_len_full),
        _ptr(committed), _ptr(context_lens), _ptr(p_t_at_draft), _ptr(p_d_at_draft),
        _ptr(labels), _ptr(device_status), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def sts_fit_workspace_size(N):
    return lib().rva_sts_fit_workspace_size(N)


def sts_fit(N, G1, z, accept_len, observed_len, T_lo, T_hi, T_out, nll_out, workspace,
            stream=None):
    _check("rva_sts_fit", lib().rva_sts_fit(
        N, G1, _ptr(z), _ptr(accept_len), _ptr(observed_len), float(T_lo), float(T_hi),
        _ptr(T_out), _ptr(nll_out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def calibration_ece_workspace_size(N, G1, n_bins):
    return lib().rva_calibration_ece_workspace_size(N, G1, n_bins)


def calibration_ece(N, G1, z, accept_len, observed_len, T, n_bins, ece_out, bin_counts,
                    workspace, stream=None):
    _check("rva_calibration_ece", lib().rva_calibration_ece(
        N, G1, _ptr(z), _ptr(accept_len), _ptr(observed_len), _ptr(T), n_bins, _ptr(ece_out),
        _ptr(bin_counts), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def markov_workspace_size(B, V):
    return lib().rva_markov_workspace_size(B, V)


def markov_sample(B, G1, V, r, base_logits, anchor, u, w1, w1_scale, w2, w2_scale, draft_logits,
                  draft_tokens, p_at, workspace, device_status=None, stream=None):
    _check("rva_markov_sample", lib().rva_markov_sample(
        B, G1, V, r, dtype_code(base_logits), _ptr(base_logits), _ptr(anchor), _ptr(u), _ptr(w1),
        _ptr(w1_scale), _ptr(w2), _ptr(w2_scale), _ptr(draft_logits), _ptr(draft_tokens),
        _ptr(p_at), _ptr(device_status), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
