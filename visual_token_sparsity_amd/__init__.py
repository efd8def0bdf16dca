"""SparseVILA decoupled visual sparsity on MI355X: Python binding of libsv.

A thin ctypes layer over the C ABI in include/sv.h.  It marshals torch
tensors (device memory and the current HIP stream) into pointers and sizes;
every step of the computation runs in the HIP kernels of libsv.so.  There is
no CPU fallback: if libsv.so is missing or a tensor is not on a GPU, the call
raises.

    idx = retrieve(q, k_vis, k)                          # query-aware retrieval
    out = sparse_decode_attn(q, k_vis, v_vis, idx,       # attention over the
                             k_txt, v_txt, txt_len)      #   selected + text entries
    out, idx = retrieve_attend(q, k_vis, v_vis, k,       # both, one launch per layer
                               k_txt, v_txt, txt_len)
    sal, keep_idx = salience_prune(vis_q, vis_k, keep)   # prefill salience prune
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch  # loaded first so libsv binds to torch's HIP runtime

__all__ = [
    "SvError", "lib_path", "load", "retrieve", "retrieve_workspace_bytes",
    "sparse_decode_attn", "sparse_decode_attn_workspace_bytes", "salience_prune",
    "salience_prune_workspace_bytes", "new_workspace", "retrieve_attend",
    "retrieve_attend_workspace_bytes", "pack_selected", "summary_salience_prune",
    "summary_salience_prune_workspace_bytes", "workspace_status", "set_wait_limit",
    "prefill_attend_retrieve", "prefill_attend_retrieve_workspace_bytes",
    "SV_F32", "SV_BF16",
]

SV_F32, SV_BF16 = 0, 1
_STATUS = {0: "SV_OK", 1: "SV_EINVAL", 2: "SV_EUNSUPPORTED", 3: "SV_EWORKSPACE", 4: "SV_EHIP"}
_LIB: Optional[ctypes.CDLL] = None


class SvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


def lib_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsv.so")


def load() -> ctypes.CDLL:
    """Load libsv.so (built in-tree by visual_token_sparsity_amd.build)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m visual_token_sparsity_amd.build`")
    lib = ctypes.CDLL(path)
    c_i, c_i64, c_p, c_sz, c_f = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float
    lib.sv_version.restype = c_i
    lib.sv_last_error.restype = ctypes.c_char_p
    lib.sv_retrieve_workspace.argtypes = [c_i, c_i, c_i]
    lib.sv_retrieve_workspace.restype = c_sz
    lib.sv_retrieve.argtypes = [c_p, c_i, c_i, c_i, c_p, c_i64, c_i64, c_i, c_i, c_i, c_i, c_i,
                                c_p, c_p, c_p, c_sz, c_p]
    lib.sv_retrieve.restype = c_i
    lib.sv_sparse_decode_attn_workspace.argtypes = [c_i, c_i, c_i, c_i, c_i, c_i]
    lib.sv_sparse_decode_attn_workspace.restype = c_sz
    lib.sv_sparse_decode_attn.argtypes = [c_p, c_i, c_i, c_p, c_p, c_i64, c_i64, c_i, c_i, c_i,
                                          c_p, c_i, c_p, c_p, c_i64, c_i64, c_p, c_i, c_i, c_f,
                                          c_p, c_p, c_sz, c_p]
    lib.sv_sparse_decode_attn.restype = c_i
    lib.sv_retrieve_attend_workspace.argtypes = [c_i, c_i, c_i, c_i, c_i, c_i, c_i]
    lib.sv_retrieve_attend_workspace.restype = c_sz
    lib.sv_retrieve_attend.argtypes = [c_p, c_i, c_i, c_p, c_p, c_i64, c_i64, c_i, c_i, c_i, c_i,
                                       c_p, c_p, c_i64, c_i64, c_p, c_i, c_i, c_f, c_p, c_p, c_p,
                                       c_p, c_sz, c_p]
    lib.sv_retrieve_attend.restype = c_i
    lib.sv_pack_selected.argtypes = [c_p, c_p, c_i64, c_i64, c_i, c_i, c_i, c_i, c_p, c_i, c_i,
                                     c_p, c_p, c_p]
    lib.sv_pack_selected.restype = c_i
    lib.sv_salience_prune_workspace.argtypes = [c_i, c_i, c_i]
    lib.sv_salience_prune_workspace.restype = c_sz
    lib.sv_salience_prune.argtypes = [c_p, c_p, c_i, c_i, c_i, c_i, c_i, c_f, c_i, c_p, c_p,
                                      c_p, c_sz, c_p]
    lib.sv_salience_prune.restype = c_i
    lib.sv_summary_salience_prune_workspace.argtypes = [c_i, c_i, c_i]
    lib.sv_summary_salience_prune_workspace.restype = c_sz
    lib.sv_summary_salience_prune.argtypes = [c_p, c_p, c_i, c_i, c_i, c_i, c_i, c_f, c_i, c_i,
                                              c_p, c_p, c_p, c_sz, c_p]
    lib.sv_summary_salience_prune.restype = c_i
    lib.sv_prefill_attend_retrieve_workspace.argtypes = [c_i, c_i, c_i, c_i, c_i, c_i, c_i]
    lib.sv_prefill_attend_retrieve_workspace.restype = c_sz
    lib.sv_prefill_attend_retrieve.argtypes = [c_p, c_i, c_i, c_i, c_p, c_p, c_i64, c_i64, c_i,
                                               c_i, c_i, c_p, c_p, c_i64, c_i64, c_p, c_i, c_i,
                                               c_f, c_i, c_p, c_p, c_p, c_p, c_sz, c_p]
    lib.sv_prefill_attend_retrieve.restype = c_i
    lib.sv_workspace_status.argtypes = [c_p, c_p]
    lib.sv_workspace_status.restype = c_i
    lib.sv_set_wait_limit.argtypes = [ctypes.c_uint32]
    lib.sv_set_wait_limit.restype = ctypes.c_uint32
    _LIB = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        raise SvError(status, load().sv_last_error().decode())


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _on_gpu(*ts: torch.Tensor) -> torch.device:
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("libsv runs on the GPU only: every tensor must be on a HIP device")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same device")
    return dev


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _cache_strides(t: torch.Tensor, name: str) -> Tuple[int, int]:
    """[B][T][H][D] cache with contiguous [H][D] rows; returns (batch, token) strides."""
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B][T][H][D]")
    if t.stride(3) != 1 or t.stride(2) != t.shape[3]:
        raise ValueError(f"{name}: each token row must be a contiguous [H][D] block")
    return t.stride(0), t.stride(1)


def _workspace(nbytes: int, dev, ws: Optional[torch.Tensor]) -> torch.Tensor:
    """The caller's workspace, or a fresh zero-filled one.

    Workspaces must be zero-filled before their first use; each call leaves
    its completion counters at zero, so a workspace can be reused as is.
    """
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return ws
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """A zero-filled workspace of ``nbytes`` bytes, reusable across calls."""
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)


def prefill_attend_retrieve_workspace_bytes(B: int, Tq: int, Hq: int, Hkv: int, D: int, N: int,
                                            Tmax: int) -> int:
    return int(load().sv_prefill_attend_retrieve_workspace(B, Tq, Hq, Hkv, D, N, Tmax))


def prefill_attend_retrieve(q: torch.Tensor, k_vis: torch.Tensor, v_vis: torch.Tensor,
                            k_txt: Optional[torch.Tensor], v_txt: Optional[torch.Tensor],
                            txt_len: Optional[torch.Tensor], k: int,
                            scale: Optional[float] = None, *, scores: bool = False,
                            workspace: Optional[torch.Tensor] = None,
                            out: Optional[torch.Tensor] = None,
                            idx_out: Optional[torch.Tensor] = None):
    """Causal prefill attention of a question chunk plus the query-aware retrieval
    of its top-k visual tokens, from one pass over the caches.

    q        [B][Tq][Hq][D] bf16 (the question's tokens)
    k_vis, v_vis  [B][N][Hkv][D] (same strides)
    k_txt, v_txt  [B][Tmax][Hkv][D] (same strides; the last Tq of the txt_len[b]
             valid rows are the question's own) or None
    txt_len  int32 [B] on the device, or None when there is no text
    returns (out fp32 [B][Tq][Hq][D], idx int32 [B][k] ascending[, scores fp32 [B][N]])
    """
    lib = load()
    dev = _on_gpu(q, k_vis, v_vis, k_txt, v_txt, txt_len)
    if q.dtype != torch.bfloat16 or k_vis.dtype != q.dtype or v_vis.dtype != q.dtype:
        raise TypeError("prefill_attend_retrieve takes bf16 q and caches")
    q = q.contiguous()
    B, Tq, Hq, D = q.shape
    _, N, Hkv, Dk = k_vis.shape
    if Dk != D or k_vis.shape[0] != B:
        raise ValueError("q and k_vis shapes disagree")
    if k_vis.stride() != v_vis.stride() or k_vis.shape != v_vis.shape:
        raise ValueError("k_vis and v_vis must share shape and strides")
    vbs, vts = _cache_strides(k_vis, "k_vis")
    if k_txt is not None:
        if k_txt.stride() != v_txt.stride() or k_txt.shape != v_txt.shape:
            raise ValueError("k_txt and v_txt must share shape and strides")
        tbs, tts = _cache_strides(k_txt, "k_txt")
        Tmax = k_txt.shape[1]
        if txt_len is None or txt_len.dtype != torch.int32:
            raise TypeError("txt_len must be an int32 device tensor")
        txt_len = txt_len.contiguous()
    else:
        tbs = tts = Tmax = 0
    res = out if out is not None else torch.empty((B, Tq, Hq, D), dtype=torch.float32, device=dev)
    idx = idx_out if idx_out is not None else torch.empty((B, max(k, 0)), dtype=torch.int32, device=dev)
    sc = torch.empty((B, N), dtype=torch.float32, device=dev) if scores else None
    ws = _workspace(prefill_attend_retrieve_workspace_bytes(B, Tq, Hq, Hkv, D, N, Tmax), dev,
                    workspace)
    ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
    _check(lib.sv_prefill_attend_retrieve(
        q.data_ptr(), B, Tq, Hq, k_vis.data_ptr(), v_vis.data_ptr(), vbs, vts, N, Hkv, D,
        ptr(k_txt), ptr(v_txt), tbs, tts, ptr(txt_len) if Tmax else None, Tmax, SV_BF16,
        float(scale) if scale else 0.0, k, res.data_ptr(), idx.data_ptr() if k > 0 else None,
        ptr(sc), ws.data_ptr(), ws.numel() * ws.element_size(), _stream(dev)))
    return (res, idx, sc) if scores else (res, idx)


def workspace_status(workspace: torch.Tensor) -> None:
    """Raise SvError if a bounded in-kernel wait of a call on this workspace
    (retrieve on rows over 2048 tokens, retrieve_attend) gave up since it was
    zeroed.  Waits for the current stream."""
    dev = _on_gpu(workspace)
    _check(load().sv_workspace_status(ctypes.c_void_p(workspace.data_ptr()), _stream(dev)))


def set_wait_limit(polls: int) -> int:
    """Bound of the in-kernel waits, in polls, for later launches (0: the
    default); returns the previous bound.  For testing the give-up path."""
    return int(load().sv_set_wait_limit(polls))


def retrieve_workspace_bytes(B: int, N: int, k: int) -> int:
    return int(load().sv_retrieve_workspace(B, N, k))


def retrieve(q: torch.Tensor, k_vis: torch.Tensor, k: int, *, scores: bool = False,
             workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None):
    """Top-k visual tokens per sequence for the query ``q``.

    q      [B][Tq][Hq][D] (or [B][Hq][D]) bf16/fp32, contiguous
    k_vis  [B][N][Hkv][D] same dtype, token rows contiguous
    returns idx int32 [B][k] ascending (and fp32 scores [B][N] if ``scores``)
    """
    lib = load()
    if q.dim() == 3:
        q = q.unsqueeze(1)
    dev = _on_gpu(q, k_vis)
    if q.dtype != k_vis.dtype:
        raise TypeError("q and k_vis must share a dtype")
    q = q.contiguous()
    B, Tq, Hq, D = q.shape
    _, N, Hkv, Dk = k_vis.shape
    if Dk != D or k_vis.shape[0] != B:
        raise ValueError("q and k_vis shapes disagree")
    bs, ts = _cache_strides(k_vis, "k_vis")
    idx = out if out is not None else torch.empty((B, max(k, 0)), dtype=torch.int32, device=dev)
    sc = torch.empty((B, N), dtype=torch.float32, device=dev) if scores else None
    ws = _workspace(retrieve_workspace_bytes(B, N, k), dev, workspace)
    _check(lib.sv_retrieve(q.data_ptr(), B, Tq, Hq, k_vis.data_ptr(), bs, ts, N, Hkv, D,
                           _dtype(q), k, idx.data_ptr(), sc.data_ptr() if sc is not None else None,
                           ws.data_ptr(), ws.numel() * ws.element_size(), _stream(dev)))
    return (idx, sc) if scores else idx


def sparse_decode_attn_workspace_bytes(B: int, Hq: int, Hkv: int, D: int, k: int, Tmax: int) -> int:
    return int(load().sv_sparse_decode_attn_workspace(B, Hq, Hkv, D, k, Tmax))


def sparse_decode_attn(q: torch.Tensor, k_vis: torch.Tensor, v_vis: torch.Tensor,
                       idx: "torch.Tensor | int", k_txt: Optional[torch.Tensor],
                       v_txt: Optional[torch.Tensor], txt_len: Optional[torch.Tensor],
                       scale: Optional[float] = None, *,
                       workspace: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Attention of the current token over the selected visual entries plus the text entries.

    q        [B][Hq][D] (or [B][1][Hq][D])
    k_vis, v_vis  [B][N][Hkv][D] (same strides)
    idx      int32 [B][k], or an int k: the visual rows 0..k-1 (a packed cache; no index list)
    k_txt, v_txt  [B][Tmax][Hkv][D] (same strides) or None
    txt_len  int32 [B] on the device (rows attended), or None when there is no text
    returns fp32 [B][Hq][D]
    """
    lib = load()
    if q.dim() == 4:
        q = q[:, 0]
    rows = isinstance(idx, int)
    dev = _on_gpu(q, k_vis, v_vis, None if rows else idx, k_txt, v_txt, txt_len)
    q = q.contiguous()
    B, Hq, D = q.shape
    _, N, Hkv, _ = k_vis.shape
    if k_vis.stride() != v_vis.stride() or k_vis.shape != v_vis.shape:
        raise ValueError("k_vis and v_vis must share shape and strides")
    vbs, vts = _cache_strides(k_vis, "k_vis")
    if rows:
        k = idx
        idx = None
    else:
        if idx.dtype != torch.int32:
            raise TypeError("idx must be int32")
        idx = idx.contiguous()
        k = idx.shape[1]
    if k_txt is not None:
        if k_txt.stride() != v_txt.stride() or k_txt.shape != v_txt.shape:
            raise ValueError("k_txt and v_txt must share shape and strides")
        tbs, tts = _cache_strides(k_txt, "k_txt")
        Tmax = k_txt.shape[1]
        if txt_len is None or txt_len.dtype != torch.int32:
            raise TypeError("txt_len must be an int32 device tensor")
        txt_len = txt_len.contiguous()
    else:
        tbs = tts = Tmax = 0
    res = out if out is not None else torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws = _workspace(sparse_decode_attn_workspace_bytes(B, Hq, Hkv, D, k, Tmax), dev, workspace)
    ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
    _check(lib.sv_sparse_decode_attn(
        q.data_ptr(), B, Hq, k_vis.data_ptr(), v_vis.data_ptr(), vbs, vts, N, Hkv, D,
        ptr(idx), k, ptr(k_txt), ptr(v_txt), tbs, tts, ptr(txt_len) if Tmax else None, Tmax,
        _dtype(q), float(scale) if scale else 0.0, res.data_ptr(), ws.data_ptr(),
        ws.numel() * ws.element_size(), _stream(dev)))
    return res


def pack_selected(k_vis: torch.Tensor, v_vis: torch.Tensor, idx: torch.Tensor, *,
                  out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None
                  ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Copy the selected visual rows into contiguous [B][k][Hkv][D] buffers.

    k_vis, v_vis  [B][N][Hkv][D] (same strides), bf16/fp32
    idx           int32 [B][k]; an index outside [0, N) gives a zero row
    returns (k_pack, v_pack), same dtype as the caches
    """
    lib = load()
    dev = _on_gpu(k_vis, v_vis, idx)
    if k_vis.stride() != v_vis.stride() or k_vis.shape != v_vis.shape or k_vis.dtype != v_vis.dtype:
        raise ValueError("k_vis and v_vis must share shape, strides and dtype")
    bs, ts = _cache_strides(k_vis, "k_vis")
    if idx.dtype != torch.int32 or idx.dim() != 2 or idx.shape[0] != k_vis.shape[0]:
        raise TypeError("idx must be int32 [B][k]")
    idx = idx.contiguous()
    B, N, Hkv, D = k_vis.shape
    k = idx.shape[1]
    if out is not None:
        kp, vp = out
        for t in (kp, vp):
            if t.shape != (B, k, Hkv, D) or t.dtype != k_vis.dtype or not t.is_contiguous():
                raise ValueError("out buffers must be contiguous [B][k][Hkv][D] of the cache dtype")
    else:
        kp = torch.empty((B, k, Hkv, D), dtype=k_vis.dtype, device=dev)
        vp = torch.empty_like(kp)
    _check(lib.sv_pack_selected(k_vis.data_ptr(), v_vis.data_ptr(), bs, ts, N, Hkv, D,
                                _dtype(k_vis), idx.data_ptr(), B, k, kp.data_ptr(), vp.data_ptr(),
                                _stream(dev)))
    return kp, vp


def retrieve_attend_workspace_bytes(B: int, Hq: int, Hkv: int, D: int, N: int, k: int,
                                    Tmax: int) -> int:
    return int(load().sv_retrieve_attend_workspace(B, Hq, Hkv, D, N, k, Tmax))


def retrieve_attend(q: torch.Tensor, k_vis: torch.Tensor, v_vis: torch.Tensor, k: int,
                    k_txt: Optional[torch.Tensor], v_txt: Optional[torch.Tensor],
                    txt_len: Optional[torch.Tensor], scale: Optional[float] = None, *,
                    scores: bool = False, workspace: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, idx_out: Optional[torch.Tensor] = None):
    """One decode layer in one launch: top-k retrieval for ``q`` and attention over
    the selected visual entries plus the text entries.

    q        [B][Hq][D] (or [B][1][Hq][D]): one decode token
    k_vis, v_vis  [B][N][Hkv][D] (same strides)
    k        visual tokens selected and attended (1 <= k <= N)
    k_txt, v_txt  [B][Tmax][Hkv][D] (same strides) or None
    txt_len  int32 [B] on the device, or None when there is no text
    returns (out fp32 [B][Hq][D], idx int32 [B][k] ascending[, scores fp32 [B][N]])
    """
    lib = load()
    if q.dim() == 4:
        if q.shape[1] != 1:
            raise ValueError("retrieve_attend takes one decode token per sequence")
        q = q[:, 0]
    dev = _on_gpu(q, k_vis, v_vis, k_txt, v_txt, txt_len)
    if q.dtype != k_vis.dtype or v_vis.dtype != k_vis.dtype:
        raise TypeError("q, k_vis and v_vis must share a dtype")
    q = q.contiguous()
    B, Hq, D = q.shape
    _, N, Hkv, Dk = k_vis.shape
    if Dk != D or k_vis.shape[0] != B:
        raise ValueError("q and k_vis shapes disagree")
    if k_vis.stride() != v_vis.stride() or k_vis.shape != v_vis.shape:
        raise ValueError("k_vis and v_vis must share shape and strides")
    vbs, vts = _cache_strides(k_vis, "k_vis")
    if k_txt is not None:
        if k_txt.stride() != v_txt.stride() or k_txt.shape != v_txt.shape:
            raise ValueError("k_txt and v_txt must share shape and strides")
        if k_txt.dtype != q.dtype:
            raise TypeError("k_txt must share the dtype of q")
        tbs, tts = _cache_strides(k_txt, "k_txt")
        Tmax = k_txt.shape[1]
        if txt_len is None or txt_len.dtype != torch.int32:
            raise TypeError("txt_len must be an int32 device tensor")
        txt_len = txt_len.contiguous()
    else:
        tbs = tts = Tmax = 0
    res = out if out is not None else torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    idx = idx_out if idx_out is not None else torch.empty((B, max(k, 0)), dtype=torch.int32, device=dev)
    sc = torch.empty((B, N), dtype=torch.float32, device=dev) if scores else None
    ws = _workspace(retrieve_attend_workspace_bytes(B, Hq, Hkv, D, N, k, Tmax), dev, workspace)
    ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
    _check(lib.sv_retrieve_attend(
        q.data_ptr(), B, Hq, k_vis.data_ptr(), v_vis.data_ptr(), vbs, vts, N, Hkv, D, k,
        ptr(k_txt), ptr(v_txt), tbs, tts, ptr(txt_len) if Tmax else None, Tmax, _dtype(q),
        float(scale) if scale else 0.0, idx.data_ptr(), ptr(sc), res.data_ptr(), ws.data_ptr(),
        ws.numel() * ws.element_size(), _stream(dev)))
    return (res, idx, sc) if scores else (res, idx)


def salience_prune_workspace_bytes(F: int, H: int, N: int) -> int:
    return int(load().sv_salience_prune_workspace(F, H, N))


def salience_prune(vis_q: torch.Tensor, vis_k: torch.Tensor, keep: int,
                   scale: Optional[float] = None, *, workspace: Optional[torch.Tensor] = None,
                   salience_out: Optional[torch.Tensor] = None,
                   idx_out: Optional[torch.Tensor] = None):
    """Column-mean salience per token and the ``keep`` most salient tokens per frame.

    vis_q, vis_k  [F][H][N][D] bf16, contiguous
    returns (salience fp32 [F][N], idx int32 [F][keep] ascending)
    """
    lib = load()
    dev = _on_gpu(vis_q, vis_k)
    if vis_q.shape != vis_k.shape or vis_q.dim() != 4:
        raise ValueError("vis_q and vis_k must both be [F][H][N][D]")
    vis_q, vis_k = vis_q.contiguous(), vis_k.contiguous()
    F, H, N, D = vis_q.shape
    sal = salience_out if salience_out is not None else torch.empty((F, N), dtype=torch.float32, device=dev)
    idx = idx_out if idx_out is not None else torch.empty((F, max(keep, 0)), dtype=torch.int32, device=dev)
    ws = _workspace(salience_prune_workspace_bytes(F, H, N), dev, workspace)
    _check(lib.sv_salience_prune(vis_q.data_ptr(), vis_k.data_ptr(), F, H, N, D, _dtype(vis_q),
                                 float(scale) if scale else 0.0, keep, sal.data_ptr(),
                                 idx.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                                 _stream(dev)))
    return sal, idx


def summary_salience_prune_workspace_bytes(F: int, H: int, N: int) -> int:
    return int(load().sv_summary_salience_prune_workspace(F, H, N))


def summary_salience_prune(vis_q: torch.Tensor, vis_k: torch.Tensor, S: int, keep: int,
                           scale: Optional[float] = None, *,
                           workspace: Optional[torch.Tensor] = None,
                           salience_out: Optional[torch.Tensor] = None,
                           idx_out: Optional[torch.Tensor] = None):
    """Salience from the attention of the first ``S`` (summary) tokens, and the
    ``keep`` most salient tokens per frame.

    vis_q, vis_k  [F][H][N][D] bf16, contiguous (rows 0..S-1 of vis_q are read)
    returns (salience fp32 [F][N], idx int32 [F][keep] ascending)
    """
    lib = load()
    dev = _on_gpu(vis_q, vis_k)
    if vis_q.shape != vis_k.shape or vis_q.dim() != 4:
        raise ValueError("vis_q and vis_k must both be [F][H][N][D]")
    vis_q, vis_k = vis_q.contiguous(), vis_k.contiguous()
    F, H, N, D = vis_q.shape
    sal = salience_out if salience_out is not None else torch.empty((F, N), dtype=torch.float32, device=dev)
    idx = idx_out if idx_out is not None else torch.empty((F, max(keep, 0)), dtype=torch.int32, device=dev)
    ws = _workspace(summary_salience_prune_workspace_bytes(F, H, N), dev, workspace)
    _check(lib.sv_summary_salience_prune(vis_q.data_ptr(), vis_k.data_ptr(), F, H, N, D,
                                         _dtype(vis_q), float(scale) if scale else 0.0, S, keep,
                                         sal.data_ptr(), idx.data_ptr(), ws.data_ptr(),
                                         ws.numel() * ws.element_size(), _stream(dev)))
    return sal, idx
