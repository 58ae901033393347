"""ctypes binding of libtt (include/tt.h).

Argument marshalling only: shape/dtype/device checks, device pointers, the
current torch stream, and workspace buffers allocated through torch.  Every
step of the computation runs in the HIP kernels of libtt.so; there is no CPU
or PyTorch fallback.  If the library is missing, every call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtt.so")

TT_OK, TT_EINVAL, TT_EUNSUPPORTED, TT_ENODEV, TT_EHIP = range(5)
TT_FP32, TT_BF16 = 0, 1
TT_ATTN_AUTO, TT_ATTN_MFMA, TT_ATTN_SHUFFLE = 0, 1, 2
_PATHS = {"auto": TT_ATTN_AUTO, "mfma": TT_ATTN_MFMA, "shuffle": TT_ATTN_SHUFFLE}
SIZE_MAX = ctypes.c_size_t(-1).value
NOALLOC_SCRATCH_BYTES = 8 << 20     # TT_NOALLOC_SCRATCH_BYTES


class TTError(RuntimeError):
    """A libtt entry point returned a status other than TT_OK."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


class AttnOpts(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int), ("kv_splits", ctypes.c_int), ("kv_groups", ctypes.c_int),
                ("rows_per_wave", ctypes.c_int), ("stream_waves", ctypes.c_int)]


class Select(ctypes.Structure):
    """tt_select: the selection rule of one unmasking step."""
    _fields_ = [("mode", ctypes.c_int), ("k", ctypes.c_int), ("gamma", ctypes.c_float),
                ("steps_left", ctypes.c_int), ("step", ctypes.c_int), ("n_steps", ctypes.c_int)]


SELECT_MODES = {"top_k": 0, "threshold": 1, "schedule": 2, "leftmost": 3}


def select_rule(mode: str, *, k: int = 0, gamma: float = 0.0, steps_left: int = 1, step: int = 1,
                n_steps: int = 1) -> Select:
    """Build a tt_select: "top_k" (k), "threshold" (gamma, steps_left),
    "schedule" (step, n_steps) or "leftmost" (k)."""
    _require(mode in SELECT_MODES, f"unknown selection mode {mode!r}")
    return Select(SELECT_MODES[mode], int(k), float(gamma), int(steps_left), int(step),
                  int(n_steps))


_lib = None
_lock = threading.Lock()

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_SIGNATURES = {
    "tt_status_string": (ctypes.c_char_p, [_i]),
    "tt_version": (ctypes.c_char_p, []),
    "tt_block_attn_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, ctypes.POINTER(AttnOpts)]),
    "tt_block_attn": (_i, [_vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _f, _vp, _i, _i, _i, _i,
                           _vp, _sz, _vp]),
    "tt_block_attn_ex": (_i, [_vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _f, _vp, _i, _i, _i,
                              _i, _vp, _sz, _vp, ctypes.POINTER(AttnOpts)]),
    "tt_block_attn_varlen": (_i, [_vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _f, _vp, _i,
                                  _i, _i, _i, _vp, _sz, _vp, ctypes.POINTER(AttnOpts)]),
    "tt_block_attn_multiblock_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i,
                                                       ctypes.POINTER(AttnOpts)]),
    "tt_block_attn_multiblock": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _i,
                                      _i, _i, _i, _vp, _sz, _vp, ctypes.POINTER(AttnOpts)]),
    "tt_lmhead_unmask_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "tt_lmhead_unmask_step": (_i, [_vp, _vp, _vp, ctypes.POINTER(Select), _vp, _vp, _i, _i, _i, _i,
                                   _vp, _vp, _vp, _sz, _vp]),
    "tt_unmask_workspace_bytes": (_sz, [_i, _i, _i]),
    "tt_unmask_step": (_i, [_vp, _vp, _i, _vp, _vp, _i, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "tt_unmask_step_noalloc": (_i, [_vp, _vp, _i, _vp, _vp, _i, _i, _i, _vp, _vp, _vp]),
    "tt_unmask_reduce": (_i, [_vp, _vp, _i, _i, _i, _vp, _sz, _vp]),
    "tt_unmask_commit": (_i, [_vp, _i, _vp, _vp, _i, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "tt_unmask_step_ex": (_i, [_vp, _vp, ctypes.POINTER(Select), _vp, _vp, _i, _i, _i, _vp, _vp,
                               _vp, _sz, _vp]),
    "tt_unmask_commit_ex": (_i, [_vp, ctypes.POINTER(Select), _vp, _vp, _i, _i, _i, _vp, _vp, _vp,
                                 _sz, _vp]),
}


def lib() -> ctypes.CDLL:
    """Load libtt.so (once).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m denoiser_attention_amd.build` "
                    "(hipcc, gfx950).  There is no fallback implementation.")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().tt_status_string(status).decode()


def version() -> str:
    return lib().tt_version().decode()


def _check(status: int, what: str) -> None:
    if status != TT_OK:
        raise TTError(status, what)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return TT_FP32
    if t == torch.bfloat16:
        return TT_BF16
    raise TypeError(f"unsupported dtype {t}; expected float32 or bfloat16")


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device, stream) -> int:
    s = torch.cuda.current_stream(device) if stream is None else stream
    return s.cuda_stream


def _on(stream):
    """Context in which the binding allocates its own workspaces and outputs:
    the launch stream, so that the caching allocator never hands such a
    buffer to another stream while a kernel on `stream` may still use it."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _cuda_contig(name: str, t: torch.Tensor, device: torch.device) -> None:
    _require(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _require(t.is_cuda and t.device == device, f"{name} must be on {device}")
    _require(t.is_contiguous(), f"{name} must be contiguous")


def attn_workspace_bytes(batch, prefix_len, block_len, n_q_heads, n_kv_heads, head_dim,
                         dtype: torch.dtype, path: str = "auto", kv_splits: int = 0,
                         kv_groups: int = 0, rows_per_wave: int = 0, stream_waves: int = 0) -> int:
    opts = AttnOpts(_PATHS[path], kv_splits, kv_groups, rows_per_wave, stream_waves)
    n = lib().tt_block_attn_workspace_bytes(batch, prefix_len, block_len, n_q_heads, n_kv_heads,
                                            head_dim, _dtype_code(dtype), ctypes.byref(opts))
    if n == SIZE_MAX:
        raise ValueError("invalid attention shape")
    return n


def block_attn(q, k_ctx, v_ctx, prefix_len, k_blk, v_blk, scale, *, out=None, out_dtype=None,
               path: str = "auto", kv_splits: int = 0, kv_groups: int = 0, rows_per_wave: int = 0,
               stream_waves: int = 0, workspace=None, stream=None):
    """Eq. (1) block attention through tt_block_attn_ex; returns ``out``.

    q [B,Hq,L,D]; k_ctx/v_ctx [B,Hkv,Pcap,D] (or None when prefix_len == 0);
    k_blk/v_blk [B,Hkv,L,D]; all float32 or all bfloat16 on one GPU.
    """
    _require(q.dim() == 4, "q must be [B, Hq, L, D]")
    device = q.device
    B, Hq, L, D = q.shape
    for name, t in (("q", q), ("k_blk", k_blk), ("v_blk", v_blk)):
        _cuda_contig(name, t, device)
        _require(t.dtype == q.dtype, f"{name} dtype differs from q")
    _require(k_blk.dim() == 4 and k_blk.shape[0] == B and k_blk.shape[2] == L
             and k_blk.shape[3] == D, "k_blk must be [B, Hkv, L, D]")
    _require(v_blk.shape == k_blk.shape, "v_blk must match k_blk")
    Hkv = k_blk.shape[1]
    if k_ctx is None or v_ctx is None:
        _require(k_ctx is None and v_ctx is None and prefix_len == 0,
                 "k_ctx/v_ctx may be omitted only when prefix_len == 0")
        Pcap = 0
    else:
        for name, t in (("k_ctx", k_ctx), ("v_ctx", v_ctx)):
            _cuda_contig(name, t, device)
            _require(t.dtype == q.dtype, f"{name} dtype differs from q")
        _require(k_ctx.dim() == 4 and k_ctx.shape[0] == B and k_ctx.shape[1] == Hkv
                 and k_ctx.shape[3] == D, "k_ctx must be [B, Hkv, Pcap, D]")
        _require(v_ctx.shape == k_ctx.shape, "v_ctx must match k_ctx")
        Pcap = k_ctx.shape[2]
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        with _on(stream):
            out = torch.empty((B, Hq, L, D), dtype=out_dtype, device=device)
    _cuda_contig("out", out, device)
    _require(tuple(out.shape) == (B, Hq, L, D), "out must be [B, Hq, L, D]")
    opts = AttnOpts(_PATHS[path], kv_splits, kv_groups, rows_per_wave, stream_waves)
    need = attn_workspace_bytes(B, prefix_len, L, Hq, Hkv, D, q.dtype, path, kv_splits, kv_groups,
                                rows_per_wave, stream_waves)
    if need and workspace is None:
        with _on(stream):
            workspace = torch.empty(need, dtype=torch.uint8, device=device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().tt_block_attn_ex(
        _ptr(q), _ptr(k_ctx), _ptr(v_ctx), prefix_len, _ptr(k_blk), _ptr(v_blk), L, Hq, Hkv, D,
        float(scale), _ptr(out), B, Pcap, _dtype_code(q.dtype), _dtype_code(out.dtype),
        _ptr(workspace), ws_bytes, _stream(device, stream), ctypes.byref(opts))
    _check(st, "tt_block_attn")
    return out


def _ctx_checks(k_ctx, v_ctx, q, B, Hkv, D, device, need_rows):
    if k_ctx is None or v_ctx is None:
        _require(k_ctx is None and v_ctx is None and need_rows == 0,
                 "k_ctx/v_ctx may be omitted only when no cache row is visible")
        return 0
    for name, t in (("k_ctx", k_ctx), ("v_ctx", v_ctx)):
        _cuda_contig(name, t, device)
        _require(t.dtype == q.dtype, f"{name} dtype differs from q")
    _require(k_ctx.dim() == 4 and k_ctx.shape[0] == B and k_ctx.shape[1] == Hkv
             and k_ctx.shape[3] == D, "k_ctx must be [B, Hkv, cap, D]")
    _require(v_ctx.shape == k_ctx.shape, "v_ctx must match k_ctx")
    return k_ctx.shape[2]


def block_attn_varlen(q, k_ctx, v_ctx, prefix_lens, max_prefix_len, k_blk, v_blk, scale, *,
                      out=None, out_dtype=None, path: str = "auto", kv_splits: int = 0,
                      kv_groups: int = 0, rows_per_wave: int = 0,
                      stream_waves: int = 0, workspace=None, stream=None):
    """Eq. (1) with a prefix length per batch entry (tt_block_attn_varlen).
    ``prefix_lens`` is an int32 tensor [B] on the same GPU, every value in
    [0, max_prefix_len]."""
    args, out, _ = _varlen_args(q, k_ctx, v_ctx, prefix_lens, max_prefix_len, k_blk, v_blk, scale,
                                out, out_dtype, path, kv_splits, kv_groups, rows_per_wave,
                                stream_waves, workspace, stream)
    _check(lib().tt_block_attn_varlen(*args), "tt_block_attn_varlen")
    return out


def prepare_block_attn_varlen(q, k_ctx, v_ctx, prefix_lens, max_prefix_len, k_blk, v_blk, scale,
                              out, *, path: str = "auto", kv_splits: int = 0, kv_groups: int = 0,
                              rows_per_wave: int = 0, stream_waves: int = 0, workspace=None,
                              stream=None):
    """Validate once (same checks as block_attn_varlen), make one call, and
    return a Prepared call."""
    args, out, keep = _varlen_args(q, k_ctx, v_ctx, prefix_lens, max_prefix_len, k_blk, v_blk,
                                   scale, out, None, path, kv_splits, kv_groups, rows_per_wave,
                                   stream_waves, workspace, stream)
    call = Prepared(lib().tt_block_attn_varlen, args, "tt_block_attn_varlen", keep)
    call()
    return call


def _varlen_args(q, k_ctx, v_ctx, prefix_lens, max_prefix_len, k_blk, v_blk, scale, out, out_dtype,
                 path, kv_splits, kv_groups, rows_per_wave, stream_waves, workspace, stream):
    _require(q.dim() == 4, "q must be [B, Hq, L, D]")
    device = q.device
    B, Hq, L, D = q.shape
    for name, t in (("q", q), ("k_blk", k_blk), ("v_blk", v_blk)):
        _cuda_contig(name, t, device)
        _require(t.dtype == q.dtype, f"{name} dtype differs from q")
    _require(k_blk.dim() == 4 and k_blk.shape[0] == B and k_blk.shape[2] == L
             and k_blk.shape[3] == D and v_blk.shape == k_blk.shape, "k_blk/v_blk: [B, Hkv, L, D]")
    Hkv = k_blk.shape[1]
    _cuda_contig("prefix_lens", prefix_lens, device)
    _require(prefix_lens.dtype == torch.int32 and tuple(prefix_lens.shape) == (B,),
             "prefix_lens: int32 [B]")
    Pcap = _ctx_checks(k_ctx, v_ctx, q, B, Hkv, D, device, max_prefix_len)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        with _on(stream):
            out = torch.empty((B, Hq, L, D), dtype=out_dtype, device=device)
    _cuda_contig("out", out, device)
    _require(tuple(out.shape) == (B, Hq, L, D), "out must be [B, Hq, L, D]")
    opts = AttnOpts(_PATHS[path], kv_splits, kv_groups, rows_per_wave, stream_waves)
    need = attn_workspace_bytes(B, max_prefix_len, L, Hq, Hkv, D, q.dtype, path, kv_splits,
                                kv_groups, rows_per_wave, stream_waves)
    if need and workspace is None:
        with _on(stream):
            workspace = torch.empty(need, dtype=torch.uint8, device=device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(q), _ptr(k_ctx), _ptr(v_ctx), _ptr(prefix_lens), int(max_prefix_len), _ptr(k_blk),
            _ptr(v_blk), L, Hq, Hkv, D, float(scale), _ptr(out), B, Pcap, _dtype_code(q.dtype),
            _dtype_code(out.dtype), _ptr(workspace), ws_bytes, _stream(device, stream),
            ctypes.byref(opts))
    return args, out, (q, k_ctx, v_ctx, prefix_lens, k_blk, v_blk, out, workspace, opts)


def attn_multiblock_workspace_bytes(batch, block_size, n_blocks, n_q_heads, n_kv_heads, head_dim,
                                    dtype: torch.dtype, path: str = "auto", kv_splits: int = 0,
                                    kv_groups: int = 0, rows_per_wave: int = 0,
                                    stream_waves: int = 0) -> int:
    opts = AttnOpts(_PATHS[path], kv_splits, kv_groups, rows_per_wave, stream_waves)
    n = lib().tt_block_attn_multiblock_workspace_bytes(batch, block_size, n_blocks, n_q_heads,
                                                       n_kv_heads, head_dim, _dtype_code(dtype),
                                                       ctypes.byref(opts))
    if n == SIZE_MAX:
        raise ValueError("invalid attention shape")
    return n


def block_attn_multiblock(q, k_ctx, v_ctx, k_noisy, v_noisy, block_size, scale, *, out=None,
                          out_dtype=None, path: str = "auto", kv_splits: int = 0,
                          kv_groups: int = 0, rows_per_wave: int = 0,
                          stream_waves: int = 0, workspace=None, stream=None):
    """Training-style pass over all noisy blocks (tt_block_attn_multiblock).
    q [B,Hq,N*S,D]; k_ctx/v_ctx [B,Hkv,cap,D] with cap >= (N-1)*S;
    k_noisy/v_noisy [B,Hkv,N*S,D]."""
    args, out, _ = _multiblock_args(q, k_ctx, v_ctx, k_noisy, v_noisy, block_size, scale, out,
                                    out_dtype, path, kv_splits, kv_groups, rows_per_wave,
                                    stream_waves, workspace, stream)
    _check(lib().tt_block_attn_multiblock(*args), "tt_block_attn_multiblock")
    return out


def prepare_block_attn_multiblock(q, k_ctx, v_ctx, k_noisy, v_noisy, block_size, scale, out, *,
                                  path: str = "auto", kv_splits: int = 0, kv_groups: int = 0,
                                  rows_per_wave: int = 0, stream_waves: int = 0, workspace=None,
                                  stream=None):
    """Validate once (same checks as block_attn_multiblock), make one call,
    and return a Prepared call."""
    args, out, keep = _multiblock_args(q, k_ctx, v_ctx, k_noisy, v_noisy, block_size, scale, out,
                                       None, path, kv_splits, kv_groups, rows_per_wave,
                                       stream_waves, workspace, stream)
    call = Prepared(lib().tt_block_attn_multiblock, args, "tt_block_attn_multiblock", keep)
    call()
    return call


def _multiblock_args(q, k_ctx, v_ctx, k_noisy, v_noisy, block_size, scale, out, out_dtype, path,
                     kv_splits, kv_groups, rows_per_wave, stream_waves, workspace, stream):
    _require(q.dim() == 4, "q must be [B, Hq, N*S, D]")
    device = q.device
    B, Hq, T, D = q.shape
    S = int(block_size)
    _require(S >= 1 and T % S == 0, "the query length must be a whole number of blocks")
    N = T // S
    for name, t in (("q", q), ("k_noisy", k_noisy), ("v_noisy", v_noisy)):
        _cuda_contig(name, t, device)
        _require(t.dtype == q.dtype, f"{name} dtype differs from q")
    _require(k_noisy.dim() == 4 and k_noisy.shape[0] == B and k_noisy.shape[2] == T
             and k_noisy.shape[3] == D and v_noisy.shape == k_noisy.shape,
             "k_noisy/v_noisy: [B, Hkv, N*S, D]")
    Hkv = k_noisy.shape[1]
    cap = _ctx_checks(k_ctx, v_ctx, q, B, Hkv, D, device, (N - 1) * S)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        with _on(stream):
            out = torch.empty((B, Hq, T, D), dtype=out_dtype, device=device)
    _cuda_contig("out", out, device)
    _require(tuple(out.shape) == (B, Hq, T, D), "out must be [B, Hq, N*S, D]")
    opts = AttnOpts(_PATHS[path], kv_splits, kv_groups, rows_per_wave, stream_waves)
    need = attn_multiblock_workspace_bytes(B, S, N, Hq, Hkv, D, q.dtype, path, kv_splits,
                                           kv_groups, rows_per_wave, stream_waves)
    if need and workspace is None:
        with _on(stream):
            workspace = torch.empty(need, dtype=torch.uint8, device=device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(q), _ptr(k_ctx), _ptr(v_ctx), _ptr(k_noisy), _ptr(v_noisy), S, N, Hq, Hkv, D,
            float(scale), _ptr(out), B, cap, _dtype_code(q.dtype), _dtype_code(out.dtype),
            _ptr(workspace), ws_bytes, _stream(device, stream), ctypes.byref(opts))
    return args, out, (q, k_ctx, v_ctx, k_noisy, v_noisy, out, workspace, opts)


def unmask_workspace_bytes(batch, block_len, vocab) -> int:
    n = lib().tt_unmask_workspace_bytes(batch, block_len, vocab)
    if n == SIZE_MAX:
        raise ValueError("invalid unmask shape")
    return n


def _unmask_checks(logits, mask_state, tokens, mask_out, conf_out, pred_out):
    device = mask_state.device
    _cuda_contig("mask_state", mask_state, device)
    _require(mask_state.dtype == torch.uint8 and mask_state.dim() == 2, "mask_state: [B, L] uint8")
    B, L = mask_state.shape
    if logits is not None:
        _cuda_contig("logits", logits, device)
        _require(logits.dtype == torch.float32 and logits.dim() == 3
                 and tuple(logits.shape[:2]) == (B, L), "logits: [B, L, V] float32")
    for name, t, dt in (("tokens", tokens, torch.int32), ("mask_out", mask_out, torch.uint8),
                        ("conf_out", conf_out, torch.float32), ("pred_out", pred_out, torch.int32)):
        if t is not None:
            _cuda_contig(name, t, device)
            _require(t.dtype == dt and tuple(t.shape) == (B, L), f"{name}: [B, L] {dt}")
    return device, B, L


def unmask_step(logits, mask_state, k, tokens, *, mask_out=None, conf_out=None, pred_out=None,
                workspace=None, stream=None):
    """One fixed-k unmask step through tt_unmask_step.  ``tokens`` is updated in
    place at committed positions; returns (tokens, mask_out)."""
    device, B, L = _unmask_checks(logits, mask_state, tokens, mask_out, conf_out, pred_out)
    V = logits.shape[2]
    if mask_out is None:
        with _on(stream):
            mask_out = torch.empty_like(mask_state)
    need = unmask_workspace_bytes(B, L, V)
    if need and workspace is None:
        with _on(stream):
            workspace = torch.empty(need, dtype=torch.uint8, device=device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    st = lib().tt_unmask_step(_ptr(logits), _ptr(mask_state), int(k), _ptr(tokens),
                              _ptr(mask_out), B, L, V, _ptr(conf_out), _ptr(pred_out),
                              _ptr(workspace), ws_bytes, _stream(device, stream))
    _check(st, "tt_unmask_step")
    return tokens, mask_out


def unmask_step_noalloc(logits, mask_state, k, tokens, *, mask_out=None, conf_out=None,
                        pred_out=None, stream=None):
    """tt_unmask_step_noalloc: tt_unmask_step with the library's static
    device scratch in place of a workspace (no allocation in the library;
    pass ``mask_out`` to allocate nothing here either)."""
    device, B, L = _unmask_checks(logits, mask_state, tokens, mask_out, conf_out, pred_out)
    V = logits.shape[2]
    if mask_out is None:
        with _on(stream):
            mask_out = torch.empty_like(mask_state)
    st = lib().tt_unmask_step_noalloc(_ptr(logits), _ptr(mask_state), int(k), _ptr(tokens),
                                      _ptr(mask_out), B, L, V, _ptr(conf_out), _ptr(pred_out),
                                      _stream(device, stream))
    _check(st, "tt_unmask_step_noalloc")
    return tokens, mask_out


def unmask_step_ex(logits, mask_state, select: Select, tokens, *, mask_out=None, conf_out=None,
                   pred_out=None, workspace=None, stream=None):
    """One unmask step under any selection rule (tt_unmask_step_ex)."""
    device, B, L = _unmask_checks(logits, mask_state, tokens, mask_out, conf_out, pred_out)
    V = logits.shape[2]
    if mask_out is None:
        with _on(stream):
            mask_out = torch.empty_like(mask_state)
    need = unmask_workspace_bytes(B, L, V)
    if need and workspace is None:
        with _on(stream):
            workspace = torch.empty(need, dtype=torch.uint8, device=device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    st = lib().tt_unmask_step_ex(_ptr(logits), _ptr(mask_state), ctypes.byref(select),
                                 _ptr(tokens), _ptr(mask_out), B, L, V, _ptr(conf_out),
                                 _ptr(pred_out), _ptr(workspace), ws_bytes,
                                 _stream(device, stream))
    _check(st, "tt_unmask_step_ex")
    return tokens, mask_out


def unmask_reduce(logits, mask_state, workspace, *, stream=None):
    """First half of tt_unmask_step (vocabulary pass into ``workspace``)."""
    device, B, L = _unmask_checks(logits, mask_state, None, None, None, None)
    st = lib().tt_unmask_reduce(_ptr(logits), _ptr(mask_state), B, L, logits.shape[2],
                                _ptr(workspace), workspace.numel(), _stream(device, stream))
    _check(st, "tt_unmask_reduce")


def unmask_commit(mask_state, k, tokens, mask_out, vocab, workspace, *, conf_out=None,
                  pred_out=None, stream=None):
    """Second half of tt_unmask_step (merge, top-k, commit)."""
    device, B, L = _unmask_checks(None, mask_state, tokens, mask_out, conf_out, pred_out)
    st = lib().tt_unmask_commit(_ptr(mask_state), int(k), _ptr(tokens), _ptr(mask_out), B, L,
                                vocab, _ptr(conf_out), _ptr(pred_out), _ptr(workspace),
                                workspace.numel(), _stream(device, stream))
    _check(st, "tt_unmask_commit")


def unmask_commit_ex(mask_state, select: Select, tokens, mask_out, vocab, workspace, *,
                     conf_out=None, pred_out=None, stream=None):
    """Second half of tt_unmask_step_ex (merge, select, commit)."""
    device, B, L = _unmask_checks(None, mask_state, tokens, mask_out, conf_out, pred_out)
    st = lib().tt_unmask_commit_ex(_ptr(mask_state), ctypes.byref(select), _ptr(tokens),
                                   _ptr(mask_out), B, L, vocab, _ptr(conf_out), _ptr(pred_out),
                                   _ptr(workspace), workspace.numel(), _stream(device, stream))
    _check(st, "tt_unmask_commit_ex")


class Prepared:
    """A libtt call whose arguments were validated once; calling it re-issues
    the same C call (same tensors, same stream).  Keeps per-launch host cost to
    one ctypes call, e.g. for timing loops or graph capture."""

    __slots__ = ("_fn", "_args", "_what", "keepalive")

    def __init__(self, fn, args, what, keepalive):
        self._fn, self._args, self._what, self.keepalive = fn, args, what, keepalive

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != TT_OK:
            raise TTError(st, self._what)


def prepare_block_attn(q, k_ctx, v_ctx, prefix_len, k_blk, v_blk, scale, out, *,
                       path: str = "auto", kv_splits: int = 0, kv_groups: int = 0,
                       rows_per_wave: int = 0, stream_waves: int = 0, workspace=None, stream=None):
    """Validate once (same checks as block_attn) and return a Prepared call."""
    device = q.device
    B, Hq, L, D = q.shape
    Hkv = k_blk.shape[1]
    Pcap = 0 if k_ctx is None else k_ctx.shape[2]
    need = attn_workspace_bytes(B, prefix_len, L, Hq, Hkv, D, q.dtype, path, kv_splits, kv_groups,
                                rows_per_wave, stream_waves)
    if need and workspace is None:
        with _on(stream):
            workspace = torch.empty(need, dtype=torch.uint8, device=device)
    # one validating call through the checked path
    block_attn(q, k_ctx, v_ctx, prefix_len, k_blk, v_blk, scale, out=out, path=path,
               kv_splits=kv_splits, kv_groups=kv_groups, rows_per_wave=rows_per_wave,
               stream_waves=stream_waves,
               workspace=workspace, stream=stream)
    opts = AttnOpts(_PATHS[path], kv_splits, kv_groups, rows_per_wave, stream_waves)
    ws_bytes = 0 if workspace is None else workspace.numel()
    args = (_ptr(q), _ptr(k_ctx), _ptr(v_ctx), prefix_len, _ptr(k_blk), _ptr(v_blk), L, Hq, Hkv,
            D, float(scale), _ptr(out), B, Pcap, _dtype_code(q.dtype), _dtype_code(out.dtype),
            _ptr(workspace), ws_bytes, _stream(device, stream), ctypes.byref(opts))
    keep = (q, k_ctx, v_ctx, k_blk, v_blk, out, workspace, opts)
    return Prepared(lib().tt_block_attn_ex, args, "tt_block_attn", keep)


def prepare_unmask_reduce(logits, mask_state, workspace, *, stream=None):
    device, B, L = _unmask_checks(logits, mask_state, None, None, None, None)
    V = logits.shape[2]
    _require(workspace.numel() >= unmask_workspace_bytes(B, L, V), "workspace too small")
    args = (_ptr(logits), _ptr(mask_state), B, L, V, _ptr(workspace), workspace.numel(),
            _stream(device, stream))
    return Prepared(lib().tt_unmask_reduce, args, "tt_unmask_reduce",
                    (logits, mask_state, workspace))


def prepare_unmask_commit(mask_state, k, tokens, mask_out, vocab, workspace, *, conf_out=None,
                          pred_out=None, stream=None):
    device, B, L = _unmask_checks(None, mask_state, tokens, mask_out, conf_out, pred_out)
    _require(workspace.numel() >= unmask_workspace_bytes(B, L, vocab), "workspace too small")
    args = (_ptr(mask_state), int(k), _ptr(tokens), _ptr(mask_out), B, L, vocab, _ptr(conf_out),
            _ptr(pred_out), _ptr(workspace), workspace.numel(), _stream(device, stream))
    return Prepared(lib().tt_unmask_commit, args, "tt_unmask_commit",
                    (mask_state, tokens, mask_out, workspace, conf_out, pred_out))


def prepare_unmask_commit_ex(mask_state, select: Select, tokens, mask_out, vocab, workspace, *,
                             conf_out=None, pred_out=None, stream=None):
    device, B, L = _unmask_checks(None, mask_state, tokens, mask_out, conf_out, pred_out)
    _require(workspace.numel() >= unmask_workspace_bytes(B, L, vocab), "workspace too small")
    sel = Select(select.mode, select.k, select.gamma, select.steps_left, select.step,
                 select.n_steps)
    args = (_ptr(mask_state), ctypes.byref(sel), _ptr(tokens), _ptr(mask_out), B, L, vocab,
            _ptr(conf_out), _ptr(pred_out), _ptr(workspace), workspace.numel(),
            _stream(device, stream))
    return Prepared(lib().tt_unmask_commit_ex, args, "tt_unmask_commit_ex",
                    (mask_state, tokens, mask_out, workspace, conf_out, pred_out, sel))


def lmhead_unmask_workspace_bytes(batch, block_len, vocab, d_model) -> int:
    n = lib().tt_lmhead_unmask_workspace_bytes(batch, block_len, vocab, d_model)
    if n == SIZE_MAX:
        raise ValueError("invalid or unsupported LM-head unmask shape")
    return n


def _lmhead_args(hidden, weight, mask_state, select, tokens, mask_out, conf_out, pred_out,
                 workspace, stream):
    device, B, L = _unmask_checks(None, mask_state, tokens, mask_out, conf_out, pred_out)
    for name, t in (("hidden", hidden), ("weight", weight)):
        _cuda_contig(name, t, device)
        _require(t.dtype == torch.bfloat16 and t.dim() == (3 if name == "hidden" else 2),
                 f"{name}: bfloat16")
    _require(tuple(hidden.shape[:2]) == (B, L), "hidden: [B, L, d_model]")
    V, d = weight.shape
    _require(hidden.shape[2] == d, "weight: [vocab, d_model] with the hidden width")
    if mask_out is None:
        with _on(stream):
            mask_out = torch.empty_like(mask_state)
    need = lmhead_unmask_workspace_bytes(B, L, V, d)
    if need and workspace is None:
        with _on(stream):
            workspace = torch.empty(need, dtype=torch.uint8, device=device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    sel = Select(select.mode, select.k, select.gamma, select.steps_left, select.step,
                 select.n_steps)
    args = (_ptr(hidden), _ptr(weight), _ptr(mask_state), ctypes.byref(sel), _ptr(tokens),
            _ptr(mask_out), B, L, V, d, _ptr(conf_out), _ptr(pred_out), _ptr(workspace), ws_bytes,
            _stream(device, stream))
    return args, mask_out, (hidden, weight, mask_state, tokens, mask_out, conf_out, pred_out,
                            workspace, sel)


def lmhead_unmask_step(hidden, weight, mask_state, select: Select, tokens, *, mask_out=None,
                       conf_out=None, pred_out=None, workspace=None, stream=None):
    """Unmask step with the LM-head projection fused in (tt_lmhead_unmask_step).
    hidden [B, L, d] and weight [V, d] bfloat16; returns (tokens, mask_out)."""
    args, mask_out, keep = _lmhead_args(hidden, weight, mask_state, select, tokens, mask_out,
                                        conf_out, pred_out, workspace, stream)
    _check(lib().tt_lmhead_unmask_step(*args), "tt_lmhead_unmask_step")
    return tokens, mask_out


def prepare_lmhead_unmask_step(hidden, weight, mask_state, select: Select, tokens, mask_out, *,
                               conf_out=None, pred_out=None, workspace=None, stream=None):
    args, mask_out, keep = _lmhead_args(hidden, weight, mask_state, select, tokens, mask_out,
                                        conf_out, pred_out, workspace, stream)
    return Prepared(lib().tt_lmhead_unmask_step, args, "tt_lmhead_unmask_step", keep)
