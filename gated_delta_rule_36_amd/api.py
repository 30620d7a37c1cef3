"""Python binding of the KDA forward library: ``fwd(...)``.

Argument marshalling only.  Every step of the forward pass runs in the HIP
kernels of ``libkda.so``; there is no other implementation to fall back on,
so a missing library raises :class:`KdaLibraryMissing`.

The call form and the tensor contract follow the FlashKDA input-tensor page
("Complete Forward Pass Example" and the sections above it): bf16
``[B,T,H,128]`` q/k/v/g/out, bf16 ``[B,T,H]`` beta logits, fp32 ``A_log [H]``
and ``dt_bias [H,128]``, ``lower_bound`` in [-5, 0], optional bf16/fp32
``[N,H,V,K]`` states and an optional int64 ``cu_seqlens [N+1]`` with B = 1.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Union

import torch

from . import _lib

_STATE_CODES = {torch.bfloat16: _lib.KDA_DTYPE_BF16, torch.float32: _lib.KDA_DTYPE_FP32}
_KERNELS = {None: _lib.KDA_KERNEL_AUTO, "auto": _lib.KDA_KERNEL_AUTO, "mfma": _lib.KDA_KERNEL_CHUNKED,
            "chunked": _lib.KDA_KERNEL_CHUNKED, "recurrent": _lib.KDA_KERNEL_RECURRENT,
            "single": _lib.KDA_KERNEL_SINGLE}
_INVERSES = {None: _lib.KDA_INVERSE_SUBSTITUTION, "substitution": _lib.KDA_INVERSE_SUBSTITUTION,
             "neumann": _lib.KDA_INVERSE_NEUMANN}
_SIGMOIDS = {None: _lib.KDA_SIGMOID_EXP2, "exp2": _lib.KDA_SIGMOID_EXP2, "tanh": _lib.KDA_SIGMOID_TANH}


def _options(kernel, inverse, sigmoid):
    """struct kda_options for the keyword choices, or None for all defaults."""
    if kernel is None and inverse is None and sigmoid is None:
        return None
    for name, value, table in (("kernel", kernel, _KERNELS), ("inverse", inverse, _INVERSES),
                               ("sigmoid", sigmoid, _SIGMOIDS)):
        if value not in table:
            raise ValueError(f"{name} must be one of {sorted(k for k in table if k)}, got {value!r}")
    return _lib.Options(_KERNELS[kernel], _INVERSES[inverse], _SIGMOIDS[sigmoid], 0)


class KdaError(RuntimeError):
    """The library rejected a call; ``status`` holds the kda_status code."""

    def __init__(self, status: int):
        self.status = status
        super().__init__(f"kda_fwd failed: {_lib.status_string(status)} (status {status})")


class KdaArgumentError(KdaError, ValueError):
    """An argument error reported by the library before any launch."""


def _check_tensor(name, t, dtype, device, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
        beta: torch.Tensor, scale: float, out: torch.Tensor,
        A_log: Optional[torch.Tensor], dt_bias: Optional[torch.Tensor],
        lower_bound: float, initial_state: Optional[torch.Tensor] = None,
        final_state: Optional[torch.Tensor] = None,
        cu_seqlens: Optional[torch.Tensor] = None, *,
        check_cu_seqlens: bool = True,
        segment_chunks: Union[None, int, str] = None,
        kernel: Optional[str] = None, inverse: Optional[str] = None,
        sigmoid: Optional[str] = None) -> torch.Tensor:
    """Run the chunked KDA forward pass; writes ``out`` (and ``final_state``).

    Enqueued on the current stream of ``q``'s device; returns ``out``.
    ``check_cu_seqlens`` copies ``cu_seqlens`` to the host (a synchronising
    copy) to check it is nondecreasing from 0 to T; the kernels never read
    outside the tensors either way.

    ``segment_chunks`` selects the segmented form (``kda_fwd_scan``: each
    sequence cut into segments of that many 16-token chunks, processed in
    parallel and stitched by an fp32 combine step) for workloads with few
    (sequence, head) chains; ``"auto"`` picks a segment length from the
    sizes (:func:`auto_segment_chunks`), ``None`` runs ``kda_fwd``.  The
    workspace is a temporary allocation on the same stream.

    ``kernel`` ("auto", "mfma", "recurrent", "single"), ``inverse``
    ("substitution", "neumann") and ``sigmoid`` ("exp2", "tanh") fill the
    library's ``kda_options`` (``None``: the default); they choose how the
    same result is computed.  A combination no kernel implements for the call
    raises :class:`KdaArgumentError`.
    """
    if not isinstance(q, torch.Tensor):
        raise TypeError("q must be a torch.Tensor")
    device = q.device
    # dtypes first, so a wrong dtype is reported as such wherever it lives
    for name, t, dt in (("q", q, torch.bfloat16), ("k", k, torch.bfloat16),
                        ("v", v, torch.bfloat16), ("g", g, torch.bfloat16),
                        ("beta", beta, torch.bfloat16), ("out", out, torch.bfloat16),
                        ("A_log", A_log, torch.float32), ("dt_bias", dt_bias, torch.float32),
                        ("cu_seqlens", cu_seqlens, torch.int64)):
        if t is None and name in ("A_log", "dt_bias", "cu_seqlens"):
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
    for name, t in (("q", q), ("k", k), ("g", g)):
        _check_tensor(name, t, torch.bfloat16, device, ndim=4)
    _check_tensor("v", v, torch.bfloat16, device, ndim=4)
    _check_tensor("out", out, torch.bfloat16, device, ndim=4)
    _check_tensor("beta", beta, torch.bfloat16, device, ndim=3)
    B, T, H, K = q.shape
    V = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape:
        raise ValueError("q, k and g must share the shape [B,T,H,K]")
    if v.shape[:3] != q.shape[:3] or out.shape != v.shape:
        raise ValueError("v and out must be [B,T,H,V] with q's B, T, H")
    if beta.shape != q.shape[:3]:
        raise ValueError("beta must be [B,T,H]")
    if A_log is not None:
        _check_tensor("A_log", A_log, torch.float32, device, ndim=1)
        if A_log.shape != (H,):
            raise ValueError("A_log must be [H]")
    if dt_bias is not None:
        _check_tensor("dt_bias", dt_bias, torch.float32, device, ndim=2)
        if dt_bias.shape != (H, K):
            raise ValueError("dt_bias must be [H,K]")

    num_seqs = 0
    if cu_seqlens is not None:
        _check_tensor("cu_seqlens", cu_seqlens, torch.int64, device, ndim=1)
        if cu_seqlens.numel() < 1:
            raise ValueError("cu_seqlens must have N+1 >= 1 entries")
        num_seqs = cu_seqlens.numel() - 1
        if check_cu_seqlens:
            host = cu_seqlens.cpu()
            if int(host[0]) != 0 or int(host[-1]) != T or bool((host[1:] < host[:-1]).any()):
                raise ValueError("cu_seqlens must be nondecreasing from 0 to T")
    N = num_seqs if cu_seqlens is not None else B

    codes = []
    for name, st in (("initial_state", initial_state), ("final_state", final_state)):
        if st is None:
            codes.append(_lib.KDA_DTYPE_NONE)
            continue
        if st.dtype not in _STATE_CODES:
            raise TypeError(f"{name} must be bfloat16 or float32, got {st.dtype}")
        _check_tensor(name, st, st.dtype, device, ndim=4)
        if st.shape != (N, H, V, K):
            raise ValueError(f"{name} must be [N,H,V,K] = {(N, H, V, K)}, got {tuple(st.shape)}")
        codes.append(_STATE_CODES[st.dtype])

    if segment_chunks == "auto":
        segment_chunks = auto_segment_chunks(N * H, T)
    elif segment_chunks is not None and (not isinstance(segment_chunks, int)
                                         or isinstance(segment_chunks, bool) or segment_chunks < 1):
        raise ValueError(f"segment_chunks must be a positive int, 'auto' or None, got {segment_chunks!r}")

    opts = _options(kernel, inverse, sigmoid)
    opts_ref = None if opts is None else ctypes.byref(opts)
    lib = _lib.load()
    with torch.cuda.device(device):
        stream = torch.cuda.current_stream(device).cuda_stream
        args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(out),
                _ptr(A_log), _ptr(dt_bias), float(lower_bound),
                _ptr(initial_state), codes[0], _ptr(final_state), codes[1],
                _ptr(cu_seqlens), num_seqs, B, T, H, K, V)
        if segment_chunks is None:
            status = lib.kda_fwd_ex(*args, opts_ref, stream)
        else:
            nbytes = lib.kda_fwd_scan_workspace_bytes(_ptr(cu_seqlens), num_seqs, B, T, H,
                                                      segment_chunks)
            if nbytes < 0:
                raise ValueError("bad sizes for the segmented form")
            # freed right after the call: the caching allocator hands it out
            # again only to work ordered after this call on the same stream
            workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
            status = lib.kda_fwd_scan(*args, segment_chunks, workspace.data_ptr(), nbytes, opts_ref,
                                      stream)
    if status != _lib.KDA_OK:
        if status == _lib.KDA_ERR_LAUNCH:
            raise KdaError(status)
        raise KdaArgumentError(status)
    return out


def fwd_kernel(T: int, varlen: bool = False, *, kernel: Optional[str] = None,
               inverse: Optional[str] = None, sigmoid: Optional[str] = None) -> str:
    """Name of the kernel ``fwd`` runs for a call with ``T`` tokens per batch
    row (``varlen``: cu_seqlens given) and these options, as the library
    decides it: "recurrent", "single" or "mfma".  Raises ValueError when the
    options are invalid for such a call.  The segmented form
    (``segment_chunks``) always runs the chunked kernel."""
    opts = _options(kernel, inverse, sigmoid)
    name = _lib.load().kda_fwd_kernel(int(T), 1 if varlen else 0,
                                      None if opts is None else ctypes.byref(opts))
    if name is None:
        raise ValueError(f"no kernel implements kernel={kernel!r}, inverse={inverse!r}, "
                         f"sigmoid={sigmoid!r} for T={T}, varlen={varlen}")
    return name.decode()


def auto_segment_chunks(chains: int, T: int, target_blocks: int = 256,
                        min_chunks: int = 8, min_segments: int = 6) -> Optional[int]:
    """Segment length (in 16-token chunks) for the segmented form, or None
    when it would not help.  With ``chains`` (sequence, head) chains of at
    most ``T`` tokens, each chain is cut into about ``target_blocks / chains``
    segments (one workgroup per CU on a 256-CU part) of at least
    ``min_chunks`` chunks.  The segmented form walks every segment about
    three times (end state, transition matrix, output) against once for a
    whole chain, so it needs ``min_segments`` segments or more to pay off."""
    chunks = -(-T // 16)
    if chains <= 0 or target_blocks // chains < min_segments:
        return None
    seg = max(min_chunks, -(-chunks // (target_blocks // chains)))
    return None if -(-chunks // seg) < min_segments else seg
