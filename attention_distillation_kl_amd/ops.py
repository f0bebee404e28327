"""Torch-facing wrappers over the C ABI: allocation of outputs with torch,
the current HIP stream, and an autograd Function.  All arithmetic happens in
the HIP kernels behind ``libstreamkl.so``.
"""
import math

import torch

from . import _lib


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return _lib.BF16
    if t.dtype == torch.float32:
        return _lib.F32
    raise TypeError(f"unsupported dtype {t.dtype}: expected bfloat16 or float32")


def _check_inputs(q1, k1, q2, k2):
    for name, t in (("q1", q1), ("k1", k1), ("q2", q2), ("k2", k2)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on the GPU (got {t.device}); there is no CPU path")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d], got shape {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if len({t.dtype for t in (q1, k1, q2, k2)}) != 1:
        raise TypeError("q1, k1, q2, k2 must share one dtype")
    if len({t.device for t in (q1, k1, q2, k2)}) != 1:
        raise ValueError("q1, k1, q2, k2 must be on one device")
    B, H, NQ, d = q1.shape
    NK = k1.shape[2]
    if tuple(q2.shape) != (B, H, NQ, d) or tuple(k1.shape) != (B, H, NK, d) or tuple(k2.shape) != (B, H, NK, d):
        raise ValueError("shape mismatch: q1,q2 must be [B,H,N_Q,d] and k1,k2 [B,H,N_K,d]")
    return B, H, NQ, NK, d


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def streamkl_fwd(q1, k1, q2, k2, scale=None, causal=False, splits=None):
    """Per-row (KL(P1||P2), LSE1, LSE2), each [B, H, N_Q] float32.

    ``splits``: key partitions of the split-K forward; None takes the
    library's choice (streamkl_fwd_splits), 1 runs the unsplit kernel.  The
    partitions' row states live in a workspace allocated here with torch."""
    B, H, NQ, NK, d = _check_inputs(q1, k1, q2, k2)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dev = q1.device
    dt = _dtype_code(q1)
    causal = int(bool(causal))
    kl = torch.empty(B, H, NQ, device=dev, dtype=torch.float32)
    lse1 = torch.empty_like(kl)
    lse2 = torch.empty_like(kl)
    if splits is None:
        splits = _lib.fwd_splits(B, H, NQ, NK, d, causal, dt)
    splits = int(splits)
    if splits == 1:
        st = _lib.fwd(_ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), B, H, NQ, NK, d, scale, causal,
                      dt, _ptr(kl), _ptr(lse1), _ptr(lse2), _stream(dev))
        where = "streamkl_fwd"
    else:
        ws_bytes = _lib.fwd_workspace_size(B, H, NQ, NK, d, causal, dt, splits)
        ws = torch.empty(max(1, (ws_bytes + 3) // 4), device=dev, dtype=torch.float32)
        st = _lib.fwd_splitk(_ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), B, H, NQ, NK, d, scale, causal,
                             dt, splits, _ptr(kl), _ptr(lse1), _ptr(lse2), _ptr(ws), ws_bytes, _stream(dev))
        where = "streamkl_fwd_splitk"
    if st != _lib.OK:
        raise _lib.StreamKLError(st, where)
    return kl, lse1, lse2


def streamkl_bwd(q1, k1, q2, k2, kl, lse1, lse2, dkl=None, scale=None, causal=False,
                 grad_mask=_lib.GRAD_ALL):
    """(dq1, dk1, dq2, dk2); gradients outside ``grad_mask`` are None."""
    B, H, NQ, NK, d = _check_inputs(q1, k1, q2, k2)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dev = q1.device
    for name, t in (("kl", kl), ("lse1", lse1), ("lse2", lse2)):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, H, NQ) or not t.is_contiguous() or t.device != dev:
            raise ValueError(f"{name} must be a contiguous float32 [B, H, N_Q] tensor on {dev}")
    if dkl is not None:
        dkl = dkl.to(device=dev, dtype=torch.float32).expand(B, H, NQ).contiguous()
    g1, g2 = bool(grad_mask & 1), bool(grad_mask & 2)
    dq1 = torch.empty_like(q1) if g1 else None
    dk1 = torch.empty_like(k1) if g1 else None
    dq2 = torch.empty_like(q2) if g2 else None
    dk2 = torch.empty_like(k2) if g2 else None
    dt = _dtype_code(q1)
    ws_bytes = _lib.bwd_workspace_size(B, H, NQ, NK, d, int(bool(causal)), dt, grad_mask)
    ws = torch.empty(ws_bytes, device=dev, dtype=torch.uint8) if ws_bytes else None
    st = _lib.bwd(_ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(kl), _ptr(lse1), _ptr(lse2), _ptr(dkl),
                  B, H, NQ, NK, d, scale, int(bool(causal)), dt, int(grad_mask),
                  _ptr(dq1), _ptr(dk1), _ptr(dq2), _ptr(dk2), _ptr(ws), ws_bytes, _stream(dev))
    if st != _lib.OK:
        raise _lib.StreamKLError(st, "streamkl_bwd")
    return dq1, dk1, dq2, dk2


def streamkl_bwd_fused(q1, k1, q2, k2, kl, lse1, lse2, dkl=None, scale=None, causal=False,
                       grad_mask=_lib.GRAD_ALL, workspace=None, out=None):
    """The single-pass backward (bf16 only): (dq1, dk1, dq2, dk2) as
    streamkl_bwd returns them.  ``workspace``: a device tensor of at least
    streamkl_bwd_fused_workspace_size bytes (the fp32 query-gradient sums);
    allocated here when None.  ``out``: preallocated (dq1, dk1, dq2, dk2),
    None for unrequested gradients."""
    B, H, NQ, NK, d = _check_inputs(q1, k1, q2, k2)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dev = q1.device
    for name, t in (("kl", kl), ("lse1", lse1), ("lse2", lse2)):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, H, NQ) or not t.is_contiguous() or t.device != dev:
            raise ValueError(f"{name} must be a contiguous float32 [B, H, N_Q] tensor on {dev}")
    if dkl is not None:
        dkl = dkl.to(device=dev, dtype=torch.float32).expand(B, H, NQ).contiguous()
    g1, g2 = bool(grad_mask & 1), bool(grad_mask & 2)
    if out is None:
        out = (torch.empty_like(q1) if g1 else None, torch.empty_like(k1) if g1 else None,
               torch.empty_like(q2) if g2 else None, torch.empty_like(k2) if g2 else None)
    dq1, dk1, dq2, dk2 = out
    dt = _dtype_code(q1)
    need = _lib.bwd_fused_workspace_size(B, H, NQ, NK, d, int(bool(causal)), dt, grad_mask)
    if workspace is None:
        workspace = torch.empty(max(need, 16), device=dev, dtype=torch.uint8)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {dev}")
    st = _lib.bwd_fused(_ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(kl), _ptr(lse1), _ptr(lse2), _ptr(dkl),
                        B, H, NQ, NK, d, scale, int(bool(causal)), dt, int(grad_mask),
                        _ptr(dq1), _ptr(dk1), _ptr(dq2), _ptr(dk2), _ptr(workspace),
                        workspace.numel() * workspace.element_size(), _stream(dev))
    if st != _lib.OK:
        raise _lib.StreamKLError(st, "streamkl_bwd_fused")
    return dq1, dk1, dq2, dk2


def streamkl_bwd_workspace(q1, k1, causal=False, grad_mask=_lib.GRAD_ALL):
    """The backward's workspace for these sizes (a uint8 device tensor), or
    None where the library needs none (query- and key-gradient grids that
    fill the GPU)."""
    B, H, NQ, d = q1.shape
    n = _lib.bwd_workspace_size(B, H, NQ, k1.shape[2], d, int(bool(causal)), _dtype_code(q1), int(grad_mask))
    return torch.empty(n, device=q1.device, dtype=torch.uint8) if n else None


def streamkl_bwd_half(which, q1, k1, q2, k2, kl, lse1, lse2, dkl=None, scale=None, causal=False,
                     grad_mask=_lib.GRAD_ALL, out=None, workspace=None):
    """One half of the backward: which='dq' -> (dq1, dq2), 'dk' -> (dk1, dk2).
    ``out`` may supply preallocated output tensors (a pair, None for unrequested).
    ``workspace`` (see streamkl_bwd_workspace) selects streamkl_bwd_dq_ws or
    streamkl_bwd_dk_ws, which partition the streamed rows where streamkl_bwd
    does (the keys of short query blocks, the queries of small key grids);
    without it neither half partitions."""
    B, H, NQ, NK, d = _check_inputs(q1, k1, q2, k2)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dev = q1.device
    if which not in ("dq", "dk"):
        raise ValueError(f"which must be 'dq' or 'dk', not {which!r}")
    if dkl is not None:
        dkl = dkl.to(device=dev, dtype=torch.float32).expand(B, H, NQ).contiguous()
    like = (q1, q2) if which == "dq" else (k1, k2)
    if out is None:
        out = (torch.empty_like(like[0]) if grad_mask & 1 else None,
               torch.empty_like(like[1]) if grad_mask & 2 else None)
    if workspace is not None:
        if workspace.device != dev or not workspace.is_contiguous():
            raise ValueError(f"workspace must be a contiguous tensor on {dev}")
        fn = _lib.bwd_dq_ws if which == "dq" else _lib.bwd_dk_ws
        st = fn(_ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(kl), _ptr(lse1), _ptr(lse2),
                _ptr(dkl), B, H, NQ, NK, d, scale, int(bool(causal)), _dtype_code(q1),
                int(grad_mask), _ptr(out[0]), _ptr(out[1]), _ptr(workspace),
                workspace.numel() * workspace.element_size(), _stream(dev))
        if st != _lib.OK:
            raise _lib.StreamKLError(st, f"streamkl_bwd_{which}_ws")
        return out
    st = _lib.bwd_half(which, _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(kl), _ptr(lse1), _ptr(lse2),
                       _ptr(dkl), B, H, NQ, NK, d, scale, int(bool(causal)), _dtype_code(q1),
                       int(grad_mask), _ptr(out[0]), _ptr(out[1]), _stream(dev))
    if st != _lib.OK:
        raise _lib.StreamKLError(st, f"streamkl_bwd_{which}")
    return out


class StreamKLFunction(torch.autograd.Function):
    """KL(softmax(scale Q1 K1^T) || softmax(scale Q2 K2^T)) per query row.

    Saves only the inputs and the per-row KL / LSE vectors for the backward
    pass, which recomputes the probabilities.
    """

    @staticmethod
    def forward(ctx, q1, k1, q2, k2, scale, causal):
        kl, lse1, lse2 = streamkl_fwd(q1, k1, q2, k2, scale, causal)
        ctx.save_for_backward(q1, k1, q2, k2, kl, lse1, lse2)
        ctx.scale, ctx.causal = scale, causal
        ctx.mark_non_differentiable(lse1, lse2)
        return kl, lse1, lse2

    @staticmethod
    def backward(ctx, gkl, _glse1, _glse2):
        q1, k1, q2, k2, kl, lse1, lse2 = ctx.saved_tensors
        need = ctx.needs_input_grad
        mask = (_lib.GRAD_Q1K1 if (need[0] or need[1]) else 0) | (_lib.GRAD_Q2K2 if (need[2] or need[3]) else 0)
        if mask == 0 or gkl is None:
            return None, None, None, None, None, None
        dq1, dk1, dq2, dk2 = streamkl_bwd(q1, k1, q2, k2, kl, lse1, lse2, gkl, ctx.scale, ctx.causal, mask)
        return dq1, dk1, dq2, dk2, None, None


def kl(q1, k1, q2, k2, scale=None, causal=False):
    """Differentiable per-row attention KL: returns (kl, lse1, lse2)."""
    if scale is None:
        scale = 1.0 / math.sqrt(q1.shape[-1])
    return StreamKLFunction.apply(q1, k1, q2, k2, float(scale), bool(causal))
