"""Python binding of the attention library: marshals torch tensors (device
memory and the current stream) into the C ABI of include/attn.h.  Every step
of the computation runs in the library's HIP kernels; this module only checks
tensor metadata, allocates outputs when asked to, and forwards pointers.

Layouts: q, out [n, l_q, h, d]; k, v [n, l_k, h_kv, d]; lse [n, h, l_q]
float32.  Masking: absolute positions q_offset + i and k_offset + j, causal
kpos <= qpos, inclusive window (win_l, win_r) with -1 for an open side.
"""
from __future__ import annotations

import contextlib
import ctypes
import math

import torch

from . import _lib
from ._lib import ATTN_BF16, ATTN_F32, check

_DT = {torch.bfloat16: ATTN_BF16, torch.float32: ATTN_F32}


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _on(stream):
    """Context under which buffers for work launched on `stream` are
    allocated: the caching allocator then ties them to that stream, so a block
    freed after the call is reused only by work ordered after it."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _dtype_code(t):
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _dev(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def attn_fwd(q, k, v, out, lse, scale, causal=False, win_l=-1, win_r=-1,
             q_offset=0, k_offset=0, stream=None):
    """Forward into caller-provided `out` (q's dtype) and `lse` (float32)."""
    _dev(q, k, v, out, lse)
    n, l_q, h, d = q.shape
    _, l_k, h_kv, _ = k.shape
    if k.shape != v.shape or k.shape[0] != n or k.shape[3] != d:
        raise ValueError("k and v must be [n, l_k, h_kv, d] matching q")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if tuple(lse.shape) != (n, h, l_q) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [n, h, l_q]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    st = _lib.lib().attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                             out.data_ptr(), lse.data_ptr(), n, l_q, l_k, h,
                             h_kv, d, float(scale), int(bool(causal)),
                             int(win_l), int(win_r), int(q_offset),
                             int(k_offset), _stream(stream), _dtype_code(q))
    check("attn_fwd", st)
    return out, lse


def fwd_kernel_name(n, l_q, l_k, h, h_kv, d, causal=False, win_l=-1, win_r=-1,
                    q_offset=0, k_offset=0, dtype=torch.bfloat16, fused=False,
                    scale=None):
    """Name of the kernel attn_fwd (or, fused, attn_fwd_acc) launches for
    these arguments, as kernel traces show it; None if none would run."""
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    r = _lib.lib().attn_fwd_kernel_name(n, l_q, l_k, h, h_kv, d, float(scale),
                                        int(bool(causal)), int(win_l), int(win_r),
                                        int(q_offset), int(k_offset), _DT[dtype],
                                        int(bool(fused)))
    return None if r is None else r.decode()


def attention_forward(q, k, v, scale=None, causal=False, window=(-1, -1),
                      q_offset=0, k_offset=0, stream=None):
    """Allocate (O, LSE) and run the forward; scale defaults to 1/sqrt(d)."""
    n, l_q, h, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    with _on(stream):
        out = torch.empty_like(q)
        lse = torch.empty((n, h, l_q), dtype=torch.float32, device=q.device)
    return attn_fwd(q, k, v, out, lse, scale, causal, window[0], window[1],
                    q_offset, k_offset, stream)


def attn_merge(out_acc, lse_acc, out_blk, lse_blk, stream=None):
    """In-place merge of (out_blk, lse_blk) into the float32 accumulator."""
    _dev(out_acc, lse_acc, out_blk, lse_blk)
    n, l, h, d = out_acc.shape
    if out_acc.dtype != torch.float32 or lse_acc.dtype != torch.float32 \
            or lse_blk.dtype != torch.float32:
        raise ValueError("accumulator and LSEs must be float32")
    if out_blk.shape != out_acc.shape or tuple(lse_acc.shape) != (n, h, l) \
            or lse_blk.shape != lse_acc.shape:
        raise ValueError("shape mismatch")
    st = _lib.lib().attn_merge(out_acc.data_ptr(), lse_acc.data_ptr(),
                               out_blk.data_ptr(), lse_blk.data_ptr(), n, l, h,
                               d, _dtype_code(out_blk), _stream(stream))
    check("attn_merge", st)
    return out_acc, lse_acc


def attn_fwd_acc(q, k, v, out_acc, lse_acc, scale, causal=False, win_l=-1,
                 win_r=-1, q_offset=0, k_offset=0, stream=None):
    """One fused ring step: attention of bf16 q against this k/v chunk merged
    into the float32 accumulator (out_acc [n,l_q,h,d], lse_acc [n,h,l_q])."""
    _dev(q, k, v, out_acc, lse_acc)
    n, l_q, h, d = q.shape
    _, l_k, h_kv, _ = k.shape
    if k.shape != v.shape or k.shape[0] != n or k.shape[3] != d:
        raise ValueError("k and v must be [n, l_k, h_kv, d] matching q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    if out_acc.shape != q.shape or out_acc.dtype != torch.float32:
        raise ValueError("out_acc must be float32 shaped like q")
    if tuple(lse_acc.shape) != (n, h, l_q) or lse_acc.dtype != torch.float32:
        raise ValueError("lse_acc must be float32 [n, h, l_q]")
    st = _lib.lib().attn_fwd_acc(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                 out_acc.data_ptr(), lse_acc.data_ptr(), n, l_q,
                                 l_k, h, h_kv, d, float(scale),
                                 int(bool(causal)), int(win_l), int(win_r),
                                 int(q_offset), int(k_offset), _stream(stream),
                                 _dtype_code(q))
    check("attn_fwd_acc", st)
    return out_acc, lse_acc


def attn_fwd_ring(q, k_chunks, v_chunks, k_offsets, out, lse, scale, causal=False,
                  win_l=-1, win_r=-1, q_offset=0, stream=None):
    """A whole ring share in one launch: bf16 q against every k/v chunk (key j
    of chunk c at absolute position k_offsets[c] + j), written to `out` (bf16,
    like q) and `lse` (float32 [n, h, l_q])."""
    nc = len(k_chunks)
    if len(v_chunks) != nc or len(k_offsets) != nc:
        raise ValueError("k_chunks, v_chunks and k_offsets must have one entry per chunk")
    if not 1 <= nc <= _lib.ATTN_RING_MAX_CHUNKS:
        raise ValueError(f"1 to {_lib.ATTN_RING_MAX_CHUNKS} chunks, got {nc}")
    _dev(q, out, lse, *k_chunks, *v_chunks)
    n, l_q, h, d = q.shape
    h_kv = k_chunks[0].shape[2]
    for kc, vc in zip(k_chunks, v_chunks):
        if kc.shape != vc.shape or kc.dim() != 4 or kc.shape[0] != n or \
                kc.shape[2] != h_kv or kc.shape[3] != d:
            raise ValueError("every k and v chunk must be [n, l_k, h_kv, d] matching q")
        if kc.dtype != q.dtype or vc.dtype != q.dtype:
            raise ValueError("q and the chunks must share a dtype")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if tuple(lse.shape) != (n, h, l_q) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [n, h, l_q]")
    ptrs = ctypes.c_void_p * nc
    kp = ptrs(*[c.data_ptr() for c in k_chunks])
    vp = ptrs(*[c.data_ptr() for c in v_chunks])
    lk = (ctypes.c_int * nc)(*[c.shape[1] for c in k_chunks])
    ko = (ctypes.c_longlong * nc)(*[int(o) for o in k_offsets])
    st = _lib.lib().attn_fwd_ring(q.data_ptr(), kp, vp, lk, ko, nc, out.data_ptr(),
                                  lse.data_ptr(), n, l_q, h, h_kv, d, float(scale),
                                  int(bool(causal)), int(win_l), int(win_r),
                                  int(q_offset), _stream(stream), _dtype_code(q))
    check("attn_fwd_ring", st)
    return out, lse


def hbm_copy(src, dst, stream=None):
    """The library's plain streaming copy (bandwidth reference) of src's bytes
    into dst (same byte size, a multiple of 16)."""
    _dev(src, dst)
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nb:
        raise ValueError("src and dst must have the same byte size")
    check("attn_hbm_copy", _lib.lib().attn_hbm_copy(src.data_ptr(), dst.data_ptr(), nb,
                                                      _stream(stream)))
    return dst


def attn_acc_init(out_acc, lse_acc=None, stream=None):
    """O = 0 and (unless lse_acc is None) LSE = -inf."""
    _dev(out_acc, *([] if lse_acc is None else [lse_acc]))
    n, l, h, d = out_acc.shape
    if out_acc.dtype != torch.float32:
        raise ValueError("the accumulator must be float32")
    if lse_acc is not None and tuple(lse_acc.shape) != (n, h, l):
        raise ValueError("shape mismatch")
    st = _lib.lib().attn_acc_init(out_acc.data_ptr(),
                                  None if lse_acc is None else lse_acc.data_ptr(),
                                  n, l, h, d, _stream(stream))
    check("attn_acc_init", st)
    return out_acc, lse_acc


def attn_acc_cast(out_acc, out, stream=None):
    _dev(out_acc, out)
    n, l, h, d = out_acc.shape
    if out.shape != out_acc.shape:
        raise ValueError("shape mismatch")
    st = _lib.lib().attn_acc_cast(out_acc.data_ptr(), out.data_ptr(), n, l, h,
                                  d, _dtype_code(out), _stream(stream))
    check("attn_acc_cast", st)
    return out


def bwd_workspace_bytes(n, l_q, l_k, h, h_kv, d):
    return int(_lib.lib().attn_bwd_workspace_bytes(n, l_q, l_k, h, h_kv, d))


def _check_bwd(dout, q, k, v, out, lse, dq, dk, dv, acc):
    """Shapes and dtypes of the backward's tensors against q and k: the C
    ABI receives bare pointers, so a short tensor here would be read or
    written past its end.  acc: the gradients are float32 accumulators.
    Metadata first, then the device: every mismatch raises before anything
    reaches the library."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [n, l_q, h, d] and k [n, l_k, h_kv, d]")
    n, l_q, h, d = q.shape
    if k.shape[0] != n or k.shape[3] != d or v.shape != k.shape:
        raise ValueError("k and v must be [n, l_k, h_kv, d] matching q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    for name, t in (("dout", dout), ("out", out)):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    if tuple(lse.shape) != (n, h, l_q) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [n, h, l_q]")
    gdt = torch.float32 if acc else q.dtype
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, k)):
        if t.shape != ref.shape or t.dtype != gdt:
            what = "float32 accumulators" if acc else "gradients in q's dtype"
            raise ValueError(f"{name} must be shaped like {'q' if ref is q else 'k'} "
                             f"({what})")
    _dev(dout, q, k, v, out, lse, dq, dk, dv)


def _workspace(workspace, need, device, stream):
    if workspace is None:
        with _on(stream):
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    _dev(workspace)
    return workspace


def attn_bwd(dout, q, k, v, out, lse, dq, dk, dv, scale, causal=False,
             win_l=-1, win_r=-1, q_offset=0, k_offset=0, workspace=None,
             stream=None):
    """Backward into caller-provided dq, dk, dv; `workspace` is a uint8 device
    tensor of at least bwd_workspace_bytes(...) bytes (allocated on `stream`
    if None)."""
    _check_bwd(dout, q, k, v, out, lse, dq, dk, dv, acc=False)
    n, l_q, h, d = q.shape
    _, l_k, h_kv, _ = k.shape
    need = bwd_workspace_bytes(n, l_q, l_k, h, h_kv, d)
    workspace = _workspace(workspace, need, q.device, stream)
    st = _lib.lib().attn_bwd(dout.data_ptr(), q.data_ptr(), k.data_ptr(),
                             v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                             dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), n,
                             l_q, l_k, h, h_kv, d, float(scale),
                             int(bool(causal)), int(win_l), int(win_r),
                             int(q_offset), int(k_offset), workspace.data_ptr(),
                             workspace.numel() * workspace.element_size(),
                             _stream(stream), _dtype_code(q))
    check("attn_bwd", st)
    return dq, dk, dv


def attn_bwd_prepare(dout, out, lse, workspace, stream=None):
    """D = rowsum(dout * out) and the LSE in base-2 units of the query rows,
    into the leading bwd_prepare_bytes(...) bytes of `workspace` (a uint8
    device tensor), for attn_bwd_acc(..., prepared=True)."""
    if dout.dim() != 4 or out.shape != dout.shape or out.dtype != dout.dtype:
        raise ValueError("dout and out must be [n, l_q, h, d] of one dtype")
    n, l_q, h, d = dout.shape
    if tuple(lse.shape) != (n, h, l_q) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [n, h, l_q]")
    _dev(dout, out, lse, workspace)
    st = _lib.lib().attn_bwd_prepare(dout.data_ptr(), out.data_ptr(), lse.data_ptr(), n,
                                     l_q, h, d, workspace.data_ptr(),
                                     workspace.numel() * workspace.element_size(),
                                     _stream(stream), _dtype_code(dout))
    check("attn_bwd_prepare", st)
    return workspace


def attn_bwd_ring(dout, q, out, lse, k_chunks, v_chunks, k_offsets, dk_acc, dv_acc, dq,
                  scale, causal=False, win_l=-1, win_r=-1, q_offset=0, workspace=None,
                  stream=None):
    """The whole ring backward share in three launches: dq (q's dtype) written
    with the gradient over every chunk; chunk c's dK, dV added to the float32
    accumulators dk_acc[c], dv_acc[c] (shaped like the chunk)."""
    nc = len(k_chunks)
    if not (len(v_chunks) == len(k_offsets) == len(dk_acc) == len(dv_acc) == nc):
        raise ValueError("one entry per chunk in every list")
    if not 1 <= nc <= _lib.ATTN_RING_MAX_CHUNKS:
        raise ValueError(f"1 to {_lib.ATTN_RING_MAX_CHUNKS} chunks, got {nc}")
    if q.dim() != 4:
        raise ValueError("q must be [n, l_q, h, d]")
    n, l_q, h, d = q.shape
    h_kv = k_chunks[0].shape[2] if k_chunks[0].dim() == 4 else -1
    for name, t in (("dout", dout), ("out", out), ("dq", dq)):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    if tuple(lse.shape) != (n, h, l_q) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [n, h, l_q]")
    for kc, vc, dka, dva in zip(k_chunks, v_chunks, dk_acc, dv_acc):
        if kc.dim() != 4 or kc.shape != vc.shape or kc.shape[0] != n or \
                kc.shape[2] != h_kv or kc.shape[3] != d:
            raise ValueError("every k and v chunk must be [n, l_k, h_kv, d] matching q")
        if kc.dtype != q.dtype or vc.dtype != q.dtype:
            raise ValueError("q and the chunks must share a dtype")
        if dka.shape != kc.shape or dva.shape != kc.shape or \
                dka.dtype != torch.float32 or dva.dtype != torch.float32:
            raise ValueError("dk_acc and dv_acc must be float32 shaped like their chunk")
    _dev(dout, q, out, lse, dq, *k_chunks, *v_chunks, *dk_acc, *dv_acc)
    need = bwd_prepare_bytes(n, l_q, h)
    workspace = _workspace(workspace, need, q.device, stream)
    arr = lambda ts: (ctypes.c_void_p * nc)(*[t.data_ptr() for t in ts])
    lk = (ctypes.c_int * nc)(*[t.shape[1] for t in k_chunks])
    ko = (ctypes.c_longlong * nc)(*[int(o) for o in k_offsets])
    st = _lib.lib().attn_bwd_ring(dout.data_ptr(), q.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                  arr(k_chunks), arr(v_chunks), lk, ko, arr(dk_acc),
                                  arr(dv_acc), nc, dq.data_ptr(), n, l_q, h, h_kv, d,
                                  float(scale), int(bool(causal)), int(win_l), int(win_r),
                                  int(q_offset), workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(),
                                  _stream(stream), _dtype_code(q))
    check("attn_bwd_ring", st)
    return dq, dk_acc, dv_acc


def bwd_prepare_bytes(n, l_q, h):
    return int(_lib.lib().attn_bwd_prepare_bytes(n, l_q, h))


def attn_bwd_acc(dout, q, k, v, out, lse, dq_acc, dk_acc, dv_acc, scale,
                 causal=False, win_l=-1, win_r=-1, q_offset=0, k_offset=0,
                 workspace=None, stream=None, prepared=False):
    """One ring backward step: this chunk's gradients added to the float32
    accumulators dq_acc (shaped like q), dk_acc and dv_acc (shaped like k);
    out and lse are the query rows' results over the whole sequence.
    prepared=True: `workspace` already holds what attn_bwd_prepare wrote for
    these dout, out and lse (attn_bwd_acc_prepared, no preprocessing)."""
    if prepared and workspace is None:
        raise ValueError("prepared=True needs the prepared workspace")
    _check_bwd(dout, q, k, v, out, lse, dq_acc, dk_acc, dv_acc, acc=True)
    n, l_q, h, d = q.shape
    _, l_k, h_kv, _ = k.shape
    need = bwd_workspace_bytes(n, l_q, l_k, h, h_kv, d)
    workspace = _workspace(workspace, need, q.device, stream)
    fn = _lib.lib().attn_bwd_acc_prepared if prepared else _lib.lib().attn_bwd_acc
    st = fn(dout.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
            lse.data_ptr(), dq_acc.data_ptr(), dk_acc.data_ptr(), dv_acc.data_ptr(), n, l_q,
            l_k, h, h_kv, d, float(scale), int(bool(causal)), int(win_l), int(win_r),
            int(q_offset), int(k_offset), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), _stream(stream), _dtype_code(q))
    check("attn_bwd_acc_prepared" if prepared else "attn_bwd_acc", st)
    return dq_acc, dk_acc, dv_acc


def attn_bwd_static(dout, q, k, v, out, lse, dq, dk, dv, scale, causal=False,
                    win_l=-1, win_r=-1, q_offset=0, k_offset=0, stream=None):
    """attn_bwd with the library's static per-device workspace: allocates
    nothing.  Calls that overlap in time on one device race (they share the
    workspace)."""
    _check_bwd(dout, q, k, v, out, lse, dq, dk, dv, acc=False)
    n, l_q, h, d = q.shape
    _, l_k, h_kv, _ = k.shape
    st = _lib.lib().attn_bwd_static(dout.data_ptr(), q.data_ptr(), k.data_ptr(),
                                    v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                    dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), n,
                                    l_q, l_k, h, h_kv, d, float(scale),
                                    int(bool(causal)), int(win_l), int(win_r),
                                    int(q_offset), int(k_offset), _stream(stream),
                                    _dtype_code(q))
    check("attn_bwd_static", st)
    return dq, dk, dv


def attention_backward(dout, q, k, v, out, lse, scale=None, causal=False,
                       window=(-1, -1), q_offset=0, k_offset=0, stream=None):
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    with _on(stream):
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dv = torch.empty_like(v)
    return attn_bwd(dout, q, k, v, out, lse, dq, dk, dv, scale, causal,
                    window[0], window[1], q_offset, k_offset, None, stream)


class _Attention(torch.autograd.Function):
    """attn_fwd as the forward and attn_bwd as the backward of one autograd
    node (the pages' custom_vjp pairing of the kernel's fwd and bwd).  The
    node keeps q, k, v, O and LSE for the backward; LSE is returned as a
    non-differentiable output."""

    @staticmethod
    def forward(ctx, q, k, v, scale, causal, window, q_offset, k_offset):
        o, lse = attention_forward(q, k, v, scale, causal, window, q_offset,
                                   k_offset)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.args = (scale, causal, window, q_offset, k_offset)
        ctx.mark_non_differentiable(lse)
        return o, lse

    @staticmethod
    def backward(ctx, do, _dlse):
        q, k, v, o, lse = ctx.saved_tensors
        scale, causal, window, q_offset, k_offset = ctx.args
        dq, dk, dv = attention_backward(do.contiguous(), q, k, v, o, lse, scale,
                                        causal, window, q_offset, k_offset)
        return dq, dk, dv, None, None, None, None, None


def flash_attention(q, k, v, scale=None, causal=False, window=(-1, -1),
                    q_offset=0, k_offset=0, return_lse=False):
    """Differentiable exact attention: O (and LSE with return_lse) from
    attn_fwd, gradients of q, k, v from attn_bwd (bf16 or float32).  scale
    defaults to 1/sqrt(d)."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    o, lse = _Attention.apply(q, k, v, float(scale), bool(causal),
                              (int(window[0]), int(window[1])), int(q_offset),
                              int(k_offset))
    return (o, lse) if return_lse else o


class RingShare:
    """One device's share of ring attention, with its buffers allocated once:
    the float32 accumulator (O, LSE), one block (O, LSE) per step and the
    final output.  `run` launches acc_init, then per key/value chunk (with
    that chunk's absolute offset) either attn_fwd + attn_merge or, with
    fused=True, the single attn_fwd_acc step, then the final cast - all on
    one stream, nothing synchronised (flash_sharding.py, ring_fwd).  With
    one_launch=True (at most ATTN_RING_MAX_CHUNKS chunks) the whole share is
    the attn_fwd_ring call instead (one launch for bf16; float32 merges one
    fused step per chunk into the output itself), writing the final O and
    LSE directly."""

    def __init__(self, q, scale, causal, q_offset, window=(-1, -1)):
        n, l, h, d = q.shape
        self.q = q
        self.scale = scale
        self.causal = causal
        self.q_offset = q_offset
        self.window = (int(window[0]), int(window[1]))
        dev = q.device
        self.acc = torch.empty((n, l, h, d), dtype=torch.float32, device=dev)
        self.lse_acc = torch.empty((n, h, l), dtype=torch.float32, device=dev)
        self.blk = torch.empty_like(q)
        self.lse_blk = torch.empty((n, h, l), dtype=torch.float32, device=dev)
        self.out = torch.empty_like(q)

    def run(self, k_chunks, v_chunks, k_offsets, stream=None, fused=False,
            one_launch=False):
        if one_launch:
            wl, wr = self.window
            # lse_acc holds the share's final LSE, as after the other forms
            attn_fwd_ring(self.q, k_chunks, v_chunks, k_offsets, self.out, self.lse_acc,
                          self.scale, self.causal, wl, wr, self.q_offset, stream)
            return self.out, self.lse_acc
        attn_acc_init(self.acc, self.lse_acc, stream)
        for kc, vc, ko in zip(k_chunks, v_chunks, k_offsets):
            wl, wr = self.window
            if fused:
                attn_fwd_acc(self.q, kc, vc, self.acc, self.lse_acc, self.scale,
                             self.causal, wl, wr, self.q_offset, ko, stream)
            else:
                attn_fwd(self.q, kc, vc, self.blk, self.lse_blk, self.scale,
                         self.causal, wl, wr, self.q_offset, ko, stream)
                attn_merge(self.acc, self.lse_acc, self.blk, self.lse_blk,
                           stream)
        attn_acc_cast(self.acc, self.out, stream)
        return self.out, self.lse_acc

    def capture(self, k_chunks, v_chunks, k_offsets, fused=True):
        """Record `run` on these chunk buffers into a HIP graph and return it
        (a torch.cuda.CUDAGraph).  Each replay recomputes the share from what
        q and the chunk buffers hold at that moment, into the same output
        buffers; the buffers must outlive the graph."""
        return _capture(lambda: self.run(k_chunks, v_chunks, k_offsets,
                                         fused=fused))


def _capture(fn):
    # one eager call first, so that the kernels' code objects are loaded and
    # every buffer is allocated before the capture
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def ring_share(q, k_chunks, v_chunks, k_offsets, q_offset, scale=None,
               causal=True, stream=None, fused=False, window=(-1, -1),
               one_launch=False):
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return RingShare(q, scale, causal, q_offset, window).run(
        k_chunks, v_chunks, k_offsets, stream, fused, one_launch)


class RingShareBwd:
    """One device's share of the ring backward (picotron
    ring_attention_backward): given its query block q with the forward ring
    share's final (out, lse) and the incoming gradient dout, `run` prepares
    the per-row D and LSE once (attn_bwd_prepare), adds every key/value
    chunk's contribution with attn_bwd_acc_prepared - dQ accumulating
    locally in float32, one float32 (dK, dV) accumulator per chunk (in a real
    ring those travel with the chunk) - and casts dQ to q's dtype at the end.
    Buffers are allocated once; everything runs on one stream."""

    def __init__(self, q, out, lse, dout, scale, causal, q_offset,
                 window=(-1, -1)):
        self.q, self.out, self.lse, self.dout = q, out, lse, dout
        self.scale = scale
        self.causal = causal
        self.q_offset = q_offset
        self.window = (int(window[0]), int(window[1]))
        self.dq_acc = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        self.dq = torch.empty_like(q)
        self.kv_acc = None
        self.dk_acc = []
        self.dv_acc = []
        self.ws = None

    def run(self, k_chunks, v_chunks, k_offsets, stream=None, one_launch=False):
        """one_launch=True: the share as attn_bwd_ring (prepare, one dK/dV
        launch over all chunks, one dQ launch; at most ATTN_RING_MAX_CHUNKS
        chunks) instead of a step per chunk."""
        n, l_q, h, d = self.q.shape
        P = len(k_chunks)
        shape = tuple(k_chunks[0].shape)
        if len(self.dk_acc) != P or tuple(self.dk_acc[0].shape) != shape:
            # all chunks' (dK, dV) accumulators in one buffer, zeroed by a
            # single launch per run
            self.kv_acc = torch.empty((2 * P * shape[0],) + shape[1:],
                                      dtype=torch.float32, device=self.q.device)
            self.dk_acc = [self.kv_acc[s * shape[0]:(s + 1) * shape[0]]
                           for s in range(P)]
            self.dv_acc = [self.kv_acc[(P + s) * shape[0]:(P + s + 1) * shape[0]]
                           for s in range(P)]
        need = max([bwd_workspace_bytes(n, l_q, c.shape[1], h, c.shape[2], d)
                    for c in k_chunks] + [bwd_prepare_bytes(n, l_q, h), 1])
        if self.ws is None or self.ws.numel() < need:
            with _on(stream):
                self.ws = torch.empty(need, dtype=torch.uint8, device=self.q.device)
        if one_launch:
            attn_acc_init(self.kv_acc, None, stream)
            attn_bwd_ring(self.dout, self.q, self.out, self.lse, k_chunks, v_chunks,
                          k_offsets, self.dk_acc, self.dv_acc, self.dq, self.scale,
                          self.causal, self.window[0], self.window[1], self.q_offset,
                          self.ws, stream)
            return self.dq, self.dk_acc, self.dv_acc
        attn_acc_init(self.dq_acc, None, stream)
        attn_acc_init(self.kv_acc, None, stream)
        attn_bwd_prepare(self.dout, self.out, self.lse, self.ws, stream)
        for kc, vc, ko, dka, dva in zip(k_chunks, v_chunks, k_offsets,
                                        self.dk_acc, self.dv_acc):
            attn_bwd_acc(self.dout, self.q, kc, vc, self.out, self.lse,
                         self.dq_acc, dka, dva, self.scale, self.causal,
                         self.window[0], self.window[1], self.q_offset, ko,
                         self.ws, stream, prepared=True)
        attn_acc_cast(self.dq_acc, self.dq, stream)
        return self.dq, self.dk_acc, self.dv_acc

    def capture(self, k_chunks, v_chunks, k_offsets):
        """Record `run` into a HIP graph (see RingShare.capture)."""
        return _capture(lambda: self.run(k_chunks, v_chunks, k_offsets))
