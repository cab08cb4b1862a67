"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every function the header declares, and rejects bad arguments before making
any HIP call.  Pointers here are fake addresses: each call must fail its
argument checks, so nothing is ever dereferenced or launched."""
import ctypes
import os
import re

import numpy as np
import pytest

from blockwise_exact_attention_amd import _lib
from blockwise_exact_attention_amd._lib import (
    ATTN_BF16, ATTN_ERR_ALIAS, ATTN_ERR_ALIGN, ATTN_ERR_NULL, ATTN_ERR_SHAPE,
    ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_F32, ATTN_OK)
from blockwise_exact_attention_amd.flops import allowed_pairs
import oracle

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include",
                      "attn.h")

A = 1 << 32          # fake, well-aligned, far-apart device addresses
B = 2 << 32
C = 3 << 32
D_ = 4 << 32
E = 5 << 32
F = 6 << 32


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(attn_\w+)\s*\(", text,
                                 flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("attn_fwd", "attn_fwd_acc", "attn_fwd_ring", "attn_merge", "attn_bwd",
              "attn_bwd_acc", "attn_acc_init", "attn_acc_cast",
              "attn_bwd_workspace_bytes", "attn_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(declared_functions()) == set(_lib.SIGNATURES)


def test_python_constants_match_the_header():
    text = open(HEADER).read()
    consts = {m[0]: int(m[1]) for m in re.findall(r"\b(ATTN_\w+)\s*=\s*(\d+)", text)}
    assert len(consts) == 10
    for name, value in consts.items():
        assert getattr(_lib, name) == value, name
    defines = dict(re.findall(r"#define\s+(ATTN_\w+)\s+(.+)", text))
    assert int(defines["ATTN_RING_MAX_CHUNKS"]) == _lib.ATTN_RING_MAX_CHUNKS
    assert defines["ATTN_BWD_STATIC_MAX_WORKSPACE"].strip() == "(64 << 20)"
    assert _lib.ATTN_BWD_STATIC_MAX_WORKSPACE == 64 << 20


def test_status_strings():
    for s in range(8):
        assert _lib.status_string(s)
    assert _lib.status_string(ATTN_OK) == "ok"


def _fwd(**kw):
    a = dict(q=A, k=B, v=C, out=D_, lse=E, n=1, l_q=128, l_k=128, h=2, h_kv=2,
             d=64, scale=0.125, causal=0, win_l=-1, win_r=-1, q_offset=0,
             k_offset=0, stream=None, dtype=ATTN_BF16)
    a.update(kw)
    return _lib.lib().attn_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"],
                               a["n"], a["l_q"], a["l_k"], a["h"], a["h_kv"],
                               a["d"], a["scale"], a["causal"], a["win_l"],
                               a["win_r"], a["q_offset"], a["k_offset"],
                               a["stream"], a["dtype"])


def _fwd_acc(**kw):
    a = dict(q=A, k=B, v=C, acc=D_, lse=E, n=1, l_q=128, l_k=128, h=2, h_kv=2,
             d=64, scale=0.125, causal=0, win_l=-1, win_r=-1, q_offset=0,
             k_offset=0, stream=None, dtype=ATTN_BF16)
    a.update(kw)
    return _lib.lib().attn_fwd_acc(a["q"], a["k"], a["v"], a["acc"], a["lse"],
                                   a["n"], a["l_q"], a["l_k"], a["h"], a["h_kv"],
                                   a["d"], a["scale"], a["causal"], a["win_l"],
                                   a["win_r"], a["q_offset"], a["k_offset"],
                                   a["stream"], a["dtype"])


def test_fwd_acc_argument_checks():
    """The fused ring step rejects what attn_fwd rejects (the accumulator
    here is 128*2*64*4 = 64 KiB from D_); float32 inputs are checked with
    their own element size."""
    for f in ("q", "k", "v", "acc", "lse"):
        assert _fwd_acc(**{f: None}) == ATTN_ERR_NULL
    assert _fwd_acc(h=6, h_kv=4) == ATTN_ERR_SHAPE
    assert _fwd_acc(d=96) == ATTN_ERR_UNSUPPORTED
    # q is 32 KiB in bf16 and 64 KiB in float32: an accumulator 48 KiB past
    # q overlaps only the float32 one
    assert _fwd_acc(dtype=ATTN_F32, acc=A + 49152) == ATTN_ERR_ALIAS
    assert _fwd_acc(dtype=ATTN_F32, lse=E + 2) == ATTN_ERR_ALIGN
    assert _fwd_acc(acc=D_ + 8) == ATTN_ERR_ALIGN
    assert _fwd_acc(lse=E + 2) == ATTN_ERR_ALIGN
    assert _fwd_acc(acc=A + 64) == ATTN_ERR_ALIAS
    assert _fwd_acc(lse=D_ + 1024) == ATTN_ERR_ALIAS
    assert _fwd_acc(lse=C + 16) == ATTN_ERR_ALIAS


def _fwd_ring(chunks=None, **kw):
    """chunks: list of (k, v, l_k, k_offset); default two chunks of 128 keys
    at B/C and F/F+2^30."""
    a = dict(q=A, out=D_, lse=E, n=1, l_q=128, h=2, h_kv=2, d=64, scale=0.125,
             causal=0, win_l=-1, win_r=-1, q_offset=0, stream=None, dtype=ATTN_BF16,
             n_chunks=None, arrays=True)
    a.update(kw)
    if chunks is None:
        chunks = [(B, C, 128, 0), (F, F + (1 << 30), 128, 128)]
    nc = len(chunks) if a["n_chunks"] is None else a["n_chunks"]
    m = max(len(chunks), 1)
    kp = (ctypes.c_void_p * m)(*[c[0] for c in chunks])
    vp = (ctypes.c_void_p * m)(*[c[1] for c in chunks])
    lk = (ctypes.c_int * m)(*[c[2] for c in chunks])
    ko = (ctypes.c_longlong * m)(*[c[3] for c in chunks])
    if not a["arrays"]:
        kp = None
    return _lib.lib().attn_fwd_ring(a["q"], kp, vp, lk, ko, nc, a["out"], a["lse"],
                                    a["n"], a["l_q"], a["h"], a["h_kv"], a["d"],
                                    a["scale"], a["causal"], a["win_l"], a["win_r"],
                                    a["q_offset"], a["stream"], a["dtype"])


def test_fwd_ring_argument_checks():
    """The one-launch share checks the chunk count, the host arrays and every
    chunk as attn_fwd checks k and v, before any HIP call."""
    assert _fwd_ring(n_chunks=0) == ATTN_ERR_SHAPE
    many = [(B, C, 16, 16 * i) for i in range(_lib.ATTN_RING_MAX_CHUNKS + 1)]
    assert _fwd_ring(many) == ATTN_ERR_SHAPE
    assert _fwd_ring(arrays=False) == ATTN_ERR_NULL
    for f in ("q", "out", "lse"):
        assert _fwd_ring(**{f: None}) == ATTN_ERR_NULL
    assert _fwd_ring([(B, C, 128, 0), (None, C, 128, 0)]) == ATTN_ERR_NULL
    assert _fwd_ring([(B, C, 128, 0), (F, None, 128, 0)]) == ATTN_ERR_NULL
    assert _fwd_ring([(B, C, 128, 0), (F, F + 4096, -1, 0)]) == ATTN_ERR_SHAPE
    assert _fwd_ring(h=6, h_kv=4) == ATTN_ERR_SHAPE
    assert _fwd_ring(d=96) == ATTN_ERR_UNSUPPORTED
    # q is 32 KiB in bf16 and 64 KiB in float32: an output 48 KiB past q
    # overlaps only the float32 one
    assert _fwd_ring(dtype=ATTN_F32, out=A + 49152) == ATTN_ERR_ALIAS
    assert _fwd_ring(scale=float("nan")) == ATTN_ERR_UNSUPPORTED
    assert _fwd_ring(out=D_ + 8) == ATTN_ERR_ALIGN
    assert _fwd_ring([(B, C, 128, 0), (F + 8, F + 4096, 128, 0)]) == ATTN_ERR_ALIGN
    assert _fwd_ring(out=A + 64) == ATTN_ERR_ALIAS
    assert _fwd_ring(lse=D_ + 64) == ATTN_ERR_ALIAS
    # out over the second chunk's v
    assert _fwd_ring(out=F + (1 << 30) + 64) == ATTN_ERR_ALIAS
    # no rows: valid, nothing launched, chunk pointers may then be anything
    assert _fwd_ring(l_q=0, q=None, out=None, lse=None) == ATTN_OK
    # an empty chunk needs no pointers (rows are still there: checked only
    # up to the launch, so use zero rows to stay on the host)
    assert _fwd_ring([(None, None, 0, 0)], l_q=0, q=None, out=None, lse=None) == ATTN_OK


@pytest.mark.parametrize("field", ["q", "k", "v", "out", "lse"])
def test_fwd_null(field):
    assert _fwd(**{field: None}) == ATTN_ERR_NULL


@pytest.mark.parametrize("kw", [dict(n=-1), dict(l_q=-1), dict(l_k=-1),
                                dict(h=0), dict(h_kv=0), dict(h=6, h_kv=4),
                                dict(d=0), dict(n=1 << 30, l_q=1 << 30),
                                dict(h=1 << 18, h_kv=1 << 18),
                                dict(n=1 << 20, l_q=64, l_k=1 << 20, h=64, h_kv=64),
                                dict(n=1 << 20, l_q=64, l_k=64, h=1 << 10, h_kv=1),
                                # 2^30 query rows (2^32 work-items at four per row)
                                dict(n=1, l_q=1 << 30, l_k=64, h=1, h_kv=1),
                                # 2^30 key rows (2^32 work-items at four per row)
                                dict(n=1, l_q=64, l_k=1 << 30, h=1, h_kv=1)])
def test_fwd_shape(kw):
    assert _fwd(**kw) == ATTN_ERR_SHAPE


def test_empty_inputs_need_no_pointers_and_launch_nothing():
    """Zero rows (n = 0 or l_q = 0), or an empty chunk for the calls that then
    leave their outputs alone, return ATTN_OK before any HIP call, with NULL
    for every tensor that has no elements.  A NULL pointer to a non-empty
    tensor is still an error.  (A fused ring step over an empty chunk does
    launch: accumulator rows still at -inf are cleared to O = 0; the GPU
    tests cover it.)"""
    L = _lib.lib()
    nul = dict(q=None, k=None, v=None, out=None, lse=None)
    assert _fwd(n=0, **nul) == ATTN_OK
    assert _fwd(l_q=0, l_k=0, **nul) == ATTN_OK
    assert _fwd(l_q=0, q=None, out=None, lse=None) == ATTN_OK
    assert _fwd(l_k=0, k=None, v=None, out=None) == ATTN_ERR_NULL   # O has rows
    assert _fwd(n=0, h=0, **nul) == ATTN_ERR_SHAPE
    assert _fwd_acc(l_q=0, q=None, acc=None, lse=None) == ATTN_OK
    assert _fwd_acc(l_k=0, k=None, v=None, acc=None) == ATTN_ERR_NULL
    assert L.attn_merge(None, None, None, None, 1, 0, 2, 64, ATTN_BF16, None) == ATTN_OK
    assert L.attn_merge(None, None, None, None, 0, 5, 2, 64, ATTN_BF16, None) == ATTN_OK
    assert L.attn_merge(A, B, None, D_, 1, 5, 2, 64, ATTN_BF16, None) == ATTN_ERR_NULL
    assert L.attn_acc_init(None, None, 0, 5, 2, 64, None) == ATTN_OK
    assert L.attn_acc_cast(None, None, 3, 0, 2, 64, ATTN_BF16, None) == ATTN_OK
    for sizes in ((0, 128, 128), (1, 0, 128), (1, 128, 0)):
        assert L.attn_bwd_workspace_bytes(*sizes, 2, 2, 64) == 0
    bwd_args = lambda n, l_q, l_k, ptrs: (*ptrs, n, l_q, l_k, 2, 2, 64, 0.125, 1,
                                          -1, -1, 0, 0, None, 0, None, ATTN_BF16)
    assert L.attn_bwd(*bwd_args(0, 128, 128, [None] * 9)) == ATTN_OK
    assert L.attn_bwd(*bwd_args(1, 0, 0, [None] * 9)) == ATTN_OK
    # accumulating backward with no keys or no queries adds nothing
    kv_none = [A, A + (1 << 28), None, None, C, C + (1 << 28), D_, None, None]
    assert L.attn_bwd_acc(*bwd_args(1, 128, 0, kv_none)) == ATTN_OK
    q_none = [None, None, B, B + (1 << 28), None, None, None, D_, D_ + (1 << 28)]
    assert L.attn_bwd_acc(*bwd_args(1, 0, 128, q_none)) == ATTN_OK
    assert L.attn_bwd(*bwd_args(1, 128, 0, kv_none[:6] + [None] * 3)) == ATTN_ERR_NULL


@pytest.mark.parametrize("kw", [dict(d=96), dict(d=256), dict(dtype=7),
                                dict(scale=float("inf")),
                                dict(scale=float("nan"))])
def test_fwd_unsupported(kw):
    assert _fwd(**kw) == ATTN_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(q=A + 2), dict(out=D_ + 8),
                                dict(lse=E + 2)])
def test_fwd_align(kw):
    assert _fwd(**kw) == ATTN_ERR_ALIGN


@pytest.mark.parametrize("kw", [dict(out=A), dict(out=A + 64), dict(lse=C + 16),
                                dict(lse=D_ + 32)])
def test_fwd_alias(kw):
    assert _fwd(**kw) == ATTN_ERR_ALIAS


def test_merge_checks():
    L = _lib.lib()
    ok = dict(a=A, la=B, b=C, lb=D_, n=1, l=16, h=2, d=64, dt=ATTN_BF16)

    def call(**kw):
        x = dict(ok)
        x.update(kw)
        return L.attn_merge(x["a"], x["la"], x["b"], x["lb"], x["n"], x["l"],
                            x["h"], x["d"], x["dt"], None)
    assert call(a=None) == ATTN_ERR_NULL
    assert call(lb=None) == ATTN_ERR_NULL
    assert call(l=-1) == ATTN_ERR_SHAPE
    assert call(n=1 << 12, l=1 << 20, h=1 << 10, d=4) == ATTN_ERR_SHAPE  # 2^42 rows
    assert call(h=0) == ATTN_ERR_SHAPE
    assert call(dt=3) == ATTN_ERR_UNSUPPORTED
    assert call(a=A + 4) == ATTN_ERR_ALIGN
    assert call(b=A + 16) == ATTN_ERR_ALIAS
    assert call(lb=B) == ATTN_ERR_ALIAS
    assert L.attn_acc_init(None, B, 1, 2, 3, 4, None) == ATTN_ERR_NULL
    assert L.attn_acc_init(A, A + 8, 1, 2, 3, 4, None) == ATTN_ERR_ALIAS
    assert L.attn_acc_cast(A, B, 1, 2, 3, 4, 9, None) == ATTN_ERR_UNSUPPORTED
    assert L.attn_acc_cast(A, A + 16, 1, 2, 3, 4, ATTN_F32, None) == ATTN_ERR_ALIAS


def test_bwd_checks():
    L = _lib.lib()
    need = L.attn_bwd_workspace_bytes(1, 128, 128, 2, 2, 64)
    assert need > 0
    assert L.attn_bwd_workspace_bytes(1, 128, 128, 3, 2, 64) == 0

    ptrs = [A, A + (1 << 28), B, B + (1 << 28), C, C + (1 << 28), D_,
            D_ + (1 << 28), E]

    def call(ptrs=ptrs, ws=F, wsb=need, d=64, h=2, h_kv=2, dtype=ATTN_BF16):
        return L.attn_bwd(*ptrs, 1, 128, 128, h, h_kv, d, 0.125, 1, -1, -1, 0,
                          0, ws, wsb, None, dtype)
    bad = list(ptrs)
    bad[3] = None
    assert call(ptrs=bad) == ATTN_ERR_NULL
    assert call(h=3) == ATTN_ERR_SHAPE
    assert call(d=32) == ATTN_ERR_UNSUPPORTED
    # dout is 32 KiB in bf16 and 64 KiB in float32: a dq 40 KiB past it
    # overlaps only the float32 one
    f32_alias = list(ptrs)
    f32_alias[6] = A + 40960
    assert call(ptrs=f32_alias, dtype=ATTN_F32) == ATTN_ERR_ALIAS
    assert call(ws=None) == ATTN_ERR_WORKSPACE
    assert call(wsb=need - 1) == ATTN_ERR_WORKSPACE
    alias = list(ptrs)
    alias[6] = ptrs[1]          # dq on top of q
    assert call(ptrs=alias) == ATTN_ERR_ALIAS
    assert call(ws=ptrs[7]) == ATTN_ERR_ALIAS   # workspace on top of dk


def test_bwd_static_checks():
    """The allocation-free backward checks what attn_bwd checks, and refuses
    sizes whose workspace exceeds its static array, before any HIP call."""
    L = _lib.lib()
    ptrs = [A, A + (1 << 28), B, B + (1 << 28), C, C + (1 << 28), D_,
            D_ + (1 << 28), E]

    def call(ptrs=ptrs, n=1, l=128, d=64, h=2, h_kv=2, dtype=ATTN_BF16):
        return L.attn_bwd_static(*ptrs, n, l, l, h, h_kv, d, 0.125, 1, -1, -1, 0, 0, None,
                                 dtype)
    bad = list(ptrs)
    bad[3] = None
    assert call(ptrs=bad) == ATTN_ERR_NULL
    assert call(h=3) == ATTN_ERR_SHAPE
    assert call(d=32) == ATTN_ERR_UNSUPPORTED
    # dout is 32 KiB in bf16 and 64 KiB in float32: a dq 40 KiB past it
    # overlaps only the float32 one
    f32_alias = list(ptrs)
    f32_alias[6] = A + 40960
    assert call(ptrs=f32_alias, dtype=ATTN_F32) == ATTN_ERR_ALIAS
    alias = list(ptrs)
    alias[6] = ptrs[1]          # dq on top of q
    assert call(ptrs=alias) == ATTN_ERR_ALIAS
    # 2^21 rows of 4 heads: D and LSE take exactly the 64 MiB (accepted, up
    # to the launch); of 5 heads, 80 MiB (refused)
    big = [i << 40 for i in range(1, 10)]
    assert L.attn_bwd_workspace_bytes(1, 1 << 21, 1 << 21, 4, 4, 64) == \
        _lib.ATTN_BWD_STATIC_MAX_WORKSPACE
    assert L.attn_bwd_workspace_bytes(1, 1 << 21, 1 << 21, 5, 5, 64) > \
        _lib.ATTN_BWD_STATIC_MAX_WORKSPACE
    assert call(ptrs=big, l=1 << 21, h=5, h_kv=5) == ATTN_ERR_WORKSPACE
    # no rows: nothing to do, no workspace needed
    assert call(ptrs=[None] * 9, l=0) == ATTN_OK


def test_allowed_pairs_matches_oracle_mask():
    rng = np.random.default_rng(0)
    for _ in range(200):
        l_q = int(rng.integers(1, 40))
        l_k = int(rng.integers(1, 40))
        causal = bool(rng.integers(0, 2))
        wl = int(rng.integers(-1, 8))
        wr = int(rng.integers(-1, 8))
        qo = int(rng.integers(-20, 20))
        ko = int(rng.integers(-20, 20))
        m = oracle.allowed_mask(np.arange(l_q), np.arange(l_k), causal, wl, wr,
                                qo, ko)
        assert allowed_pairs(l_q, l_k, causal, wl, wr, qo, ko) == int(m.sum())
    # the workloads' pair counts
    assert allowed_pairs(2048, 2048, True) == 2098176
    assert allowed_pairs(4096, 4096, True, 256, 0) == 1019776
    assert allowed_pairs(1024, 1024, True, -1, -1, 7168, 7168) == 524800
    assert allowed_pairs(16384, 16384, True) == 134225920


def test_bwd_acc_checks():
    """The accumulating backward checks its arguments like attn_bwd, with
    float32 gradient accumulators: dk_acc starting 48 KiB into dq_acc
    (128*2*64*4 = 64 KiB) is an alias.  Every call here fails a check, so
    nothing is launched."""
    L = _lib.lib()
    need = L.attn_bwd_workspace_bytes(1, 128, 128, 2, 2, 64)
    ptrs = [A, A + (1 << 28), B, B + (1 << 28), C, C + (1 << 28), D_,
            D_ + (1 << 28), E]

    def call(ptrs=ptrs, ws=F, wsb=need, dtype=ATTN_BF16):
        return L.attn_bwd_acc(*ptrs, 1, 128, 128, 2, 2, 64, 0.125, 1, -1, -1,
                              0, 0, ws, wsb, None, dtype)
    for i in range(9):
        bad = list(ptrs)
        bad[i] = None
        assert call(ptrs=bad) == ATTN_ERR_NULL
    f32_alias = list(ptrs)
    f32_alias[6] = A + 40960    # inside a float32 dout only
    assert call(ptrs=f32_alias, dtype=ATTN_F32) == ATTN_ERR_ALIAS
    assert call(wsb=need - 1) == ATTN_ERR_WORKSPACE
    mis = list(ptrs)
    mis[6] = D_ + 4
    assert call(ptrs=mis) == ATTN_ERR_ALIGN
    near = list(ptrs)
    near[7] = D_ + 48 * 1024    # dk_acc inside dq_acc's 64 KiB
    assert call(ptrs=near) == ATTN_ERR_ALIAS


def test_missing_library_fails_loudly(monkeypatch):
    """No fallback: without libattn.so the binding raises instead of
    computing anything elsewhere."""
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", "/nonexistent/libattn.so")
    with pytest.raises(RuntimeError, match="missing"):
        _lib.lib()


def test_host_tensors_are_rejected():
    """The binding takes device tensors only: host tensors are refused before
    any library call (there is no CPU path)."""
    import torch
    from blockwise_exact_attention_amd import attention as A
    q = torch.zeros((1, 8, 2, 64), dtype=torch.bfloat16)
    lse = torch.zeros((1, 2, 8))
    with pytest.raises(ValueError, match="GPU"):
        A.attn_fwd(q, q, q, q.clone(), lse, 0.125)
    with pytest.raises(ValueError, match="GPU"):
        A.attn_merge(lse.new_zeros((1, 8, 2, 64)), lse.clone(), q, lse)


def _bwd_set(acc=False):
    """Consistent host tensors for the backward wrappers: q-shaped dout, q,
    out, dq and k-shaped k, v, dk, dv (GQA 4/2), LSE [n, h, l_q]."""
    import torch
    bf = torch.bfloat16
    gd = torch.float32 if acc else bf
    n, l_q, l_k, h, h_kv, d = 1, 8, 12, 4, 2, 64
    t = dict(dout=torch.zeros((n, l_q, h, d), dtype=bf),
             q=torch.zeros((n, l_q, h, d), dtype=bf),
             k=torch.zeros((n, l_k, h_kv, d), dtype=bf),
             v=torch.zeros((n, l_k, h_kv, d), dtype=bf),
             out=torch.zeros((n, l_q, h, d), dtype=bf),
             lse=torch.zeros((n, h, l_q)),
             dq=torch.zeros((n, l_q, h, d), dtype=gd),
             dk=torch.zeros((n, l_k, h_kv, d), dtype=gd),
             dv=torch.zeros((n, l_k, h_kv, d), dtype=gd))
    return t


@pytest.mark.parametrize("acc", [False, True])
@pytest.mark.parametrize("field,bad", [
    ("dout", "short"), ("out", "short"), ("out", "dtype"), ("v", "short"),
    ("v", "dtype"), ("lse", "short"), ("lse", "dtype"), ("dq", "short"),
    ("dq", "dtype"), ("dk", "short"), ("dv", "short"), ("dv", "dtype"),
    ("k", "head_dim")])
def test_bwd_wrapper_rejects_mismatched_tensors(acc, field, bad):
    """The backward wrappers check all nine tensors against q and k before
    anything reaches the library (which receives bare pointers and could not
    tell a short tensor): each mismatch raises ValueError naming the shape
    problem, not the device."""
    import torch
    from blockwise_exact_attention_amd import attention as A
    t = _bwd_set(acc)
    x = t[field]
    if bad == "short":
        t[field] = x[..., :-1].contiguous() if field == "lse" else x[:, :-1].contiguous()
    elif bad == "dtype":
        t[field] = x.to(torch.float16 if x.dtype == torch.float32 else torch.float32)
    else:
        t["k"] = x[..., :32].contiguous()
    fn = A.attn_bwd_acc if acc else A.attn_bwd
    with pytest.raises(ValueError) as e:
        fn(t["dout"], t["q"], t["k"], t["v"], t["out"], t["lse"], t["dq"], t["dk"],
           t["dv"], 0.125, True)
    assert "GPU" not in str(e.value)


@pytest.mark.parametrize("acc", [False, True])
def test_bwd_wrapper_consistent_host_tensors_reach_the_device_check(acc):
    """A consistent set passes every shape check and is then refused only
    because it is on the host."""
    from blockwise_exact_attention_amd import attention as A
    t = _bwd_set(acc)
    fn = A.attn_bwd_acc if acc else A.attn_bwd
    with pytest.raises(ValueError, match="GPU"):
        fn(t["dout"], t["q"], t["k"], t["v"], t["out"], t["lse"], t["dq"], t["dk"],
           t["dv"], 0.125, True)


def test_fwd_kernel_name_reports_the_dispatch():
    """Host-side dispatch: short key loops (the 256-key window) run the
    one-phase kernel, longer ones (12 and more key tiles per 128-row q tile
    on average) the pipelined one; rejected or kernel-free calls name
    nothing."""
    from blockwise_exact_attention_amd.attention import fwd_kernel_name
    import torch
    assert fwd_kernel_name(2, 2048, 2048, 16, 16, 128, True).startswith("fwd_pipe_kernel<128")
    assert fwd_kernel_name(4, 4096, 4096, 16, 16, 64, True, 256, 0).startswith(
        "fwd_bf16_kernel<64")
    assert fwd_kernel_name(1, 700, 700, 2, 2, 128, True).startswith("fwd_bf16_kernel<128")
    assert fwd_kernel_name(1, 16384, 16384, 16, 16, 128, True).startswith("fwd_pipe_kernel<128")
    assert fwd_kernel_name(1, 1024, 8192, 32, 8, 128, True, q_offset=7168).startswith(
        "fwd_pipe_kernel<128")
    assert fwd_kernel_name(1, 1024, 1024, 32, 8, 128, True, q_offset=7168,
                           fused=True) == "fwd_pipe_kernel<128, 2, true, false>"
    assert fwd_kernel_name(1, 512, 512, 4, 4, 128, True,
                           fused=True) == "fwd_bf16_kernel<128, 64, 2, true>"
    assert fwd_kernel_name(1, 128, 128, 2, 2, 64,
                           dtype=torch.float32) == "fwd_f32_kernel<64, false>"
    assert fwd_kernel_name(1, 128, 128, 2, 2, 128, dtype=torch.float32,
                           fused=True) == "fwd_f32_kernel<128, true>"
    assert fwd_kernel_name(1, 0, 128, 2, 2, 64) is None
    assert fwd_kernel_name(1, 128, 0, 2, 2, 64) is None
    assert fwd_kernel_name(1, 128, 128, 2, 2, 96) is None


def test_hbm_copy_checks():
    L = _lib.lib()
    assert L.attn_hbm_copy(A, B, 100, None) == ATTN_ERR_SHAPE      # not a multiple of 16
    assert L.attn_hbm_copy(A, B, -16, None) == ATTN_ERR_SHAPE
    assert L.attn_hbm_copy(None, B, 64, None) == ATTN_ERR_NULL
    assert L.attn_hbm_copy(A + 8, B, 64, None) == ATTN_ERR_ALIGN
    assert L.attn_hbm_copy(A, A + 32, 64, None) == ATTN_ERR_ALIAS
    assert L.attn_hbm_copy(None, None, 0, None) == ATTN_OK


def test_bwd_prepare_checks():
    """The once-per-share preprocessing and the prepared step check their
    arguments before any HIP call (fake addresses)."""
    L = _lib.lib()
    need = L.attn_bwd_prepare_bytes(1, 128, 2)
    assert need >= 2 * 128 * 2 * 4
    assert L.attn_bwd_prepare_bytes(1, 0, 2) == 0
    assert L.attn_bwd_prepare_bytes(-1, 128, 2) == 0

    def prep(dout=A, out=B, lse=C, ws=D_, wsb=need, d=64, h=2, dtype=ATTN_BF16, l_q=128):
        return L.attn_bwd_prepare(dout, out, lse, 1, l_q, h, d, ws, wsb, None, dtype)
    assert prep(dout=None) == ATTN_ERR_NULL
    assert prep(lse=None) == ATTN_ERR_NULL
    assert prep(d=96) == ATTN_ERR_UNSUPPORTED
    assert prep(dtype=ATTN_F32, ws=A + 40960) == ATTN_ERR_ALIAS   # inside a float32 dout only
    assert prep(l_q=-1) == ATTN_ERR_SHAPE
    assert prep(ws=None) == ATTN_ERR_WORKSPACE
    assert prep(wsb=need - 1) == ATTN_ERR_WORKSPACE
    assert prep(out=B + 8) == ATTN_ERR_ALIGN
    assert prep(ws=A + 256) == ATTN_ERR_ALIAS
    assert prep(l_q=0, dout=None, out=None, lse=None, ws=None) == ATTN_OK

    ptrs = [A, A + (1 << 28), B, B + (1 << 28), C, C + (1 << 28), D_,
            D_ + (1 << 28), E]
    wneed = L.attn_bwd_workspace_bytes(1, 128, 128, 2, 2, 64)

    def step(ptrs=ptrs, ws=F, wsb=wneed, h=2, dtype=ATTN_BF16):
        return L.attn_bwd_acc_prepared(*ptrs, 1, 128, 128, h, 2, 64, 0.125, 1, -1, -1, 0, 0,
                                       ws, wsb, None, dtype)
    bad = list(ptrs)
    bad[2] = None
    assert step(ptrs=bad) == ATTN_ERR_NULL
    assert step(h=3) == ATTN_ERR_SHAPE
    f32_alias = list(ptrs)
    f32_alias[6] = A + 40960    # inside a float32 dout only
    assert step(ptrs=f32_alias, dtype=ATTN_F32) == ATTN_ERR_ALIAS
    assert step(ws=None) == ATTN_ERR_WORKSPACE
    assert step(wsb=wneed - 1) == ATTN_ERR_WORKSPACE
    assert step(ws=ptrs[7]) == ATTN_ERR_ALIAS


def test_bwd_ring_checks():
    """The one-launch ring backward checks the chunk count, the host arrays,
    every tensor and the workspace before any HIP call (fake addresses)."""
    L = _lib.lib()
    G = 7 << 32
    H = 8 << 32

    def call(n_chunks=2, arrays=True, l_k=(128, 64), k=(B, B + (1 << 30)),
             dka=(F, F + (1 << 30)), dva=(G, G + (1 << 30)), dq=D_ + (1 << 28), ws=H,
             wsb=None, dtype=ATTN_BF16, h=2, d=64):
        m = max(n_chunks, 1)
        pad = lambda t, x: list(t[:m]) + [x] * (m - len(t[:m]))
        kp = (ctypes.c_void_p * m)(*pad(k, B))
        vp = (ctypes.c_void_p * m)(*[C + (i << 30) for i in range(m)])
        lk = (ctypes.c_int * m)(*pad(l_k, 16))
        ko = (ctypes.c_longlong * m)(*[64 * i for i in range(m)])
        ka = (ctypes.c_void_p * m)(*pad(dka, F))
        va = (ctypes.c_void_p * m)(*pad(dva, G))
        need = L.attn_bwd_prepare_bytes(1, 128, h) if wsb is None else wsb
        return L.attn_bwd_ring(A, A + (1 << 28), D_, E, kp if arrays else None, vp, lk, ko,
                               ka, va, n_chunks, dq, 1, 128, h, 2, d, 0.125, 1, -1, -1, 64,
                               ws, need, None, dtype)
    assert call(n_chunks=0) == ATTN_ERR_SHAPE
    assert call(n_chunks=_lib.ATTN_RING_MAX_CHUNKS + 1) == ATTN_ERR_SHAPE
    assert call(arrays=False) == ATTN_ERR_NULL
    assert call(dq=None) == ATTN_ERR_NULL
    assert call(dka=(F, None)) == ATTN_ERR_NULL
    assert call(l_k=(128, -1)) == ATTN_ERR_SHAPE
    assert call(h=3) == ATTN_ERR_SHAPE
    assert call(d=96) == ATTN_ERR_UNSUPPORTED
    # dout is 32 KiB in bf16 and 64 KiB in float32: a dq 40 KiB past it
    # overlaps only the float32 one
    assert call(dtype=ATTN_F32, dq=A + 40960) == ATTN_ERR_ALIAS
    assert call(ws=None) == ATTN_ERR_WORKSPACE
    assert call(wsb=16) == ATTN_ERR_WORKSPACE
    assert call(dka=(F + 8, F + (1 << 30))) == ATTN_ERR_ALIGN
    assert call(dq=A + 64) == ATTN_ERR_ALIAS                 # dq over dout
    assert call(dka=(F, F)) == ATTN_ERR_ALIAS                # two accumulators
    assert call(dva=(G, B + (1 << 30) + 64)) == ATTN_ERR_ALIAS   # accumulator over a K chunk
