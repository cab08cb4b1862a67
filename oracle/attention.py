"""Plain fp64 oracle of exact attention, its backward, the (O, LSE) merge and
the ring share of one device.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py. It shares no code with the HIP library.

Everything here is the definition written out, in float64, with library
matmuls as steps and no online softmax: each query row's softmax is taken over
its whole allowed key set at once.

Sources (page titles, then the function on the page):
  * "picotron/parallel/context_parallel.py": ring_attention_forward (scores
    scaled after the dot product, upper-triangular causal mask, max-shifted
    exponentials, log-sum-exp, P.V), ring_attention_backward (recompute P from
    the LSE; dV, dP, D = rowsum(dO*O), dS = P*(dP - D), dQ, dK),
    update_out_and_lse (the sigmoid form of the merge; the first call returns
    the block itself), RingAttention._repeat_kv (grouped-query heads: each
    key/value head serves a run of consecutive query heads).
  * "flash_sharding.py" (flash_attn_jax): ring_fwd (accumulator starts at
    O = 0, LSE = -inf; a chunk that lies wholly in the causal future yields
    O = 0 and LSE = -inf; the log1p form of the merge; block outputs are
    upcast before merging), partition_fwd (window_size = (-1, -1) means no
    local window).

Readings where the pages are silent (each one is listed with its reason in the
design notes of the repository):
  * positions are absolute: a query row i sits at q_offset + i and a key row j
    at k_offset + j; causal allows kpos <= qpos;
  * a window (win_l, win_r) is inclusive, kpos in [qpos - win_l, qpos + win_r];
    a negative side is unbounded; causal and window intersect;
  * a row with no allowed key has O = 0 and LSE = -inf and gets zero
    gradients (the ring_fwd convention for a skipped chunk);
  * merging with an LSE of -inf on either side is the identity on the other
    side, never NaN;
  * GQA: query head hq reads key/value head hq // (h // h_kv).

Layouts: q, o, dO, dq [n, l_q, h, d]; k, v, dk, dv [n, l_k, h_kv, d];
lse [n, h, l_q].
"""
from __future__ import annotations

import numpy as np

_NEG_INF = -np.inf


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def allowed_mask(i_idx, j_idx, causal, win_l, win_r, q_offset, k_offset):
    """Boolean [len(i_idx), len(j_idx)]: may query row i attend to key row j.

    qpos = q_offset + i, kpos = k_offset + j; causal keeps kpos <= qpos (the
    upper-triangular mask of ring_attention_forward, for equal offsets), the
    window keeps qpos - win_l <= kpos <= qpos + win_r, each side only when
    non-negative (window_size == (-1, -1) means no window in flash_sharding.py,
    partition_fwd).
    """
    assert abs(int(q_offset)) < 2**62 and abs(int(k_offset)) < 2**62
    qpos = np.int64(q_offset) + np.asarray(i_idx, dtype=np.int64)[:, None]
    kpos = np.int64(k_offset) + np.asarray(j_idx, dtype=np.int64)[None, :]
    ok = np.ones((qpos.shape[0], kpos.shape[1]), dtype=bool)
    if causal:
        ok &= kpos <= qpos
    if win_l >= 0:
        ok &= kpos >= qpos - np.int64(win_l)
    if win_r >= 0:
        ok &= kpos <= qpos + np.int64(win_r)
    return ok


def _group(h, h_kv):
    assert h % h_kv == 0, "query heads must be a multiple of key/value heads"
    return h // h_kv


def _row_blocks(rows, block):
    for s in range(0, len(rows), block):
        yield rows[s:s + block]


def _scores_block(qh, kh, rows, scale, causal, win_l, win_r, q_offset,
                  k_offset):
    """Scaled scores of `rows` against every key, masked keys = -inf.

    Returns (S, keys, nonempty): S is [len(rows), len(keys)] over the key
    columns that at least one row of the block may see (columns nobody may
    see contribute exactly zero and are dropped), `nonempty` marks rows with
    at least one allowed key.
    """
    l_k = kh.shape[0]
    mask = allowed_mask(rows, np.arange(l_k), causal, win_l, win_r, q_offset,
                        k_offset)
    keys = np.nonzero(mask.any(axis=0))[0]
    mask = mask[:, keys]
    s = (qh[rows] @ kh[keys].T) * scale
    s = np.where(mask, s, _NEG_INF)
    return s, keys, mask, mask.any(axis=1)


def _softmax_rows(s, nonempty):
    """Row max, LSE and P of masked scores (picotron ring_attention_forward).

    Empty rows get LSE = -inf and P = 0 (flash_sharding.py ring_fwd, the
    skipped-chunk branch)."""
    m = np.where(nonempty, np.max(s, axis=1, initial=_NEG_INF), 0.0)
    e = np.exp(s - m[:, None])
    tot = e.sum(axis=1)
    lse = np.where(nonempty, np.log(np.where(nonempty, tot, 1.0)) + m,
                   _NEG_INF)
    p = np.where(nonempty[:, None], e / np.where(nonempty, tot, 1.0)[:, None],
                 0.0)
    return lse, p


def attention_fwd(q, k, v, scale, causal=False, win_l=-1, win_r=-1,
                  q_offset=0, k_offset=0, heads=None, rows=None, block=512):
    """Exact attention forward in fp64: returns (O [n,l_q,h,d], LSE [n,h,l_q]).

    `heads` (iterable of (b, hq)) and `rows` (query indices) restrict the work
    to a sample; entries outside the sample are NaN.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, l_q, h, d = q.shape
    _, l_k, h_kv, dk = k.shape
    assert dk == d and v.shape == k.shape and k.shape[0] == n
    grp = _group(h, h_kv)
    o = np.full((n, l_q, h, d), np.nan)
    lse = np.full((n, h, l_q), np.nan)
    if heads is None:
        heads = [(b, hq) for b in range(n) for hq in range(h)]
    rows = np.arange(l_q) if rows is None else np.asarray(rows, np.int64)
    for b, hq in heads:
        g = hq // grp
        qh, kh, vh = q[b, :, hq, :], k[b, :, g, :], v[b, :, g, :]
        for rb in _row_blocks(rows, block):
            s, keys, _, nonempty = _scores_block(qh, kh, rb, scale, causal,
                                                 win_l, win_r, q_offset,
                                                 k_offset)
            lse_b, p = _softmax_rows(s, nonempty)
            o[b, rb, hq, :] = p @ vh[keys]
            lse[b, hq, rb] = lse_b
    return o, lse


def attention_bwd(q, k, v, do, scale, causal=False, win_l=-1, win_r=-1,
                  q_offset=0, k_offset=0, kv_heads=None, block=512):
    """Exact attention backward in fp64 (picotron ring_attention_backward).

    Recomputes the forward itself (O and LSE in fp64), then per row block:
    P = exp(S - LSE), dV += P^T dO, dP = dO V^T, D = rowsum(dO * O),
    dS = P * (dP - D) (zero where masked), dQ = scale dS K,
    dK += scale dS^T Q.  Grouped heads: dK and dV of a key/value head are the
    sums over the query heads that read it, which is what differentiating
    through RingAttention._repeat_kv gives.

    `kv_heads` (iterable of (b, g)) restricts the work to whole key/value
    groups; entries outside are NaN.  Returns (dq, dk, dv).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    n, l_q, h, d = q.shape
    _, l_k, h_kv, _ = k.shape
    grp = _group(h, h_kv)
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    if kv_heads is None:
        kv_heads = [(b, g) for b in range(n) for g in range(h_kv)]
    rows = np.arange(l_q)
    for b, g in kv_heads:
        kh, vh = k[b, :, g, :], v[b, :, g, :]
        dk_acc = np.zeros((l_k, d))
        dv_acc = np.zeros((l_k, d))
        for hq in range(g * grp, (g + 1) * grp):
            qh, doh = q[b, :, hq, :], do[b, :, hq, :]
            for rb in _row_blocks(rows, block):
                s, keys, mask, nonempty = _scores_block(
                    qh, kh, rb, scale, causal, win_l, win_r, q_offset,
                    k_offset)
                _, p = _softmax_rows(s, nonempty)
                o_rb = p @ vh[keys]
                dv_acc[keys] += p.T @ doh[rb]
                dp = doh[rb] @ vh[keys].T
                dd = np.sum(doh[rb] * o_rb, axis=1)
                ds = np.where(mask, p * (dp - dd[:, None]), 0.0)
                dq[b, rb, hq, :] = scale * (ds @ kh[keys])
                dk_acc[keys] += scale * (ds.T @ qh[rb])
        dk[b, :, g, :] = dk_acc
        dv[b, :, g, :] = dv_acc
    return dq, dk, dv


def merge(o1, lse1, o2, lse2):
    """Merge two partial results over disjoint key sets, log1p form
    (flash_sharding.py, ring_fwd): lse = mx + log1p(exp(mn - mx)),
    o = o1 exp(lse1 - lse) + o2 exp(lse2 - lse).

    o* [n,l,h,d], lse* [n,h,l].  An LSE of -inf on one side returns the other
    side unchanged (both -inf: O = 0, LSE = -inf).
    """
    o1, lse1, o2, lse2 = _f64(o1), _f64(lse1), _f64(o2), _f64(lse2)
    e1 = np.isneginf(lse1)
    e2 = np.isneginf(lse2)
    both = e1 | e2
    a = np.where(both, 0.0, lse1)
    b = np.where(both, 0.0, lse2)
    mx = np.maximum(a, b)
    mn = np.minimum(a, b)
    lse = mx + np.log1p(np.exp(mn - mx))
    w1 = np.exp(a - lse)
    w2 = np.exp(b - lse)
    o = (o1 * np.transpose(w1, (0, 2, 1))[..., None]
         + o2 * np.transpose(w2, (0, 2, 1))[..., None])
    # identity guards: a -inf side carries no mass
    lse = np.where(e2, lse1, np.where(e1, lse2, lse))
    r1 = np.transpose(e1, (0, 2, 1))[..., None]
    r2 = np.transpose(e2, (0, 2, 1))[..., None]
    o = np.where(r2, np.where(r1, 0.0, o1), np.where(r1, o2, o))
    return o, lse


def merge_sigmoid(o1, lse1, o2, lse2):
    """Same merge in the sigmoid form of picotron update_out_and_lse:
    out -= sigmoid(blse - lse) (out - bout); lse -= logsigmoid(lse - blse),
    with the same -inf identity guards as `merge`."""
    o1, lse1, o2, lse2 = _f64(o1), _f64(lse1), _f64(o2), _f64(lse2)
    e1 = np.isneginf(lse1)
    e2 = np.isneginf(lse2)
    both = e1 | e2
    a = np.where(both, 0.0, lse1)
    b = np.where(both, 0.0, lse2)
    sig = 1.0 / (1.0 + np.exp(-(b - a)))
    # logsigmoid(x) = -log1p(exp(-x)), written for either sign of x
    x = a - b
    logsig = np.where(x >= 0, -np.log1p(np.exp(-x)), x - np.log1p(np.exp(x)))
    o = o1 - np.transpose(sig, (0, 2, 1))[..., None] * (o1 - o2)
    lse = a - logsig
    lse = np.where(e2, lse1, np.where(e1, lse2, lse))
    r1 = np.transpose(e1, (0, 2, 1))[..., None]
    r2 = np.transpose(e2, (0, 2, 1))[..., None]
    o = np.where(r2, np.where(r1, 0.0, o1), np.where(r1, o2, o))
    return o, lse


def ring_share(q, k_chunks, v_chunks, scale, causal, q_offset, k_offsets,
               heads=None):
    """One device's share of ring attention (flash_sharding.py ring_fwd):
    start at (O = 0, LSE = -inf), then for every key/value chunk s attend the
    local queries to it with absolute offsets and merge the result in.
    Returns (O, LSE) in fp64."""
    q = _f64(q)
    n, l, h, d = q.shape
    o = np.zeros((n, l, h, d))
    lse = np.full((n, h, l), _NEG_INF)
    for kc, vc, ko in zip(k_chunks, v_chunks, k_offsets):
        ob, lb = attention_fwd(q, kc, vc, scale, causal, -1, -1, q_offset, ko,
                               heads=heads)
        if heads is not None:
            ob = np.nan_to_num(ob)
            lb = np.where(np.isnan(lb), _NEG_INF, lb)
        o, lse = merge(o, lse, ob, lb)
    return o, lse
