"""Brute-force exact attention in pure Python (loops, math.fsum), for tiny
shapes only.  It is a pin for the fp64 oracle: it shares nothing with it but
the definition (positions q_offset + i and k_offset + j, causal kpos <= qpos,
inclusive window, grouped heads hq // (h // h_kv), empty rows -> (0, -inf)).
"""
import math


def _allowed(i, j, causal, win_l, win_r, q_offset, k_offset):
    qp = q_offset + i
    kp = k_offset + j
    if causal and kp > qp:
        return False
    if win_l >= 0 and kp < qp - win_l:
        return False
    if win_r >= 0 and kp > qp + win_r:
        return False
    return True


def brute_attention(q, k, v, scale, causal=False, win_l=-1, win_r=-1,
                    q_offset=0, k_offset=0):
    """q [n][l_q][h][d], k, v [n][l_k][h_kv][d] as nested sequences.
    Returns (O nested [n][l_q][h][d], LSE nested [n][h][l_q])."""
    n = len(q)
    l_q = len(q[0])
    h = len(q[0][0])
    d = len(q[0][0][0])
    l_k = len(k[0])
    h_kv = len(k[0][0])
    grp = h // h_kv
    o = [[[[0.0] * d for _ in range(h)] for _ in range(l_q)] for _ in range(n)]
    lse = [[[0.0] * l_q for _ in range(h)] for _ in range(n)]
    for b in range(n):
        for hq in range(h):
            g = hq // grp
            for i in range(l_q):
                js = [j for j in range(l_k)
                      if _allowed(i, j, causal, win_l, win_r, q_offset,
                                  k_offset)]
                if not js:
                    lse[b][hq][i] = -math.inf
                    continue
                s = [scale * math.fsum(float(q[b][i][hq][c]) *
                                       float(k[b][j][g][c]) for c in range(d))
                     for j in js]
                m = max(s)
                tot = math.fsum(math.exp(x - m) for x in s)
                ls = m + math.log(tot)
                lse[b][hq][i] = ls
                for c in range(d):
                    o[b][i][hq][c] = math.fsum(
                        math.exp(x - ls) * float(v[b][j][g][c])
                        for x, j in zip(s, js))
    return o, lse
