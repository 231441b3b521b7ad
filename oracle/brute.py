"""Pure-Python brute force for tiny inputs (TEST INFRASTRUCTURE ONLY).

Loops over every (i, j, d) with math.exp and math.fsum; no numpy, no library
matmul.  It restates the definition in oracle/attention.py independently so the
two can be checked against each other for L <= 16.
"""
import math


def _visible(mode, i, j, block_size):
    if mode == "none":
        return True
    if mode == "causal":
        return j <= i
    if mode == "block_diag":
        return i // block_size == j // block_size
    raise ValueError(mode)


def attn_brute(q, k, v, mode, sm_scale, block_size=0):
    """q, k, v: nested lists [L][D] of floats for one head. Returns [L][D] floats."""
    L = len(q)
    D = len(v[0])
    out = []
    for i in range(L):
        keys = [j for j in range(L) if _visible(mode, i, j, block_size)]
        s = {j: sm_scale * math.fsum(q[i][d] * k[j][d] for d in range(len(q[i]))) for j in keys}
        top = max(s.values())
        w = {j: math.exp(s[j] - top) for j in keys}
        denom = math.fsum(w.values())
        out.append([math.fsum(w[j] * v[j][d] for j in keys) / denom for d in range(D)])
    return out


def lse_brute(q, k, mode, sm_scale, block_size=0):
    """ln(sum_j visible exp(S[i, j])) per row with math.log / math.fsum; [L] floats."""
    L = len(q)
    out = []
    for i in range(L):
        s = [sm_scale * math.fsum(q[i][d] * k[j][d] for d in range(len(q[i])))
             for j in range(L) if _visible(mode, i, j, block_size)]
        top = max(s)
        out.append(top + math.log(math.fsum(math.exp(x - top) for x in s)))
    return out
