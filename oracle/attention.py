"""Plain fp64 attention forward (TEST INFRASTRUCTURE ONLY).

What the pages compute, per (batch b, head h), on [B, H, L, D] tensors:

  S[i, j] = sm_scale * sum_d Q[i, d] K[j, d]
        -- the scale multiplies the dot product: [TLX, tlx_block_attn_kernel],
           [TCA, _flash_attn_fwd_kernel], [FA-A, _attn_fwd_inner].
  visible(i, j):
        none        every key                   [TCA, full example; FA-A, non-causal range]
        causal      j <= i                      [FA-A, _attn_fwd_inner, stage-2 mask]
        block_diag  floor(i/bs) == floor(j/bs)  [TLX, problem statement: only the
                                                 diagonal B x B blocks are nonzero]
  P[i, j] = exp(S[i, j] - m_i) on visible entries, 0 elsewhere, m_i = max visible S[i, :]
  l_i     = sum_j P[i, j]
  O[i, :] = sum_j Phat[i, j] V[j, :] / l_i
        -- normalising after P.V as in [TCA, online softmax core] and [FA-A, _attn_fwd].
           Phat = P, or P rounded to a narrow format when the caller asks for the
           cast the fp8-V path performs before P.V ([FA-A, _attn_fwd_inner], fp8 branch);
           l_i always uses the unrounded P ([TCA, online softmax core]: the row sum is
           taken over p itself; [FA-A, _attn_fwd_inner]: l_ij sums p, not p_cast).

attn_ref is the plain definition: full masked score rows (materialised in row
chunks, every row complete inside its chunk) and a standard, non-online softmax.
The online recurrence of the pages reaches the same O in exact arithmetic, so the
definition is the oracle for every unrounded case.

attn_online_ref writes the pages' online recurrence out in fp64 (running max m_i,
running sum l_i, rescaled accumulator, O = acc / l_i).  It only matters when Phat
is rounded: the rounding then happens against the running max, so the result
depends on the key-tile width.  It is the oracle for that case.
"""
import numpy as np

from .fp_formats import round_e5m2, round_bf16, round_f16

MODES = ("none", "causal", "block_diag")
_ROUNDERS = {None: None, "e5m2": round_e5m2, "bf16": round_bf16, "f16": round_f16}


def _check_mode(mode, L, block_size):
    if mode not in MODES:
        raise ValueError(f"unknown mask mode {mode!r}")
    if mode == "block_diag":
        # [TLX, tlx_block_attn wrapper]: the sequence length must split into whole blocks.
        if block_size <= 0 or L % block_size != 0:
            raise ValueError(f"block_diag needs block_size dividing L (L={L}, bs={block_size})")


def visible_mask(mode, L, block_size=0, rows=None):
    """Boolean [R, L]: which keys j each query row i may attend to."""
    _check_mode(mode, L, block_size)
    i = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    j = np.arange(L)
    if mode == "none":
        return np.ones((i.size, L), dtype=bool)
    if mode == "causal":
        return j[None, :] <= i[:, None]
    return (j[None, :] // block_size) == (i[:, None] // block_size)


def visible_pairs(mode, L, block_size=0):
    """Number of visible (i, j) pairs per head."""
    if mode == "none":
        return L * L
    if mode == "causal":
        return L * (L + 1) // 2
    return L * block_size


def attn_flops(mode, B, H, L, D, block_size=0):
    """Algorithmic FLOPs: 2*D for S[i,j] plus 2*D for P[i,j]*V[j,:], per visible pair."""
    return 4 * D * visible_pairs(mode, L, block_size) * B * H


def _as_f64(x):
    return np.asarray(x, dtype=np.float64)


def _row_chunks(rows, chunk):
    for s in range(0, rows.size, chunk):
        yield rows[s:s + chunk]


def attn_weights(q, k, mode, sm_scale, block_size=0, rows=None):
    """Normalised softmax weights P / l for one head: q [L, D], k [L, D] -> [R, L] fp64."""
    q = _as_f64(q)
    k = _as_f64(k)
    L = k.shape[0]
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    vis = visible_mask(mode, L, block_size, rows)
    S = sm_scale * (q[rows] @ k.T)
    S = np.where(vis, S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    assert np.all(np.isfinite(m)), "every row sees at least one key in every mode"
    P = np.where(vis, np.exp(S - m), 0.0)
    return P / P.sum(axis=1, keepdims=True)


def _head_ref(q, k, v, mode, sm_scale, block_size, rows, rounder, chunk):
    L = k.shape[0]
    out = np.empty((rows.size, v.shape[1]), dtype=np.float64)
    pos = 0
    for r in _row_chunks(rows, chunk):
        vis = visible_mask(mode, L, block_size, r)
        S = sm_scale * (q[r] @ k.T)                      # [R, L] full score rows
        S = np.where(vis, S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        assert np.all(np.isfinite(m)), "every row sees at least one key in every mode"
        P = np.where(vis, np.exp(S - m), 0.0)            # masked entries weigh exactly 0
        l = P.sum(axis=1, keepdims=True)                 # denominator from unrounded P
        Ph = P if rounder is None else rounder(P)
        out[pos:pos + r.size] = (Ph @ v) / l
        pos += r.size
    return out


def attn_ref(q, k, v, mode, sm_scale, block_size=0, rows=None, p_round=None, chunk=512):
    """Attention forward by the plain definition.

    q, k, v : real arrays [B, H, L, D] (any dtype that converts exactly to fp64)
    mode    : "none" | "causal" | "block_diag"
    rows    : optional 1-D array of query rows to evaluate (all rows if None)
    p_round : None, or "e5m2" | "bf16" | "f16" to round the unnormalised weights
              exp(S - m_i) (final-max frame) before P.V; l_i stays unrounded
    Returns fp64 [B, H, R, D].
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, L, D = q.shape
    _check_mode(mode, L, block_size)
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    rounder = _ROUNDERS[p_round]
    out = np.empty((B, H, rows.size, v.shape[3]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h] = _head_ref(q[b, h], k[b, h], v[b, h], mode, sm_scale, block_size,
                                  rows, rounder, chunk)
    return out


def attn_lse_ref(q, k, mode, sm_scale, block_size=0, rows=None):
    """Natural-log row normaliser lse_i = m_i + ln(sum_j visible exp(S[i, j] - m_i)).

    The fused-attention page stores this per row for a backward pass ([FA-A, _attn_fwd]
    epilogue: m_i += log(l_i)).  q, k: [B, H, L, D]; returns fp64 [B, H, R].
    """
    q, k = _as_f64(q), _as_f64(k)
    B, H, L, D = q.shape
    _check_mode(mode, L, block_size)
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((B, H, rows.size), dtype=np.float64)
    vis = visible_mask(mode, L, block_size, rows)
    for b in range(B):
        for h in range(H):
            S = np.where(vis, sm_scale * (q[b, h][rows] @ k[b, h].T), -np.inf)
            m = S.max(axis=1)
            out[b, h] = m + np.log(np.where(vis, np.exp(S - m[:, None]), 0.0).sum(axis=1))
    return out


def attn_online_ref(q, k, v, mode, sm_scale, block_n, block_size=0, rows=None, p_round=None):
    """The pages' online-softmax recurrence in fp64, key tiles of width block_n.

    For each query row, walk key tiles [t*block_n, (t+1)*block_n) in order
    ([TCA, online softmax core]; [FA-A, _attn_fwd_inner]):
        m_new = max(m, max of the tile's visible scores)
        p     = exp(s - m_new) on visible keys, 0 on masked keys
        alpha = exp(m - m_new)
        l     = l * alpha + sum(p)                  (unrounded p)
        acc   = acc * alpha + round(p) . V_tile     (round = identity unless p_round)
        m     = m_new
    then O = acc / l.  Tiles with no visible key for a row leave its state unchanged
    (the causal stage split of [FA-A, _attn_fwd] never visits them, and a tile whose
    keys are all masked contributes exp(-inf) = 0).  The state starts at m = -inf,
    l = 0, acc = 0; the pages start l at 1.0, which the first alpha = exp(-inf) = 0
    wipes out.  Returns fp64 [B, H, R, D].
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, L, D = q.shape
    _check_mode(mode, L, block_size)
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    rounder = _ROUNDERS[p_round]
    vis_all = visible_mask(mode, L, block_size, rows)       # [R, L]
    out = np.empty((B, H, rows.size, v.shape[3]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            S_all = sm_scale * (q[b, h][rows] @ k[b, h].T)   # [R, L]
            R = rows.size
            m = np.full(R, -np.inf)
            l = np.zeros(R)
            acc = np.zeros((R, v.shape[3]))
            for t0 in range(0, L, block_n):
                t1 = min(t0 + block_n, L)
                vis = vis_all[:, t0:t1]
                live = vis.any(axis=1)
                s = np.where(vis, S_all[:, t0:t1], -np.inf)
                m_new = np.where(live, np.maximum(m, s.max(axis=1)), m)
                shift = np.where(live, m_new, 0.0)[:, None]
                p = np.where(vis, np.exp(s - shift), 0.0)
                with np.errstate(invalid="ignore"):
                    alpha = np.where(live, np.exp(m - m_new), 1.0)
                alpha = np.where(np.isnan(alpha), 0.0, alpha)     # first live tile: exp(-inf)
                ph = p if rounder is None else rounder(p)
                l = l * alpha + p.sum(axis=1)
                acc = acc * alpha[:, None] + ph @ v[b, h][t0:t1]
                m = m_new
            out[b, h] = acc / l[:, None]
    return out
