"""Pins for the CPU oracle: it is checked against things other than itself.

P1 brute force (pure-Python loops) on L <= 16        P6 block_diag == full attention on each block
P2 library routine (torch SDPA, fp64, CPU)            P7 closed forms (bs=L, bs=1, Q=0 means)
P3 weights of each row sum to 1, masked weights 0    P8 invariance to a common shift of K; sharp rows
P4 constant V reproduces V                            P9 causal row i == dense attention on prefix
P5 causal row 0 returns v_0 exactly                   P10 narrow-format rounding vs torch's casts
plus hand-worked values (tests/golden/hand_worked.json), the online recurrence
against the definition, and planted mistakes that the pins must catch.
"""
import importlib.util
import json
import math
import os
import sys
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MODES_BS = [("none", 0), ("causal", 0), ("block_diag", 1), ("block_diag", 2),
            ("block_diag", 4), ("block_diag", 8), ("block_diag", 16)]


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _qkv(B, H, L, D, seed, scale=1.0):
    return (_rand((B, H, L, D), seed, scale), _rand((B, H, L, D), seed + 1, scale),
            _rand((B, H, L, D), seed + 2))


# ---------------------------------------------------------------- P1 brute force
@pytest.mark.parametrize("mode,bs", MODES_BS)
@pytest.mark.parametrize("L,D", [(1, 1), (5, 3), (16, 8)])
def test_p1_brute_force(mode, bs, L, D):
    if mode == "block_diag" and L % bs:
        pytest.skip("block size must divide L")
    q, k, v = _qkv(1, 2, L, D, seed=L * 100 + D, scale=1.5)
    got = oracle.attn_ref(q, k, v, mode, 0.37, bs)
    for h in range(2):
        ref = np.array(oracle.attn_brute(q[0, h].tolist(), k[0, h].tolist(), v[0, h].tolist(),
                                         mode, 0.37, bs))
        assert np.abs(got[0, h] - ref).max() <= 1e-12


# ---------------------------------------------------------------- P2 library routine
@pytest.mark.parametrize("mode,bs", [("none", 0), ("causal", 0), ("block_diag", 32),
                                     ("block_diag", 64)])
@pytest.mark.parametrize("L", [64, 256])
def test_p2_torch_sdpa(mode, bs, L):
    q, k, v = _qkv(2, 3, L, 32, seed=7 + L)
    scale = 1.0 / math.sqrt(32)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    if mode == "none":
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
    elif mode == "causal":
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                                               scale=scale)
    else:
        idx = torch.arange(L)
        mask = (idx[:, None] // bs) == (idx[None, :] // bs)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                               scale=scale)
    got = oracle.attn_ref(q, k, v, mode, scale, bs)
    assert np.abs(got - ref.numpy()).max() <= 1e-12


# ---------------------------------------------------------------- P3 rows sum to one
@pytest.mark.parametrize("mode,bs", [("none", 0), ("causal", 0), ("block_diag", 8)])
def test_p3_weights_sum_to_one(mode, bs):
    q, k, _ = _qkv(1, 1, 64, 16, seed=3, scale=2.0)
    W = oracle.attn_weights(q[0, 0], k[0, 0], mode, 0.25, bs)
    assert np.abs(W.sum(axis=1) - 1.0).max() <= 1e-14
    vis = oracle.visible_mask(mode, 64, bs)
    assert np.all(W[~vis] == 0.0)
    assert np.all(W[vis] > 0.0)


# ---------------------------------------------------------------- P4 constant V
@pytest.mark.parametrize("mode,bs", [("none", 0), ("causal", 0), ("block_diag", 16)])
def test_p4_constant_v(mode, bs):
    q, k, _ = _qkv(2, 2, 48, 8, seed=11, scale=3.0)
    c = np.linspace(-2.0, 5.0, 8)
    v = np.broadcast_to(c, q.shape).copy()
    got = oracle.attn_ref(q, k, v, mode, 0.5, bs)
    assert np.abs(got - c).max() <= 1e-13


# ---------------------------------------------------------------- P5 causal row 0
def test_p5_causal_row0_is_v0():
    q, k, v = _qkv(2, 3, 40, 8, seed=5, scale=4.0)
    got = oracle.attn_ref(q, k, v, "causal", 0.8)
    assert np.array_equal(got[:, :, 0, :], v[:, :, 0, :])


# ---------------------------------------------------------------- P6 block restriction
@pytest.mark.parametrize("bs", [4, 16, 64])
def test_p6_block_diag_is_full_attention_per_block(bs):
    L = 128
    q, k, v = _qkv(2, 2, L, 16, seed=bs)
    got = oracle.attn_ref(q, k, v, "block_diag", 0.3, bs)
    for blk in range(L // bs):
        sl = slice(blk * bs, (blk + 1) * bs)
        ref = oracle.attn_ref(q[:, :, sl], k[:, :, sl], v[:, :, sl], "none", 0.3)
        assert np.abs(got[:, :, sl] - ref).max() <= 1e-13


# ---------------------------------------------------------------- P7 closed forms
def test_p7_closed_forms():
    L, D = 32, 8
    q, k, v = _qkv(1, 2, L, D, seed=9)
    # block size L is dense attention; block size 1 returns V
    assert np.abs(oracle.attn_ref(q, k, v, "block_diag", 0.4, L)
                  - oracle.attn_ref(q, k, v, "none", 0.4)).max() <= 1e-13
    assert np.abs(oracle.attn_ref(q, k, v, "block_diag", 0.4, 1) - v).max() <= 1e-14
    # Q = 0: every visible key weighs the same
    z = np.zeros_like(q)
    assert np.abs(oracle.attn_ref(z, k, v, "none", 0.4) - v.mean(axis=2, keepdims=True)).max() <= 1e-14
    prefix = np.cumsum(v, axis=2) / np.arange(1, L + 1)[None, None, :, None]
    assert np.abs(oracle.attn_ref(z, k, v, "causal", 0.4) - prefix).max() <= 1e-14
    bmean = v.reshape(1, 2, L // 4, 4, D).mean(axis=3, keepdims=True)
    bmean = np.broadcast_to(bmean, (1, 2, L // 4, 4, D)).reshape(1, 2, L, D)
    assert np.abs(oracle.attn_ref(z, k, v, "block_diag", 0.4, 4) - bmean).max() <= 1e-14


# ---------------------------------------------------------------- P8 shift invariance, sharp rows
@pytest.mark.parametrize("mode,bs", [("none", 0), ("causal", 0), ("block_diag", 8)])
def test_p8_shift_and_sharp(mode, bs):
    q, k, v = _qkv(1, 2, 64, 16, seed=21)
    u = _rand((16,), 99, 3.0)
    # adding one vector u to every key adds q_i.u to the whole row i of S
    a = oracle.attn_ref(q, k, v, mode, 0.5, bs)
    b = oracle.attn_ref(q, k + u, v, mode, 0.5, bs)
    assert np.abs(a - b).max() <= 1e-11
    sharp = oracle.attn_ref(q * 8.0, k, v, mode, 0.5, bs)
    assert np.all(np.isfinite(sharp))
    # a very sharp row picks the arg-max key's value (rows whose top two scores are
    # more than 60 apart, so the runner-up weighs below e^-60)
    big = oracle.attn_ref(q * 1e4, k, v, mode, 0.5, bs)
    S = 0.5 * 1e4 * (q[0, 0] @ k[0, 0].T)
    S = np.where(oracle.visible_mask(mode, 64, bs), S, -np.inf)
    top2 = np.sort(S, axis=1)[:, -2:]
    clear = (top2[:, 1] - top2[:, 0]) > 60.0
    assert clear.sum() >= 32
    arg = S.argmax(axis=1)
    assert np.abs(big[0, 0][clear] - v[0, 0][arg][clear]).max() <= 1e-12


# ---------------------------------------------------------------- P9 causal prefix
def test_p9_causal_row_is_dense_on_prefix():
    L = 40
    q, k, v = _qkv(1, 1, L, 8, seed=33)
    c = oracle.attn_ref(q, k, v, "causal", 0.6)
    for i in (0, 1, 7, 23, L - 1):
        d = oracle.attn_ref(q[:, :, :i + 1], k[:, :, :i + 1], v[:, :, :i + 1], "none", 0.6)
        assert np.abs(c[:, :, i] - d[:, :, i]).max() <= 1e-14
    assert np.abs(c[:, :, -1] - oracle.attn_ref(q, k, v, "none", 0.6)[:, :, -1]).max() <= 1e-14


# ---------------------------------------------------------------- row subsets
def test_rows_subset_matches_full():
    q, k, v = _qkv(1, 2, 100, 8, seed=4)
    rows = np.array([0, 3, 50, 99])
    for mode, bs in (("none", 0), ("causal", 0), ("block_diag", 25)):
        full = oracle.attn_ref(q, k, v, mode, 0.7, bs)
        sub = oracle.attn_ref(q, k, v, mode, 0.7, bs, rows=rows, chunk=3)
        assert np.array_equal(sub, full[:, :, rows]) or np.abs(sub - full[:, :, rows]).max() <= 1e-15


# ---------------------------------------------------------------- hand-worked values
def test_hand_worked_cases():
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        scale = math.log(3.0) if c["sm_scale"] == "ln3" else float(c["sm_scale"])
        q, k, v = (np.array(c[x], dtype=np.float64)[None, None] for x in ("q", "k", "v"))
        got = oracle.attn_ref(q, k, v, c["mode"], scale, c["block_size"])[0, 0]
        assert np.abs(got - np.array(c["o"])).max() <= 1e-14, c["name"]


# ---------------------------------------------------------------- online recurrence
@pytest.mark.parametrize("mode,bs", [("none", 0), ("causal", 0), ("block_diag", 16)])
@pytest.mark.parametrize("block_n", [1, 7, 16, 64, 1000])
def test_online_recurrence_equals_definition(mode, bs, block_n):
    q, k, v = _qkv(1, 2, 96, 8, seed=block_n, scale=2.0)
    a = oracle.attn_ref(q, k, v, mode, 0.5, bs)
    b = oracle.attn_online_ref(q, k, v, mode, 0.5, block_n, bs)
    assert np.abs(a - b).max() <= 1e-13


def test_online_single_tile_rounding_matches_final_frame():
    # with one key tile the running max is the final max, so both readings of the
    # rounded-P path coincide
    q, k, v = _qkv(1, 2, 64, 16, seed=3)
    for mode in ("none", "causal"):
        a = oracle.attn_ref(q, k, v, mode, 0.25, p_round="e5m2")
        b = oracle.attn_online_ref(q, k, v, mode, 0.25, 64, p_round="e5m2")
        assert np.abs(a - b).max() <= 1e-14
    # and rounding P does change the answer (so the option is live)
    c = oracle.attn_ref(q, k, v, "none", 0.25)
    assert np.abs(a - c).max() > 1e-3


def _frame_case():
    """One query row, two keys with scores 0 and ln 2.6 (sm_scale 1), v = (7, 14).

    Worked by hand from the fused-attention page's fp8 branch (_attn_fwd_inner: p is taken
    against the running max, cast to e5m2 for P.V, the row sum uses the uncast p):
      tile width 1, running frame: tile 0 has m = 0, p = 1 (exact in e5m2), acc = 7, l = 1;
        tile 1 has m = ln 2.6, alpha = 1/2.6, p = 1, so acc = 7/2.6 + 14, l = 1/2.6 + 1 and
        o = (7 + 14 * 2.6) / 3.6 = 217/18 = 12.0555...
      one tile (width 2), i.e. the final-max frame of the plain definition with the cast:
        weights 1/2.6 -> e5m2 0.375 (the grid in [0.25, 0.5) is 0.25, 0.3125, 0.375, 0.4375)
        and 1; o = (0.375 * 7 + 14) / (1/2.6 + 1) = 1729/144 = 12.00694...
      rounding in the previous frame instead (tile 1's weight taken against m = 0 is 2.6 ->
        e5m2 2.5, then rescaled by 1/2.6): o = (7 + 2.5 * 14) / 3.6 = 35/3 = 11.666...
    The three frames give three different answers, so the rounding frame is pinned.
    """
    q = np.array([[[[1.0], [1.0]]]])
    k = np.array([[[[0.0], [math.log(2.6)]]]])
    v = np.array([[[[7.0], [14.0]]]])
    return q, k, v


RUNNING_FRAME_O = 217.0 / 18.0
FINAL_FRAME_O = 1729.0 / 144.0


def test_online_rounding_uses_running_max_frame():
    q, k, v = _frame_case()
    o = oracle.attn_online_ref(q, k, v, "none", 1.0, 1, p_round="e5m2")
    assert abs(o[0, 0, 1, 0] - RUNNING_FRAME_O) <= 1e-12
    # one tile: the running max is the final max
    o1 = oracle.attn_online_ref(q, k, v, "none", 1.0, 2, p_round="e5m2")
    assert abs(o1[0, 0, 1, 0] - FINAL_FRAME_O) <= 1e-12
    # row 0 sees its own key only in causal mode: weight 1, exact
    oc = oracle.attn_online_ref(q, k, v, "causal", 1.0, 1, p_round="e5m2")
    assert oc[0, 0, 0, 0] == 7.0 and abs(oc[0, 0, 1, 0] - RUNNING_FRAME_O) <= 1e-12


def test_plain_definition_rounds_in_final_frame():
    # the plain definition with the cast rounds exp(S - m_final), divides by the uncast sum
    q, k, v = _frame_case()
    o = oracle.attn_ref(q, k, v, "none", 1.0, p_round="e5m2")
    assert abs(o[0, 0, 1, 0] - FINAL_FRAME_O) <= 1e-12
    # an earlier hand-built row whose weights (1 and 1/8) are exact in e5m2: every frame agrees
    q8 = np.array([[[[1.0], [1.0]]]])
    k8 = np.array([[[[0.0], [math.log(8.0)]]]])
    v8 = np.array([[[[9.0], [18.0]]]])
    for fn in (lambda: oracle.attn_online_ref(q8, k8, v8, "none", 1.0, 1, p_round="e5m2"),
               lambda: oracle.attn_ref(q8, k8, v8, "none", 1.0, p_round="e5m2")):
        assert abs(fn()[0, 0, 1, 0] - (9.0 + 8 * 18.0) / 9.0) <= 1e-12


# ---------------------------------------------------------------- row normaliser (LSE)
@pytest.mark.parametrize("mode,bs", [("none", 0), ("causal", 0), ("block_diag", 4)])
def test_lse_brute_and_closed_form(mode, bs):
    q, k, _ = _qkv(1, 2, 16, 8, seed=12, scale=2.0)
    got = oracle.attn_lse_ref(q, k, mode, 0.6, bs)
    for h in range(2):
        ref = oracle.lse_brute(q[0, h].tolist(), k[0, h].tolist(), mode, 0.6, bs)
        assert np.abs(got[0, h] - np.array(ref)).max() <= 1e-12
    # Q = 0: every visible score is 0, so lse_i = ln(number of visible keys)
    z = oracle.attn_lse_ref(np.zeros_like(q), k, mode, 0.6, bs)
    counts = oracle.visible_mask(mode, 16, bs).sum(axis=1)
    assert np.abs(z[0, 0] - np.log(counts)).max() <= 1e-15


# ---------------------------------------------------------------- P10 narrow formats
def test_p10_e5m2_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    got = oracle.e5m2_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])


def test_p10_e5m2_round_codes_and_midpoints():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e5m2_decode(codes)
    fin = np.sort(vals[np.isfinite(vals)])
    fin = np.unique(fin)
    mids = (fin[:-1] + fin[1:]) / 2.0
    rng = np.random.default_rng(0)
    rnd = np.concatenate([rng.standard_normal(20000),
                          rng.standard_normal(20000) * 1e-5,
                          rng.uniform(0, 1, 20000),
                          rng.uniform(5e4, 7e4, 2000)])
    x = np.concatenate([fin, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf), rnd])
    x = x.astype(np.float32).astype(np.float64)       # values torch can take exactly
    ref = torch.from_numpy(x).to(torch.float32).to(torch.float8_e5m2).to(torch.float64).numpy()
    got = oracle.round_e5m2(x)
    assert np.array_equal(got, ref)
    # the encoder agrees with torch's byte for byte on finite values
    b_ref = torch.from_numpy(x).to(torch.float32).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e5m2_encode(x), b_ref)


@pytest.mark.parametrize("fmt,tdt", [("bf16", torch.bfloat16), ("f16", torch.float16)])
def test_p10_bf16_f16_rounding(fmt, tdt):
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(50000), rng.standard_normal(5000) * 1e-6,
                        rng.standard_normal(5000) * 1e4]).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x).to(torch.float32).to(tdt).to(torch.float64).numpy()
    got = oracle.round_bf16(x) if fmt == "bf16" else oracle.round_f16(x)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- counting helpers
def test_flop_counts():
    assert oracle.visible_pairs("none", 10) == 100
    assert oracle.visible_pairs("causal", 10) == 55
    assert oracle.visible_pairs("block_diag", 12, 4) == 48
    assert oracle.attn_flops("causal", 4, 32, 4096, 128) == 549890031616
    assert oracle.visible_mask("causal", 10).sum() == 55
    assert oracle.visible_mask("block_diag", 12, 4).sum() == 48


# ---------------------------------------------------------------- planted mistakes
def _pin_suite(mod):
    """Run a compact version of the pins against module `mod`; True if all pass."""
    q, k, v = _qkv(1, 2, 16, 4, seed=77, scale=1.5)
    for mode, bs in (("none", 0), ("causal", 0), ("block_diag", 4)):
        got = mod.attn_ref(q, k, v, mode, 0.45, bs)
        for h in range(2):
            ref = np.array(oracle.attn_brute(q[0, h].tolist(), k[0, h].tolist(),
                                             v[0, h].tolist(), mode, 0.45, bs))
            if not np.abs(got[0, h] - ref).max() <= 1e-12:
                return False
        if mode != "none":
            got_on = mod.attn_online_ref(q, k, v, mode, 0.45, 5, bs)
            if not np.abs(got_on - got).max() <= 1e-12:
                return False
    if not np.array_equal(mod.attn_ref(q, k, v, "causal", 0.45)[:, :, 0], v[:, :, 0]):
        return False
    # rounded P: the running-max frame of the recurrence and the final frame of the definition
    fq, fk, fv = _frame_case()
    if abs(mod.attn_online_ref(fq, fk, fv, "none", 1.0, 1, p_round="e5m2")[0, 0, 1, 0]
           - RUNNING_FRAME_O) > 1e-12:
        return False
    if abs(mod.attn_ref(fq, fk, fv, "none", 1.0, p_round="e5m2")[0, 0, 1, 0] - FINAL_FRAME_O) > 1e-12:
        return False
    # one tile of width 2: the weight 1/2.6 is cast to 0.375 for P.V, the sum keeps 1/2.6
    if abs(mod.attn_online_ref(fq, fk, fv, "none", 1.0, 2, p_round="e5m2")[0, 0, 1, 0]
           - FINAL_FRAME_O) > 1e-12:
        return False
    return True


MUTATIONS = [
    ("transposed causal mask", "return j[None, :] <= i[:, None]", "return j[None, :] >= i[:, None]"),
    ("off-by-one causal mask", "return j[None, :] <= i[:, None]", "return j[None, :] < i[:, None] + 0 * i[:, None] + (i[:, None] == 0)"),
    ("block index from wrong axis", "return (j[None, :] // block_size) == (i[:, None] // block_size)",
     "return (j[None, :] // block_size) == (j[None, :] * 0 + i[:, None] % block_size)"),
    ("scale dropped", "S = sm_scale * (q[r] @ k.T)", "S = (q[r] @ k.T)"),
    ("K not transposed (uses Q twice)", "S = sm_scale * (q[r] @ k.T)", "S = sm_scale * (q[r] @ q.T)"),
    ("mask not applied to the scores", "# [R, L] full score rows\n        S = np.where(vis, S, -np.inf)",
     "# [R, L] full score rows\n        vis = np.ones_like(vis)"),
    ("P.V uses K in place of V", "out[pos:pos + r.size] = (Ph @ v) / l", "out[pos:pos + r.size] = (Ph @ k) / l"),
    ("normalised by wrong axis", "l = P.sum(axis=1, keepdims=True)", "l = P.sum(axis=0, keepdims=True)[:, :1].T[:P.shape[0]] if P.shape[0] == P.shape[1] else P.sum(axis=1, keepdims=True)"),
    ("online alpha sign flipped", "alpha = np.where(live, np.exp(m - m_new), 1.0)",
     "alpha = np.where(live, np.exp(m_new - m), 1.0)"),
    ("online sum uses no rescale", "l = l * alpha + p.sum(axis=1)", "l = l + p.sum(axis=1)"),
    # rounding frame of the fp8 cast in the recurrence: against the previous running max (then
    # rescaled into the new frame), or against the row's final max, instead of the running max
    ("online rounds in the previous frame", "ph = p if rounder is None else rounder(p)",
     "ph = p if rounder is None else rounder(p * np.exp(shift - np.where(np.isfinite(m), m, shift[:, 0])[:, None])) * np.exp(np.where(np.isfinite(m), m, shift[:, 0])[:, None] - shift)"),
    ("online rounds in the final frame", "ph = p if rounder is None else rounder(p)",
     "ph = p if rounder is None else rounder(p * np.exp(shift - np.where(vis_all, S_all, -np.inf).max(axis=1)[:, None])) * np.exp(np.where(vis_all, S_all, -np.inf).max(axis=1)[:, None] - shift)"),
    ("online sum over the cast weights", "l = l * alpha + p.sum(axis=1)", "l = l * alpha + ph.sum(axis=1)"),
    ("definition rounds the normalised weights", "Ph = P if rounder is None else rounder(P)",
     "Ph = P if rounder is None else rounder(P / l) * l"),
    ("definition sums the cast weights", "out[pos:pos + r.size] = (Ph @ v) / l",
     "out[pos:pos + r.size] = (Ph @ v) / (Ph.sum(axis=1, keepdims=True) if rounder is not None else l)"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistakes_are_caught(name, old, new):
    src_path = oatt.__file__
    with open(src_path) as f:
        src = f.read()
    assert old in src, f"mutation anchor missing: {name}"
    mutated = src.replace(old, new, 1)
    mod = types.ModuleType("oracle._mutant")
    mod.__dict__["__package__"] = "oracle"
    mod.__dict__["__name__"] = "oracle._mutant"
    exec(compile(mutated, src_path + "<mutant>", "exec"), mod.__dict__)
    assert _pin_suite(oatt), "unmutated oracle must pass the compact pin suite"
    assert not _pin_suite(mod), f"planted mistake not caught: {name}"
