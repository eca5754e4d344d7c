"""Pins for the float64 CPU oracle (no GPU).

Each test ties the oracle to something other than itself: numbers the pages
print (fixtures under tests/golden, each with its citation), closed forms,
invariants of the mathematics, finite differences and a pure-Python brute
force.  A dropped term, a wrong sign or index, or a transposed operand in
oracle/attention.py fails at least one of these.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import (
    attention_backward,
    attention_forward,
    attention_probs,
    brute_force_forward,
    causal_tile_count,
    key_tile_words,
    merge_states,
    online_forward,
)


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _heads(x):
    return x[None, None]


# --------------------------------------------------------------------------
# Worked example of the MI50 notes, section 2.2
# --------------------------------------------------------------------------
def test_worked_row_block_merge(golden_dir):
    g = _load(golden_dir, "worked_row_mi50.json")
    (a, b) = g["blocks"]
    # each block's own state: its max and sum exp(s - max)
    m_a, l_a = max(a), sum(math.exp(x - max(a)) for x in a)
    m_b, l_b = max(b), sum(math.exp(x - max(b)) for x in b)
    assert m_a == g["block1_max"] and m_b == g["block2_max"]
    nd = g["printed_decimals"]
    assert round(l_a, nd) == g["block1_sum_printed"]
    assert round(l_b, nd) == g["block2_sum_printed"]
    assert round(math.exp(m_a - m_b), nd) == g["rescale_printed"]
    m, l, _ = merge_states([m_a], [l_a], None, [m_b], [l_b], None)
    closed = 1.0 + math.exp(-1) + math.exp(-2) + math.exp(-3)
    assert m[0] == 4.0
    assert abs(l[0] - closed) < 1e-15
    assert round(l[0], nd) == g["merged_sum_printed"]


def test_worked_row_through_forward(golden_dir):
    g = _load(golden_dir, "worked_row_mi50.json")
    row = np.array(g["row"])
    # one query, D=1, q=1 and k_j = s_j gives the score row exactly (scale 1)
    q = np.ones((1, 1))
    k = row[:, None]
    v = np.eye(4)[:, :1] * 0 + np.arange(4.0)[:, None]  # v_j = j
    closed_l = 1.0 + math.exp(-1) + math.exp(-2) + math.exp(-3)
    qq = np.zeros((4, 1)); qq[:1] = q  # 4 queries so shapes are square
    o, lse = attention_forward(_heads(qq), _heads(k), _heads(v), False, 1.0)
    assert abs(lse[0, 0, 0] - (4.0 + math.log(closed_l))) < 1e-14
    p = np.exp(row - 4.0) / closed_l
    assert abs(o[0, 0, 0, 0] - float(p @ np.arange(4.0))) < 1e-14
    # the online pass with key tiles [1,2] | [3,4] reaches the same state
    _, lse_on, info = online_forward(qq, k, v, False, 1.0, block_q=4, block_k=2, trace_row=0)
    (j0, m1, l1, c1), (j1, m2, l2, c2) = info["trace"]
    assert (m1, m2) == (2.0, 4.0)
    assert abs(l1 - (math.exp(-1) + 1)) < 1e-15
    assert abs(c2 - math.exp(-2)) < 1e-15
    assert abs(l2 - closed_l) < 1e-15
    assert abs(lse_on[0] - lse[0, 0, 0]) < 1e-14


# --------------------------------------------------------------------------
# "Why FlashAttention ..." section 4.1 trace, 4.2 table, 4.5 count, 09 ablation
# --------------------------------------------------------------------------
def _page_qkv(seed, n, d):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(n, d))
    k = rng.normal(size=(n, d))
    v = rng.normal(size=(n, d))
    return q, k, v


def test_recurrence_trace_matches_page(golden_dir):
    g = _load(golden_dir, "recurrence_trace_why.json")
    q, k, v = _page_qkv(g["seed"], g["N"], g["D"])
    _, _, info = online_forward(q, k, v, False, 1.0 / math.sqrt(g["D"]),
                                block_q=g["N"], block_k=g["block_k"], trace_row=0)
    tol = 0.5 * 10.0 ** (-g["printed_decimals"]) + 1e-12
    assert len(info["trace"]) == len(g["rows"])
    for (j0, m, l, corr), row in zip(info["trace"], g["rows"]):
        assert j0 == row["j"]
        assert abs(m - row["m"]) <= tol
        assert abs(l - row["l"]) <= tol
        assert abs(corr - row["corr"]) <= tol


@pytest.mark.parametrize("n", [256, 1024])
@pytest.mark.parametrize("causal", [False, True])
def test_online_equals_definition_float64(golden_dir, n, causal):
    g = _load(golden_dir, "exactness_table_why.json")
    q, k, v = _page_qkv(n, n, 64)
    scale = 1.0 / 8.0
    ref, lse_ref = attention_forward(_heads(q), _heads(k), _heads(v), causal, scale)
    got, lse, _ = online_forward(q, k, v, causal, scale, block_q=64, block_k=64)
    err = np.abs(ref[0, 0] - got).max()
    page = max(r["max_abs"] for r in g["rows"])
    # rounding level: the page's table tops out below 1e-15
    assert err <= 10 * page
    assert np.abs(lse_ref[0, 0] - lse).max() <= 1e-13


def test_rescale_ablation_matches_page(golden_dir):
    g = _load(golden_dir, "rescale_ablation_why.json")
    q, k, v = _page_qkv(g["seed"], g["N"], g["D"])
    scale = 1.0 / math.sqrt(g["D"])
    ref, _ = attention_forward(_heads(q), _heads(k), _heads(v), False, scale)
    bad, _, _ = online_forward(q, k, v, False, scale, ablate_rescale=True)
    diff = np.abs(ref[0, 0] - bad)
    assert round(float(diff.max()), 3) == g["max_abs_printed"]
    assert round(float(diff.mean()), 4) == g["mean_abs_printed"]
    good, _, _ = online_forward(q, k, v, False, scale)
    assert np.abs(ref[0, 0] - good).max() < 1e-14


def test_causal_tile_count(golden_dir):
    g = _load(golden_dir, "causal_tiles_why.json")
    t = g["N"] // g["block"]
    assert t * t == g["tiles_noncausal"]
    cnt = causal_tile_count(g["N"], g["block"])
    assert cnt == g["tiles_causal"] == t * (t + 1) // 2
    assert round(100.0 * (1 - cnt / (t * t)), 1) == g["skipped_percent_printed"]
    # the online pass visits exactly that many tiles
    q, k, v = (np.ones((g["N"], 2)),) * 3
    _, _, info = online_forward(q, k, v, True, 1.0, block_q=g["block"], block_k=g["block"])
    assert info["tiles"] == cnt


# --------------------------------------------------------------------------
# Closed forms and special cases
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one(causal):
    q, k = _rand(3, 33, 16), _rand(4, 33, 16)
    p = attention_probs(q, k, causal, 0.25)
    assert np.abs(p.sum(axis=1) - 1.0).max() < 1e-14
    if causal:
        assert np.all(p[np.triu_indices(33, 1)] == 0.0)


def test_causal_row_zero_is_first_value():
    q, k, v = _rand(5, 1, 1, 17, 8), _rand(6, 1, 1, 17, 8), _rand(7, 1, 1, 17, 8)
    o, lse = attention_forward(q, k, v, True, 0.3)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0])
    assert lse[0, 0, 0] == 0.3 * float(q[0, 0, 0] @ k[0, 0, 0])


@pytest.mark.parametrize("causal", [False, True])
def test_constant_keys_give_prefix_mean(causal):
    n, d = 19, 6
    q = _rand(8, 1, 1, n, d)
    k = np.tile(_rand(9, d), (1, 1, n, 1))
    v = _rand(10, 1, 1, n, d)
    o, lse = attention_forward(q, k, v, causal, 0.7)
    for i in range(n):
        cnt = i + 1 if causal else n
        assert np.abs(o[0, 0, i] - v[0, 0, :cnt].mean(axis=0)).max() < 1e-14
        s = 0.7 * float(q[0, 0, i] @ k[0, 0, 0])
        assert abs(lse[0, 0, i] - (s + math.log(cnt))) < 1e-13


def test_largest_fp16_inputs_scale_one():
    # the page on MI50 tuning stresses every input equal to 65504 with scale 1
    x = np.full((1, 2, 9, 4), 65504.0)
    o, lse = attention_forward(x, x, x, True, 1.0)
    assert np.abs(o - 65504.0).max() <= 65504.0 * 4e-16 * 9
    s = 65504.0 * 65504.0 * 4
    for i in range(9):
        assert lse[0, 0, i] == s + math.log(i + 1)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    q, k, v = _rand(11, 1, 2, 23, 8), _rand(12, 1, 2, 23, 8), _rand(13, 1, 2, 23, 8)
    do = _rand(14, 1, 2, 23, 8)
    u = _rand(15, 8)
    scale = 0.4
    o1, l1 = attention_forward(q, k, v, causal, scale)
    o2, l2 = attention_forward(q, k + u, v, causal, scale)
    assert np.abs(o1 - o2).max() < 1e-13
    assert np.abs((l2 - l1) - scale * (q @ u)).max() < 1e-12
    g1 = attention_backward(q, k, v, do, causal, scale)
    g2 = attention_backward(q, k + u, v, do, causal, scale)
    for a, b in zip(g1, g2):
        assert np.abs(a - b).max() < 1e-12


def test_joint_key_value_permutation_invariance():
    q, k, v = _rand(16, 1, 1, 29, 8), _rand(17, 1, 1, 29, 8), _rand(18, 1, 1, 29, 8)
    perm = np.random.default_rng(19).permutation(29)
    o1, l1 = attention_forward(q, k, v, False, 0.5)
    o2, l2 = attention_forward(q, k[:, :, perm], v[:, :, perm], False, 0.5)
    assert np.abs(o1 - o2).max() < 1e-14 and np.abs(l1 - l2).max() < 1e-13


@pytest.mark.parametrize("n", [1, 2, 5, 8])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_agrees(n, causal):
    d = 4
    q, k, v = _rand(20 + n, n, d), _rand(30 + n, n, d), _rand(40 + n, n, d)
    scale = 1.0 / math.sqrt(d)
    ob, lb = brute_force_forward(q.tolist(), k.tolist(), v.tolist(), causal, scale)
    o, lse = attention_forward(_heads(q), _heads(k), _heads(v), causal, scale)
    on, lon, _ = online_forward(q, k, v, causal, scale, block_q=3, block_k=2)
    assert np.abs(o[0, 0] - np.array(ob)).max() < 1e-14
    assert np.abs(lse[0, 0] - np.array(lb)).max() < 1e-14
    assert np.abs(on - np.array(ob)).max() < 1e-14
    assert np.abs(lon - np.array(lb)).max() < 1e-14


def test_row_block_split_does_not_change_result():
    q, k, v = _rand(50, 1, 1, 70, 8), _rand(51, 1, 1, 70, 8), _rand(52, 1, 1, 70, 8)
    for causal in (False, True):
        a = attention_forward(q, k, v, causal, 0.3, row_block=256)
        b = attention_forward(q, k, v, causal, 0.3, row_block=7)
        assert np.abs(a[0] - b[0]).max() < 1e-15


def test_merge_guard_for_empty_side():
    # a side that has seen no visible key (m = -inf) contributes nothing
    m, l, o = merge_states([-np.inf], [0.0], [[0.0, 0.0]], [1.5], [2.0], [[3.0, 4.0]])
    assert m[0] == 1.5 and l[0] == 2.0 and np.array_equal(o[0], [3.0, 4.0])
    assert not np.any(np.isnan(o))


# --------------------------------------------------------------------------
# Backward
# --------------------------------------------------------------------------
def _loss(q, k, v, do, causal, scale):
    o, _ = attention_forward(q, k, v, causal, scale)
    return float((o * do).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences(causal):
    n, d = 7, 4
    q, k, v = _rand(60, 1, 1, n, d), _rand(61, 1, 1, n, d), _rand(62, 1, 1, n, d)
    do = _rand(63, 1, 1, n, d)
    scale = 0.6
    grads = attention_backward(q, k, v, do, causal, scale)
    h = 1e-6
    for gi, name in enumerate("qkv"):
        base = [q, k, v]
        num = np.zeros_like(base[gi])
        for idx in np.ndindex(base[gi].shape):
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[gi][idx] += h
            minus[gi][idx] -= h
            num[idx] = (_loss(*plus, do, causal, scale) - _loss(*minus, do, causal, scale)) / (2 * h)
        assert np.abs(num - grads[gi]).max() < 1e-8, name


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    n, d = 40, 8
    q, k, v = _rand(70, 1, 2, n, d), _rand(71, 1, 2, n, d), _rand(72, 1, 2, n, d)
    do = _rand(73, 1, 2, n, d)
    dq, dk, dv = attention_backward(q, k, v, do, causal, 0.35, row_block=16)
    # softmax rows sum to one, so dS rows sum to zero and sum_j dK_j = 0
    assert np.abs(dk.sum(axis=2)).max() < 1e-12
    # dV = P^T dO and P's rows sum to one
    assert np.abs(dv.sum(axis=2) - do.sum(axis=2)).max() < 1e-12
    # Delta_i = rowsum(P * dP) equals rowsum(dO * O) because O = P V
    o, _ = attention_forward(q, k, v, causal, 0.35)
    p = attention_probs(q[0, 0], k[0, 0], causal, 0.35)
    dp = do[0, 0] @ v[0, 0].T
    assert np.abs((p * dp).sum(axis=1) - (do[0, 0] * o[0, 0]).sum(axis=1)).max() < 1e-12


def test_constant_keys_give_zero_dq():
    n, d = 12, 4
    q, v, do = _rand(80, 1, 1, n, d), _rand(81, 1, 1, n, d), _rand(82, 1, 1, n, d)
    k = np.tile(_rand(83, d), (1, 1, n, 1))
    dq, _, _ = attention_backward(q, k, v, do, True, 0.5)
    assert np.abs(dq).max() < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_selected_rows_match_brute_force(causal):
    n, d = 8, 3
    q, k, v = _rand(90, n, d), _rand(91, n, d), _rand(92, n, d)
    rows = np.array([7, 0, 3, 3, 5])
    o, lse = attention_forward(_heads(q), _heads(k), _heads(v), causal, 0.8, rows=rows, row_block=2)
    ob, lb = brute_force_forward(q.tolist(), k.tolist(), v.tolist(), causal, 0.8)
    assert np.abs(o[0, 0] - np.array(ob)[rows]).max() < 1e-14
    assert np.abs(lse[0, 0] - np.array(lb)[rows]).max() < 1e-14


# --------------------------------------------------------------------------
# Key splits and their merge ("CUDA FlashAttention ...", §7)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cuts", [(0, 40), (0, 13, 27, 40), (0, 1, 39, 40), (0, 20, 20, 40)])
def test_merged_key_splits_equal_full_attention(causal, cuts):
    from oracle import attention_partial, merge_lse
    q, k, v = _rand(100, 1, 2, 40, 8), _rand(101, 1, 2, 40, 8), _rand(102, 1, 2, 40, 8)
    parts = [attention_partial(q, k, v, causal, 0.3, lo, hi) for lo, hi in zip(cuts[:-1], cuts[1:])]
    o, lse = merge_lse([p[1] for p in parts], [p[0] for p in parts])
    o_ref, lse_ref = attention_forward(q, k, v, causal, 0.3)
    assert np.abs(o - o_ref).max() < 1e-13
    assert np.abs(lse - lse_ref).max() < 1e-13


def test_partial_of_unseen_keys_is_empty():
    from oracle import attention_partial
    q, k, v = _rand(103, 1, 1, 16, 4), _rand(104, 1, 1, 16, 4), _rand(105, 1, 1, 16, 4)
    o, lse = attention_partial(q, k, v, True, 0.5, 8, 16)
    assert np.all(np.isneginf(lse[0, 0, :8])) and np.all(o[0, 0, :8] == 0)
    assert np.all(np.isfinite(lse[0, 0, 8:]))
    # a single key: the output is that key's value row
    o1, lse1 = attention_partial(q, k, v, False, 0.5, 3, 4)
    assert np.abs(o1[0, 0] - v[0, 0, 3]).max() < 1e-15
    assert np.abs(lse1[0, 0] - 0.5 * (q[0, 0] @ k[0, 0, 3])).max() < 1e-14


# --------------------------------------------------------------------------
# Key-padding masks (variable-length batches) and their block-level flags
# --------------------------------------------------------------------------
def _mask(seed, b, n, p=0.6):
    return (np.random.default_rng(seed).random((b, n)) < p).astype(np.uint8)


@pytest.mark.parametrize("causal", [False, True])
def test_all_visible_mask_changes_nothing(causal):
    q, k, v = _rand(400, 2, 2, 70, 8), _rand(401, 2, 2, 70, 8), _rand(402, 2, 2, 70, 8)
    a = attention_forward(q, k, v, causal, 0.3)
    b = attention_forward(q, k, v, causal, 0.3, key_mask=np.ones((2, 70), np.uint8))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_masked_keys_equal_deleted_keys():
    # without a causal mask, an invisible key is the same as no key at all
    n, d = 50, 8
    q, k, v = _rand(410, 1, 1, n, d), _rand(411, 1, 1, n, d), _rand(412, 1, 1, n, d)
    mask = _mask(413, 1, n)
    keep = mask[0] != 0
    o, lse = attention_forward(q, k, v, False, 0.4, key_mask=mask)
    o2, lse2 = attention_forward(q, k[:, :, keep], v[:, :, keep], False, 0.4)
    assert np.abs(o - o2).max() < 1e-14 and np.abs(lse - lse2).max() < 1e-13


@pytest.mark.parametrize("n", [1, 3, 8])
@pytest.mark.parametrize("causal", [False, True])
def test_masked_brute_force_agrees(n, causal):
    d = 4
    q, k, v = _rand(420 + n, n, d), _rand(430 + n, n, d), _rand(440 + n, n, d)
    for seed in range(4):
        vis = _mask(450 + seed, 1, n, 0.5)
        ob, lb = brute_force_forward(q.tolist(), k.tolist(), v.tolist(), causal, 0.5, visible=vis[0].tolist())
        o, lse = attention_forward(_heads(q), _heads(k), _heads(v), causal, 0.5, key_mask=vis)
        assert np.abs(o[0, 0] - np.array(ob)).max() < 1e-14
        lb = np.array(lb)
        assert np.array_equal(np.isneginf(lse[0, 0]), np.isneginf(lb))
        fin = np.isfinite(lb)
        assert np.abs(lse[0, 0][fin] - lb[fin]).max(initial=0.0) < 1e-14


def test_row_without_visible_key_is_zero_with_minus_inf_lse():
    n, d = 6, 4
    q, k, v = _rand(460, 1, 1, n, d), _rand(461, 1, 1, n, d), _rand(462, 1, 1, n, d)
    mask = np.array([[0, 0, 1, 1, 0, 1]], np.uint8)
    o, lse = attention_forward(q, k, v, True, 1.0, key_mask=mask)
    # causal rows 0 and 1 see only keys 0..1, both invisible
    assert np.array_equal(o[0, 0, :2], np.zeros((2, d))) and np.all(np.isneginf(lse[0, 0, :2]))
    # row 2 sees only key 2: O = v_2, LSE = s_22
    assert np.abs(o[0, 0, 2] - v[0, 0, 2]).max() < 1e-15
    assert abs(lse[0, 0, 2] - float(q[0, 0, 2] @ k[0, 0, 2])) < 1e-14
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse[0, 0, 2:]))


def test_length_mask_equals_shorter_sequences():
    # a right-padded variable-length batch: element b holds L_b real tokens
    n, d, lens = 40, 8, [40, 17, 1]
    q, k, v = _rand(470, 3, 2, n, d), _rand(471, 3, 2, n, d), _rand(472, 3, 2, n, d)
    mask = (np.arange(n)[None, :] < np.array(lens)[:, None]).astype(np.uint8)
    for causal in (False, True):
        o, lse = attention_forward(q, k, v, causal, 0.3, key_mask=mask)
        for b, L in enumerate(lens):
            sl = slice(0, L)
            o2, lse2 = attention_forward(q[b:b + 1, :, sl], k[b:b + 1, :, sl], v[b:b + 1, :, sl], causal, 0.3)
            assert np.abs(o[b:b + 1, :, sl] - o2).max() < 1e-14
            assert np.abs(lse[b:b + 1, :, sl] - lse2).max() < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_masked_backward_matches_finite_differences(causal):
    n, d = 7, 3
    q, k, v = _rand(480, 1, 1, n, d), _rand(481, 1, 1, n, d), _rand(482, 1, 1, n, d)
    do = _rand(483, 1, 1, n, d)
    mask = np.array([[0, 1, 1, 0, 1, 0, 1]], np.uint8)  # causal row 0 has no key
    scale = 0.7
    grads = attention_backward(q, k, v, do, causal, scale, key_mask=mask)

    def loss(q_, k_, v_):
        o, _ = attention_forward(q_, k_, v_, causal, scale, key_mask=mask)
        return float((o * do).sum())

    h = 1e-6
    for gi, name in enumerate("qkv"):
        base = [q, k, v]
        num = np.zeros_like(base[gi])
        for idx in np.ndindex(base[gi].shape):
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[gi][idx] += h
            minus[gi][idx] -= h
            num[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        assert np.abs(num - grads[gi]).max() < 1e-8, name
    # invisible keys receive exactly zero gradient; so does a row with no key
    hidden = mask[0] == 0
    assert np.all(grads[1][0, 0, hidden] == 0) and np.all(grads[2][0, 0, hidden] == 0)
    if causal:
        assert np.all(grads[0][0, 0, 0] == 0)


def test_key_tile_words_by_hand():
    n = 130  # tiles of 64, 64 and 2 keys
    words, tiles = key_tile_words(np.ones((1, n), np.uint8))
    assert words == [[(1 << 64) - 1, (1 << 64) - 1, 0b11]] and tiles == [[0, 1, 2]]
    words, tiles = key_tile_words(np.zeros((1, n), np.uint8))
    assert words == [[0, 0, 0]] and tiles == [[]]
    m = np.zeros((2, n), np.uint8)
    m[0, 65] = 1
    m[1, 0] = m[1, 63] = m[1, 129] = 1
    words, tiles = key_tile_words(m)
    assert words == [[0, 2, 0], [1 | (1 << 63), 0, 0b10]] and tiles == [[1], [0, 2]]


# --------------------------------------------------------------------------
# Grouped K/V heads (GQA / MQA)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("H,Hkv", [(4, 2), (6, 1), (3, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_grouped_heads_equal_repeated_kv(H, Hkv, causal):
    n, d = 33, 8
    q = _rand(500, 2, H, n, d)
    k, v, do = _rand(501, 2, Hkv, n, d), _rand(502, 2, Hkv, n, d), _rand(503, 2, H, n, d)
    rep = H // Hkv
    k_rep, v_rep = np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1)
    o, lse = attention_forward(q, k, v, causal, 0.3)
    o2, lse2 = attention_forward(q, k_rep, v_rep, causal, 0.3)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    dq, dk, dv = attention_backward(q, k, v, do, causal, 0.3)
    dq2, dk2, dv2 = attention_backward(q, k_rep, v_rep, do, causal, 0.3)
    assert dk.shape == k.shape and dv.shape == v.shape
    assert np.abs(dq - dq2).max() < 1e-13
    # a shared head's gradient is the sum over the query heads that read it
    assert np.abs(dk - dk2.reshape(2, Hkv, rep, n, d).sum(axis=2)).max() < 1e-12
    assert np.abs(dv - dv2.reshape(2, Hkv, rep, n, d).sum(axis=2)).max() < 1e-12


def test_grouped_heads_brute_force():
    n, d, H, Hkv = 5, 3, 4, 2
    q, k, v = _rand(510, 1, H, n, d), _rand(511, 1, Hkv, n, d), _rand(512, 1, Hkv, n, d)
    o, lse = attention_forward(q, k, v, True, 0.8)
    for h in range(H):
        ob, lb = brute_force_forward(q[0, h].tolist(), k[0, h * Hkv // H].tolist(), v[0, h * Hkv // H].tolist(),
                                     True, 0.8)
        assert np.abs(o[0, h] - np.array(ob)).max() < 1e-14 and np.abs(lse[0, h] - np.array(lb)).max() < 1e-14


def test_grouped_heads_finite_differences():
    n, d, H, Hkv = 6, 3, 4, 1
    q, k, v = _rand(520, 1, H, n, d), _rand(521, 1, Hkv, n, d), _rand(522, 1, Hkv, n, d)
    do = _rand(523, 1, H, n, d)
    grads = attention_backward(q, k, v, do, True, 0.5)

    def loss(q_, k_, v_):
        return float((attention_forward(q_, k_, v_, True, 0.5)[0] * do).sum())

    h = 1e-6
    for gi, name in enumerate("qkv"):
        base = [q, k, v]
        num = np.zeros_like(base[gi])
        for idx in np.ndindex(base[gi].shape):
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[gi][idx] += h
            minus[gi][idx] -= h
            num[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        assert np.abs(num - grads[gi]).max() < 1e-8, name


def test_grouped_heads_reject_non_divisor():
    with pytest.raises(ValueError):
        attention_forward(_rand(530, 1, 3, 4, 2), _rand(531, 1, 2, 4, 2), _rand(532, 1, 2, 4, 2), False, 1.0)


# --------------------------------------------------------------------------
# Dropout regenerated from Philox4x64-10 (seed, offset)
# --------------------------------------------------------------------------
from oracle import dropout_keep, dropout_threshold, philox4x64, philox4x64_array  # noqa: E402


def _numpy_philox_block(counter, key):
    """numpy's own Philox4x64-10 bit generator: it raises the 256-bit counter
    by one before each block, so start it one below the wanted counter."""
    c = sum(int(x) << (64 * i) for i, x in enumerate(counter)) - 1
    c %= 1 << 256
    words = np.array([(c >> (64 * i)) & ((1 << 64) - 1) for i in range(4)], dtype=np.uint64)
    bg = np.random.Philox(counter=words, key=np.array(key, dtype=np.uint64))
    return [int(x) for x in bg.random_raw(4)]


@pytest.mark.parametrize("counter,key", [
    ([0, 0, 0, 0], [0, 0]),
    ([1, 2, 3, 4], [5, 6]),
    ([0, 7, 0, 0], [0xFFFFFFFFFFFFFFFF, 1]),
    ([(1 << 64) - 1, (1 << 64) - 1, 12, 99], [0x0123456789ABCDEF, 0xFEDCBA9876543210]),
    ([0x5555, 4095, 31, 2 ** 40], [42, 0]),
])
def test_philox_matches_numpy_bit_generator(counter, key):
    assert philox4x64(counter, key) == _numpy_philox_block(counter, key)


def test_philox_array_matches_scalar():
    rng = np.random.default_rng(600)
    c = rng.integers(0, 2 ** 63, size=(4, 50), dtype=np.uint64) * np.uint64(2) + np.uint64(1)
    key = (0x9E3779B97F4A7C15, 0x123456789)
    w = philox4x64_array(c[0], c[1], c[2], c[3], *key)
    for n in range(50):
        assert [int(x[n]) for x in w] == philox4x64([int(c[r, n]) for r in range(4)], key)


def test_dropout_keep_mapping_per_element():
    B, H, N, p, seed, offset = 2, 3, 70, 0.37, 0xABCDEF, 5
    keep = dropout_keep(B, H, N, p, seed, offset)
    thr, _ = dropout_threshold(p)
    rng = np.random.default_rng(601)
    for _ in range(200):
        b, h, i, j = (int(rng.integers(0, x)) for x in (B, H, N, N))
        w = philox4x64([j // 16, i, b * H + h, offset], [seed, 0])
        value = (w[(j % 16) // 4] >> (16 * (j % 4))) & 0xFFFF
        assert keep[b, h, i, j] == (value >= thr)


def test_dropout_keep_rate_and_streams():
    B, H, N, p = 1, 2, 600, 0.3
    keep = dropout_keep(B, H, N, p, 7, 0)
    thr, scale = dropout_threshold(p)
    q_keep = 1 - thr / 65536
    n = keep.size
    assert abs(keep.mean() - q_keep) < 5 * math.sqrt(q_keep * (1 - q_keep) / n)
    assert abs(scale - 1 / q_keep) < 1e-15 and thr == 19660
    assert np.array_equal(keep, dropout_keep(B, H, N, p, 7, 0))          # regenerated, not stored
    other = dropout_keep(B, H, N, p, 7, 1)                               # the next offset
    assert 0.3 < np.mean(keep != other) < 0.5
    assert dropout_keep(1, 1, 20, 0.0, 3, 0).all()


def test_dropout_zero_probability_changes_nothing():
    q, k, v = _rand(610, 1, 2, 50, 8), _rand(611, 1, 2, 50, 8), _rand(612, 1, 2, 50, 8)
    a = attention_forward(q, k, v, True, 0.3)
    b = attention_forward(q, k, v, True, 0.3, dropout=(0.0, 99, 3))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_brute_force_agrees(causal):
    n, d, p, seed, offset = 7, 3, 0.4, 77, 2
    q, k, v = _rand(620, n, d), _rand(621, n, d), _rand(622, n, d)
    keep = dropout_keep(1, 1, n, p, seed, offset)[0, 0]
    _, ks = dropout_threshold(p)
    ob, lb = brute_force_forward(q.tolist(), k.tolist(), v.tolist(), causal, 0.5, keep=keep.tolist(), keep_scale=ks)
    o, lse = attention_forward(_heads(q), _heads(k), _heads(v), causal, 0.5, dropout=(p, seed, offset))
    assert np.abs(o[0, 0] - np.array(ob)).max() < 1e-14
    assert np.abs(lse[0, 0] - np.array(lb)).max() < 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_backward_matches_finite_differences(causal):
    n, d = 6, 3
    q, k, v = _rand(630, 1, 2, n, d), _rand(631, 1, 2, n, d), _rand(632, 1, 2, n, d)
    do = _rand(633, 1, 2, n, d)
    drop = (0.35, 1234, 9)
    grads = attention_backward(q, k, v, do, causal, 0.6, dropout=drop)

    def loss(q_, k_, v_):
        return float((attention_forward(q_, k_, v_, causal, 0.6, dropout=drop)[0] * do).sum())

    h = 1e-6
    for gi, name in enumerate("qkv"):
        base = [q, k, v]
        num = np.zeros_like(base[gi])
        for idx in np.ndindex(base[gi].shape):
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[gi][idx] += h
            minus[gi][idx] -= h
            num[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        assert np.abs(num - grads[gi]).max() < 1e-8, name


def test_dropout_delta_equals_rowsum_do_o():
    # the backward's correction term still equals rowsum(dO * O) with the
    # dropped O, which is what the GPU's preprocessing pass computes
    n, d, p, seed, offset = 30, 8, 0.25, 5, 0
    q, k, v, do = (_rand(640 + i, 1, 1, n, d) for i in range(4))
    o, _ = attention_forward(q, k, v, True, 0.4, dropout=(p, seed, offset))
    prob = attention_probs(q[0, 0], k[0, 0], True, 0.4)
    keep = dropout_keep(1, 1, n, p, seed, offset)[0, 0]
    _, ks = dropout_threshold(p)
    dp = (do[0, 0] @ v[0, 0].T) * keep * ks
    assert np.abs((prob * dp).sum(axis=1) - (do[0, 0] * o[0, 0]).sum(axis=1)).max() < 1e-13


def test_dropout_head_numbers_select_a_head_of_a_larger_problem():
    B, H, n, d, drop = 2, 3, 20, 4, (0.3, 8, 2)
    q, k, v = _rand(650, B, H, n, d), _rand(651, B, H, n, d), _rand(652, B, H, n, d)
    o, lse = attention_forward(q, k, v, False, 0.5, dropout=drop)
    o1, _ = attention_forward(q[1:2, 2:3], k[1:2, 2:3], v[1:2, 2:3], False, 0.5, dropout=drop + ([[1 * H + 2]],))
    assert np.array_equal(o[1:2, 2:3], o1)


@pytest.mark.parametrize("causal", [False, True])
def test_masked_dropout_brute_force_agrees(causal):
    # a key-padding mask and dropout together: hidden keys leave the softmax,
    # then the kept probabilities of the visible ones are scaled
    n, d, p, seed, offset = 8, 3, 0.3, 91, 4
    q, k, v = _rand(650, n, d), _rand(651, n, d), _rand(652, n, d)
    vis = np.array([0, 0, 1, 1, 0, 1, 1, 0], dtype=np.uint8)
    keep = dropout_keep(1, 1, n, p, seed, offset)[0, 0]
    _, ks = dropout_threshold(p)
    ob, lb = brute_force_forward(q.tolist(), k.tolist(), v.tolist(), causal, 0.7, visible=vis.tolist(),
                                 keep=keep.tolist(), keep_scale=ks)
    o, lse = attention_forward(_heads(q), _heads(k), _heads(v), causal, 0.7, key_mask=vis[None],
                               dropout=(p, seed, offset))
    fin = np.isfinite(np.array(lb))
    assert np.abs(o[0, 0] - np.array(ob)).max() < 1e-14
    assert np.abs(lse[0, 0][fin] - np.array(lb)[fin]).max() < 1e-14
    assert np.array_equal(np.isneginf(lse[0, 0]), ~fin)  # causal rows 0 and 1 see only hidden keys
    assert (~fin).sum() == (2 if causal else 0)


def test_masked_dropout_backward_matches_finite_differences():
    n, d = 6, 3
    q, k, v = _rand(660, 1, 2, n, d), _rand(661, 1, 2, n, d), _rand(662, 1, 2, n, d)
    do = _rand(663, 1, 2, n, d)
    m = np.array([[1, 1, 0, 1, 0, 1]], dtype=np.uint8)
    drop = (0.3, 4321, 1)
    grads = attention_backward(q, k, v, do, True, 0.6, key_mask=m, dropout=drop)

    def loss(q_, k_, v_):
        return float((attention_forward(q_, k_, v_, True, 0.6, key_mask=m, dropout=drop)[0] * do).sum())

    h = 1e-6
    for gi, name in enumerate("qkv"):
        base = [q, k, v]
        num = np.zeros_like(base[gi])
        for idx in np.ndindex(base[gi].shape):
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[gi][idx] += h
            minus[gi][idx] -= h
            num[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        assert np.abs(num - grads[gi]).max() < 1e-8, name
