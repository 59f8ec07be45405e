"""Pins of the oracle's log-sum-exp merge (CPU only): a hand-derived worked example,
the merge's identity, order independence and associativity."""

import ast
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "three_keys_hand.json")


def _expr(x):
    """Value of one fixture entry: a number, or an arithmetic expression over numbers
    with + - * / and ln() (evaluated exactly as written, nothing else is accepted)."""
    if isinstance(x, (int, float)):
        return float(x)
    node = ast.parse(x, mode="eval").body

    def ev(n):
        if isinstance(n, ast.Constant) and isinstance(n.value, (int, float)):
            return float(n.value)
        if isinstance(n, ast.UnaryOp) and isinstance(n.op, ast.USub):
            return -ev(n.operand)
        if isinstance(n, ast.BinOp) and isinstance(n.op, (ast.Add, ast.Sub, ast.Mult, ast.Div)):
            a, b = ev(n.left), ev(n.right)
            return {ast.Add: a + b, ast.Sub: a - b, ast.Mult: a * b, ast.Div: a / b if b else math.nan}[type(n.op)]
        if (isinstance(n, ast.Call) and isinstance(n.func, ast.Name) and n.func.id == "ln" and len(n.args) == 1
                and not n.keywords):
            return math.log(ev(n.args[0]))
        raise ValueError(f"unsupported fixture expression {x!r}")

    return ev(node)


def _arr(x):
    return np.vectorize(_expr, otypes=[np.float64])(np.asarray(x, dtype=object))


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _three_keys(g):
    """q [1, 2, 1, 2], k/v [1, 3, 1, 2] of the fixture (one batch row, one head)."""
    q = _arr(g["q"])[None, :, None, :]
    k = _arr(g["k"])[None, :, None, :]
    v = _arr(g["v"])[None, :, None, :]
    return q, k, v


def test_golden_expressions_parse_as_numbers():
    assert _expr("ln(3)/3 - ln(2)/9") == pytest.approx(math.log(3) / 3 - math.log(2) / 9, abs=1e-16)
    assert _expr("-2/9") == pytest.approx(-2 / 9, abs=1e-16)
    with pytest.raises(ValueError):
        _expr("__import__('os')")


def test_hand_derived_three_key_example():
    g = _golden()
    ex = g["expected"]
    q, k, v = _three_keys(g)
    scale, causal = float(g["scale"]), bool(g["causal"])
    q_idx, k_idx = np.asarray(g["q_idx"]), np.asarray(g["k_idx"])
    o, lse = oracle.attention_full(q, k, v, q_idx, k_idx, scale, causal)
    np.testing.assert_allclose(o[0, :, 0], _arr(ex["forward"]["O"]), atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], _arr(ex["forward"]["LSE"]), atol=1e-15)
    # row 0 against each key chunk on its own, then the merge of the two partials
    qa = q[:, :1]
    parts = []
    for ch in ex["row0_chunks"]:
        keys = np.asarray(ch["keys"])
        oc, lc = oracle.attention_full(qa, k[:, keys], v[:, keys], q_idx[:1], k_idx[keys], scale, causal)
        np.testing.assert_allclose(oc[0, 0, 0], _arr(ch["O"]), atol=1e-15)
        assert abs(lc[0, 0, 0] - _expr(ch["LSE"])) < 1e-15
        parts.append((oc, lc))
    om, lm = oracle.lse_merge(parts[0][0], parts[0][1], parts[1][0], parts[1][1])
    np.testing.assert_allclose(om[0, 0, 0], _arr(ex["row0_merge"]["O"]), atol=1e-15)
    assert abs(lm[0, 0, 0] - _expr(ex["row0_merge"]["LSE"])) < 1e-15


def test_hand_derived_three_key_backward():
    g = _golden()
    bw = g["expected"]["row0_backward"]
    q, k, v = _three_keys(g)
    scale, causal = float(g["scale"]), bool(g["causal"])
    q_idx, k_idx = np.asarray(g["q_idx"])[:1], np.asarray(g["k_idx"])
    qa = q[:, :1]
    o, lse = oracle.attention_full(qa, k, v, q_idx, k_idx, scale, causal)
    do = _arr(bw["dO"])[None, None, None, :]
    delta = oracle.bwd_delta(o, do)
    assert abs(delta[0, 0, 0] - _expr(bw["delta"])) < 1e-15
    dq, dk, dv = oracle.attention_bwd_full(qa, k, v, do, lse, delta, q_idx, k_idx, scale, causal)
    np.testing.assert_allclose(dq[0, 0, 0], _arr(bw["dQ"]), atol=1e-15)
    np.testing.assert_allclose(dk[0, :, 0], _arr(bw["dK"]), atol=1e-15)
    np.testing.assert_allclose(dv[0, :, 0], _arr(bw["dV"]), atol=1e-15)


def _partials(rng, B=1, Sq=6, Hq=4, d=5, CP=4, masked=()):
    parts = []
    for c in range(CP):
        o = rng.standard_normal((B, Sq, Hq, d))
        lse = rng.standard_normal((B, Hq, Sq)) * 3
        if c in masked:
            o[:] = 0
            lse[:] = -np.inf
        parts.append((o, lse))
    return parts


def _merge_all(parts, order):
    o = np.zeros_like(parts[0][0])
    lse = np.full_like(parts[0][1], -np.inf)
    for c in order:
        o, lse = oracle.lse_merge(o, lse, *parts[c])
    return o, lse


def test_merge_into_empty_is_the_partial_exactly():
    rng = np.random.default_rng(1)
    (o, lse), = _partials(rng, CP=1)
    om, lm = oracle.lse_merge(np.zeros_like(o), np.full_like(lse, -np.inf), o, lse)
    np.testing.assert_array_equal(om, o)
    np.testing.assert_array_equal(lm, lse)


def test_merge_one_chunk_equals_plain_attention_over_it():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 5, 2, 4))
    k = rng.standard_normal((1, 7, 1, 4))
    v = rng.standard_normal((1, 7, 1, 4))
    o, lse = oracle.attention_full(q, k, v, 10 + np.arange(5), np.arange(7), 0.5, True)
    om, lm = oracle.lse_merge(np.zeros_like(o), np.full_like(lse, -np.inf), o, lse)
    np.testing.assert_array_equal(om, o)
    np.testing.assert_array_equal(lm, lse)


def test_merge_with_masked_chunk_leaves_state_unchanged():
    rng = np.random.default_rng(3)
    parts = _partials(rng, CP=2, masked=(1,))
    om, lm = oracle.lse_merge(*parts[0], *parts[1])
    np.testing.assert_array_equal(om, parts[0][0])
    np.testing.assert_array_equal(lm, parts[0][1])
    # and both -inf: unchanged (rows stay O = 0 / -inf)
    dead = _partials(rng, CP=2, masked=(0, 1))
    om, lm = oracle.lse_merge(*dead[0], *dead[1])
    assert np.all(om == 0) and np.all(lm == -np.inf)


def test_merge_order_does_not_matter():
    rng = np.random.default_rng(4)
    parts = _partials(rng, CP=4, masked=(2,))
    ref_o, ref_l = _merge_all(parts, [0, 1, 2, 3])
    for perm in itertools.permutations(range(4)):
        o, lse = _merge_all(parts, perm)
        np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-13)


def test_merge_is_associative():
    rng = np.random.default_rng(5)
    a, b, c = _partials(rng, CP=3)
    left = oracle.lse_merge(*oracle.lse_merge(*a, *b), *c)
    right = oracle.lse_merge(*a, *oracle.lse_merge(*b, *c))
    np.testing.assert_allclose(left[0], right[0], atol=1e-13)
    np.testing.assert_allclose(left[1], right[1], atol=1e-13)


def test_merge_of_key_partition_equals_attention_over_union():
    """Partials over a partition of the keys merge into attention over all keys,
    for every way to cut the key range in two."""
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 3, 2, 4))
    k = rng.standard_normal((1, 9, 2, 4))
    v = rng.standard_normal((1, 9, 2, 4))
    qi = np.array([20, 21, 22])
    full = oracle.attention_full(q, k, v, qi, np.arange(9), 0.6, False)
    for cut in range(10):
        a = oracle.attention_full(q, k[:, :cut], v[:, :cut], qi, np.arange(cut), 0.6, False)
        b = oracle.attention_full(q, k[:, cut:], v[:, cut:], qi, np.arange(cut, 9), 0.6, False)
        o, lse = oracle.lse_merge(*a, *b)
        np.testing.assert_allclose(o, full[0], atol=1e-14)
        np.testing.assert_allclose(lse, full[1], atol=1e-14)


@pytest.mark.parametrize("big", [700.0, -700.0])
def test_merge_is_stable_for_large_lse(big):
    """The max-shift keeps the merge finite where e^L itself would overflow/underflow."""
    o1 = np.ones((1, 1, 1, 1)); o2 = 3 * np.ones((1, 1, 1, 1))
    l1 = np.full((1, 1, 1), big); l2 = np.full((1, 1, 1), big + math.log(3))
    o, lse = oracle.lse_merge(o1, l1, o2, l2)
    assert abs(lse[0, 0, 0] - (big + math.log(4))) < 1e-12
    assert abs(o[0, 0, 0, 0] - (0.25 * 1 + 0.75 * 3)) < 1e-12  # ulp(700) ~ 1e-13
