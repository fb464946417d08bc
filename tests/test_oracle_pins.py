"""Pins for the CPU oracle: values the pages print, closed forms, invariants,
special cases that reduce to a library routine, and brute force on tiny inputs.

None of these re-derive an expected value from the oracle itself.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import GOLDEN
from oracle import moe_oracle as O


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _frac(p):
    return Fraction(p[0], p[1])


# ---------------------------------------------------------------------------
# Worked example W1: "MoE token routing" section 2-3
# ---------------------------------------------------------------------------

def _w1_router():
    g = _golden("w1_token_routing_example.json")
    probs = np.array(g["probs"])
    x = np.ones((1, 1))
    # logits = ln p, so softmax returns p exactly (up to fp32 rounding of the logits)
    w_r = np.log(probs).astype(np.float32).reshape(4, 1)
    return g, x, w_r


def test_w1_renorm_weights_and_ids():
    g, x, w_r = _w1_router()
    rt = O.route(x, w_r, None, k=2, mode=O.GATE_RENORM)
    assert rt.ids.tolist() == [g["selected_ids_rank_order"]]
    np.testing.assert_allclose(rt.w[0], g["renorm_weights"], atol=1e-6)


def test_w1_topk_then_softmax_equals_printed_weights():
    g, x, w_r = _w1_router()
    rt = O.route(x, w_r, None, k=2, mode=O.GATE_RENORM, renorm_form=O.RENORM_FORM_TOPK_THEN_SOFTMAX)
    np.testing.assert_allclose(rt.w[0], g["renorm_weights"], atol=1e-6)


def test_w1_switch_keeps_full_probabilities():
    g, x, w_r = _w1_router()
    rt = O.route(x, w_r, None, k=2, mode=O.GATE_SWITCH)
    probs = g["probs"]
    np.testing.assert_allclose(rt.w[0], [probs[i] for i in g["selected_ids_rank_order"]], atol=1e-6)


def test_w1_combine_gives_printed_output():
    g, x, w_r = _w1_router()
    rt = O.route(x, w_r, None, k=2, mode=O.GATE_RENORM)
    disp = O.assign_slots(rt.ids, 4, C=1)
    path_out = np.zeros((int(disp.offsets[-1]), 2))
    for r in range(2):
        path_out[disp.row_of[0, r]] = g["expert_outputs"][str(int(rt.ids[0, r]))]
    y = O.combine(1, 2, disp.row_of, rt.w, path_out)
    np.testing.assert_allclose(y[0], g["combined_output"], atol=1e-6)


# ---------------------------------------------------------------------------
# Worked example W2: "LLM from scratch" ch. 36, section 36.4
# ---------------------------------------------------------------------------

def _w2():
    g = _golden("w2_ch36_worked_example.json")
    P = np.array(g["probs"])
    x = np.eye(4)
    w_r = np.log(P).T.astype(np.float32)      # [E=3, d=4]: w_r[e, i] = ln P[i, e]
    return g, x, w_r


def _linear_path_outputs(g, x, ids, disp):
    """Expert e maps x to scale[e]*x (the page's linear experts)."""
    out = np.zeros((int(disp.offsets[-1]), x.shape[1]))
    T, k = ids.shape
    for t in range(T):
        for r in range(k):
            row = disp.row_of[t, r]
            if row >= 0:
                out[row] = g["expert_scale"][ids[t, r]] * x[t]
    return out


def test_w2_selection_and_weights():
    g, x, w_r = _w2()
    rt = O.route(x, w_r, None, k=2, mode=O.GATE_RENORM)
    for t in range(4):
        assert sorted(rt.ids[t].tolist()) == g["selected_sets"][t]
        by_id = {int(e): float(w) for e, w in zip(rt.ids[t], rt.w[t])}
        for e, wf in zip(g["selected_sets"][t], g["weights_by_expert_id"][t]):
            assert abs(by_id[e] - float(_frac(wf))) < 1e-6
    # rank order is by score, which differs from id order on the last token
    assert rt.ids[3].tolist() == [2, 1]


def test_w2_unlimited_capacity_output_is_diagonal():
    g, x, w_r = _w2()
    rt = O.route(x, w_r, None, k=2, mode=O.GATE_RENORM)
    disp = O.assign_slots(rt.ids, 3, C=4)
    y = O.combine(4, 4, disp.row_of, rt.w, _linear_path_outputs(g, x, rt.ids, disp))
    # closed form: Y_tt = sum over the printed weights of weight * scale
    for t in range(4):
        want = sum(_frac(wf) * g["expert_scale"][e]
                   for e, wf in zip(g["selected_sets"][t], g["weights_by_expert_id"][t]))
        assert abs(y[t, t] - float(want)) < 1e-6
    assert abs(y[3, 3] - float(_frac(g["token4_undropped_coefficient"]))) < 1e-6
    assert np.count_nonzero(y - np.diag(np.diag(y))) == 0
    assert disp.load.tolist() == g["requested_load"]
    assert int(disp.load.sum()) == g["total_paths"]
    assert disp.rho_max == pytest.approx(g["rho_max"])


def test_w2_capacity_three_drops_token4_at_expert1():
    g, x, w_r = _w2()
    C = O.capacity(4, 2, 3, *g["capacity_factor"])
    assert C == g["capacity"]
    rt = O.route(x, w_r, None, k=2, mode=O.GATE_RENORM)
    disp = O.assign_slots(rt.ids, 3, C)
    assert disp.accepted.tolist() == g["accepted"]
    assert disp.load.tolist() == g["requested_load"]
    rej = [(t, int(rt.ids[t, r])) for t in range(4) for r in range(2) if disp.slot[t, r] < 0]
    assert rej == [(g["rejected"]["token"], g["rejected"]["expert"])]
    assert disp.overflow == 1
    assert Fraction(disp.rejected_paths, 8) == _frac(g["path_rejection_rate"])
    assert Fraction(disp.tokens_affected, 4) == _frac(g["tokens_affected_rate"])
    assert disp.tokens_dropped == g["tokens_fully_skipped_rate"]
    assert disp.rho_max == pytest.approx(g["rho_max"])
    # slots are token-order first-come-first-served
    assert disp.slot[:, 0].tolist()[:3] == [0, 1, 2]
    y = O.combine(4, 4, disp.row_of, rt.w, _linear_path_outputs(g, x, rt.ids, disp))
    # the rejected path adds nothing and the surviving weight is not renormalised:
    # only expert 2 (scale 3) with its printed weight 7/9 remains for token 4
    surviving = _frac(g["weights_by_expert_id"][3][1]) * g["expert_scale"][2]
    assert abs(y[3, 3] - float(surviving)) < 1e-6
    assert abs(y[3, 3] - float(_frac(g["token4_undropped_coefficient"]))) > 0.1
    assert abs(y[3, 3] - g["token4_renormalise_variant_coefficient"]) > 0.1
    for t in range(3):  # the other tokens keep their undropped outputs
        want = sum(_frac(wf) * g["expert_scale"][e]
                   for e, wf in zip(g["selected_sets"][t], g["weights_by_expert_id"][t]))
        assert abs(y[t, t] - float(want)) < 1e-6


def test_w2_balance_statistics():
    g, x, w_r = _w2()
    rt = O.route(x, w_r, None, k=2, mode=O.GATE_RENORM)
    f, p_bar, aux = O.balance_stats(rt.g32, rt.ids, 3)
    np.testing.assert_allclose(f, np.array(g["requested_load"]) / g["total_paths"], atol=1e-12)
    np.testing.assert_allclose(p_bar, np.array(g["probs"]).mean(axis=0), atol=1e-6)
    assert f.sum() == pytest.approx(1.0) and p_bar.sum() == pytest.approx(1.0)
    # the most requested expert is not the one with the highest mean probability
    assert int(np.argmax(f)) == 1 and int(np.argmax(p_bar)) == 0


def test_balance_value_is_one_at_uniform():
    # all-equal logits: f_e = p_bar_e = 1/E  => E * sum f p_bar = 1
    E, k, T = 4, 4, 8
    g32 = np.zeros((T, E))
    ids = O.select_topk(g32, k)
    _, _, aux = O.balance_stats(g32, ids, E)
    assert aux == pytest.approx(1.0)


# ---------------------------------------------------------------------------
# Capacity and accounting numbers printed on the pages
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", _golden("capacity_examples.json")["cases"])
def test_capacity_examples(case):
    assert O.capacity(case["T"], case["k"], case["E"], *case["cf"]) == case["C"]


def test_capacity_is_exact_integer_ceiling():
    # 1.25 * 8192 * 8 / 128 = 640 exactly: no spurious rounding up
    assert O.capacity(8192, 8, 128, 5, 4) == 640
    assert O.capacity(8193, 8, 128, 5, 4) == 641
    for T, k, E, a, b in itertools.product([1, 7, 1000], [1, 2, 3], [3, 8], [1, 5], [1, 4]):
        want = math.ceil(Fraction(a, b) * T * k / E)
        assert O.capacity(T, k, E, a, b) == want


@pytest.mark.parametrize("case", _golden("accounting.json")["cases"])
def test_accounting(case):
    w = case["what"]
    if w == "expert_params":
        got = O.expert_params(case["d"], case["m"])
    elif w == "all_routed_params":
        got = case["E"] * O.expert_params(case["d"], case["m"])
    elif w == "active_routed_params":
        got = case["k"] * O.expert_params(case["d"], case["m"])
    elif w == "routed_bytes_2B":
        got = 2 * case["E"] * O.expert_params(case["d"], case["m"])
    elif w == "router_params":
        got = O.router_params(case["d"], case["E"])
    assert got == case["value"]


# ---------------------------------------------------------------------------
# Selection: brute force with deliberate ties
# ---------------------------------------------------------------------------

def test_select_topk_matches_brute_force_with_ties():
    rng = np.random.default_rng(7)
    for E, k in [(3, 1), (4, 2), (8, 3), (8, 8), (16, 5)]:
        g = rng.integers(-2, 3, size=(200, E)).astype(np.float64)  # many exact ties
        ids = O.select_topk(g, k)
        for t in range(g.shape[0]):
            brute = sorted(range(E), key=lambda e: (-g[t, e], e))[:k]
            assert ids[t].tolist() == brute


def test_negative_zero_ties_with_positive_zero():
    x = np.array([[1.0]])
    w_r = np.array([[-0.0], [0.0], [-1.0]], dtype=np.float32)
    rt = O.route(x, w_r, None, k=1, mode=O.GATE_RENORM)
    assert rt.ids[0, 0] == 0           # equal scores: the lower id wins


def test_route_margins_hand_computed():
    """The score gaps that decide the selection, worked by hand on a small table.
    Row 0 scores (3.0 at id 1, 2.0 at id 3, 0.5 at id 0, -1.0 at id 2) are listed
    out of rank order, so a margin taken over ids instead of ranks, a sort in the
    wrong direction or a flipped sign fails.  Row 1 holds an exact tie at the
    boundary (margin 0), row 2 a tie inside the set."""
    g = np.array([[0.5, 3.0, -1.0, 2.0],
                  [1.0, 1.0, -2.0, 1.0],
                  [-4.0, -0.25, -0.25, -3.0]])
    # k < E: boundary = k-th minus (k+1)-th largest; adjacent gaps between ranks 0..k-1
    b, a = O.route_margins(g, 2)
    np.testing.assert_array_equal(b, [2.0 - 0.5, 1.0 - 1.0, -0.25 - (-3.0)])
    np.testing.assert_array_equal(a, [[3.0 - 2.0], [0.0], [0.0]])
    b, a = O.route_margins(g, 3)
    np.testing.assert_array_equal(b, [0.5 - (-1.0), 1.0 - (-2.0), -3.0 - (-4.0)])
    np.testing.assert_array_equal(a, [[1.0, 1.5], [0.0, 0.0], [0.0, 2.75]])
    # k = 1: no adjacent in-set gap
    b, a = O.route_margins(g, 1)
    np.testing.assert_array_equal(b, [1.0, 0.0, 0.0])
    assert a.shape == (3, 0)
    # k = E: every expert is selected, the set cannot change (boundary = inf)
    b, a = O.route_margins(g, 4)
    assert np.isinf(b).all() and (b > 0).all()
    np.testing.assert_array_equal(a, [[1.0, 1.5, 1.5], [0.0, 0.0, 3.0], [0.0, 2.75, 1.0]])
    # the margins are never negative and do not depend on the order of the ids
    perm = [2, 0, 3, 1]
    for k in (1, 2, 3, 4):
        b0, a0 = O.route_margins(g, k)
        b1, a1 = O.route_margins(g[:, perm], k)
        np.testing.assert_array_equal(b0, b1)
        np.testing.assert_array_equal(a0, a1)
        assert (b0 >= 0).all() and (a0 >= 0).all()


def test_selection_by_probability_equals_selection_by_score():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 16))
    w_r = rng.standard_normal((10, 16)).astype(np.float32)
    rt = O.route(x, w_r, None, k=3, mode=O.GATE_RENORM)
    p = O.softmax_rows(rt.g32)
    by_prob = np.argsort(-p, axis=1, kind="stable")[:, :3]
    assert (by_prob == rt.ids).all()


# ---------------------------------------------------------------------------
# Weights: equivalences and special cases
# ---------------------------------------------------------------------------

def test_two_renorm_forms_agree():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((256, 32))
    w_r = (rng.standard_normal((16, 32)) * 2).astype(np.float32)
    a = O.route(x, w_r, None, 4, O.GATE_RENORM, O.RENORM_FORM_SOFTMAX_THEN_RENORM).w
    b = O.route(x, w_r, None, 4, O.GATE_RENORM, O.RENORM_FORM_TOPK_THEN_SOFTMAX).w
    np.testing.assert_allclose(a, b, atol=1e-12)
    np.testing.assert_allclose(a.sum(axis=1), 1.0, atol=1e-12)
    assert (a >= 0).all()


def test_k1_renorm_weight_is_exactly_one():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((50, 8))
    w_r = rng.standard_normal((6, 8)).astype(np.float32)
    rt = O.route(x, w_r, None, 1, O.GATE_RENORM)
    assert (rt.w == 1.0).all()


def test_switch_weights_sum_to_at_most_one_and_kE_is_full_softmax():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((40, 8))
    w_r = rng.standard_normal((5, 8)).astype(np.float32)
    rt = O.route(x, w_r, None, 2, O.GATE_SWITCH)
    assert (rt.w.sum(axis=1) <= 1.0 + 1e-15).all()
    full = O.route(x, w_r, None, 5, O.GATE_RENORM)
    # k = E renormalised weights are the full softmax (compare to torch's softmax)
    ref = torch.softmax(torch.tensor(full.g32), dim=1).numpy()
    np.testing.assert_allclose(full.w, ref[np.arange(40)[:, None], full.ids], atol=1e-12)


def test_router_logits_match_library_matmul_and_bias():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((9, 33)).astype(np.float32)
    w_r = rng.standard_normal((7, 33)).astype(np.float32)
    b = rng.standard_normal(7).astype(np.float32)
    g64, g32 = O.router_logits(x, w_r, b)
    ref = torch.nn.functional.linear(torch.tensor(x, dtype=torch.float64),
                                     torch.tensor(w_r, dtype=torch.float64),
                                     torch.tensor(b, dtype=torch.float64)).numpy()
    np.testing.assert_allclose(g64, ref, rtol=1e-13, atol=1e-13)
    assert (g32 == g32.astype(np.float32)).all()


def test_nonfinite_logits_are_an_input_failure():
    x = np.array([[1.0, np.nan]])
    w_r = np.ones((3, 2), dtype=np.float32)
    with pytest.raises(O.NonFiniteLogit):
        O.route(x, w_r, None, 1, O.GATE_RENORM)
    x = np.array([[1e30, 1e30]])
    w_r = np.full((3, 2), 1e30, dtype=np.float32)      # overflows fp32
    with pytest.raises(O.NonFiniteLogit):
        O.route(x, w_r, None, 1, O.GATE_RENORM)


def test_argument_checks_and_empty_group():
    x = np.zeros((0, 4))
    w_r = np.ones((3, 4), dtype=np.float32)
    experts = (np.zeros((3, 2, 4)), np.zeros((3, 2, 4)), np.zeros((3, 4, 2)))
    res = O.forward(x, w_r, None, experts, k=2, mode=O.GATE_RENORM, C=3)
    assert res.y.shape == (0, 4) and res.dispatch.load.tolist() == [0, 0, 0]
    x1 = np.ones((2, 4))
    with pytest.raises(O.OracleError):
        O.forward(x1, w_r, None, experts, k=0, mode=O.GATE_RENORM)
    with pytest.raises(O.OracleError):
        O.forward(x1, w_r, None, experts, k=4, mode=O.GATE_RENORM)
    with pytest.raises(O.OracleError):
        O.forward(x1, w_r, None, experts, k=1, mode=O.GATE_RENORM, C=0)


# ---------------------------------------------------------------------------
# Dispatch invariants (Algorithm 36.1) and properties
# ---------------------------------------------------------------------------

def _random_ids(rng, T, E, k, skew=0.0):
    logits = rng.standard_normal((T, E)) - skew * np.log1p(np.arange(E))[None, :]
    return O.select_topk(O.round_to_f32(logits), k)


@pytest.mark.parametrize("T,E,k,C", [(300, 8, 2, 40), (500, 16, 4, 90), (257, 5, 5, 300), (64, 4, 1, 1)])
def test_dispatch_invariants(T, E, k, C):
    rng = np.random.default_rng(T + E + k)
    ids = _random_ids(rng, T, E, k, skew=1.0)
    disp = O.assign_slots(ids, E, C)
    assert int(disp.load.sum()) == T * k
    assert (disp.accepted <= C).all()
    assert (disp.load == disp.accepted + np.maximum(disp.load - C, 0)).all()
    assert disp.overflow == disp.rejected_paths
    assert int(disp.offsets[-1]) == int(disp.accepted.sum()) == len(disp.src_token)
    for e in range(E):
        mine = [(t, r) for t in range(T) for r in range(k) if ids[t, r] == e]
        slots = [disp.slot[t, r] for t, r in mine]
        # first-come-first-served in token order: the first C requests get 0..C-1
        assert slots == [i if i < C else -1 for i in range(len(mine))]
        rows = disp.src_token[disp.offsets[e]:disp.offsets[e + 1]]
        assert rows.tolist() == [t for t, r in mine][:C]      # token order in each group
    # each accepted record maps to a distinct grouped row that points back to it
    acc = disp.row_of[disp.row_of >= 0]
    assert len(set(acc.tolist())) == len(acc)


def test_causal_prefix_property():
    """Acceptance of token t depends only on tokens before it ([CH36] §36.3)."""
    rng = np.random.default_rng(21)
    T, E, k, C = 200, 8, 2, 30
    ids = _random_ids(rng, T, E, k, skew=1.5)
    full = O.assign_slots(ids, E, C)
    for tp in [1, 17, 99, 150]:
        part = O.assign_slots(ids[:tp], E, C)
        assert (part.slot == full.slot[:tp]).all()


def _tiny_layer(rng, T, d, m, E):
    x = rng.standard_normal((T, d))
    w_r = (rng.standard_normal((E, d)) / math.sqrt(d)).astype(np.float32)
    wg = rng.standard_normal((E, m, d)) / math.sqrt(d)
    wu = rng.standard_normal((E, m, d)) / math.sqrt(d)
    wd = rng.standard_normal((E, d, m)) / math.sqrt(m)
    return x, w_r, (wg, wu, wd)


def test_permutation_equivariance_without_capacity():
    rng = np.random.default_rng(4)
    x, w_r, ex = _tiny_layer(rng, 24, 6, 10, 5)
    perm = rng.permutation(24)
    a = O.forward(x, w_r, None, ex, k=2, mode=O.GATE_RENORM).y
    b = O.forward(x[perm], w_r, None, ex, k=2, mode=O.GATE_RENORM).y
    np.testing.assert_allclose(a[perm], b, atol=1e-12)


def test_sparse_with_k_equal_E_reduces_to_dense_brute_force():
    rng = np.random.default_rng(17)
    for E in [1, 3, 6]:
        x, w_r, ex = _tiny_layer(rng, 12, 5, 7, E)
        b = rng.standard_normal(E).astype(np.float32)
        sparse = O.forward(x, w_r, b, ex, k=E, mode=O.GATE_RENORM).y
        dense = O.dense_forward(x, w_r, b, ex)
        np.testing.assert_allclose(sparse, dense, atol=1e-12)


def test_single_expert_single_choice_is_the_ffn():
    """E = k = 1: the weight is exactly one and the layer is that expert's FFN."""
    rng = np.random.default_rng(23)
    x, w_r, ex = _tiny_layer(rng, 10, 4, 6, 1)
    y = O.forward(x, w_r, None, ex, k=1, mode=O.GATE_RENORM).y
    xt = torch.tensor(x)
    ref = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(xt, torch.tensor(ex[0][0])))
        * torch.nn.functional.linear(xt, torch.tensor(ex[1][0])), torch.tensor(ex[2][0]))
    np.testing.assert_allclose(y, ref.numpy(), atol=1e-12)


# ---------------------------------------------------------------------------
# SwiGLU expert: closed forms and library routines
# ---------------------------------------------------------------------------

def test_swiglu_identity_weights_closed_form():
    x = np.linspace(-6, 6, 25).reshape(5, 5)
    eye = np.eye(5)
    y = O.swiglu_ffn(x, eye, eye, eye, round_h_bf16=False)
    # SiLU(x) * x = x^2 * sigmoid(x); sigmoid via tanh: (1 + tanh(x/2)) / 2
    np.testing.assert_allclose(y, x * x * (1 + np.tanh(x / 2)) / 2, rtol=1e-13, atol=1e-15)


def test_swiglu_orientation_with_permutations():
    """Permutation weights expose a transposed operand: out[j] must equal
    SiLU(x[pg[pd[j]]]) * x[pu[pd[j]]] with P[a, b] = 1 iff b == p[a]."""
    rng = np.random.default_rng(2)
    d = m = 7
    pg, pu, pd = rng.permutation(m), rng.permutation(m), rng.permutation(d)
    Pg, Pu, Pd = np.zeros((m, d)), np.zeros((m, d)), np.zeros((d, m))
    Pg[np.arange(m), pg] = 1
    Pu[np.arange(m), pu] = 1
    Pd[np.arange(d), pd] = 1
    x = rng.standard_normal((3, d))
    y = O.swiglu_ffn(x, Pg, Pu, Pd, round_h_bf16=False)
    for t in range(3):
        for j in range(d):
            i = pd[j]
            a, b = x[t, pg[i]], x[t, pu[i]]
            assert y[t, j] == pytest.approx(a * b * (1 + math.tanh(a / 2)) / 2, rel=1e-13, abs=1e-15)


def test_swiglu_matches_torch_fp64_and_zero_down_gives_zero():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((11, 9))
    wg, wu, wd = rng.standard_normal((13, 9)), rng.standard_normal((13, 9)), rng.standard_normal((9, 13))
    y = O.swiglu_ffn(x, wg, wu, wd, round_h_bf16=False)
    xt = torch.tensor(x)
    ref = (torch.nn.functional.silu(xt @ torch.tensor(wg).T) * (xt @ torch.tensor(wu).T)) @ torch.tensor(wd).T
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)
    assert (O.swiglu_ffn(x, wg, wu, np.zeros_like(wd), False) == 0).all()


def test_round_to_bf16_matches_torch_conversion_including_ties():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 20000)
    # exact halfway points between neighbouring bf16 values (ties to even)
    base = torch.tensor(rng.standard_normal(4000).astype(np.float32)).to(torch.bfloat16).float()
    bits = base.view(torch.int32)
    half = (bits + 0x8000).view(torch.float32).numpy()
    v = np.concatenate([v, half, np.array([0.0, -0.0, 1e-40, -3e-39], dtype=np.float32)])
    ref = torch.tensor(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_to_bf16(v.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


# ---------------------------------------------------------------------------
# Combine: dropped paths, shared expert
# ---------------------------------------------------------------------------

def test_fully_dropped_token_contributes_nothing_and_shared_is_unweighted():
    rng = np.random.default_rng(31)
    T, d, m, E = 40, 6, 8, 4
    x, w_r, ex = _tiny_layer(rng, T, d, m, E)
    b = np.array([50, 50, 0, 0], dtype=np.float32)  # everyone wants experts 0 and 1
    res = O.forward(x, w_r, b, ex, k=2, mode=O.GATE_RENORM, C=3)
    dropped = np.where((res.dispatch.slot < 0).all(axis=1))[0]
    assert len(dropped) == T - 3 and res.dispatch.tokens_dropped == T - 3
    assert (res.y[dropped] == 0).all()
    sh = (rng.standard_normal((5, d)), rng.standard_normal((5, d)), rng.standard_normal((d, 5)))
    with_shared = O.forward(x, w_r, b, ex, k=2, mode=O.GATE_RENORM, C=3, shared=sh)
    s = O.swiglu_ffn(x, *sh, round_h_bf16=False)
    np.testing.assert_allclose(with_shared.y - res.y, s, atol=1e-12)
    zero_routed = (ex[0], ex[1], np.zeros_like(ex[2]))
    only_shared = O.forward(x, w_r, b, zero_routed, k=2, mode=O.GATE_RENORM, shared=sh)
    np.testing.assert_allclose(only_shared.y, s, atol=1e-12)


def test_token_subset_matches_full_evaluation():
    rng = np.random.default_rng(12)
    x, w_r, ex = _tiny_layer(rng, 60, 6, 8, 5)
    full = O.forward(x, w_r, None, ex, k=2, mode=O.GATE_RENORM, C=20)
    sub = O.forward(x, w_r, None, ex, k=2, mode=O.GATE_RENORM, C=20, tokens=[0, 13, 59])
    np.testing.assert_allclose(sub.y, full.y[[0, 13, 59]], atol=1e-14)


# --------------------------------------------------------------------------
# overflow variants ([CH36] §36.3 acceptance rules and overflow, §36.4 example)
# --------------------------------------------------------------------------

def test_w2_renormalised_survivors_gives_printed_3x4():
    """The worked example's variant: renormalising over the surviving paths
    gives token 4 the coefficient 3 (its only surviving expert, scale 3, with
    weight one); the tokens without a rejected path keep their outputs."""
    g, x, w_r = _w2()
    rt = O.route(x, w_r, None, k=2, mode=O.GATE_RENORM)
    disp = O.assign_slots(rt.ids, 3, g["capacity"])
    outs = _linear_path_outputs(g, x, rt.ids, disp)
    drop = O.combine(4, 4, disp.row_of, rt.w, outs)
    ren = O.combine(4, 4, disp.row_of, O.survivor_weights(disp.row_of, rt.w), outs)
    assert abs(ren[3, 3] - g["token4_renormalise_variant_coefficient"]) < 1e-9
    np.testing.assert_allclose(ren[:3], drop[:3], atol=1e-12)
    # without any rejection the renormalised weights are the weights themselves
    free = O.assign_slots(rt.ids, 3, 4)
    np.testing.assert_allclose(O.survivor_weights(free.row_of, rt.w), rt.w, atol=1e-12)


def test_gate_priority_constructed_example():
    """tests/golden/w2_gate_priority_variant.json: at expert 1 the four requests
    carry weights 2/9, 1/3, 7/18, 2/3 in token order; C = 3 rejects the last
    arrival first-come-first-served but the lowest weight (token 0) by gate
    weight, and the accepted rows keep token order."""
    with open(os.path.join(GOLDEN, "w2_gate_priority_variant.json")) as f:
        g = json.load(f)
    P = np.array(g["probs"])
    x = np.eye(4)
    w_r = np.log(P).T.astype(np.float32)
    rt = O.route(x, w_r, None, k=2, mode=O.GATE_RENORM)
    for t in range(4):
        assert sorted(rt.ids[t].tolist()) == g["selected_sets"][t]
        by_id = {int(e): float(w) for e, w in zip(rt.ids[t], rt.w[t])}
        for e, wf in zip(g["selected_sets"][t], g["weights_by_expert_id"][t]):
            assert abs(by_id[e] - float(_frac(wf))) < 1e-6
    C = g["capacity"]
    fcfs = O.assign_slots(rt.ids, 3, C)
    gate = O.assign_slots_by_gate(rt.ids, O.round_to_f32(rt.w), 3, C)

    def rejected(d):
        return [[t, int(rt.ids[t, r])] for t in range(4) for r in range(2) if d.slot[t, r] < 0]

    assert rejected(fcfs) == g["first_come_first_served"]["rejected"]
    assert rejected(gate) == g["by_gate_weight"]["rejected"]
    for t, c in g["by_gate_weight"]["expert1_slots_by_token"]:
        r = int(np.where(rt.ids[t] == 1)[0][0])
        assert gate.slot[t, r] == c
    cases = ((fcfs, rt.w, "first_come_first_served"), (gate, rt.w, "by_gate_weight"),
             (gate, O.survivor_weights(gate.row_of, rt.w), "by_gate_weight_renormalised_survivors"))
    for d, w, key in cases:
        y = O.combine(4, 4, d.row_of, w, _linear_path_outputs(g, x, rt.ids, d))
        want = [float(_frac(v)) for v in g[key]["y_diag"]]
        np.testing.assert_allclose(np.diag(y), want, atol=1e-6)
        assert np.count_nonzero(y - np.diag(np.diag(y))) == 0
    # the load statistics do not depend on the acceptance order
    assert gate.load.tolist() == fcfs.load.tolist()
    assert gate.overflow == fcfs.overflow == 1


@pytest.mark.parametrize("seed", range(6))
def test_gate_priority_invariants(seed):
    """Brute-force properties on random small groups: per expert exactly
    min(L_e, C) requests are accepted; no rejected request outweighs an accepted
    one (equal weights: the earlier token wins); accepted slots run 0.. in token
    order; with C >= every load nothing changes from first-come-first-served."""
    rng = np.random.default_rng(100 + seed)
    T, E, k = int(rng.integers(5, 40)), int(rng.integers(2, 7)), 2
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    w = rng.choice([0.125, 0.25, 0.375, 0.5], size=(T, k))   # many exact ties
    C = int(rng.integers(1, 6))
    d = O.assign_slots_by_gate(ids, w, E, C)
    for e in range(E):
        req = [(t, r) for t in range(T) for r in range(k) if ids[t, r] == e]
        acc = [(t, r) for t, r in req if d.slot[t, r] >= 0]
        rej = [(t, r) for t, r in req if d.slot[t, r] < 0]
        assert len(acc) == min(len(req), C)
        for ta, ra in acc:
            for tr, rr in rej:
                assert w[ta, ra] > w[tr, rr] or (w[ta, ra] == w[tr, rr] and ta < tr)
        assert [int(d.slot[t, r]) for t, r in acc] == list(range(len(acc)))
    big = O.assign_slots_by_gate(ids, w, E, T)
    ref = O.assign_slots(ids, E, T)
    assert np.array_equal(big.slot, ref.slot) and np.array_equal(big.row_of, ref.row_of)


# ---------------------------------------------------------------------------
# Overflow variant: rerouting a rejected path to the next-choice expert
# (hand-worked fixtures; the reading is stated in the fixture and the oracle)
# ---------------------------------------------------------------------------

def _reroute_case(c, mode):
    P = np.array(c["probs"])
    T, E = P.shape
    k = c["k"]
    x = np.eye(T)
    w_r = np.log(P).T.astype(np.float32)        # [E, d = T]: the scores are ln p
    rt = O.route(x, w_r, None, k, mode)
    n = min(2 * k, E)
    ids2 = np.full((T, 2 * k), -1, dtype=np.int64)
    ids2[:, :n] = O.select_topk(rt.g32, n)
    w2 = np.zeros((T, 2 * k))
    w2[:, :k] = O.gate_weights(rt.g32, ids2[:, :k], mode)
    w2[:, k:] = O.spare_weights(rt.g32, ids2[:, :k], ids2[:, k:], mode)
    return x, w_r, ids2, w2


@pytest.mark.parametrize("case", _golden("reroute_next_choice.json")["cases"], ids=lambda c: c["name"])
def test_reroute_hand_worked_examples(case):
    C = O.capacity(len(case["probs"]), case["k"], len(case["probs"][0]), *case["capacity_factor"])
    assert C == case["capacity"]
    for mode, key in ((O.GATE_RENORM, "y_diag_renorm"), (O.GATE_SWITCH, "y_diag_switch")):
        if key not in case:
            continue
        x, w_r, ids2, w2 = _reroute_case(case, mode)
        assert ids2.tolist() == case["ids_2k"]
        rr = O.assign_slots_reroute(ids2, case["k"], len(case["expert_scale"]), C)
        d = rr.dispatch
        assert d.slot.tolist() == case["slot_2k"]
        assert d.load.tolist() == case["requested_load"]
        assert d.offsets.tolist() == case["offsets"]
        assert d.src_token.tolist() == case["src_token"]
        assert d.overflow == case["first_pass_overflow"]
        assert (rr.rerouted, rr.tokens_affected, rr.tokens_dropped) == (
            case["rerouted"], case["tokens_affected"], case["tokens_dropped"])
        # linear experts on the grouped rows, combined over the 2k columns
        out = np.zeros((int(d.offsets[-1]), x.shape[1]))
        T = x.shape[0]
        for t in range(T):
            for c in range(ids2.shape[1]):
                if d.row_of[t, c] >= 0:
                    out[d.row_of[t, c]] = case["expert_scale"][ids2[t, c]] * x[t]
        y = O.combine(T, x.shape[1], d.row_of, w2, out)
        want = [float(Fraction(*v)) for v in case[key]]
        np.testing.assert_allclose(np.diag(y), want, atol=1e-6)
        assert np.count_nonzero(y - np.diag(np.diag(y))) == 0


def _reroute_by_expert(ids2, k, E, C):
    """The same acceptance written per expert instead of as one ordered sweep:
    an expert keeps its first min(L_e, C) candidate requests in token order,
    then, of the spare requests made to it (the j-th rejected candidate of a
    token asks for its spare j), the first C - min(L_e, C) in token order."""
    T = ids2.shape[0]
    slot = np.full((T, 2 * k), -1, dtype=np.int64)
    first = {e: [(t, r) for t in range(T) for r in range(k) if ids2[t, r] == e] for e in range(E)}
    for e, reqs in first.items():
        for c, (t, r) in enumerate(reqs[:C]):
            slot[t, r] = c
    spare_reqs = {e: [] for e in range(E)}
    for t in range(T):
        rejected = [r for r in range(k) if slot[t, r] < 0]
        for j in range(len(rejected)):
            if ids2[t, k + j] >= 0:
                spare_reqs[int(ids2[t, k + j])].append((t, k + j))
    for e, reqs in spare_reqs.items():
        base = min(len(first[e]), C)
        for c, (t, col) in enumerate(reqs[:max(C - base, 0)]):
            slot[t, col] = base + c
    return slot


@pytest.mark.parametrize("seed", range(6))
def test_reroute_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    for _ in range(20):
        E = int(rng.integers(2, 9))
        k = int(rng.integers(1, E + 1))
        T = int(rng.integers(1, 40))
        C = int(rng.integers(1, max(2, T * k // E + 2)))
        g = rng.integers(-3, 4, size=(T, E)).astype(np.float64)     # many exact ties
        n = min(2 * k, E)
        ids2 = np.full((T, 2 * k), -1, dtype=np.int64)
        ids2[:, :n] = O.select_topk(g, n)
        rr = O.assign_slots_reroute(ids2, k, E, C)
        d = rr.dispatch
        # the same slots from the per-expert formulation
        np.testing.assert_array_equal(d.slot, _reroute_by_expert(ids2, k, E, C))
        # the candidates' acceptance is Algorithm 36.1's, unchanged by the reroutes
        np.testing.assert_array_equal(d.slot[:, :k], O.assign_slots(ids2[:, :k], E, C).slot)
        # capacity holds, every row is used once, served experts are distinct per token
        acc = np.bincount(ids2[d.slot >= 0], minlength=E)
        assert (acc <= C).all() and int(d.offsets[-1]) == int((d.slot >= 0).sum())
        assert sorted(d.row_of[d.row_of >= 0].tolist()) == list(range(int(d.offsets[-1])))
        for t in range(T):
            served = ids2[t][d.slot[t] >= 0].tolist()
            assert len(served) == len(set(served)) and len(served) <= k
            # spare j is used only when at least j + 1 candidates were rejected
            nrej = int((d.slot[t, :k] < 0).sum())
            assert all(d.slot[t, k + j] < 0 for j in range(nrej, k))
        assert d.load.tolist() == np.bincount(ids2[:, :k].ravel(), minlength=E).tolist()
        assert rr.rerouted == int((d.slot[:, k:] >= 0).sum()) <= d.overflow
        assert rr.tokens_dropped == int((~(d.slot >= 0).any(axis=1)).sum())
        if d.overflow == 0:
            assert rr.rerouted == 0 and (d.slot[:, k:] < 0).all()


def test_reroute_without_overflow_is_the_plain_layer():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((40, 16))
    w_r = rng.standard_normal((6, 16)).astype(np.float32)
    ex = tuple(rng.standard_normal((6, 8, 16)) * 0.2 for _ in range(2)) + (rng.standard_normal((6, 16, 8)) * 0.2,)
    plain = O.forward(x, w_r, None, ex, 2, O.GATE_RENORM, C=None)
    rer = O.forward(x, w_r, None, ex, 2, O.GATE_RENORM, C=None, reroute=True)
    np.testing.assert_array_equal(rer.route.ids[:, :2], plain.route.ids)
    np.testing.assert_allclose(rer.y, plain.y, rtol=0, atol=1e-12)
    assert rer.stats["rerouted"] == 0
