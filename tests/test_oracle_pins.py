"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test fixes a value by a closed form, a brute-force enumeration, a
textbook/library routine on a special case, or an invariant, chosen so that a
plausible slip in the oracle (a dropped term, a sign, an index, a transposed
operand) fails at least one of them.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import moe_oracle as O


def rng(seed=0):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# router logits
# --------------------------------------------------------------------------
def test_logits_unit_vector_router_picks_input_columns():
    # W_r rows are unit vectors e_e (d > E): logits are exactly x[:, :E]; a
    # transposed router ([d, E] read as [E, d]) would not even have the shape.
    T, d, E = 5, 12, 7
    x = rng(1).standard_normal((T, d))
    w = np.zeros((E, d))
    w[np.arange(E), np.arange(E)] = 1.0
    np.testing.assert_array_equal(O.router_logits(x, w), x[:, :E])


def test_logits_permuted_unit_router_and_bias():
    T, d, E = 4, 9, 5
    x = rng(2).standard_normal((T, d))
    cols = np.array([8, 0, 3, 6, 1])
    w = np.zeros((E, d))
    w[np.arange(E), cols] = 2.0
    b = np.array([0.5, -1.0, 0.0, 3.0, -0.25])
    np.testing.assert_array_equal(O.router_logits(x, w, b), 2.0 * x[:, cols] + b)
    # zero router: the logits are the bias alone
    np.testing.assert_array_equal(O.router_logits(x, np.zeros((E, d)), b), np.broadcast_to(b, (T, E)))


def test_logits_widen_bf16_bits():
    # 0x3F80 = 1.0, 0xC000 = -2.0, 0x3E80 = 0.25 in bf16
    x = np.array([[0x3F80, 0xC000, 0x3E80]], dtype=np.uint16)
    w = np.array([[0x3F80, 0x3F80, 0x3F80], [0x0000, 0x3F80, 0x0000]], dtype=np.uint16)
    np.testing.assert_array_equal(O.router_logits(x, w), [[1.0 - 2.0 + 0.25, -2.0]])


# --------------------------------------------------------------------------
# top-k selection (the bit-exact part)
# --------------------------------------------------------------------------
def brute_force_topk_set(row, k):
    """The k-subset with the largest logit sum (unique when logits are distinct)."""
    best, best_sum = None, -math.inf
    for sub in itertools.combinations(range(len(row)), k):
        s = sum(row[e] for e in sub)
        if s > best_sum:
            best, best_sum = sub, s
    return set(best)


@pytest.mark.parametrize("k", [1, 2, 3, 5])
def test_topk_matches_subset_enumeration(k):
    g = rng(3)
    for _ in range(60):
        row = g.permutation(8).astype(np.float64) * 0.37 - 1.1  # distinct values
        chosen = O.select_experts(row, k)
        assert set(chosen) == brute_force_topk_set(row, k)
        vals = [row[e] for e in chosen]
        assert all(vals[i] > vals[i + 1] for i in range(k - 1)), "slots must be largest first"


def test_topk_k1_is_argmax_lowest_id():
    g = rng(4)
    for _ in range(200):
        row = g.integers(-3, 3, size=16).astype(np.float64)  # many ties
        assert O.select_experts(row, 1) == [int(np.argmax(row))]  # numpy returns the first maximum


def test_topk_k_equals_E_is_full_descending_sort_with_id_ties():
    g = rng(5)
    for _ in range(100):
        row = g.integers(-4, 4, size=12).astype(np.float64)
        order = np.lexsort((np.arange(12), -row))  # key 1: -value, key 2: id
        assert O.select_experts(row, 12) == order.tolist()


def test_topk_all_equal_gives_lowest_ids():
    for E, k in [(8, 2), (64, 8), (64, 6), (256, 16)]:
        assert O.select_experts(np.full(E, 0.3), k) == list(range(k))


def test_topk_signed_zero_ties_and_infinities():
    row = np.array([0.0, -0.0, -np.inf, np.inf, -0.0])
    # +inf first, then the three zeros by id, then -inf
    assert O.select_experts(row, 5) == [3, 0, 1, 4, 2]


def test_topk_nan_ranks_last():
    row = np.array([np.nan, -5.0, np.nan, -np.inf, 1.0])
    assert O.select_experts(row, 3) == [4, 1, 3]
    assert O.select_experts(row, 5) == [4, 1, 3, 0, 2]


# --------------------------------------------------------------------------
# gate weights
# --------------------------------------------------------------------------
@pytest.mark.parametrize("L,E", [(0.0, 8), (2.5, 8), (-1.0, 64), (7.0, 64)])
def test_softmax_closed_form_one_hot_logit(L, E):
    row = np.zeros(E)
    row[3] = L
    p = O.softmax_row(row)
    den = math.exp(L) + (E - 1)
    assert p[3] == pytest.approx(math.exp(L) / den, rel=1e-15)
    for e in range(E):
        if e != 3:
            assert p[e] == pytest.approx(1.0 / den, rel=1e-15)


def test_route_weights_closed_form_with_and_without_renormalisation():
    E, L = 8, 1.5
    logits = np.zeros((1, E))
    logits[0, 5] = L
    # without renormalisation the weights are the softmax probabilities
    ids, w = O.route(logits, 2, renormalize=False)
    assert ids.tolist() == [[5, 0]]
    den = math.exp(L) + E - 1
    np.testing.assert_allclose(w, [[math.exp(L) / den, 1.0 / den]], rtol=1e-15)
    # with renormalisation over the two slots: e^L/(e^L+1), 1/(e^L+1)
    ids, w = O.route(logits, 2, renormalize=True)
    np.testing.assert_allclose(w, [[math.exp(L) / (math.exp(L) + 1), 1 / (math.exp(L) + 1)]], rtol=1e-15)


def test_route_weights_invariants():
    g = rng(6)
    logits = g.standard_normal((50, 64)) * 2
    _, w = O.route(logits, 8, renormalize=True)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-14)
    _, w2 = O.route(logits, 8, renormalize=False)
    assert np.all(w2.sum(1) < 1.0) and np.all(w2 > 0)
    assert np.all(np.diff(w2, axis=1) <= 0), "weights follow the slot (descending logit) order"
    # k = E with renormalisation: the weights are the full softmax (a library routine)
    from scipy.special import softmax
    ids, w3 = O.route(logits[:5, :10], 10, renormalize=True)
    for t in range(5):
        np.testing.assert_allclose(w3[t], softmax(logits[t, :10])[ids[t]], rtol=1e-13)


# --------------------------------------------------------------------------
# permutation (the bit-exact part)
# --------------------------------------------------------------------------
def bucket_permutation(ids, E):
    """Independent construction: walk the experts in order, collect rows in flat order."""
    flat = ids.ravel().tolist()
    perm = []
    counts = []
    for e in range(E):
        rows = [f for f, v in enumerate(flat) if v == e]
        counts.append(len(rows))
        perm += rows
    return counts, perm


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (16, 8, 2), (37, 64, 8), (100, 64, 6), (5, 256, 16)])
def test_permutation_matches_bucket_walk_and_invariants(T, E, k):
    g = rng(T * 1000 + E + k)
    ids = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)])
    counts, offsets, perm, inv = O.permute(ids, E)
    c_ref, p_ref = bucket_permutation(ids, E)
    assert counts.tolist() == c_ref
    assert perm.tolist() == p_ref
    assert offsets[0] == 0 and offsets[-1] == T * k and np.all(np.diff(offsets) == counts)
    assert sorted(perm.tolist()) == list(range(T * k)), "perm is a bijection"
    assert np.array_equal(inv[perm], np.arange(T * k))
    flat = ids.ravel()
    assert np.all(np.diff(flat[perm]) >= 0), "expert ids non-decreasing along perm"
    tok = perm // k
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0), "flat index strictly increasing within a segment"
        assert np.all(np.diff(tok[offsets[e]:offsets[e + 1]]) > 0)
    # every token appears exactly k times
    assert np.all(np.bincount(tok, minlength=T) == k)


# --------------------------------------------------------------------------
# expert FFN and the layer
# --------------------------------------------------------------------------
def silu_scalar(z):
    return z / (1.0 + math.exp(-z))


def test_silu_closed_forms():
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert O.silu(np.array([2.0]))[0] == pytest.approx(2.0 / (1.0 + math.exp(-2.0)), rel=1e-15)
    assert O.silu(np.array([-2.0]))[0] == pytest.approx(-2.0 / (1.0 + math.exp(2.0)), rel=1e-15)
    assert O.silu(np.array([40.0]))[0] == pytest.approx(40.0, rel=1e-15)
    assert abs(O.silu(np.array([-40.0]))[0]) < 1e-15


def probe_layer(E=3, d=6, I=4, S=0):
    """Experts with one nonzero weight per matrix, at distinct positions.

    Expert e: W_gate[e][ng, cg] = a, W_up[e][ng, cu] = b, W_down[e][m, ng] = c,
    so FFN_e(x) = c * silu(a x[cg]) * (b x[cu]) in output m and 0 elsewhere.
    Shapes are [I, d], [I, d], [d, I] with d != I, so a swapped index or a
    transposed matrix moves or drops the value.
    """
    G = E + S
    wg = np.zeros((G, I, d))
    wu = np.zeros((G, I, d))
    wd = np.zeros((G, d, I))
    spec = []
    for e in range(G):
        ng, cg, cu, m = (e + 1) % I, (2 * e + 1) % d, (3 * e + 4) % d, (5 * e + 2) % d
        a, b, c = 0.7 + 0.1 * e, -1.3 + 0.2 * e, 0.9 - 0.3 * e
        wg[e, ng, cg], wu[e, ng, cu], wd[e, m, ng] = a, b, c
        spec.append((ng, cg, cu, m, a, b, c))
    return O.Experts(wg, wu, wd), spec


def probe_output(spec, x_t, d):
    ng, cg, cu, m, a, b, c = spec
    y = np.zeros(d)
    y[m] = c * silu_scalar(a * x_t[cg]) * (b * x_t[cu])
    return y


def test_layer_probe_experts_closed_form():
    E, d, k = 3, 6, 2
    ex, spec = probe_layer(E=E, d=d)
    x = np.array([[1.5, -0.5, 2.0, 0.25, -1.25, 0.75],
                  [-2.0, 1.0, -0.5, 3.0, 0.5, -1.0]])
    ids = np.array([[2, 0], [1, 2]])
    w = np.array([[0.6, 0.4], [0.25, 0.75]])
    y = O.moe_layer(x, ex, ids, w, n_shared=0, n_experts=E)
    for t in range(2):
        ref = sum(w[t, j] * probe_output(spec[ids[t, j]], x[t], d) for j in range(k))
        np.testing.assert_allclose(y[t], ref, rtol=1e-15, atol=0)


def test_layer_probe_shared_experts_weight_one_after_routed():
    E, S, d = 2, 2, 6
    ex, spec = probe_layer(E=E, S=S, d=d)
    x = np.array([[0.3, -1.0, 2.5, -0.75, 1.25, 0.5]])
    ids = np.array([[1]])
    w = np.array([[0.4]])
    res = np.array([[10.0, 20.0, 30.0, 40.0, 50.0, 60.0]])
    y = O.moe_layer(x, ex, ids, w, n_shared=S, n_experts=E, residual=res)
    ref = 0.4 * probe_output(spec[1], x[0], d) + probe_output(spec[2], x[0], d) \
        + probe_output(spec[3], x[0], d) + res[0]
    np.testing.assert_allclose(y[0], ref, rtol=1e-15)


def random_experts(G, d, I, seed, scale=0.3):
    g = rng(seed)
    return O.Experts(g.standard_normal((G, I, d)) * scale, g.standard_normal((G, I, d)) * scale,
                     g.standard_normal((G, d, I)) * scale)


def test_layer_single_expert_is_dense_swiglu():
    # E = 1, k = 1: the weight is 1 (renormalised or not) and the layer is one SwiGLU FFN
    d, I, T = 5, 7, 4
    ex = random_experts(1, d, I, 7)
    x = rng(8).standard_normal((T, d))
    logits = rng(9).standard_normal((T, 1))
    for ren in (False, True):
        ids, w = O.route(logits, 1, ren)
        np.testing.assert_array_equal(w, 1.0)
        y = O.moe_layer(x, ex, ids, w, 0, 1)
        wg, wu, wd = ex.get(0)
        for t in range(T):
            g_ = [sum(wg[n, c] * x[t, c] for c in range(d)) for n in range(I)]
            u_ = [sum(wu[n, c] * x[t, c] for c in range(d)) for n in range(I)]
            h_ = [silu_scalar(g_[n]) * u_[n] for n in range(I)]
            o_ = [sum(wd[m, n] * h_[n] for n in range(I)) for m in range(d)]
            np.testing.assert_allclose(y[t], o_, rtol=1e-12)


def test_layer_zero_input_gives_residual():
    E, d, I, T = 4, 6, 5, 3
    ex = random_experts(E + 1, d, I, 10)
    ids = np.array([[0, 3], [1, 2], [3, 1]])
    w = np.full((T, 2), 0.5)
    res = rng(11).standard_normal((T, d))
    y = O.moe_layer(np.zeros((T, d)), ex, ids, w, 1, E, residual=res)
    np.testing.assert_array_equal(y, res)


def test_layer_power_of_two_scaling_is_exact():
    E, d, I, T, S = 4, 6, 5, 3, 1
    g = rng(12)
    wg, wu, wd = g.standard_normal((E + S, I, d)), g.standard_normal((E + S, I, d)), g.standard_normal((E + S, d, I))
    x = g.standard_normal((T, d))
    ids = np.array([[0, 3], [1, 2], [3, 1]])
    w = g.random((T, 2))
    y1 = O.moe_layer(x, O.Experts(wg, wu, wd), ids, w, S, E)
    y2 = O.moe_layer(x, O.Experts(wg, wu, 2 * wd), ids, w, S, E)
    y3 = O.moe_layer(x, O.Experts(wg, 4 * wu, wd), ids, w, S, E)
    np.testing.assert_array_equal(y2, 2 * y1)
    np.testing.assert_array_equal(y3, 4 * y1)


def test_shared_experts_equal_one_wider_expert():
    # two shared SwiGLUs of width I equal one SwiGLU of width 2I (gate/up rows and
    # down columns concatenated)
    d, I, T = 6, 4, 3
    g = rng(13)
    wg, wu, wd = g.standard_normal((2, I, d)), g.standard_normal((2, I, d)), g.standard_normal((2, d, I))
    x = g.standard_normal((T, d))
    none_ids = np.zeros((T, 0), dtype=np.int64)
    none_w = np.zeros((T, 0))
    y2 = O.moe_layer(x, O.Experts(wg, wu, wd), none_ids, none_w, n_shared=2, n_experts=0)
    wide = O.Experts(np.concatenate([wg[0], wg[1]])[None], np.concatenate([wu[0], wu[1]])[None],
                     np.concatenate([wd[0], wd[1]], axis=1)[None])
    y1 = O.moe_layer(x, wide, none_ids, none_w, n_shared=1, n_experts=0)
    np.testing.assert_allclose(y2, y1, rtol=1e-13)


def test_slot_loop_equals_dense_masked_gates():
    E, d, I, T, k, S = 8, 16, 12, 20, 3, 2
    ex = random_experts(E + S, d, I, 14)
    g = rng(15)
    x = g.standard_normal((T, d))
    logits = g.standard_normal((T, E))
    ids, w = O.route(logits, k, True)
    res = g.standard_normal((T, d))
    y_loop = O.moe_layer(x, ex, ids, w, S, E, residual=res)
    y_dense = O.moe_layer_dense(x, ex, ids, w, S, E, residual=res)
    np.testing.assert_allclose(y_loop, y_dense, rtol=1e-12, atol=1e-13)


def test_identical_experts_renormalised_output_independent_of_routing():
    E, d, I, T, k = 6, 8, 5, 7, 3
    one = random_experts(1, d, I, 16)
    wg, wu, wd = one.get(0)
    ex = O.Experts(np.repeat(wg[None], E, 0), np.repeat(wu[None], E, 0), np.repeat(wd[None], E, 0))
    x = rng(17).standard_normal((T, d))
    outs = []
    for s in range(3):
        ids, w = O.route(rng(100 + s).standard_normal((T, E)), k, True)
        outs.append(O.moe_layer(x, ex, ids, w, 0, E))
    ref = O.moe_layer(x, one, np.zeros((T, 1), dtype=np.int64), np.ones((T, 1)), 0, 1)
    for y in outs:
        np.testing.assert_allclose(y, ref, rtol=1e-13)


def test_sorted_rows_and_combine_reassemble_the_layer():
    E, d, I, T, k, S = 5, 8, 6, 9, 2, 1
    ex = random_experts(E + S, d, I, 18)
    g = rng(19)
    x = g.standard_normal((T, d))
    ids, w = O.route(g.standard_normal((T, E)), k, False)
    counts, offsets, perm, inv = O.permute(ids, E)
    h, rows = O.sorted_rows(x, ex, ids, perm, S, E)
    assert rows.shape == (T * k + S * T, d) and h.shape == (T * k + S * T, I)
    y = O.combine(rows, inv, w, S)
    np.testing.assert_allclose(y, O.moe_layer(x, ex, ids, w, S, E), rtol=1e-13)
    # the rows of expert e are exactly the tokens routed to e, in ascending token order
    for e in range(E):
        toks = perm[offsets[e]:offsets[e + 1]] // k
        for r, t in zip(range(offsets[e], offsets[e + 1]), toks):
            o, _ = O.expert_ffn(x[t], *ex.get(e))
            np.testing.assert_array_equal(rows[r], o)


def test_int8_dequantisation_scales_output_channels():
    q = np.zeros((1, 3, 4), dtype=np.int8)
    q[0, 0, 1] = 127
    q[0, 2, 3] = -5
    s = np.array([[0.5, 2.0, 0.25]], dtype=np.float32)
    w = O.dequantize(q, s)
    ref = np.zeros((1, 3, 4))
    ref[0, 0, 1] = 63.5
    ref[0, 2, 3] = -1.25
    np.testing.assert_array_equal(w, ref)


# --------------------------------------------------------------------------
# stacked workload glue
# --------------------------------------------------------------------------
@pytest.mark.parametrize("c", [0.01, 1.0, 3.0, 100.0])
def test_rmsnorm_constant_input_closed_form(c):
    eps = 1e-5
    y = O.rmsnorm(np.full((2, 16), c), eps)
    np.testing.assert_allclose(y, 1.0 / math.sqrt(1.0 + eps / (c * c)), rtol=1e-14)


def test_rmsnorm_hand_example():
    y = O.rmsnorm(np.array([[3.0, -4.0]]), 0.0)
    # mean square = (9 + 16) / 2 = 12.5
    np.testing.assert_allclose(y, [[3 / math.sqrt(12.5), -4 / math.sqrt(12.5)]], rtol=1e-15)


def test_round_to_bf16_ties_and_pattern():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1
    assert O.round_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to even -> 1 + 2^-6
    assert O.round_to_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert O.round_to_bf16(np.array([1.0 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1.0 + 2.0 ** -7
    assert O.round_to_bf16(np.array([-3.0]))[0] == -3.0
    assert O.round_to_bf16(np.array([0.0]))[0] == 0.0
    v = O.round_to_bf16(np.random.default_rng(0).standard_normal(1000))
    # every result has at most 8 significant bits
    m, _ = np.frexp(v)
    assert np.all(m * 256 == np.rint(m * 256))


def test_stack_layer_input_is_the_rounded_norm():
    # [3, -4] at eps = 0 normalises to 3/sqrt(12.5) = 0.84853..., -1.13137...: neither is a
    # bf16 value, and their nearest bf16 values are 0.84765625 (217/256) and -1.1328125 (-145/128)
    y = O.stack_layer_input(np.array([[3.0, -4.0]]), 0.0)
    assert y.tolist() == [[217 / 256, -145 / 128]]
    # a constant row normalises to exactly +-1 at eps = 0, which bf16 holds
    assert O.stack_layer_input(np.full((1, 8), -2.5), 0.0).tolist() == [[-1.0] * 8]
    # every output has at most 8 significant bits and lies within half a bf16 ulp of the norm
    h = np.random.default_rng(3).standard_normal((4, 64))
    y = O.stack_layer_input(h, 1e-5)
    m, _ = np.frexp(y)
    assert np.all(m * 256 == np.rint(m * 256))
    ref = h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + 1e-5)
    assert np.all(np.abs(y - ref) <= np.abs(ref) * 2.0 ** -8 * (1 + 1e-12))


def test_full_route_is_router_then_topk():
    # unit router rows pick columns (2, 0, 3, 1) of x, a bias adds (0, 0, 10, 0): the logits are
    # x[:, [2, 0, 3, 1]] + bias, and the top-2 is chosen from them
    x = np.array([[0.5, 1.5, -1.0, 2.0, 9.0],
                  [3.0, 0.0, 1.0, 0.25, -9.0]])
    w_r = np.zeros((4, 5))
    for e, c in enumerate((2, 0, 3, 1)):
        w_r[e, c] = 1.0
    bias = np.array([0.0, 0.0, 10.0, 0.0])
    logits, ids, w = O.full_route(x, w_r, bias, 2, True)
    np.testing.assert_array_equal(logits, [[-1.0, 0.5, 12.0, 1.5], [1.0, 3.0, 10.25, 0.0]])
    assert ids.tolist() == [[2, 3], [2, 1]]
    # renormalised over the two chosen: e^l / (e^l + e^l')
    np.testing.assert_allclose(w[0], [1 / (1 + math.exp(1.5 - 12.0)), 1 / (1 + math.exp(12.0 - 1.5))], rtol=1e-14)
    np.testing.assert_allclose(w[1], [1 / (1 + math.exp(3.0 - 10.25)), 1 / (1 + math.exp(10.25 - 3.0))], rtol=1e-14)


# --------------------------------------------------------------------------
# option: capacity-factor dropping
# --------------------------------------------------------------------------
@pytest.mark.parametrize("cf,T,k,E,C", [
    (1.0, 2048, 8, 64, 256),   # exactly T*k/E
    (2.0, 2048, 8, 64, 512),
    (2.0, 16, 2, 8, 8),
    (1.25, 10, 3, 4, 10),      # 9.375 rounds up
    (1.0, 3, 1, 2, 2),         # 1.5 rounds up
    (0.1, 1, 1, 64, 1),        # at least one row
    (0.0, 100, 8, 64, 0),      # 0: no limit
    (-1.0, 100, 8, 64, 0),
])
def test_capacity_closed_form(cf, T, k, E, C):
    assert O.capacity(cf, T, k, E) == C


def test_kept_slots_hand_example():
    # flat order: (t0: e0 e1) (t1: e0 e2) (t2: e0 e1) (t3: e1 e0), two rows per expert
    ids = np.array([[0, 1], [0, 2], [0, 1], [1, 0]])
    keep = O.kept_slots(ids, 3, 2)
    expect = np.array([[True, True], [True, True], [False, True], [False, False]])
    np.testing.assert_array_equal(keep, expect)
    # no limit, or a limit no expert reaches, keeps everything
    assert O.kept_slots(ids, 3, 0).all() and O.kept_slots(ids, 3, 4).all()


@pytest.mark.parametrize("T,E,k,cap", [(50, 8, 2, 7), (200, 16, 4, 30), (64, 4, 1, 1)])
def test_kept_slots_invariants(T, E, k, cap):
    g = rng(T + E)
    p = 1.0 / np.arange(1, E + 1) ** 1.5
    ids = np.stack([g.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(T)])
    keep = O.kept_slots(ids, E, cap)
    counts = np.bincount(ids.ravel(), minlength=E)
    kept = np.bincount(ids.ravel()[keep.ravel()], minlength=E)
    np.testing.assert_array_equal(kept, np.minimum(counts, cap))
    # every dropped pair comes after all kept pairs of its expert in flat order
    flat_ids, flat_keep = ids.ravel(), keep.ravel()
    for e in range(E):
        pos = np.nonzero(flat_ids == e)[0]
        assert flat_keep[pos].tolist() == [True] * min(len(pos), cap) + [False] * max(0, len(pos) - cap)


def test_capacity_drops_are_the_tail_of_each_sorted_segment():
    g = rng(41)
    T, E, k, cap = 120, 6, 2, 25
    ids = np.stack([g.choice(E, size=k, replace=False, p=[0.5, 0.2, 0.1, 0.1, 0.05, 0.05])
                    for _ in range(T)])
    counts, offsets, perm, inv = O.permute_with_capacity(ids, E, cap)
    c0, o0, p0, i0 = O.permute(ids, E)
    np.testing.assert_array_equal(counts, c0)
    np.testing.assert_array_equal(perm, p0)
    flat = ids.ravel()
    for f in range(T * k):
        e = flat[f]
        assert (inv[f] >= 0) == (i0[f] - o0[e] < cap)
        if inv[f] >= 0:
            assert inv[f] == i0[f]
    assert (inv < 0).sum() == np.maximum(counts - cap, 0).sum()


def test_capacity_layer_equals_dense_masked_gates_and_combine():
    E, d, I, T, k, S = 6, 12, 10, 30, 2, 1
    ex = random_experts(E + S, d, I, 42)
    g = rng(43)
    x = g.standard_normal((T, d))
    logits = g.standard_normal((T, E)) + np.array([2.0, 1.0, 0, 0, 0, 0])
    ids, w = O.route(logits, k, True)
    cap = O.capacity(0.75, T, k, E)
    keep = O.kept_slots(ids, E, cap)
    assert 0 < (~keep).sum() < keep.size
    y = O.moe_layer(x, ex, ids, w, S, E, keep=keep)
    # dropped slots behave as gates of zero in the all-experts reference
    y_dense = O.moe_layer_dense(x, ex, ids, w * keep, S, E)
    np.testing.assert_allclose(y, y_dense, rtol=1e-12, atol=1e-13)
    # the sorted rows of the kept pairs, combined, give the same layer
    _, _, perm, inv = O.permute_with_capacity(ids, E, cap)
    _, rows = O.sorted_rows(x, ex, ids, perm, S, E)
    np.testing.assert_allclose(O.combine(rows, inv, w, S), y, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# gate weights of a choice made elsewhere (the weights every end-to-end
# comparison feeds the oracle when the GPU's routing is taken as input)
# --------------------------------------------------------------------------
def test_gate_weights_for_equals_route_on_its_own_choice():
    g = rng(51)
    logits = g.standard_normal((40, 64)) * 1.5
    for ren in (False, True):
        ids, w = O.route(logits, 8, ren)
        np.testing.assert_array_equal(O.gate_weights_for(logits, ids, ren), w)


@pytest.mark.parametrize("E", [8, 64])
def test_gate_weights_for_closed_form_on_a_chosen_set(E):
    # logits (L, 0, ..., 0): p_0 = e^L / (e^L + E - 1), every other p_e = 1 / (e^L + E - 1)
    L = 1.75
    logits = np.zeros((3, E))
    logits[:, 0] = L
    eL = math.exp(L)
    den = eL + E - 1
    # token 0: the top-1 expert plus a non-top choice; token 1: the same pair in the other
    # slot order; token 2: two experts that are not the top choice
    ids = np.array([[0, 3], [3, 0], [3, 5]])
    w = O.gate_weights_for(logits, ids, renormalize=False)
    np.testing.assert_allclose(w, [[eL / den, 1 / den], [1 / den, eL / den], [1 / den, 1 / den]],
                               rtol=1e-15)
    wr = O.gate_weights_for(logits, ids, renormalize=True)
    np.testing.assert_allclose(wr, [[eL / (eL + 1), 1 / (eL + 1)], [1 / (eL + 1), eL / (eL + 1)],
                                    [0.5, 0.5]], rtol=1e-15)


def test_gate_weights_for_rows_are_per_token():
    # two tokens with different logits: each row of weights comes from its own token's softmax
    logits = np.array([[2.0, 0.0, 0.0, 0.0], [0.0, 0.0, 0.0, -1.0]])
    ids = np.array([[0, 1], [3, 2]])
    w = O.gate_weights_for(logits, ids, renormalize=False)
    d0 = math.exp(2.0) + 3
    d1 = 3 + math.exp(-1.0)
    np.testing.assert_allclose(w, [[math.exp(2.0) / d0, 1 / d0], [math.exp(-1.0) / d1, 1 / d1]],
                               rtol=1e-15)


# --------------------------------------------------------------------------
# int8 experts: which per-channel scale goes with which matrix
# --------------------------------------------------------------------------
def test_int8_experts_pair_each_matrix_with_its_own_scales():
    # one nonzero int8 weight per matrix at distinct positions, and scales that differ per
    # matrix and per channel, so that a scale taken from the wrong matrix or channel moves
    # the value: FFN(x) = sd[m] qd * silu(sg[n] qg x[cg]) * (su[n] qu x[cu]) in output m
    E, d, I = 2, 6, 4
    qg = np.zeros((E, I, d), dtype=np.int8)
    qu = np.zeros((E, I, d), dtype=np.int8)
    qd = np.zeros((E, d, I), dtype=np.int8)
    sg = np.zeros((E, I), dtype=np.float32)
    su = np.zeros((E, I), dtype=np.float32)
    sd = np.zeros((E, d), dtype=np.float32)
    for e in range(E):
        sg[e] = [1.0, 0.5, 0.25, 0.125][e:] + [3.0] * e
        su[e] = 2.0 * (e + 1) + np.arange(I)
        sd[e] = 4.0 + 0.5 * np.arange(d) + 8.0 * e
    spec = []
    for e in range(E):
        n, cg, cu, m = (e + 1) % I, (2 * e + 1) % d, (3 * e + 4) % d, (5 * e + 2) % d
        qg[e, n, cg], qu[e, n, cu], qd[e, m, n] = 7 - e, -3 - e, 5 + 2 * e
        spec.append((n, cg, cu, m))
    ex = O.Experts(qg, qu, qd, sg, su, sd)
    x = np.array([0.5, -1.0, 1.5, -0.25, 0.75, 2.0])
    for e in range(E):
        n, cg, cu, m = spec[e]
        wg, wu, wd = ex.get(e)
        # each dequantised matrix holds exactly one value: its q times its own channel scale
        assert wg[n, cg] == float(qg[e, n, cg]) * float(sg[e, n]) and np.count_nonzero(wg) == 1
        assert wu[n, cu] == float(qu[e, n, cu]) * float(su[e, n]) and np.count_nonzero(wu) == 1
        assert wd[m, n] == float(qd[e, m, n]) * float(sd[e, m]) and np.count_nonzero(wd) == 1
        a = float(qg[e, n, cg]) * float(sg[e, n]) * x[cg]
        b = float(qu[e, n, cu]) * float(su[e, n]) * x[cu]
        ref = np.zeros(d)
        ref[m] = float(qd[e, m, n]) * float(sd[e, m]) * silu_scalar(a) * b
        y = O.moe_layer(x[None], ex, np.array([[e]]), np.array([[1.0]]), n_shared=0, n_experts=E)
        np.testing.assert_allclose(y[0], ref, rtol=1e-15, atol=0)


def test_int8_experts_of_the_quantiser_reproduce_dequantised_float_experts():
    # an int8 layer equals the same layer given as the float64 arrays q * scale
    import moe_synth as S
    g = rng(52)
    G, d, I = 3, 32, 16
    w = (g.standard_normal((3, G, I, d)) * 0.02).astype(np.float32)
    wd = (g.standard_normal((G, d, I)) * 0.02).astype(np.float32)
    (qg, sg), (qu, su), (qd, sd) = S.quantize_int8_rows(w[0]), S.quantize_int8_rows(w[1]), S.quantize_int8_rows(wd)
    ex8 = O.Experts(qg, qu, qd, sg, su, sd)
    exf = O.Experts(qg * sg[..., None].astype(np.float64), qu * su[..., None].astype(np.float64),
                    qd * sd[..., None].astype(np.float64))
    x = g.standard_normal((5, d))
    ids = np.array([[0, 2], [1, 0], [2, 1], [0, 1], [2, 0]])
    wts = g.random((5, 2))
    np.testing.assert_array_equal(O.moe_layer(x, ex8, ids, wts, 0, G),
                                  O.moe_layer(x, exf, ids, wts, 0, G))


# --------------------------------------------------------------------------
# token and row subsets (every sampled comparison uses them)
# --------------------------------------------------------------------------
def test_moe_layer_token_subset_equals_rows_of_the_full_layer():
    E, d, I, T, k, S = 6, 10, 7, 12, 2, 1
    ex = random_experts(E + S, d, I, 53)
    g = rng(54)
    x = g.standard_normal((T, d))
    ids, w = O.route(g.standard_normal((T, E)), k, True)
    res = g.standard_normal((T, d))
    keep = O.kept_slots(ids, E, 3)
    assert not keep.all()
    full = O.moe_layer(x, ex, ids, w, S, E, residual=res, keep=keep)
    for sub in ([9, 2, 7], [11, 0], [5], [3, 3, 10, 1]):  # unsorted, non-contiguous, repeated
        part = O.moe_layer(x, ex, ids, w, S, E, residual=res, tokens=sub, keep=keep)
        np.testing.assert_array_equal(part, full[sub])


def test_sorted_rows_row_subset_equals_rows_of_the_full_call():
    E, d, I, T, k, S = 5, 8, 6, 9, 2, 2
    ex = random_experts(E + S, d, I, 55)
    g = rng(56)
    x = g.standard_normal((T, d))
    ids, _ = O.route(g.standard_normal((T, E)), k, False)
    _, _, perm, _ = O.permute(ids, E)
    h, rows = O.sorted_rows(x, ex, ids, perm, S, E)
    sub = [T * k + T + 4, 3, 17, 0, T * k + 1]  # shared rows of both experts and routed rows
    hs, rs = O.sorted_rows(x, ex, ids, perm, S, E, rows=sub)
    np.testing.assert_array_equal(hs, h[sub])
    np.testing.assert_array_equal(rs, rows[sub])
