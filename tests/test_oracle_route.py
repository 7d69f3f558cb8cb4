"""Pins of the oracle's Route and Dispatch stages against things other than
itself: a hand-worked example, brute force over all k-subsets, invariants,
and the k = E special case (full softmax, checked against SciPy)."""
import itertools

import numpy as np
import pytest
import scipy.special

import oracle
from golden_io import read_sections



def _floats(rows):
    return np.array([[float(v) for v in r] for r in rows])


def test_worked_example():
    g = read_sections("route_worked_example.txt")
    z = _floats(g["keys"]).astype(np.float32)
    k = 2
    r = oracle.route(z, k, oracle.SOFTMAX, True)
    np.testing.assert_array_equal(r["topk_idx"], _floats(g["topk_idx"]).astype(np.int32))
    np.testing.assert_allclose(r["topk_w"], _floats(g["topk_w_softmax_renorm"]), rtol=0, atol=1e-15)
    np.testing.assert_array_equal(r["counts"], _floats(g["counts"]).ravel())
    np.testing.assert_array_equal(r["offsets"], _floats(g["offsets"]).ravel())
    np.testing.assert_array_equal(r["src_token"], _floats(g["src_token"]).ravel())
    np.testing.assert_array_equal(r["dst_row"], _floats(g["dst_row"]).astype(np.int32))
    rs = oracle.route(z, k, oracle.SIGMOID, True)
    np.testing.assert_array_equal(rs["topk_idx"], r["topk_idx"])
    np.testing.assert_allclose(rs["topk_w"], _floats(g["topk_w_sigmoid_renorm"]), rtol=0, atol=1e-15)


def _brute_topk(zrow, k):
    """The unique k-subset S with: every chosen key > every unchosen key, or
    equal with a lower index.  Found by trying all subsets."""
    E = len(zrow)
    hits = []
    for S in itertools.combinations(range(E), k):
        ok = all((zrow[c] > zrow[u]) or (zrow[c] == zrow[u] and c < u)
                 for c in S for u in range(E) if u not in S)
        if ok:
            hits.append(S)
    assert len(hits) == 1
    S = hits[0]
    return sorted(S, key=lambda e: (-zrow[e], e))


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("E,k", [(4, 2), (6, 3), (8, 1), (5, 5)])
def test_topk_brute_force(seed, E, k):
    rng = np.random.default_rng(seed)
    T = 40
    # coarse values so that many ties occur
    z = (rng.integers(-3, 4, size=(T, E)) * 0.5).astype(np.float32)
    idx = oracle.select_topk(z, k)
    for t in range(T):
        assert list(idx[t]) == _brute_topk([float(v) for v in z[t]], k)


def test_all_equal_keys_pick_lowest_indices():
    z = np.full((3, 8), 0.25, dtype=np.float32)
    idx = oracle.select_topk(z, 3)
    np.testing.assert_array_equal(idx, np.tile(np.arange(3), (3, 1)))


@pytest.mark.parametrize("score", [oracle.SOFTMAX, oracle.SIGMOID])
@pytest.mark.parametrize("renorm", [True, False])
def test_dispatch_invariants(score, renorm):
    rng = np.random.default_rng(7)
    T, E, k = 257, 16, 4
    z = rng.standard_normal((T, E)).astype(np.float32)
    r = oracle.route(z, k, score, renorm)
    idx, dst, src = r["topk_idx"], r["dst_row"], r["src_token"]
    assert r["counts"].sum() == T * k
    assert np.all(np.diff(r["offsets"]) >= 0) and r["offsets"][-1] == T * k
    # each token's k experts are distinct
    assert all(len(set(row)) == k for row in idx)
    # src_token and dst_row are mutually inverse bijections
    assert sorted(dst.ravel()) == list(range(T * k))
    for t in range(T):
        for j in range(k):
            assert src[dst[t, j]] == t
            e = idx[t, j]
            assert r["offsets"][e] <= dst[t, j] < r["offsets"][e + 1]
    # ascending tokens inside every segment
    for e in range(E):
        seg = src[r["offsets"][e]:r["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)
    # renormalised weights sum to one
    if renorm:
        np.testing.assert_allclose(r["topk_w"].sum(1), 1.0, rtol=1e-14)


def test_k_equals_E_is_full_softmax():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((50, 6)).astype(np.float32)
    r = oracle.route(z, 6, oracle.SOFTMAX, True)
    full = scipy.special.softmax(z.astype(np.float64), axis=1)
    np.testing.assert_allclose(r["topk_w"], np.take_along_axis(full, r["topk_idx"].astype(int), 1),
                               rtol=1e-13)
    r2 = oracle.route(z, 2, oracle.SOFTMAX, False)
    np.testing.assert_allclose(r2["topk_w"], np.take_along_axis(full, r2["topk_idx"].astype(int), 1),
                               rtol=1e-13)


def test_sigmoid_no_renorm_is_scipy_expit():
    rng = np.random.default_rng(4)
    z = rng.standard_normal((20, 8)).astype(np.float32)
    r = oracle.route(z, 3, oracle.SIGMOID, False)
    np.testing.assert_allclose(r["topk_w"],
                               scipy.special.expit(np.take_along_axis(z, r["topk_idx"].astype(int), 1)
                                                   .astype(np.float64)), rtol=1e-14)


def test_router_logits_fp32_and_bias_add():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((9, 16)).astype(np.float32)
    w = rng.standard_normal((16, 4)).astype(np.float32)
    b = rng.standard_normal(4).astype(np.float32)
    l = oracle.router_logits(x, w, b)
    assert l.dtype == np.float32
    exact = x.astype(np.float64) @ w.astype(np.float64)
    # one rounding of the exact dot product, then one fp32 add
    np.testing.assert_array_equal(l, exact.astype(np.float32) + b)


@pytest.mark.parametrize("score", [oracle.SOFTMAX, oracle.SIGMOID])
@pytest.mark.parametrize("renorm", [True, False])
def test_route_bwd_finite_differences(score, renorm):
    """dz = J^T dw with J the Jacobian of the weights at fixed selection."""
    rng = np.random.default_rng(11)
    T, E, k = 6, 7, 3
    z = rng.standard_normal((T, E))
    idx = oracle.select_topk(z.astype(np.float32), k)
    dw = rng.standard_normal((T, k))
    w = oracle.gates(z, idx, score, renorm)
    dz = oracle.route_bwd(z, idx, w, dw, score, renorm)
    eps = 1e-6
    num = np.zeros_like(z)
    for t in range(T):
        for e in range(E):
            zp, zm = z.copy(), z.copy()
            zp[t, e] += eps
            zm[t, e] -= eps
            num[t, e] = ((oracle.gates(zp, idx, score, renorm) - oracle.gates(zm, idx, score, renorm))
                         * dw).sum() / (2 * eps)
    np.testing.assert_allclose(dz, num, rtol=0, atol=1e-8)


@pytest.mark.parametrize("score,renorm", [("softmax", True), ("softmax", False),
                                          ("sigmoid", True), ("sigmoid", False)])
def test_replaying_the_topk_selection_is_the_route(score, renorm):
    """Replaying the experts the top-k route chose reproduces that route: same
    weights, counts, offsets and permutation, and nothing was replaced."""
    rng = np.random.default_rng(11)
    z = rng.standard_normal((97, 13)).astype(np.float32)
    r = oracle.route(z, 3, score, renorm)
    rr = oracle.route_replay(z, r["topk_idx"], score, renorm)
    assert not rr["changed"]
    for key in ("topk_idx", "counts", "offsets", "dst_row", "src_token"):
        np.testing.assert_array_equal(rr[key], r[key])
    np.testing.assert_array_equal(rr["topk_w"], r["topk_w"])


def test_canonical_experts_rule_brute_force():
    """Invalid slots (outside [0, E) or repeating an earlier slot) get the
    smallest expert the token does not use; valid slots are untouched; the
    result is k distinct experts per token.  Checked against a direct
    enumeration of the rule on small random cases."""
    rng = np.random.default_rng(5)
    for _ in range(300):
        E = int(rng.integers(2, 7))
        k = int(rng.integers(1, E + 1))
        idx = rng.integers(-2, E + 2, size=(4, k))
        got, changed = oracle.canonical_experts(idx, E)
        any_bad = False
        for t in range(4):
            orig = list(idx[t])
            bad = [not (0 <= orig[j] < E) or orig[j] in orig[:j] for j in range(k)]
            any_bad |= any(bad)
            row = list(got[t])
            assert len(set(row)) == k and all(0 <= e < E for e in row)
            for j in range(k):
                if not bad[j]:
                    assert row[j] == orig[j]
                else:
                    others = {row[s] for s in range(k) if s != j}
                    assert row[j] == min(c for c in range(E) if c not in others)
        assert changed == any_bad


def test_balanced_assignment_is_exactly_balanced():
    """The forced assignment of the balanced workload: every expert gets
    exactly T*k/E pairs and each token's k experts are distinct."""
    from routing_grouped_gemm_router_amd import inputs
    for T, E, k in [(512, 16, 4), (8192, 256, 8), (96, 8, 8)]:
        idx = inputs.balanced_experts(T, E, k, seed=3).numpy()
        counts = np.bincount(idx.ravel(), minlength=E)
        assert (counts == T * k // E).all()
        assert all(len(set(row)) == k for row in idx)
        r = oracle.route_replay(np.zeros((T, E), np.float32), idx, "sigmoid", True)
        assert not r["changed"]
        assert (r["counts"] == T * k // E).all()


def test_capacity_keeps_the_lowest_tokens_of_each_expert():
    """Capacity-limited dropping: each expert keeps the pairs of its C lowest
    tokens; with C at least the largest count nothing is dropped (the
    dropless map); kept rows form a bijection with the kept pairs, in
    ascending token order inside each segment; dropped pairs have no row."""
    rng = np.random.default_rng(8)
    z = (rng.standard_normal((200, 6)) + np.array([2.0, 1.0, 0, 0, -1, -2])).astype(np.float32)
    r = oracle.route(z, 2, "softmax", True)
    full = oracle.apply_capacity(r, int(r["counts"].max()))
    for key in ("counts", "offsets", "dst_row", "src_token"):
        np.testing.assert_array_equal(full[key], r[key])
    for C in (0, 1, 7, 40):
        c = oracle.apply_capacity(r, C)
        np.testing.assert_array_equal(c["counts"], np.minimum(r["counts"], C))
        for e in range(6):
            toks = [t for t in range(200) for j in range(2) if r["topk_idx"][t, j] == e]
            kept = sorted(toks)[:C]
            seg = c["src_token"][c["offsets"][e]:c["offsets"][e + 1]]
            np.testing.assert_array_equal(seg, kept)
        kept_pairs = np.argwhere(c["dst_row"] >= 0)
        assert len(kept_pairs) == c["offsets"][-1]
        for t, j in kept_pairs:
            assert c["src_token"][c["dst_row"][t, j]] == t
        np.testing.assert_array_equal(c["topk_w"], r["topk_w"])
    assert oracle.capacity_of(1.0, 200, 2, 6) == 67


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_aux_loss_balanced_value_and_finite_differences(score):
    """At perfect balance (equal counts, equal probabilities) the loss is
    exactly coeff; its gradient matches central differences of the loss with
    the counts held fixed."""
    T, E, k, coeff = 40, 8, 2, 0.01
    L, dz = oracle.aux_loss(np.zeros((T, E), np.float32), np.full(E, T * k // E), k, score, coeff)
    assert abs(L - coeff) < 1e-15
    rng = np.random.default_rng(3)
    z = rng.standard_normal((T, E))
    counts = rng.multinomial(T * k, np.ones(E) / E)
    L, dz = oracle.aux_loss(z, counts, k, score, coeff)
    num = np.zeros_like(z)
    eps = 1e-6
    for pos in np.ndindex(z.shape):
        zp, zm = z.copy(), z.copy()
        zp[pos] += eps
        zm[pos] -= eps
        num[pos] = (oracle.aux_loss(zp, counts, k, score, coeff)[0] -
                    oracle.aux_loss(zm, counts, k, score, coeff)[0]) / (2 * eps)
    np.testing.assert_allclose(dz, num, rtol=0, atol=1e-10)


# ---- selection-only expert bias (auxiliary-loss-free balancing) ----------

def _sigmoid_sweep():
    rng = np.random.default_rng(0)
    return np.concatenate([np.linspace(-90, 90, 1_000_001), rng.uniform(-20, 20, 1_000_000),
                           rng.standard_normal(500_000)]).astype(np.float32)


def test_sigmoid_spec_against_the_exact_sigmoid():
    """Within 2 ulp of the correctly rounded sigmoid on |z| <= 87, inexact on
    under 30 % of a dense sweep, and non-decreasing.  (Measured: dropping the
    last Taylor term gives 3 ulp and 32 %, a wrong sign of the low part of
    ln 2 thousands of ulp.)"""
    z = _sigmoid_sweep()
    s = oracle.sigmoid_spec(z)
    assert s.dtype == np.float32
    ref = (1.0 / (1.0 + np.exp(-z.astype(np.float64)))).astype(np.float32)
    ulp = np.abs(s.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    inside = np.abs(z) <= 87
    assert ulp[inside].max() <= 2
    assert (ulp[inside] > 0).mean() < 0.30
    order = np.argsort(z, kind="stable")
    assert np.all(np.diff(s[order].astype(np.float64)) >= 0)


def test_sigmoid_spec_landmarks():
    s = oracle.sigmoid_spec(np.float32([0.0, -0.0, 17.0, 87.0, 1e30, -87.0, -88.0, -1e30]))
    assert s[0] == 0.5 and s[1] == 0.5
    assert s[2] == 1.0 and s[3] == 1.0 and s[4] == 1.0        # 1 + e^-17 rounds to 1
    assert s[5] == s[6] == s[7]                               # clamped at -87: e^87 finite
    assert np.isclose(float(s[5]), 1.0 / (1.0 + np.exp(87.0)), rtol=1e-6)
    assert float(s[5]) >= np.finfo(np.float32).tiny           # normal, never subnormal


def test_route_expert_bias_selection_and_unbiased_gates():
    rng = np.random.default_rng(3)
    T, E, k = 200, 12, 3
    z = rng.standard_normal((T, E)).astype(np.float32)
    b = np.zeros(E, np.float32)
    b[4], b[7] = 2.0, -2.0            # keys lie in (0, 1) before the bias
    r = oracle.route_expert_bias(z, b, k, renorm=True)
    assert (r["topk_idx"][:, 0] == 4).all()                  # forced into slot 0
    assert not (r["topk_idx"] == 7).any()                    # never chosen
    # the weights ignore the bias: the sigmoid of the chosen logits, renormalised
    ref = oracle.gates(z, r["topk_idx"], oracle.SIGMOID, True)
    np.testing.assert_allclose(r["topk_w"], ref, rtol=1e-6)
    np.testing.assert_allclose(oracle.route_expert_bias(z, b, k, renorm=False)["topk_w"],
                               oracle.gates(z, r["topk_idx"], oracle.SIGMOID, False), rtol=1e-6)
    # brute force: the k experts of largest key, ties to the lower index
    keys = oracle.selection_keys(z, b)
    for t in range(T):
        best = sorted(range(E), key=lambda e: (-float(keys[t, e]), e))[:k]
        assert list(r["topk_idx"][t]) == best
    # dispatch map consistent with the chosen experts
    assert r["counts"].sum() == T * k
    for t in range(T):
        for j in range(k):
            row = r["dst_row"][t, j]
            e = r["topk_idx"][t, j]
            assert r["offsets"][e] <= row < r["offsets"][e + 1] and r["src_token"][row] == t


def test_route_expert_bias_ties_on_equal_scores():
    """Scores that round to the same fp32 key tie: the lower index wins."""
    z = np.float32([[30.0, 40.0, 20.0, -3.0]])      # the first three saturate to 1.0
    r = oracle.route_expert_bias(z, np.zeros(4, np.float32), 2, renorm=False)
    assert list(r["topk_idx"][0]) == [0, 1]
    r = oracle.route_expert_bias(z, np.float32([0, 0, 1e-3, 0]), 2, renorm=False)
    assert list(r["topk_idx"][0]) == [2, 0]


def test_expert_bias_update_by_hand():
    b = oracle.expert_bias_update(np.zeros(4, np.float32), [5, 1, 2, 0], 0.25)
    np.testing.assert_array_equal(b, np.float32([-0.25, 0.25, 0.0, 0.25]))   # mean load 2
    b = oracle.expert_bias_update(np.float32([1.0, 0.0, -1.0]), [3, 0, 0], 0.5)
    np.testing.assert_array_equal(b, np.float32([0.5, 0.5, -0.5]))           # mean load 1
    b = oracle.expert_bias_update(np.float32([0.1]), [7], 1e-3)
    assert b[0] == np.float32(0.1)                                           # at the mean
    b = oracle.expert_bias_update(np.float32([1.0, 1.0]), [2, 1], 1e-8)
    assert b[0] == np.float32(1.0 - 1e-8) and b[1] == np.float32(1.0 + 1e-8)  # fp32 add


# ---- pad-to-max ------------------------------------------------------------

def test_pad_to_max_by_hand():
    """Experts 0 and 1, C = 2: expert 0 gets tokens 0, 2, 3 (keeps 0 and 2),
    expert 1 token 1; rows [0, 2 | 1, pad]."""
    z = np.float32([[1, 0], [0, 1], [1, 0], [1, 0]])
    r = oracle.pad_to_max(oracle.route(z, 1, oracle.SOFTMAX, True), 2)
    np.testing.assert_array_equal(r["offsets"], [0, 2, 4])
    np.testing.assert_array_equal(r["counts"], [2, 1])
    np.testing.assert_array_equal(r["dst_row"], [[0], [2], [1], [-1]])
    np.testing.assert_array_equal(r["src_token"], [0, 2, 1, -1])


@pytest.mark.parametrize("C", [1, 7, 40, 500])
def test_pad_to_max_is_capacity_in_a_static_layout(C):
    rng = np.random.default_rng(C)
    T, E, k = 300, 9, 3
    z = (rng.standard_normal((T, E)) + np.linspace(0, 2, E)).astype(np.float32)
    r = oracle.route(z, k, oracle.SOFTMAX, True)
    p = oracle.pad_to_max(r, C)
    cap = oracle.apply_capacity(r, C)
    np.testing.assert_array_equal(p["offsets"], np.arange(E + 1) * C)
    np.testing.assert_array_equal(p["counts"], np.minimum(r["counts"], C))
    # the same kept pairs; compacting the padded rows gives the capacity layout
    np.testing.assert_array_equal(p["dst_row"] >= 0, cap["dst_row"] >= 0)
    np.testing.assert_array_equal(p["src_token"][p["src_token"] >= 0], cap["src_token"])
    for t in range(T):
        for j in range(k):
            row = p["dst_row"][t, j]
            if row >= 0:
                e = r["topk_idx"][t, j]
                assert e * C <= row < e * C + p["counts"][e] and p["src_token"][row] == t
    assert (p["src_token"] < 0).sum() == E * C - p["counts"].sum()


def _hexrows(rows):
    return np.array([[float.fromhex(v) for v in r] for r in rows])


def test_router_logits_golden_hand_worked():
    """Hand-worked fixture (tests/golden/router_logits.txt): a dot product on
    an exact fp32 rounding tie, the bias added by one fp32 addition after
    that rounding, float64 accumulation rounded once, and the [d, E] layout
    of W_r.  Each case's expected key and choice differ from what the named
    mistakes produce (checked below on the same inputs)."""
    from golden_io import read_sections
    g = read_sections("router_logits.txt")
    # case A
    x = _hexrows(g["a_x"]).astype(np.float32)
    w = _hexrows(g["a_w"]).astype(np.float32)
    b = _hexrows(g["a_bias"]).astype(np.float32)[0]
    l0 = oracle.router_logits(x, w)
    z = oracle.router_logits(x, w, b)
    np.testing.assert_array_equal(l0, _hexrows(g["a_logits_nobias"]).astype(np.float32))
    np.testing.assert_array_equal(z, _hexrows(g["a_keys"]).astype(np.float32))
    assert oracle.select_topk(z, 1).tolist() == [[int(g["a_top1"][0][0])]]
    # the mistakes this case tells apart
    exact = x.astype(np.float64) @ w.astype(np.float64)
    bias_before_rounding = (exact + b).astype(np.float32)
    assert oracle.select_topk(bias_before_rounding, 1).tolist() == [[1]]
    assert oracle.select_topk(exact + b, 1).tolist() == [[1]]          # float64 keys
    # case B
    x = _hexrows(g["b_x"]).astype(np.float32)
    w = _hexrows(g["b_w"]).astype(np.float32)
    z = oracle.router_logits(x, w)
    np.testing.assert_array_equal(z, _hexrows(g["b_keys"]).astype(np.float32))
    assert oracle.select_topk(z, 2).tolist() == [[int(v) for v in g["b_top2"][0]]]
    f32_running = np.zeros((1, 3), np.float32)
    for i in range(3):
        f32_running = (f32_running + x[:, i:i + 1] * w[i]).astype(np.float32)
    assert f32_running[0, 0] == 1.0 and z[0, 0] != f32_running[0, 0]
    transposed = (x.astype(np.float64) @ w.T.astype(np.float64)).astype(np.float32)
    assert oracle.select_topk(transposed, 2).tolist() == [[1, 0]]
