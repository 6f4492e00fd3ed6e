"""Pins for the oracle: each test ties it to something other than itself.

Sources of truth used here: invariants and closed forms the Switch explainer
("Mixture of Experts (MoE) を1から解説 — Switch Transformerのルーティングと負荷分散",
ta-paperlens.web.app) states for eq. (1)-(4); brute-force enumeration on tiny
inputs; textbook/library routines (torch's bf16 conversion, math.exp, a dense
FFN written with torch ops); exact integer arithmetic; and central finite
differences of the oracle's own forward for every gradient.
"""
import math
import itertools

import numpy as np
import pytest
import torch

import oracle as O
from synth import CONFIGS, SMALL, LayerConfig, make_inputs


def f64(t):
    return O.f64(t)


def spec_of(cfg, mode=None):
    return O.Spec.of(cfg, mode)


def inputs64(cfg, seed=0):
    inp = make_inputs(cfg, seed=seed)
    return {k: f64(v) for k, v in inp.items()}


# ----------------------------------------------------------------- number formats

def test_bf16_round_matches_torch_on_fp32_patterns():
    # Library routine: torch's fp32 -> bf16 conversion (round to nearest even).
    rng = np.random.default_rng(0)
    hi = np.arange(0, 1 << 16, dtype=np.uint32)
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    pats = (hi[:, None] << 16 | lows[None, :]).ravel()
    pats = np.concatenate([pats, rng.integers(0, 1 << 32, 200_000, dtype=np.uint64).astype(np.uint32)])
    vals = pats.view(np.float32)
    vals = vals[np.isfinite(vals)]
    # drop values that overflow bf16 (torch gives inf, so do we, but keep the sweep finite)
    ref = torch.from_numpy(vals.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    ok = np.isfinite(ref)
    vals, ref = vals[ok], ref[ok]
    sub = np.linspace(0, len(vals) - 1, 60_000).astype(np.int64)
    got = np.array([O.round_bf16(float(v)) for v in vals[sub]])
    np.testing.assert_array_equal(got, ref[sub])


def test_exp_contract_within_2ulp_of_exp():
    xs = np.concatenate([np.linspace(-86, 86, 20001), np.linspace(-1, 1, 5001), [0.0, -0.0]])
    for x in xs.astype(np.float32):
        got = np.float32(O.exp_contract(float(x)))
        true = math.exp(float(x))
        ulp = np.spacing(np.float32(true))
        assert abs(float(got) - true) <= 2 * float(ulp), (x, got, true)
    assert O.exp_contract(0.0) == 1.0
    assert O.exp_contract(100.0) == math.inf
    assert O.exp_contract(-100.0) == 0.0


def test_sigmoid_contract_close_to_logistic():
    for x in np.linspace(-30, 30, 6001).astype(np.float32):
        s = O.sigmoid_contract(float(x))
        true = 1.0 / (1.0 + math.exp(-float(x)))
        assert abs(s - true) <= 4 * float(np.spacing(np.float32(true))) + 1e-45, (x, s, true)
    assert O.sigmoid_contract(0.0) == 0.5


def test_log1p_contract_within_3ulp_of_log1p():
    # rounding of 2 + u, the division and the final product add up to about 2.6 ulp
    us = np.concatenate([np.linspace(0, 1, 20001), np.geomspace(1e-30, 1e-3, 2001), [1.0, 0.5]])
    for u in us.astype(np.float32):
        got = O.log1p_contract(float(u))
        true = math.log1p(float(u))
        assert abs(got - true) <= 3 * float(np.spacing(np.float32(true))) + 1e-45, (u, got, true)
    assert O.log1p_contract(0.0) == 0.0


def _sqrt_softplus64(h):
    return math.sqrt(max(h, 0.0) + math.log1p(math.exp(-abs(h))))


def test_sqrt_softplus_contract_close_to_definition():
    for x in np.concatenate([np.linspace(-40, 40, 16001), np.linspace(-1, 1, 4001)]).astype(np.float32):
        s = O.sqrt_softplus_contract(float(x))
        true = _sqrt_softplus64(float(x))
        assert abs(s - true) <= 4 * float(np.spacing(np.float32(true))) + 1e-45, (x, s, true)
    # closed forms: sqrt(ln 2) at 0, sqrt(h) once e^-h is below fp32 resolution, 0 far left
    assert abs(O.sqrt_softplus_contract(0.0) - math.sqrt(math.log(2.0))) <= 2 * 2.0 ** -24
    assert O.sqrt_softplus_contract(100.0) == 10.0
    assert O.sqrt_softplus_contract(-100.0) == 0.0


@pytest.mark.parametrize("gate", ["sigmoid_bias", "sqrt_softplus_bias"])
def test_gate_derivative_from_gate_value(gate):
    # The backward sees only s = g(h); its derivative written in s must equal dg/dh,
    # checked against central differences of the plain double gate.
    g = (lambda h: 1.0 / (1.0 + math.exp(-h))) if gate == "sigmoid_bias" else _sqrt_softplus64
    gid = O.GATE_OF[gate]
    for h in np.linspace(-12, 12, 97):
        eps = 1e-4
        fd = (g(h + eps) - g(h - eps)) / (2 * eps)
        assert O.gate_deriv(gid, g(h)) == pytest.approx(fd, rel=1e-6, abs=1e-12), h
    assert O.gate_deriv(gid, 0.0) == 0.0


# ----------------------------------------------------------------- router logits

def test_logits_exact_on_integer_inputs():
    # Every product and partial sum is a small integer, so each fused multiply-add is
    # exact and the fp32 contract must return the exact integer dot product.
    rng = np.random.default_rng(1)
    x = rng.integers(-8, 9, (37, 50)).astype(np.float64)
    w = rng.integers(-8, 9, (6, 50)).astype(np.float64)
    off = rng.integers(-3, 4, 6).astype(np.float64)
    h = O.logits(O.MODE_F32, x, w, off)
    ref = x.astype(np.int64) @ w.astype(np.int64).T + off.astype(np.int64)
    np.testing.assert_array_equal(h, ref.astype(np.float64))


def test_logits_within_fp32_error_bound():
    rng = np.random.default_rng(2)
    d = 700
    x = rng.standard_normal((20, d)).astype(np.float32).astype(np.float64)
    w = (rng.standard_normal((9, d)) / math.sqrt(d)).astype(np.float32).astype(np.float64)
    h = O.logits(O.MODE_F32, x, w)
    exact = x @ w.T
    u = 2.0 ** -24
    gamma = d * u / (1 - d * u)
    bound = gamma * (np.abs(x) @ np.abs(w).T)
    assert np.all(np.abs(h - exact) <= bound)
    assert np.all(h == h.astype(np.float32))
    # the exact mode is the plain double dot product
    np.testing.assert_allclose(O.logits(O.MODE_EXACT, x, w), exact, rtol=1e-12, atol=1e-12)


def test_logits_order_is_sequential():
    # A case where the order of the fp32 sum matters: 1 + 2^-24 + 2^-24 - 1.
    # Ascending order with fused multiply-adds gives exactly 0: (1 + 2^-24) rounds to 1.
    x = np.array([[1.0, 2.0 ** -24, 2.0 ** -24, -1.0]])
    w = np.ones((1, 4))
    assert O.logits(O.MODE_F32, x, w)[0, 0] == 0.0
    # reversed order: (-1 + 2^-24) + 2^-24 + 1 = 2^-23 exactly
    assert O.logits(O.MODE_F32, x[:, ::-1].copy(), w)[0, 0] == 2.0 ** -23


# ----------------------------------------------------------------- gate + selection

def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(3)
    for E in (4, 64, 256):
        h = rng.standard_normal((50, E)).astype(np.float32).astype(np.float64) * 3
        probs, idx, w = O.gate_topk(O.MODE_F32, h, 2, O.GATE_SOFTMAX, False)
        assert np.all(np.abs(probs.sum(1) - 1.0) <= 4 * E * 2.0 ** -24)
        np.testing.assert_allclose(probs, torch.softmax(torch.from_numpy(h), 1).numpy(), rtol=2e-7)
        # top-1 gate without renormalisation is the largest probability
        np.testing.assert_array_equal(w[:, 0], probs.max(1))


def _brute_select(key, k):
    E = len(key)
    found = []
    for S in itertools.combinations(range(E), k):
        ok = all((key[i] > key[j]) or (key[i] == key[j] and i < j)
                 for i in S for j in range(E) if j not in S)
        if ok:
            found.append(set(S))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("E", [1, 2, 3, 4])
def test_selection_bruteforce_all_tie_patterns(E):
    vals = [-1.0, 0.0, 0.5, 1.0]
    rows = np.array(list(itertools.product(vals, repeat=E)), np.float64)
    for k in range(1, E + 1):
        for gate in (O.GATE_SOFTMAX, O.GATE_SIGMOID_BIAS, O.GATE_SQRT_SOFTPLUS_BIAS):
            probs, idx, w = O.gate_topk(O.MODE_F32, rows, k, gate, True,
                                        np.zeros(E) if gate else None)
            for t in range(rows.shape[0]):
                key = rows[t] if gate == O.GATE_SOFTMAX else probs[t]
                assert set(idx[t].tolist()) == _brute_select(list(key), k)
                # listed by key descending, ties by index ascending
                order = sorted(range(E), key=lambda e: (-key[e], e))[:k]
                assert idx[t].tolist() == order
                # renormalised weights sum to one
                assert abs(w[t].sum() - 1.0) < 1e-6


@pytest.mark.parametrize("gate", ["sigmoid_bias", "sqrt_softplus_bias"])
def test_gate_bias_only_selects(gate):
    rng = np.random.default_rng(4)
    h = rng.standard_normal((64, 16)).astype(np.float32).astype(np.float64)
    b = (rng.random(16) - 0.5).astype(np.float32).astype(np.float64)
    probs, idx, w = O.gate_topk(O.MODE_F32, h, 4, O.GATE_OF[gate], True, b)
    fn = O.sigmoid_contract if gate == "sigmoid_bias" else O.sqrt_softplus_contract
    for t in range(64):
        s = np.array([fn(float(v)) for v in h[t]], np.float64)
        np.testing.assert_array_equal(probs[t], s)
        key = (s.astype(np.float32) + b.astype(np.float32)).astype(np.float64)
        assert set(idx[t].tolist()) == _brute_select(list(key), 4)
        sel = s[idx[t]]
        np.testing.assert_allclose(w[t], sel / sel.sum(), rtol=1e-7)


# ----------------------------------------------------------------- selection-bias update

def test_bias_update_hand_example():
    # loads 3,1,2,2 -> mean 2: the busy expert's bias falls, the idle one's rises,
    # the two at the mean keep theirs bit for bit
    b = np.array([0.25, -0.125, 0.1, -0.3], np.float32).astype(np.float64)
    out = O.bias_update(np.array([3, 1, 2, 2]), 0.001, b)
    f = np.float32
    np.testing.assert_array_equal(out, [f(f(0.25) - f(0.001)), f(f(-0.125) + f(0.001)), f(0.1), f(-0.3)])


def test_bias_update_balanced_and_fractional_mean():
    b = np.linspace(-1, 1, 7).astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(O.bias_update(np.full(7, 5), 0.5, b), b)
    # mean 7/3: a load of 2 is below it, 3 above (an integer mean test would call both equal)
    out = O.bias_update(np.array([2, 2, 3]), 0.5, np.zeros(3))
    np.testing.assert_array_equal(out, [0.5, 0.5, -0.5])


def test_bias_update_balances_a_skewed_router():
    # Closed loop on a fixed batch: a sigmoid router with a strong per-expert skew
    # routes most tokens to a few experts; repeated sign steps on the selection bias
    # must even the loads out (a flipped sign or index makes them worse).
    rng = np.random.default_rng(11)
    T, E, k = 2048, 16, 2
    h = (rng.standard_normal((T, E)) + 2.0 * np.linspace(1, -1, E)).astype(np.float32).astype(np.float64)
    bias = np.zeros(E)

    def loads(bias):
        _, idx, _ = O.gate_topk(O.MODE_F32, h, k, O.GATE_SIGMOID_BIAS, True, bias)
        return np.bincount(idx.ravel(), minlength=E).astype(np.int32)

    c0 = loads(bias)
    mean = T * k / E
    assert c0.max() > 2.5 * mean
    for _ in range(400):
        bias = O.bias_update(loads(bias), 0.002, bias)
    c = loads(bias)
    assert c.max() < 1.2 * mean and c.min() > 0.8 * mean, c
    # the bias ends ordered against the skew: favoured experts are pushed down
    assert bias[0] < bias[-1]


def test_bias_quantile_hand_example():
    # T=3, E=2, k=1, zero bias: q = ceil(3/2) = 2. Expert 0 margins 0.8, 0.5, 0.1 (each
    # token's key minus its best rival), expert 1 the negatives; the bias moves to minus
    # the midpoint of the 2nd and 3rd largest margins
    f = np.float32
    s = np.array([[0.9, 0.1], [0.8, 0.3], [0.7, 0.6]], np.float32)
    out = O.bias_quantile(s.astype(np.float64), 1, np.zeros(2))
    m0 = [f(s[t, 0] - s[t, 1]) for t in range(3)]
    m1 = [f(s[t, 1] - s[t, 0]) for t in range(3)]
    a0, b0 = sorted(m0, reverse=True)[1:3]
    a1, b1 = sorted(m1, reverse=True)[1:3]
    np.testing.assert_array_equal(out, [f(0) - f(f(a0 + b0) * f(0.5)), f(0) - f(f(a1 + b1) * f(0.5))])
    assert O.qb_target(3, 2, 1) == 2 and O.qb_target(10, 4, 8) == 9 and O.qb_target(100, 64, 1) == 2
    # k = E: every expert takes every token, the bias stays; one token: no quantile
    np.testing.assert_array_equal(O.bias_quantile(s.astype(np.float64), 2, np.array([0.5, -0.25])), [0.5, -0.25])
    np.testing.assert_array_equal(O.bias_quantile(s[:1].astype(np.float64), 1, np.array([0.5, -0.25])),
                                  [0.5, -0.25])


def _skewed_sigmoid_router(T=1200, E=12, k=2, seed=5):
    rng = np.random.default_rng(seed)
    h = (rng.standard_normal((T, E)) + 1.5 * np.linspace(1, -1, E)).astype(np.float32).astype(np.float64)

    def route(b):
        p, idx, _ = O.gate_topk(O.MODE_F32, h, k, O.GATE_SIGMOID_BIAS, True, b)
        return p, np.bincount(idx.ravel(), minlength=E)
    return route


def test_bias_quantile_single_expert_reaches_target_exactly():
    # moving one expert's bias by its step, the others fixed, gives it exactly q tokens:
    # this fixes the margins (which cutoff, which sign) and the rank of the quantile
    T, E, k = 1200, 12, 2
    route = _skewed_sigmoid_router(T, E, k)
    b0 = np.zeros(E)
    p, c0 = route(b0)
    q = O.qb_target(T, E, k)
    bq = O.bias_quantile(p, k, b0)
    for j in range(E):
        b = b0.copy()
        b[j] = bq[j]
        assert route(b)[1][j] == q, j
    assert c0.max() > 3 * q


def test_bias_quantile_closed_loop_balances():
    T, E, k = 1200, 12, 2
    route = _skewed_sigmoid_router(T, E, k)
    q = O.qb_target(T, E, k)
    b = np.zeros(E)
    p, c = route(b)
    for _ in range(3):
        b = O.bias_quantile(p, k, b)
        p, c = route(b)
    assert np.all(np.abs(c - q) <= 0.05 * q), c


# ----------------------------------------------------------------- noisy top-k gating

def test_softplus_contract_close_to_definition():
    for x in np.concatenate([np.linspace(-40, 40, 16001), np.linspace(-1, 1, 4001)]).astype(np.float32):
        got = O.softplus_contract(float(x))
        true = max(float(x), 0.0) + math.log1p(math.exp(-abs(float(x))))
        assert abs(got - true) <= 3 * float(np.spacing(np.float32(true))) + 1e-45, (x, got, true)
    assert O.softplus_contract(100.0) == 100.0 and O.softplus_contract(-100.0) == 0.0


def _noisy_case(T=40, E=6, k=2, seed=0, noise_shift=0.0):
    rng = np.random.default_rng(seed)
    h2 = (rng.standard_normal((T, 2 * E)) * 1.5).astype(np.float32).astype(np.float64)
    h2[:, E:] += noise_shift
    eps = rng.standard_normal((T, E)).astype(np.float32).astype(np.float64)
    return h2, eps


def test_noisy_gate_without_noise_is_renormalised_softmax():
    h2, eps = _noisy_case()
    E = 6
    H = O.noisy_logits(O.MODE_F32, h2, np.zeros_like(eps))
    np.testing.assert_array_equal(H, h2[:, :E])
    # H = h + eps * softplus_c(n) with one fp32 multiply and one fp32 add
    H = O.noisy_logits(O.MODE_F32, h2, eps)
    f = np.float32
    for t in range(5):
        for e in range(E):
            sp = f(O.softplus_contract(float(h2[t, E + e])))
            assert H[t, e] == f(f(h2[t, e]) + f(f(eps[t, e]) * sp))


def _load_bruteforce(h2, eps, k, H):
    T, E = eps.shape
    load = np.zeros(E)
    for t in range(T):
        for e in range(E):
            rest = np.delete(H[t], e)
            rival = np.sort(rest)[::-1][k - 1]          # k-th largest with e left out
            sp = max(h2[t, E + e], 0) + math.log1p(math.exp(-abs(h2[t, E + e])))
            load[e] += 0.5 * math.erfc(-((h2[t, e] - rival) / sp) / math.sqrt(2))
    return load


@pytest.mark.parametrize("k", [1, 2, 5])
def test_noisy_load_rival_is_kth_largest_excluding(k):
    h2, eps = _noisy_case(T=30, E=6, seed=k)
    H = O.noisy_logits(O.MODE_F32, h2, eps)
    _, idx, w = O.gate_topk(O.MODE_F32, H, k, O.GATE_SOFTMAX, True)
    aux, imp, load = O.noisy_aux(O.MODE_F32, h2, eps, idx, w, 1.0)
    np.testing.assert_allclose(load, _load_bruteforce(h2, eps, k, H), rtol=1e-12, atol=1e-12)
    # importance = column sums of the gates; the losses are CV^2 (variance over mean^2)
    np.testing.assert_allclose(imp, np.bincount(idx.ravel(), weights=w.ravel(), minlength=6), rtol=1e-12)
    cv2 = lambda v: np.var(v) / np.mean(v) ** 2
    assert aux == pytest.approx(cv2(imp) + cv2(load), rel=1e-12)


def test_noisy_load_without_noise_scale_counts_assignments():
    # softplus(n) -> 0 makes each smoothed term a step: the load becomes the hard counts
    h2, eps = _noisy_case(T=200, E=8, k=2, seed=7, noise_shift=-80.0)
    H = O.noisy_logits(O.MODE_EXACT, h2, eps)
    _, idx, w = O.gate_topk(O.MODE_EXACT, H, 2, O.GATE_SOFTMAX, True)
    _, imp, load = O.noisy_aux(O.MODE_EXACT, h2, eps, idx, w, 1.0)
    np.testing.assert_array_equal(load, np.bincount(idx.ravel(), minlength=8).astype(np.float64))


def test_noisy_importance_loss_zero_when_balanced():
    # every token splits its weight evenly over the experts in turn: equal importance
    T, E, k = 8, 4, 2
    idx = np.array([[t % E, (t + 1) % E] for t in range(T)], np.int32)
    w = np.full((T, k), 0.5)
    h2, eps = _noisy_case(T=T, E=E, k=k)
    _, imp, _ = O.noisy_aux(O.MODE_EXACT, h2, eps, idx, w, 1.0)
    np.testing.assert_allclose(imp, np.full(E, 2.0))


# ----------------------------------------------------------------- expert-choice routing

def test_softmax_ec_contract():
    rng = np.random.default_rng(21)
    for E in (1, 3, 64, 257):
        h = (rng.standard_normal((40, E)) * 4).astype(np.float32).astype(np.float64)
        p = O.softmax_ec(O.MODE_F32, h)
        assert np.all(p == p.astype(np.float32))
        ref = torch.softmax(torch.from_numpy(h), 1).numpy()
        # error bound: the rounded difference h - m moves exp by up to |h - m| * 2^-24
        # relative, exp_c adds a few ulp, the sequential sum of E positive terms (E-1) ulp
        m = h.max(1, keepdims=True)
        bound = ref * (np.abs(h - m) + E + 4) * 2.0 ** -24 + 1e-45
        assert np.all(np.abs(p - ref) <= bound)
        assert np.all(np.abs(p.sum(1) - 1.0) <= 2 * E * 2.0 ** -24)
        # equal logits: every e_j = exp_c(0) = 1 and z = E exactly, so p = fl(1/E)
        np.testing.assert_array_equal(O.softmax_ec(O.MODE_F32, np.full((2, E), 0.75)),
                                      np.full((2, E), float(np.float32(1.0) / np.float32(E))))
    # one dominant logit: the others underflow to exactly 0
    h = np.array([[0.0, 100.0, -3.0]])
    np.testing.assert_array_equal(O.softmax_ec(O.MODE_F32, h), [[0.0, 1.0, 0.0]])


def _ec_brute_column(col, C):
    # the unique set S of size C with every member beating every non-member on
    # (probability desc, token index asc)
    return _brute_select(list(col), min(C, len(col)))


@pytest.mark.parametrize("T,E", [(3, 2), (4, 3), (5, 2)])
def test_expert_choice_bruteforce_tie_patterns(T, E):
    vals = [0.1, 0.25, 0.5]
    rng = np.random.default_rng(T * 10 + E)
    for C in (1, 2, T, T + 3):
        for _ in range(60):
            probs = rng.choice(vals, (T, E))
            slot, w, row_token, counts, offsets = O.expert_choice(probs, C)
            Cp = min(C, T)
            np.testing.assert_array_equal(counts, np.full(E, Cp))
            np.testing.assert_array_equal(offsets, np.arange(E + 1) * Cp)
            for e in range(E):
                chosen = set(np.nonzero(slot[:, e] >= 0)[0].tolist())
                assert chosen == _ec_brute_column(probs[:, e], C)
                rows = row_token[e * Cp:(e + 1) * Cp]
                assert rows.tolist() == sorted(chosen)          # seats in token order
                for r, t in enumerate(rows):
                    assert slot[t, e] == e * Cp + r and w[t, e] == probs[t, e]
            assert np.all(w[slot < 0] == 0)


def test_expert_choice_every_token_taken_is_dense_mixture():
    # C >= T: every expert takes every token, so y = x + sum_e p_e FFN_e(x)
    cfg = _tiny(5, 5, act="swiglu", renorm=False, cf=5.0, routing="expert_choice")  # C = T
    spec = spec_of(cfg, O.MODE_EXACT)
    inp = inputs64(cfg)
    fw = O.forward(spec, inp)
    assert fw["n_rows"] == 5 * cfg.T
    p = torch.softmax(torch.from_numpy(inp["x"] @ inp["w_router"].T), 1).numpy()
    ref = inp["x"].copy()
    for e in range(5):
        ref += p[:, e:e + 1] * _dense_ffn(inp["x"], inp["w1"][e], inp["w2"][e], spec.act)
    np.testing.assert_allclose(fw["y"], ref, rtol=1e-11, atol=1e-12)


def test_expert_choice_load_is_exactly_balanced():
    cfg = SMALL["gshard_top2"].replace(routing="expert_choice", k=8, renorm=False, alpha=0.0, cf=2.0)
    spec = spec_of(cfg)
    fw = O.forward(spec, inputs64(cfg))
    C = O.capacity(cfg.T, cfg.E, cfg.cf)
    np.testing.assert_array_equal(np.diff(fw["offsets"]), np.full(cfg.E, C))
    assert int((fw["slot"] >= 0).sum()) == cfg.E * C
    # tokens no expert took pass through unchanged
    none = np.all(fw["slot"] < 0, axis=1)
    np.testing.assert_array_equal(fw["y"][none], inputs64(cfg)["x"][none])


# ----------------------------------------------------------------- capacity + positions

def test_capacity_golden():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "capacity.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    for T, E, cf, C in rows:
        assert O.capacity(int(T), int(E), float(cf)) == int(C)
    assert O.capacity(100, 3, 0.0) == -1
    assert O.capacity(1000, 16, 1.25) == 79  # ceil(78.125)


def _brute_positions(idx, E, C):
    T, k = idx.shape
    pairs = [(t, r) for t in range(T) for r in range(k)]
    pos = {}
    for (t, r) in pairs:
        e = idx[t, r]
        pos[(t, r)] = sum(1 for (t2, r2) in pairs if (t2, r2) < (t, r) and idx[t2, r2] == e)
    return pos


@pytest.mark.parametrize("T,E,k", [(4, 3, 1), (4, 3, 2), (3, 4, 3), (5, 2, 1)])
def test_positions_bruteforce_all_routings(T, E, k):
    choices = list(itertools.permutations(range(E), k))
    for C in (-1, 0, 1, 2, 3):
        for routing in itertools.product(choices, repeat=T):
            idx = np.array(routing, np.int32).reshape(T, k)
            counts, offsets, slot, row_token = O.positions(idx, E, C)
            pos = _brute_positions(idx, E, C)
            cnt = np.bincount(idx.ravel(), minlength=E)
            np.testing.assert_array_equal(counts, cnt)
            kept = cnt if C < 0 else np.minimum(cnt, C)
            np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(kept)]))
            for t in range(T):
                for r in range(k):
                    p = pos[(t, r)]
                    if C < 0 or p < C:
                        assert slot[t, r] == offsets[idx[t, r]] + p
                        assert row_token[slot[t, r]] == t
                    else:
                        assert slot[t, r] == -1


def _check_routing_invariants(spec, fw):
    T, k, E = spec.T, spec.k, spec.E
    C = fw["C"]
    counts, offsets, slot, idx = fw["counts"], fw["offsets"], fw["slot"], fw["idx"]
    n = int(offsets[-1])
    if C >= 0:
        assert np.all(np.diff(offsets) <= C)
    kept = slot >= 0
    assert n + int((~kept).sum()) == T * k
    s = slot[kept]
    assert sorted(s.tolist()) == list(range(n))   # bijection onto [0, n)
    tok = np.repeat(np.arange(T), k).reshape(T, k)[kept]
    np.testing.assert_array_equal(fw["row_token"][s], tok)
    # rows of one expert are contiguous and in token order
    for e in range(E):
        rows = fw["row_token"][offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(rows) > 0)
        assert np.all((idx[rows] == e).any(1))
    assert counts.sum() == T * k


@pytest.mark.parametrize("name", list(SMALL))
def test_small_forward_invariants(name):
    cfg = SMALL[name]
    spec = spec_of(cfg)
    inp = inputs64(cfg)
    fw = O.forward(spec, inp)
    _check_routing_invariants(spec, fw)
    if spec.gate == O.GATE_SOFTMAX:
        assert np.all(np.abs(fw["probs"].sum(1) - 1) <= 4 * spec.E * 2.0 ** -24)
    # a token whose every choice was dropped leaves the layer unchanged (bitwise)
    dropped_all = np.all(fw["slot"] < 0, axis=1)
    if not spec.shared:
        np.testing.assert_array_equal(fw["y"][dropped_all], inp["x"][dropped_all])
    # x_perm rows are copies of the routed token rows
    np.testing.assert_array_equal(fw["x_perm"], inp["x"][fw["row_token"][:fw["n_rows"]]])


def test_zero_router_uniform_probs_aux_equals_alpha_and_drops():
    cfg = CONFIGS["tiny_f32"].replace(alpha=0.01)
    spec = spec_of(cfg)
    inp = inputs64(cfg)
    inp["w_router"] = np.zeros_like(inp["w_router"])
    fw = O.forward(spec, inp)
    assert np.all(fw["probs"] == 0.25)
    assert fw["aux"] == np.float32(0.01)
    assert np.all(fw["idx"][:, 0] == 0)           # ties go to the lowest index
    assert fw["C"] == 64
    assert int((fw["slot"] < 0).sum()) == 192
    dropped = fw["slot"][:, 0] < 0
    np.testing.assert_array_equal(fw["y"][dropped], inp["x"][dropped])
    assert np.all(fw["slot"][:64, 0] == np.arange(64))


@pytest.mark.parametrize("E,k", [(8, 1), (16, 2), (64, 8)])
def test_aux_equals_alpha_under_uniform_routing_any_counts(E, k):
    # P_i = 1/E for every i makes the loss alpha * sum f_i = alpha whatever the counts.
    T = 64
    probs = np.full((T, E), 1.0 / E)
    rng = np.random.default_rng(5)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts = np.bincount(idx.ravel(), minlength=E).astype(np.int32)
    assert O.aux_loss(O.MODE_EXACT, probs, counts, k, 0.01) == pytest.approx(0.01, rel=1e-15)
    # and it is minimal there: any skew of P along a skewed f raises it
    skew = probs.copy()
    top = int(np.argmax(counts))
    skew[:, top] += 0.5 / E
    skew /= skew.sum(1, keepdims=True)
    assert O.aux_loss(O.MODE_EXACT, skew, counts, k, 0.01) > 0.01


def test_aux_matches_numpy_sketch_top1():
    # eq. (4) with the sketch's definitions: f = bincount(argmax)/T, P = mean(probs)
    rng = np.random.default_rng(6)
    T, E = 200, 8
    h = rng.standard_normal((T, E))
    probs, idx, w = O.gate_topk(O.MODE_EXACT, h, 1, O.GATE_SOFTMAX, False)
    counts = np.bincount(idx[:, 0], minlength=E).astype(np.int32)
    f = np.bincount(probs.argmax(-1), minlength=E) / T
    P = probs.mean(0)
    assert O.aux_loss(O.MODE_EXACT, probs, counts, 1, 0.01) == pytest.approx(0.01 * E * (f * P).sum(), rel=1e-13)


# ----------------------------------------------------------------- closed forms

def _dense_ffn(x, w1, w2, act):
    x, w1, w2 = (torch.from_numpy(a) for a in (x, w1, w2))
    a = x @ w1.T
    if act == O.ACT_RELU:
        h = torch.relu(a)
    else:
        f = w2.shape[1]
        h = torch.nn.functional.silu(a[:, :f]) * a[:, f:]
    return (h @ w2.T).numpy()


def _tiny(E, k, act="relu", gate="softmax", renorm=True, cf=0.0, shared=0, T=24, d=8, f=12, alpha=0.0,
          sel_bias="none", routing="token_choice"):
    return LayerConfig("t", T=T, d=d, f=f, E=E, k=k, gate=gate, renorm=renorm, act=act, dtype="f32",
                       cf=cf, alpha=alpha, shared=shared, sel_bias=sel_bias, routing=routing)


@pytest.mark.parametrize("act", ["relu", "swiglu"])
def test_single_expert_is_dense_ffn(act):
    cfg = _tiny(1, 1, act=act, renorm=False)
    spec = spec_of(cfg, O.MODE_EXACT)
    inp = inputs64(cfg)
    fw = O.forward(spec, inp)
    ref = inp["x"] + _dense_ffn(inp["x"], inp["w1"][0], inp["w2"][0], spec.act)
    np.testing.assert_allclose(fw["y"], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("gate", ["softmax", "sigmoid_bias", "sqrt_softplus_bias"])
def test_identical_experts_renorm_is_dense_ffn(gate):
    cfg = _tiny(6, 3, act="swiglu", gate=gate, sel_bias="uniform" if gate != "softmax" else "none")
    spec = spec_of(cfg, O.MODE_EXACT)
    inp = inputs64(cfg)
    inp["w1"] = np.ascontiguousarray(np.repeat(inp["w1"][:1], 6, 0))
    inp["w2"] = np.ascontiguousarray(np.repeat(inp["w2"][:1], 6, 0))
    fw = O.forward(spec, inp)
    ref = inp["x"] + _dense_ffn(inp["x"], inp["w1"][0], inp["w2"][0], spec.act)
    np.testing.assert_allclose(fw["y"], ref, rtol=1e-12, atol=1e-12)


def test_k_equals_E_is_dense_mixture():
    cfg = _tiny(5, 5, act="relu")
    spec = spec_of(cfg, O.MODE_EXACT)
    inp = inputs64(cfg)
    fw = O.forward(spec, inp)
    p = torch.softmax(torch.from_numpy(inp["x"] @ inp["w_router"].T), 1).numpy()
    ref = inp["x"].copy()
    for e in range(5):
        ref += p[:, e:e + 1] * _dense_ffn(inp["x"], inp["w1"][e], inp["w2"][e], spec.act)
    np.testing.assert_allclose(fw["y"], ref, rtol=1e-11, atol=1e-12)


def test_zero_w2_is_identity_and_shared_expert_adds():
    cfg = _tiny(4, 2, act="swiglu", shared=1)
    spec = spec_of(cfg, O.MODE_EXACT)
    inp = inputs64(cfg)
    inp["w2"] = np.zeros_like(inp["w2"])
    fw = O.forward(spec, inp)
    ref = inp["x"] + _dense_ffn(inp["x"], inp["ws1"], inp["ws2"], spec.act)
    np.testing.assert_allclose(fw["y"], ref, rtol=1e-12, atol=1e-12)


def test_bf16_rounding_points_are_bf16_values():
    cfg = SMALL["switch_base"]
    spec = spec_of(cfg)
    fw = O.forward(spec, inputs64(cfg))
    for key in ("act", "h", "y_perm", "y"):
        a = fw[key].astype(np.float32)
        back = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
        np.testing.assert_array_equal(a, back)
    # h is relu of the saved pre-activation (rounding commutes with max(.,0))
    np.testing.assert_array_equal(fw["h"], np.maximum(fw["act"], 0.0))


# ----------------------------------------------------------------- gradients (finite differences)

def _loss(spec, inp, dy):
    fw = O.forward(spec, inp)
    return float((dy * fw["y"]).sum() + fw["aux"]), fw


def _signature(spec, fw):
    sig = [fw["idx"].tobytes(), fw["slot"].tobytes()]
    if spec.act == O.ACT_RELU:
        sig.append((fw["act"] > 0).tobytes())
        if spec.shared:
            sig.append((fw["act_shared"] > 0).tobytes())
    return sig


FD_CASES = [
    dict(E=4, k=1, gate="softmax", renorm=False, act="relu", cf=1.0, alpha=0.3),
    dict(E=4, k=2, gate="softmax", renorm=True, act="swiglu", cf=0.75, alpha=0.3),
    dict(E=4, k=2, gate="softmax", renorm=False, act="relu", cf=0.0, alpha=0.3),
    dict(E=4, k=2, gate="sigmoid_bias", renorm=True, act="swiglu", cf=0.0, alpha=0.0, shared=1,
         sel_bias="uniform"),
    dict(E=4, k=1, gate="sigmoid_bias", renorm=False, act="relu", cf=0.5, alpha=0.3, sel_bias="uniform"),
    dict(E=4, k=2, gate="sqrt_softplus_bias", renorm=True, act="swiglu", cf=0.0, alpha=0.3, shared=1,
         sel_bias="uniform"),
    dict(E=4, k=1, gate="sqrt_softplus_bias", renorm=False, act="relu", cf=0.5, alpha=0.3, sel_bias="uniform"),
    dict(E=4, k=2, gate="noisy_topk", renorm=True, act="swiglu", cf=0.0, alpha=0.5),
    dict(E=5, k=1, gate="noisy_topk", renorm=True, act="relu", cf=0.75, alpha=0.5, shared=1),
    dict(E=4, k=4, gate="softmax", renorm=False, act="swiglu", cf=1.0, routing="expert_choice"),
    dict(E=4, k=4, gate="softmax", renorm=False, act="relu", cf=0.5, shared=1, routing="expert_choice"),
]


@pytest.mark.parametrize("case", range(len(FD_CASES)))
def test_backward_matches_finite_differences(case):
    kw = dict(FD_CASES[case])
    cfg = _tiny(T=16, d=8, f=16, **kw)
    spec = spec_of(cfg, O.MODE_EXACT)
    inp = inputs64(cfg, seed=case)
    inp["w_router"] = inp["w_router"] * 8.0   # sharper routing -> larger gate gradients
    dy = f64(torch.randn(cfg.T, cfg.d, generator=torch.Generator().manual_seed(99 + case)))
    L0, fw = _loss(spec, inp, dy)
    bw = O.backward(spec, inp, fw, dy)
    grads = {"x": bw["dx"], "w_router": bw["dw_router"], "w1": bw["dw1"], "w2": bw["dw2"]}
    if spec.shared:
        grads.update(ws1=bw["dws1"], ws2=bw["dws2"])
    sig0 = _signature(spec, fw)
    rng = np.random.default_rng(case)
    step = 1e-6
    checked = 0
    for name, g in grads.items():
        flat = inp[name].reshape(-1)
        scale = max(np.sqrt(np.mean(g ** 2)), 1e-3)
        for i in rng.choice(flat.size, min(flat.size, 40), replace=False):
            old = flat[i]
            flat[i] = old + step
            Lp, fp = _loss(spec, inp, dy)
            flat[i] = old - step
            Lm, fm = _loss(spec, inp, dy)
            flat[i] = old
            if _signature(spec, fp) != sig0 or _signature(spec, fm) != sig0:
                continue  # a routing decision or ReLU sign flipped inside the step
            fd = (Lp - Lm) / (2 * step)
            an = g.reshape(-1)[i]
            assert abs(fd - an) <= 1e-6 * max(abs(an), scale), (name, i, fd, an)
            checked += 1
    assert checked >= 150


def test_aux_gradient_alone_matches_finite_differences():
    cfg = _tiny(E=6, k=2, gate="softmax", renorm=True, act="relu", alpha=0.5, cf=0.0)
    spec = spec_of(cfg, O.MODE_EXACT)
    inp = inputs64(cfg, seed=7)
    dy = np.zeros((cfg.T, cfg.d))
    L0, fw = _loss(spec, inp, dy)
    bw = O.backward(spec, inp, fw, dy)
    # with dy = 0 only the aux path remains: dlogits = (aE/T) p (f - sum f p)
    T, E = cfg.T, cfg.E
    f = fw["counts"] / (T * cfg.k)
    p = fw["probs"]
    ref = 0.5 * E / T * p * (f[None, :] - (p * f[None, :]).sum(1, keepdims=True))
    np.testing.assert_allclose(bw["dlogits"], ref, rtol=1e-12, atol=1e-15)
    w = inp["w_router"].reshape(-1)
    for i in range(0, w.size, 5):
        old = w[i]
        w[i] = old + 1e-6
        Lp, _ = _loss(spec, inp, dy)
        w[i] = old - 1e-6
        Lm, _ = _loss(spec, inp, dy)
        w[i] = old
        an = bw["dw_router"].reshape(-1)[i]
        assert abs((Lp - Lm) / 2e-6 - an) <= 1e-6 * max(abs(an), 1e-4)


def test_gate_gradient_is_expert_output():
    # d<dy, y>/dw[t,r] equals <dy, y_perm[slot]> for kept pairs and 0 for dropped ones.
    rng = np.random.default_rng(8)
    T, d, k, n = 10, 6, 2, 12
    x = rng.standard_normal((T, d))
    y_perm = rng.standard_normal((n, d))
    slot = np.full((T, k), -1, np.int32)
    perm = rng.permutation(n)
    flat = [(t, r) for t in range(T) for r in range(k)]
    for j, (t, r) in enumerate(flat[:n]):
        slot[t, r] = perm[j]
    w = rng.random((T, k))
    dy = rng.standard_normal((T, d))
    dO, dg = O.combine_bwd(O.MODE_EXACT, dy, y_perm, slot, w, n)
    for t in range(T):
        for r in range(k):
            w2 = w.copy()
            w2[t, r] += 1e-6
            y1 = O.combine(O.MODE_EXACT, x, y_perm, slot, w2)
            w2[t, r] -= 2e-6
            y0 = O.combine(O.MODE_EXACT, x, y_perm, slot, w2)
            fd = ((dy * y1).sum() - (dy * y0).sum()) / 2e-6
            assert abs(fd - dg[t, r]) < 1e-7
            if slot[t, r] < 0:
                assert dg[t, r] == 0.0
            else:
                np.testing.assert_allclose(dO[slot[t, r]], w[t, r] * dy[t], rtol=1e-15)


def test_empty_expert_weight_gradient_is_zero():
    G = np.zeros((0, 5))
    V = np.zeros((0, 3))
    assert np.all(O.wgrad(O.MODE_BF16, G, V) == 0.0)


def _fp32_sum(terms, order):
    acc = np.float32(0.0)
    for v in terms[order]:
        acc = np.float32(acc + v)
    return acc


def test_relu_ambiguity_bound_holds_for_fp32_accumulation():
    """oracle.relu_ambiguous (the S22 reading): outside the flagged elements, an
    fp32 accumulation of the exact bf16 products in any order gives the sign of
    the exact pre-activation. Checked on bf16 operands drawn so that many sums
    are near zero, against sequential sums in the natural, reversed and random
    orders and numpy's pairwise fp32 sum; an exactly cancelling row is flagged and
    a clearly signed one is not."""
    rng = np.random.default_rng(7)
    n, d, f = 48, 264, 40
    X = O.round_array(O.MODE_BF16, rng.standard_normal((n, d)))
    W = O.round_array(O.MODE_BF16, rng.standard_normal((f, d)) / np.sqrt(d))
    # pull some pre-activations towards zero: row n-1 of X cancels against W row 0
    # in exact arithmetic (pairs of equal and opposite products)
    X[-1, :] = 1.0
    W[0, 0::2] = O.round_array(O.MODE_BF16, np.abs(rng.standard_normal(d // 2)))
    W[0, 1::2] = -W[0, 0::2]
    exact = X @ W.T                       # products of bf16 values are exact in double
    A = O.round_array(O.MODE_BF16, exact)
    amb = O.relu_ambiguous(X, W, A)
    assert amb[-1, 0] and exact[-1, 0] == 0.0
    assert not amb[np.abs(exact) > 1e-2].any()
    X32, W32 = X.astype(np.float32), W.astype(np.float32)
    orders = [np.arange(d), np.arange(d)[::-1]] + [rng.permutation(d) for _ in range(6)]
    checked = 0
    for i in range(n):
        for j in range(f):
            if amb[i, j]:
                continue
            terms = X32[i] * W32[j]           # exact in fp32 (8-bit significands)
            s = np.sign(exact[i, j])
            for o in orders:
                assert np.sign(_fp32_sum(terms, o)) == s, (i, j)
            assert np.sign(np.sum(terms, dtype=np.float32)) == s
            checked += 1
    assert checked > 0.9 * n * f


def test_relu_ambiguity_bound_is_not_vacuous():
    """The flagged fraction at unit-scale pre-activations stays small: about
    the probability that |a| is under gamma_d * sum |x w|."""
    rng = np.random.default_rng(3)
    n, d, f = 4096, 256, 64
    X = O.round_array(O.MODE_BF16, rng.standard_normal((n, d)))
    W = O.round_array(O.MODE_BF16, rng.standard_normal((f, d)) / np.sqrt(d))
    A = O.round_array(O.MODE_BF16, X @ W.T)
    frac = O.relu_ambiguous(X, W, A).mean()
    assert 0 < frac < 1e-3


def test_relerr_sum_measures_against_the_terms():
    """helpers.relerr_sum: equal to relerr when the terms are no larger than the
    result; at a cancellation a one-ulp difference in a large term stays small."""
    from helpers import relerr, relerr_sum
    rng = np.random.default_rng(0)
    r = rng.standard_normal(1000)
    a = r * (1 + 1e-3 * rng.standard_normal(1000))
    assert relerr_sum(a, r, np.abs(r)) == pytest.approx(relerr(a, r))
    # 2.0625 - 2.15625 = -0.09375: the second term off by one bf16 ulp (2^-6)
    r2 = np.array([-0.09375, 1.0, -1.0])
    a2 = r2 + np.array([2.0 ** -6, 0.0, 0.0])
    terms = np.array([2.0625 + 2.15625, 1.0, 1.0])
    assert relerr(a2, r2) > 0.01
    assert relerr_sum(a2, r2, terms) < 0.004
    # a real error in the same cancelling sum (a dropped term of 0.25) still fails 2e-2
    a3 = r2 + np.array([0.25, 0.0, 0.0])
    assert relerr_sum(a3, r2, terms) > 0.05
