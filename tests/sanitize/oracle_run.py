"""Runs the oracle's whole-layer forward and backward on small layers (every gate,
both activations, drops, a shared expert, expert choice, noisy gating) and its
scalar contracts. Run by tests/test_sanitizers.py in a child process against an
AddressSanitizer + UndefinedBehaviorSanitizer build of the oracle (MOE_ORACLE_LIB);
it imports numpy and the oracle only."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import oracle as O  # noqa: E402


def layer(T, d, f, E, k, gate, renorm, act, cf, alpha, shared, ec=False, seed=0):
    rng = np.random.default_rng(seed)
    f1 = 2 * f if act == O.ACT_SWIGLU else f
    ER = 2 * E if gate == O.GATE_NOISY_TOPK else E
    bf = lambda a: O.round_array(O.MODE_BF16, a)  # noqa: E731
    inp = dict(x=bf(rng.standard_normal((T, d))),
               w_router=np.float32(rng.standard_normal((ER, d)) / np.sqrt(d)).astype(np.float64),
               w1=bf(rng.standard_normal((E, f1, d)) / np.sqrt(d)),
               w2=bf(rng.standard_normal((E, d, f)) / np.sqrt(f)),
               dy=bf(rng.standard_normal((T, d))))
    if gate in (O.GATE_SIGMOID_BIAS, O.GATE_SQRT_SOFTPLUS_BIAS):
        inp["sel_bias"] = np.float32(rng.uniform(-0.5, 0.5, E)).astype(np.float64)
    if gate == O.GATE_NOISY_TOPK:
        inp["noise"] = np.float32(rng.standard_normal((T, E))).astype(np.float64)
    if shared:
        inp["ws1"] = bf(rng.standard_normal((f1, d)) / np.sqrt(d))
        inp["ws2"] = bf(rng.standard_normal((d, f)) / np.sqrt(f))
    spec = O.Spec(T, d, f, E, k, gate, renorm, act, O.MODE_BF16, cf, alpha, shared, ec)
    fw = O.forward(spec, inp)
    bw = O.backward(spec, inp, fw, inp["dy"])
    assert np.all(np.isfinite(bw["dx"])) and np.all(np.isfinite(bw["dw_router"]))


def main():
    S, B, Q, N = O.GATE_SOFTMAX, O.GATE_SIGMOID_BIAS, O.GATE_SQRT_SOFTPLUS_BIAS, O.GATE_NOISY_TOPK
    R, G = O.ACT_RELU, O.ACT_SWIGLU
    layer(37, 16, 24, 4, 1, S, False, R, 1.0, 0.01, 0)
    layer(40, 16, 16, 6, 2, S, True, G, 0.75, 0.01, 1)
    layer(33, 24, 8, 8, 3, B, True, G, 0.0, 0.0, 1)
    layer(29, 16, 16, 5, 2, Q, False, R, 1.25, 0.0, 0)
    layer(31, 16, 16, 4, 2, N, True, R, 1.0, 0.3, 0)
    layer(24, 16, 16, 4, 4, S, False, R, 1.5, 0.0, 0, ec=True)
    layer(0, 16, 16, 4, 2, S, True, R, 1.0, 0.01, 0)
    for v in np.linspace(-90, 90, 2001):
        O.exp_contract(v), O.sigmoid_contract(v), O.sqrt_softplus_contract(v), O.softplus_contract(v)
    for v in np.linspace(0, 1, 501):
        O.log1p_contract(v)
    O.bias_update(np.array([3, 0, 5, 1], np.int32), 1e-3, np.zeros(4))
    O.bias_quantile(np.random.default_rng(1).random((50, 6)), 2, np.zeros(6))
    print("oracle ran clean")


if __name__ == "__main__":
    main()
