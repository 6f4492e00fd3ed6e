"""Reference oracle for the MoE layer: test infrastructure only.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library never imports it, and
this package imports nothing from the GPU library.

The arithmetic lives in ``moe_oracle.cpp`` (plain C++ loops in double; the
router follows the fp32 contract stated in that file). This module only
marshals numpy arrays in and out and strings the steps together in the order
the layer defines them:

  route   [SW] eq. (1) + top-k          -> probs, idx, w
  capacity/positions [SW] eq. (3)       -> counts, offsets, slot, row_token
  expert FFN per kept row               -> act (pre-activation), h, y_perm
  combine [SW] eq. (2) + residual       -> y
  aux     [SW] eq. (4)                  -> scalar
  backward of all of the above for L = sum <dy, y> + aux

[SW] = "Mixture of Experts (MoE) を1から解説 — Switch Transformerのルーティングと負荷分散"
(ta-paperlens.web.app).

Every floating array handed in must already hold the exact values of the
layer's storage type (bf16 or fp32 values widened to float64).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_ORACLE_LIB may point at another build of the same source (the sanitizer test's)
LIB_PATH = os.environ.get("MOE_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "moe_oracle.cpp")

MODE_EXACT, MODE_F32, MODE_BF16 = 0, 1, 2
GATE_SOFTMAX, GATE_SIGMOID_BIAS, GATE_SQRT_SOFTPLUS_BIAS, GATE_NOISY_TOPK = 0, 1, 2, 3
GATE_OF = {"softmax": GATE_SOFTMAX, "sigmoid_bias": GATE_SIGMOID_BIAS,
           "sqrt_softplus_bias": GATE_SQRT_SOFTPLUS_BIAS, "noisy_topk": GATE_NOISY_TOPK}
ACT_RELU, ACT_SWIGLU = 0, 1

_lib = None


def build(quiet: bool = True) -> str:
    """Compile the oracle with g++ (no HIP, no GPU headers)."""
    import subprocess
    cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-fast-math", "-mfma", SRC_PATH, "-o", LIB_PATH + ".tmp"]
    subprocess.run(cmd, check=True, capture_output=quiet)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        D = ctypes.POINTER(ctypes.c_double)
        I = ctypes.POINTER(ctypes.c_int)
        i, d = ctypes.c_int, ctypes.c_double
        sig = {
            "orc_round_bf16": (d, [d]),
            "orc_exp_contract": (ctypes.c_float, [ctypes.c_float]),
            "orc_sigmoid_contract": (ctypes.c_float, [ctypes.c_float]),
            "orc_log1p_contract": (ctypes.c_float, [ctypes.c_float]),
            "orc_sqrt_softplus_contract": (ctypes.c_float, [ctypes.c_float]),
            "orc_gate_deriv": (d, [i, d]),
            "orc_bias_update": (None, [i, I, d, D, D]),
            "orc_bias_quantile": (None, [i, i, i, D, D, D]),
            "orc_softplus_contract": (ctypes.c_float, [ctypes.c_float]),
            "orc_noisy_logits": (None, [i, i, i, D, D, D]),
            "orc_noisy_aux": (d, [i, i, i, i, D, D, I, D, d, D, D]),
            "orc_noisy_dlogits": (None, [i, i, i, i, D, D, I, D, D, d, D]),
            "qb_target": (i, [i, i, i]),
            "orc_capacity": (i, [i, i, d]),
            "orc_logits": (None, [i, i, i, i, D, D, D, D]),
            "orc_gate": (None, [i, i, i, i, i, i, D, D, D, I, D]),
            "orc_positions": (None, [i, i, i, i, I, I, I, I, I]),
            "orc_softmax_ec": (None, [i, i, i, D, D]),
            "orc_expert_choice": (None, [i, i, i, D, I, D, I, I, I]),
            "orc_aux": (d, [i, i, i, i, d, D, I]),
            "orc_ffn_fwd": (None, [i, i, i, i, i, D, D, D, D, D, D]),
            "orc_combine": (None, [i, i, i, i, D, D, I, D, D, D]),
            "orc_combine_bwd": (None, [i, i, i, i, D, D, I, D, D, D]),
            "orc_ffn_bwd": (None, [i, i, i, i, i, D, D, D, D, D, D]),
            "orc_wgrad": (None, [i, i, i, i, D, D, D]),
            "orc_router_dlogits": (None, [i, i, i, i, i, i, d, D, I, D, D, I, D]),
            "orc_round_array": (None, [i, ctypes.c_int64, D, D]),
            "orc_router_grads": (None, [i, i, i, i, D, D, D, D, D]),
            "orc_unpermute_bwd": (None, [i, i, i, i, D, D, I, D, D, D]),
            "orc_set_threads": (None, [i]),
            "orc_get_threads": (i, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _d(a):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _i(a):
    if a is None:
        return None
    assert a.dtype == np.int32 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int))


def f64(a) -> np.ndarray:
    """Widen a torch tensor or array (bf16/fp32/fp64) to a C-contiguous float64 array."""
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().to("cpu")
        import torch
        return np.ascontiguousarray(a.to(torch.float64).numpy())
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


# ----------------------------------------------------------------- primitives

def round_bf16(v: float) -> float:
    return lib().orc_round_bf16(float(v))


def exp_contract(x: float) -> float:
    return lib().orc_exp_contract(float(x))


def sigmoid_contract(x: float) -> float:
    return lib().orc_sigmoid_contract(float(x))


def log1p_contract(x: float) -> float:
    return lib().orc_log1p_contract(float(x))


def sqrt_softplus_contract(x: float) -> float:
    return lib().orc_sqrt_softplus_contract(float(x))


def gate_deriv(gate: int, s: float) -> float:
    return lib().orc_gate_deriv(int(gate), float(s))


def bias_update(counts, gamma: float, bias):
    """Aux-loss-free selection-bias step (fp32 values in, fp32 values out as float64)."""
    c = np.ascontiguousarray(counts, np.int32)
    b = f64(bias)
    out = np.empty_like(b)
    lib().orc_bias_update(int(c.size), _i(c), float(gamma), _d(b), _d(out))
    return out


def bias_quantile(probs, k: int, bias):
    """Quantile-Balancing bias from one batch's gate values (fp32 values as float64)."""
    p = f64(probs)
    T, E = p.shape
    b = f64(bias)
    out = np.empty_like(b)
    lib().orc_bias_quantile(T, E, int(k), _d(p), _d(b), _d(out))
    return out


def softplus_contract(x: float) -> float:
    return lib().orc_softplus_contract(float(x))


def noisy_logits(mode, logits2, eps):
    """H = h + eps * softplus(n) from the stacked [T, 2E] clean|noise logits."""
    T, E2 = logits2.shape
    H = np.empty((T, E2 // 2))
    lib().orc_noisy_logits(mode, T, E2 // 2, _d(f64(logits2)), _d(f64(eps)), _d(H))
    return H


def noisy_aux(mode, logits2, eps, idx, w, alpha):
    """(alpha (CV^2(importance) + CV^2(load)), importance [E], load [E])."""
    T, E2 = logits2.shape
    E, k = E2 // 2, idx.shape[1]
    imp, load = np.empty(E), np.empty(E)
    aux = lib().orc_noisy_aux(mode, T, E, k, _d(f64(logits2)), _d(f64(eps)), _i(np.ascontiguousarray(idx, np.int32)),
                              _d(f64(w)), float(alpha), _d(imp), _d(load))
    return aux, imp, load


def noisy_dlogits(mode, logits2, eps, idx, w, dg, alpha):
    T, E2 = logits2.shape
    out = np.empty((T, E2))
    lib().orc_noisy_dlogits(mode, T, E2 // 2, idx.shape[1], _d(f64(logits2)), _d(f64(eps)),
                            _i(np.ascontiguousarray(idx, np.int32)), _d(f64(w)), _d(f64(dg)), float(alpha), _d(out))
    return out


def qb_target(T: int, E: int, k: int) -> int:
    return lib().qb_target(int(T), int(E), int(k))


def capacity(T: int, E: int, cf: float) -> int:
    return lib().orc_capacity(T, E, float(cf))


def logits(mode, x, w_router, offset=None):
    T, d = x.shape
    E = w_router.shape[0]
    h = np.empty((T, E), np.float64)
    lib().orc_logits(mode, T, d, E, _d(x), _d(w_router), _d(offset), _d(h))
    return h


def gate_topk(mode, h, k, gate, renorm, sel_bias=None):
    T, E = h.shape
    probs = np.empty((T, E), np.float64)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    lib().orc_gate(mode, T, E, k, gate, int(renorm), _d(h), _d(sel_bias), _d(probs), _i(idx), _d(w))
    return probs, idx, w


def positions(idx, E, C):
    T, k = idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    slot = np.empty((T, k), np.int32)
    row_token = np.full(T * k, -1, np.int32)
    lib().orc_positions(T, k, E, C, _i(np.ascontiguousarray(idx, np.int32)), _i(counts),
                        _i(offsets), _i(slot), _i(row_token))
    return counts, offsets, slot, row_token


def softmax_ec(mode, h):
    """Softmax with the expert-choice fp32 contract (plain double softmax in mode 0)."""
    T, E = h.shape
    probs = np.empty((T, E))
    lib().orc_softmax_ec(mode, T, E, _d(np.ascontiguousarray(h, np.float64)), _d(probs))
    return probs


def expert_choice(probs, C):
    """Each expert takes its C most probable tokens -> slot [T,E], w [T,E], row_token,
    counts [E], offsets [E+1]."""
    T, E = probs.shape
    Cp = min(C, T)
    slot = np.empty((T, E), np.int32)
    w = np.empty((T, E))
    row_token = np.full(max(E * Cp, 1), -1, np.int32)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    lib().orc_expert_choice(T, E, C, _d(np.ascontiguousarray(probs, np.float64)), _i(slot), _d(w),
                            _i(row_token), _i(counts), _i(offsets))
    return slot, w, row_token, counts, offsets


def aux_loss(mode, probs, counts, k, alpha):
    T, E = probs.shape
    return lib().orc_aux(mode, T, E, k, float(alpha), _d(probs), _i(counts))


def ffn_fwd(mode, X, W1, W2, act):
    n, d = X.shape
    f = W2.shape[1]
    f1 = 2 * f if act == ACT_SWIGLU else f
    assert W1.shape == (f1, d) and W2.shape == (d, f)
    A = np.empty((n, f1), np.float64)
    H = np.empty((n, f), np.float64)
    Y = np.empty((n, d), np.float64)
    if n:
        lib().orc_ffn_fwd(mode, n, d, f, act, _d(X), _d(W1), _d(W2), _d(A), _d(H), _d(Y))
    return A, H, Y


def relu_ambiguous(X, W1, A):
    """Pre-activations of a ReLU expert whose sign an fp32 accumulation may not
    decide: |a| <= gamma_d * sum_j |x_j w_j| with gamma_d = d u / (1 - d u), the
    standard bound on a d-term floating-point sum. u is taken as 2^-23 (twice the
    fp32 unit roundoff, so the bound holds whichever rounding the matrix cores'
    fp32 accumulation uses), and A holds the bf16-rounded pre-activations, so the
    bound is widened by one bf16 rounding (2^-8, doubled). Both masks of such an
    element are correct results; everywhere else the mask is fixed.
    X [n, d], W1 [f, d] (the ReLU layer's first matrix), A [n, f]."""
    n, d = X.shape
    if n == 0:
        return np.zeros((0, W1.shape[0]), bool)
    u = 2.0 ** -23
    gamma = d * u / (1.0 - d * u)
    bound = np.abs(X) @ np.abs(W1).T
    return np.abs(A) <= gamma * bound * (1.0 + 2.0 ** -7)


def relu_ambiguous_rows(x_perm, w1, offsets, act):
    """relu_ambiguous over every expert's rows of the permuted buffers -> [n, f] mask."""
    n = int(offsets[-1])
    out = np.zeros((n, act.shape[1]), bool)
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            out[a:b] = relu_ambiguous(x_perm[a:b], w1[e], act[a:b])
    return out


def combine(mode, x, y_perm, slot, w, y_shared=None):
    T, d = x.shape
    k = slot.shape[1]
    y = np.empty((T, d), np.float64)
    if y_perm.shape[0] == 0:
        y_perm = np.zeros((1, d), np.float64)
    lib().orc_combine(mode, T, d, k, _d(x), _d(y_perm), _i(slot), _d(w), _d(y_shared), _d(y))
    return y


def combine_bwd(mode, dy, y_perm, slot, w, n_rows):
    T, d = dy.shape
    k = slot.shape[1]
    dO = np.zeros((max(n_rows, 1), d), np.float64)
    dg = np.empty((T, k), np.float64)
    yp = y_perm if y_perm.shape[0] else np.zeros((1, d), np.float64)
    lib().orc_combine_bwd(mode, T, d, k, _d(dy), _d(yp), _i(slot), _d(w), _d(dO), _d(dg))
    return dO[:n_rows], dg


def ffn_bwd(mode, dO, A, W1, W2, act):
    n, d = dO.shape
    f = W2.shape[1]
    f1 = 2 * f if act == ACT_SWIGLU else f
    dA = np.empty((n, f1), np.float64)
    dX = np.empty((n, d), np.float64)
    if n:
        lib().orc_ffn_bwd(mode, n, d, f, act, _d(dO), _d(A), _d(W1), _d(W2), _d(dA), _d(dX))
    return dA, dX


def wgrad(mode, G, V):
    n, M = G.shape
    N = V.shape[1]
    dW = np.empty((M, N), np.float64)
    Gc = G if n else np.zeros((1, M), np.float64)
    Vc = V if n else np.zeros((1, N), np.float64)
    lib().orc_wgrad(mode, n, M, N, _d(Gc), _d(Vc), _d(dW))
    return dW


def router_dlogits(probs, idx, w, dg, counts, gate, renorm, alpha, T_batch=None):
    """Logit gradient of the given token rows; T_batch (default: the number of
    rows) is the batch size the aux loss is normalised by."""
    T, E = probs.shape
    k = idx.shape[1]
    out = np.empty((T, E), np.float64)
    lib().orc_router_dlogits(T, T if T_batch is None else int(T_batch), E, k, gate, int(renorm), float(alpha),
                             _d(probs), _i(idx), _d(w), _d(dg), _i(counts), _d(out))
    return out


def round_array(mode, a):
    a = np.ascontiguousarray(a, np.float64)
    out = np.empty_like(a)
    lib().orc_round_array(mode, a.size, _d(a), _d(out))
    return out


def router_grads(mode, dlogits, x, w_router):
    T, E = dlogits.shape
    d = x.shape[1]
    dWr = np.empty((E, d), np.float64)
    dxr = np.empty((T, d), np.float64)
    lib().orc_router_grads(mode, T, d, E, _d(dlogits), _d(x), _d(w_router), _d(dWr), _d(dxr))
    return dWr, dxr


def unpermute_bwd(mode, dy, dX_perm, slot, dx_router=None, dx_shared=None):
    T, d = dy.shape
    k = slot.shape[1]
    dx = np.empty((T, d), np.float64)
    dXp = dX_perm if dX_perm.shape[0] else np.zeros((1, d), np.float64)
    lib().orc_unpermute_bwd(mode, T, d, k, _d(dy), _d(dXp), _i(slot), _d(dx_router),
                            _d(dx_shared), _d(dx))
    return dx


# ------------------------------------------------------------ whole-layer drivers

@dataclass
class Spec:
    """The layer description the oracle needs (duck-typed from any config object)."""
    T: int
    d: int
    f: int
    E: int
    k: int
    gate: int
    renorm: bool
    act: int
    mode: int
    cf: float
    alpha: float
    shared: int
    expert_choice: bool = False

    @staticmethod
    def of(cfg, mode=None):
        gate = GATE_OF[cfg.gate]
        act = ACT_SWIGLU if cfg.act == "swiglu" else ACT_RELU
        m = mode if mode is not None else (MODE_F32 if cfg.dtype == "f32" else MODE_BF16)
        return Spec(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, gate, bool(cfg.renorm), act, m,
                    float(cfg.cf), float(cfg.alpha), int(cfg.shared),
                    getattr(cfg, "routing", "token_choice") == "expert_choice")


def route(spec: Spec, x, w_router, logit_offset=None, sel_bias=None, noise=None):
    if spec.gate == GATE_NOISY_TOPK:
        # stacked router [W_g; W_noise] -> clean|noise logits; softmax over the top-k of H
        assert w_router.shape[0] == 2 * spec.E and logit_offset is None and spec.renorm
        h2 = logits(spec.mode, x, w_router)
        H = noisy_logits(spec.mode, h2, noise)
        probs, idx, w = gate_topk(spec.mode, H, spec.k, GATE_SOFTMAX, True)
        C = capacity(spec.T, spec.E, spec.cf)
        counts, offsets, slot, row_token = positions(idx, spec.E, C)
        aux = noisy_aux(spec.mode, h2, noise, idx, w, spec.alpha)[0] if spec.alpha else 0.0
        if spec.mode != MODE_EXACT:
            aux = float(np.float32(aux))
        return dict(h=H, logits2=h2, probs=probs, idx=idx, w=w, C=C, counts=counts, offsets=offsets,
                    slot=slot, row_token=row_token, aux=aux)
    h = logits(spec.mode, x, w_router, logit_offset)
    if spec.expert_choice:
        # the token tables have one column per expert (k = E); idx is the identity
        assert spec.k == spec.E and spec.gate == GATE_SOFTMAX and not spec.renorm and spec.cf > 0
        probs = softmax_ec(spec.mode, h)
        C = capacity(spec.T, spec.E, spec.cf)
        slot, w, row_token, counts, offsets = expert_choice(probs, C)
        idx = np.ascontiguousarray(np.broadcast_to(np.arange(spec.E, dtype=np.int32), (spec.T, spec.E)))
        return dict(h=h, probs=probs, idx=idx, w=w, C=C, counts=counts, offsets=offsets, slot=slot,
                    row_token=row_token, aux=0.0)
    probs, idx, w = gate_topk(spec.mode, h, spec.k, spec.gate, spec.renorm, sel_bias)
    C = capacity(spec.T, spec.E, spec.cf)
    counts, offsets, slot, row_token = positions(idx, spec.E, C)
    aux = aux_loss(spec.mode, probs, counts, spec.k, spec.alpha) if spec.alpha else 0.0
    return dict(h=h, probs=probs, idx=idx, w=w, C=C, counts=counts, offsets=offsets,
                slot=slot, row_token=row_token, aux=aux)


def forward(spec: Spec, inp: dict) -> dict:
    """Full forward. ``inp`` holds float64 arrays: x, w_router, w1, w2 and the optional
    logit_offset, sel_bias, ws1, ws2."""
    r = route(spec, inp["x"], inp["w_router"], inp.get("logit_offset"), inp.get("sel_bias"), inp.get("noise"))
    n = int(r["offsets"][-1])
    f1 = 2 * spec.f if spec.act == ACT_SWIGLU else spec.f
    x_perm = inp["x"][r["row_token"][:n]] if n else np.zeros((0, spec.d))
    act = np.zeros((n, f1))
    h = np.zeros((n, spec.f))
    y_perm = np.zeros((n, spec.d))
    for e in range(spec.E):
        a, b = int(r["offsets"][e]), int(r["offsets"][e + 1])
        if b > a:
            A, H, Y = ffn_fwd(spec.mode, np.ascontiguousarray(x_perm[a:b]), inp["w1"][e], inp["w2"][e], spec.act)
            act[a:b], h[a:b], y_perm[a:b] = A, H, Y
    out = dict(r, x_perm=x_perm, act=act, h=h, y_perm=y_perm, n_rows=n)
    y_shared = None
    if spec.shared:
        A, H, Y = ffn_fwd(spec.mode, inp["x"], inp["ws1"], inp["ws2"], spec.act)
        out.update(act_shared=A, h_shared=H, y_shared=Y)
        y_shared = Y
    out["y"] = combine(spec.mode, inp["x"], y_perm, r["slot"], r["w"], y_shared)
    return out


def backward(spec: Spec, inp: dict, saved: dict, dy: np.ndarray) -> dict:
    """Full backward of L = sum <dy, y> + aux, from the forward's saved tensors
    (probs, idx, w, counts, offsets, slot, row_token, x_perm, act, h, y_perm and,
    with a shared expert, act_shared and h_shared)."""
    n = int(saved["offsets"][-1])
    dO, dg = combine_bwd(spec.mode, dy, saved["y_perm"], saved["slot"], saved["w"], n)
    f1 = 2 * spec.f if spec.act == ACT_SWIGLU else spec.f
    dA = np.zeros((n, f1))
    dX_perm = np.zeros((n, spec.d))
    dw1 = np.zeros((spec.E, f1, spec.d))
    dw2 = np.zeros((spec.E, spec.d, spec.f))
    for e in range(spec.E):
        a, b = int(saved["offsets"][e]), int(saved["offsets"][e + 1])
        if b > a:
            dA_e, dX_e = ffn_bwd(spec.mode, np.ascontiguousarray(dO[a:b]), np.ascontiguousarray(saved["act"][a:b]),
                                 inp["w1"][e], inp["w2"][e], spec.act)
            dA[a:b], dX_perm[a:b] = dA_e, dX_e
        dw2[e] = wgrad(spec.mode, np.ascontiguousarray(dO[a:b]), np.ascontiguousarray(saved["h"][a:b]))
        dw1[e] = wgrad(spec.mode, np.ascontiguousarray(dA[a:b]), np.ascontiguousarray(saved["x_perm"][a:b]))
    out = dict(dO=dO, dg=dg, dA=dA, dX_perm=dX_perm, dw1=dw1, dw2=dw2)
    dx_shared = None
    if spec.shared:
        dA_s, dX_s = ffn_bwd(spec.mode, dy, saved["act_shared"], inp["ws1"], inp["ws2"], spec.act)
        out["dws2"] = wgrad(spec.mode, dy, saved["h_shared"])
        out["dws1"] = wgrad(spec.mode, dA_s, inp["x"])
        out["dA_shared"], out["dx_shared"] = dA_s, dX_s
        dx_shared = dX_s
    if spec.gate == GATE_NOISY_TOPK:
        dl = noisy_dlogits(spec.mode, saved["logits2"], inp["noise"], saved["idx"], saved["w"], dg, spec.alpha)
    else:
        dl = router_dlogits(saved["probs"], saved["idx"], saved["w"], dg, saved["counts"],
                            spec.gate, spec.renorm, spec.alpha)
    dWr, dxr = router_grads(spec.mode, dl, inp["x"], inp["w_router"])
    out.update(dlogits=dl, dw_router=dWr, dx_router=dxr)
    out["dx"] = unpermute_bwd(spec.mode, dy, dX_perm, saved["slot"], dxr, dx_shared)
    return out
