"""GPU parity, element by element against the oracle, on reduced layers sized so
that every grouped matmul runs on the tiles the large workloads use.

The grouped matmul picks its tiles on the host from the launch's row bound
(max_rows) and widths: 256x256 tiles when the groups average at least 256 rows,
every output width is at least 256 and the launch has at least 256 such tiles;
for capped layers (expert capacity <= 512) a row-ragged matmul runs as a split
pair, groups of >= 64 rows on 256x256 tiles and the rest on 128x128 tiles, and
the weight gradients (at most 512 rows deep) run on 128x128 tiles. `tile_plan`
below restates that rule and each case asserts the plan it was built for, so a
change of the rule that moves a case off its tiles fails here instead of
silently narrowing the coverage.

Kernel instantiations reached (gemm_bf16_kernel<BM, BN, BK, stages, kind,
B K-contiguous, epilogue, waves along N>):
  big_relu_dropless      <256,256,64,2,0,1,1,4> ReLU forward, <..,0,1,0,4> down
                         projection, <..,0,0,3,4> ReLU backward, <..,0,0,0,4> dgrad
                         of the up projection, <..,1,0,0,4> both weight gradients
  big_swiglu_shared      <256,256,64,2,0,1,2,4> SwiGLU forward, <..,0,0,4,4> SwiGLU
                         backward, and the rest as above, with the shared expert as
                         one more group of every launch; sigmoid gate + bias
  big_capped_relu        the split pair of every row-ragged matmul: split_part 1 on
                         the 256x256 instantiations above, split_part 2 on
                         <128,128,64,2,0,..>; both weight gradients on
                         <128,128,32,2,1,0,0,2>
  big_capped_swiglu      the same split pair with the SwiGLU epilogues
  router_big_finegrained router weight gradient <256,256,64,2,1,0,5,4> over 16 token
                         chunks (fine-grained top-8 router shape: T 32768, d 2048,
                         E 128) and the router input gradient <256,256,64,2,0,0,5,4>
  router_big_deepseek    router weight gradient over 6 token chunks (DeepSeek-V3
                         router shape: T 16384, d 7168, E 256, sigmoid + bias) and
                         the input gradient finished in the router product's
                         epilogue <256,256,64,2,0,0,6,4> with the shared expert

Each case checks, with the oracle computed once: the forward (routing, slots and
drops bit for bit; every float output within 2e-2, router outputs within 1e-5;
the layer output y and the input gradient dx, sums of terms each rounded to
bf16, measured against the sum of their terms' magnitudes, helpers.relerr_sum);
the backward end to end (GPU forward -> GPU backward, 2e-2); and the backward
stage-isolated (the oracle's saved tensors fed to moe_backward: every gradient
within 2e-2, the router weight gradient within 1e-5). ReLU pre-activations whose
sign fp32 accumulation cannot decide (oracle.relu_ambiguous) are left out of the
end-to-end comparison, and their count is printed.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from synth import LayerConfig, make_inputs

from helpers import TOL_BF16, TOL_F32, dx_terms_abs, gpu_saved_from_oracle, host64, oracle_inputs, relerr, \
    relerr_sum, run_backward, run_forward, to_dev, y_terms_abs


def _router_dw_splits(T, E, d):
    """Token chunks of the router weight gradient (restated from the library's rule)."""
    kp = (3 * E + 7) // 8 * 8
    big_tiles = math.ceil(kp / 256) * math.ceil(d / 256)
    if big_tiles * math.ceil(T / 256) >= 512:
        ns = math.ceil(512 / big_tiles)
        ns = min(ns, (128 << 20) // max(kp * d * 4, 1), T // 2048)
    else:
        tiles = math.ceil(kp / 128) * math.ceil(d / 128)
        ns = min(math.ceil(256 / tiles), T // 1024)
    return max(ns, 1)


def _tiles(kind, max_rows, groups, N, M=0, extra_group=False, row_cap=0):
    avg = max_rows // max(groups, 1)
    if kind == 0:
        n_big = math.ceil(max_rows / 256) * math.ceil(N / 256)
        dims = N >= 256
    else:
        n_big = (groups + (1 if extra_group else 0)) * math.ceil(M / 256) * math.ceil(N / 256)
        dims = M >= 256 and N >= 256
    if not (avg >= 256 and dims and n_big >= 256):
        return "128"
    if 0 < row_cap <= 512 and groups > 1:
        return "split" if kind == 0 else "128"
    return "256"


def tile_plan(c):
    """Tile choice of each matmul launch of one forward + backward step."""
    T, d, f, E, k = c.T, c.d, c.f, c.E, c.k
    f1 = 2 * f if c.act == "swiglu" else f
    C = O.capacity(T, E, c.cf)
    R = T * k if C < 0 else min(T * k, E * C)
    cap = C if C > 0 else 0
    sh = bool(c.shared)
    plan = {
        "ffn_gemm1": _tiles(0, R, E, f1, row_cap=cap),
        "ffn_gemm2": _tiles(0, R, E, d, row_cap=cap),
        "bwd_dgrad2": _tiles(0, R, E, f, row_cap=cap),
        "bwd_wgrad2": _tiles(1, R, E, f, M=d, extra_group=sh, row_cap=cap),
        "bwd_dgrad1": _tiles(0, R, E, d, row_cap=cap),
        "bwd_wgrad1": _tiles(1, R, E, d, M=f1, extra_group=sh, row_cap=cap),
    }
    kp = (3 * E + 7) // 8 * 8
    ns = _router_dw_splits(T, E, d)
    plan["router_dw"] = _tiles(1, T, ns, d, M=kp)
    plan["router_dx"] = _tiles(0, T, 1, d)
    plan["router_chunks"] = ns
    return plan


# a capped layer's split pair: groups of at least this many rows on the 256x256 launch
SPLIT_ROWS = 64
_GEMMS = ("ffn_gemm1", "ffn_gemm2", "bwd_dgrad2", "bwd_wgrad2", "bwd_dgrad1", "bwd_wgrad1")

CASES = {
    # R = 32768 rows over 64 experts: 128 row tiles x 2 column tiles of 256; d and f
    # not multiples of 64 (a partial K step in every matmul, partial column tiles)
    "big_relu_dropless": (LayerConfig("big_relu_dropless", T=16384, d=264, f=392, E=64, k=2, renorm=True,
                                      act="relu", cf=0.0, alpha=0.01, logit_offset="normal"),
                          {g: "256" for g in _GEMMS}),
    "big_swiglu_shared": (LayerConfig("big_swiglu_shared", T=16384, d=264, f=328, E=64, k=2,
                                      gate="sigmoid_bias", renorm=True, act="swiglu", cf=0.0, shared=1,
                                      sel_bias="uniform"),
                          {g: "256" for g in _GEMMS}),
    # capacity 512 (cf 2): skewed offsets leave groups from empty to full
    "big_capped_relu": (LayerConfig("big_capped_relu", T=16384, d=264, f=392, E=64, k=2, renorm=True,
                                    act="relu", cf=2.0, alpha=0.01, logit_offset="normal"),
                        {g: ("128" if "wgrad" in g else "split") for g in _GEMMS}),
    "big_capped_swiglu": (LayerConfig("big_capped_swiglu", T=16384, d=264, f=264, E=64, k=2, renorm=True,
                                      act="swiglu", cf=2.0, alpha=0.01, logit_offset="normal"),
                          {g: ("128" if "wgrad" in g else "split") for g in _GEMMS}),
    # router products at the full router shapes; a tiny expert width keeps the oracle cheap
    "router_big_finegrained": (LayerConfig("router_big_finegrained", T=32768, d=2048, f=16, E=128, k=4,
                                           renorm=True, act="relu", cf=0.0, alpha=0.01, logit_offset="logzipf"),
                               {"router_dw": "256", "router_dx": "256", "router_chunks": 16}),
    "router_big_deepseek": (LayerConfig("router_big_deepseek", T=16384, d=7168, f=16, E=256, k=2,
                                        gate="sigmoid_bias", renorm=True, act="swiglu", cf=0.0, shared=1,
                                        sel_bias="uniform"),
                            {"router_dw": "256", "router_dx": "256", "router_chunks": 6}),
}


@pytest.mark.parametrize("name", list(CASES))
def test_tile_plan(name):
    """The case reaches the tiles it was built for (host-side rule, no GPU work)."""
    c, want = CASES[name]
    plan = tile_plan(c)
    for key, v in want.items():
        assert plan[key] == v, (key, plan)


def _poison_weight_grads(t):
    for key in ("dw1", "dw2", "dws1", "dws2"):
        if t.get(key) is not None:
            t[key].fill_(float("nan"))


def run_forward_backward_again(buf, dev):
    import sparse_mixture_experts_25_amd as M
    M.forward(buf, dev, aux=True)
    run_backward(buf, dev)
    torch.cuda.synchronize()


def _report_dx(c, fw, bw, inp64, dx, what):
    """Print the worst input-gradient elements with the oracle's terms of the sum
    (dy, the kept expert rows, the router term, the shared expert)."""
    r = bw["dx"]
    rms = float(np.sqrt(np.mean(r * r)))
    err = np.abs(dx - r) / np.maximum(np.abs(r), rms)
    flat = np.argsort(err, axis=None)[-3:][::-1]
    for i in flat:
        tt, j = np.unravel_index(i, err.shape)
        rows = [int(sl) for sl in fw["slot"][tt] if sl >= 0]
        terms = [inp64["dy"][tt, j]] + [bw["dX_perm"][sl, j] for sl in rows] + [bw["dx_router"][tt, j]]
        if c.shared:
            terms.append(bw["dx_shared"][tt, j])
        print(f"  {what} dx worst: relerr {err[tt, j]:.4f} token {tt} col {j} gpu {dx[tt, j]:.6g} oracle {r[tt, j]:.6g} "
              f"rms {rms:.3g} terms " + " ".join(f"{v:.5g}" for v in terms), flush=True)


def _relu_ambiguity(c, inp64, fw):
    """(row mask [n, f] of ambiguous pre-activations, shared-expert mask [T, f] or None)."""
    if c.act != "relu":
        return np.zeros(fw["act"].shape, bool), None
    amb = O.relu_ambiguous_rows(fw["x_perm"], inp64["w1"], fw["offsets"], fw["act"])
    amb_sh = O.relu_ambiguous(inp64["x"], inp64["ws1"], fw["act_shared"]) if c.shared else None
    return amb, amb_sh


def _parity_params():
    # the router-shape cases run the oracle's router products at full router size
    # (about a minute of host work on 16 threads)
    for n in CASES:
        yield pytest.param(n, marks=[pytest.mark.timeout(900)] if n.startswith("router_big") else [])


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(_parity_params()))
def test_big_tiles_parity(name):
    c, want = CASES[name]
    plan = tile_plan(c)
    print(f"\n[big tiles] {name} T={c.T} d={c.d} f={c.f} E={c.E} k={c.k} plan={plan}", flush=True)
    inp = make_inputs(c, seed=0)
    dev = to_dev(inp)
    buf = run_forward(c, dev, backward=True)
    run_backward(buf, dev)
    torch.cuda.synchronize()
    spec = O.Spec.of(c)
    inp64 = oracle_inputs(inp)
    fw = O.forward(spec, inp64)
    bw = O.backward(spec, inp64, fw, inp64["dy"])
    t = buf.t
    n = int(fw["n_rows"])
    rows = np.diff(fw["offsets"])
    print(f"  kept rows {n}, groups >= {SPLIT_ROWS} rows: {int((rows >= SPLIT_ROWS).sum())}, "
          f"1..{SPLIT_ROWS - 1} rows: {int(((rows > 0) & (rows < SPLIT_ROWS)).sum())}, "
          f"empty: {int((rows == 0).sum())}", flush=True)
    if want.get("ffn_gemm1") == "split":
        # both launches of the split pair have groups to run
        assert (rows >= SPLIT_ROWS).any() and ((rows > 0) & (rows < SPLIT_ROWS)).any()

    # ---- forward
    np.testing.assert_array_equal(t["topk_idx"].cpu().numpy(), fw["idx"])
    np.testing.assert_array_equal(t["expert_counts"].cpu().numpy(), fw["counts"])
    np.testing.assert_array_equal(t["expert_offsets"].cpu().numpy(), fw["offsets"])
    np.testing.assert_array_equal(t["slot"].cpu().numpy(), fw["slot"])
    np.testing.assert_array_equal(t["row_token"][:n].cpu().numpy(), fw["row_token"][:n])
    assert relerr(host64(t["probs"]), fw["probs"]) <= TOL_F32
    assert relerr(host64(t["topk_w"]), fw["w"]) <= TOL_F32
    np.testing.assert_array_equal(host64(t["x_perm"][:n]), fw["x_perm"])
    if "act_saved" in t:
        assert relerr(host64(t["act_saved"][:n]), fw["act"]) <= TOL_BF16
    assert relerr(host64(t["h_saved"][:n]), fw["h"]) <= TOL_BF16
    assert relerr(host64(t["y_perm"][:n]), fw["y_perm"]) <= TOL_BF16
    assert relerr_sum(host64(t["y"]), fw["y"], y_terms_abs(fw, inp64["x"])) <= TOL_BF16
    if c.shared:
        assert relerr(host64(t["y_shared"]), fw["y_shared"]) <= TOL_BF16
    if c.alpha:
        assert abs(float(t["aux"][0]) - fw["aux"]) <= TOL_F32 * abs(fw["aux"])

    # ---- backward, stage-isolated: every element, router weight gradient at 1e-5
    # (the weight gradients start as NaN, so an element the backward leaves
    # unwritten, such as a zero tile of an expert without rows, fails below)
    saved = gpu_saved_from_oracle(c, fw, buf.info)
    _poison_weight_grads(t)
    run_backward(buf, dev, saved=saved)
    torch.cuda.synchronize()
    _report_dx(c, fw, bw, inp64, host64(t["dx"]), "stage-isolated")
    dx_terms = dx_terms_abs(fw, bw, inp64["dy"])
    assert relerr_sum(host64(t["dx"]), bw["dx"], dx_terms) <= TOL_BF16
    assert relerr(host64(t["dw1"]), bw["dw1"]) <= TOL_BF16
    assert relerr(host64(t["dw2"]), bw["dw2"]) <= TOL_BF16
    assert relerr(host64(t["dw_router"]), bw["dw_router"]) <= TOL_F32
    if c.shared:
        assert relerr(host64(t["dws1"]), bw["dws1"]) <= TOL_BF16
        assert relerr(host64(t["dws2"]), bw["dws2"]) <= TOL_BF16

    # ---- backward, end to end (ambiguous ReLU signs left out)
    _poison_weight_grads(t)
    run_forward_backward_again(buf, dev)
    _report_dx(c, fw, bw, inp64, host64(t["dx"]), "end-to-end")
    amb, amb_sh = _relu_ambiguity(c, inp64, fw)
    print(f"  ReLU pre-activations within accumulation error of zero: {int(amb.sum())}"
          + (f" (+{int(amb_sh.sum())} shared)" if amb_sh is not None else ""), flush=True)
    row_ok = ~amb.any(1)
    tok_ok = np.ones(c.T, bool)
    kt, kr = np.nonzero(fw["slot"] >= 0)
    bad = ~row_ok[fw["slot"][kt, kr]]
    tok_ok[kt[bad]] = False
    if amb_sh is not None:
        tok_ok &= ~amb_sh.any(1)
    f1 = fw["act"].shape[1]
    m1 = np.ones((c.E, f1, c.d), bool)
    for e in range(c.E):
        a, b = fw["offsets"][e], fw["offsets"][e + 1]
        m1[e, amb[a:b].any(0), :] = False
    tokm = np.repeat(tok_ok[:, None], c.d, 1)
    assert relerr_sum(host64(t["dx"]), bw["dx"], dx_terms, tokm) <= TOL_BF16
    assert relerr(host64(t["dw1"]), bw["dw1"], m1) <= TOL_BF16
    assert relerr(host64(t["dw2"]), bw["dw2"]) <= TOL_BF16
    # the router gradient sums every token's logit gradient: a token with an
    # ambiguous mask moves it by its share only, so it is compared whole
    assert relerr(host64(t["dw_router"]), bw["dw_router"]) <= TOL_BF16
    if c.shared:
        ms = np.ones_like(bw["dws1"], bool)
        if amb_sh is not None:
            ms[amb_sh.any(0), :] = False
        assert relerr(host64(t["dws1"]), bw["dws1"], ms) <= TOL_BF16
        assert relerr(host64(t["dws2"]), bw["dws2"]) <= TOL_BF16
    empty = rows == 0
    print(f"  experts without rows: {int(empty.sum())} (their weight gradients must be exact zeros)", flush=True)
    if empty.any():
        assert torch.all(t["dw1"][torch.from_numpy(empty).cuda()] == 0)
        assert torch.all(t["dw2"][torch.from_numpy(empty).cuda()] == 0)
    for key in ("dw1", "dw2", "dws1", "dws2"):
        if t.get(key) is not None:
            assert bool(torch.isfinite(t[key]).all()), key
