"""GPU: the layer with the dispatch fused into the expert matmuls gives bitwise
the same results as the layer with a permuted copy of x.

Without x_perm, moe_dispatch / moe_route_ec write only the positions,
moe_expert_ffn_rows reads each routed row of the up projection as
x[row_token[r]] as its operand loads go out, and moe_backward gathers the same
rows for the weight gradient of the up projection ([WIKI], cross-cutting
findings on fused dispatch / expert matmul pipelines). The matmuls then load
the same bytes into the same places and accumulate in the same order, so every
output and gradient must equal the x_perm layer's bit for bit; the x_perm layer
is compared with the oracle element by element in test_parity_gpu.py,
test_parity_big_tiles_gpu.py and test_full_size_gpu.py. One reduced layer is
also compared with the oracle here, end to end.

Cases: every reduced layer of the parity suite (both activations, fp32 and
bf16, capped and dropless, shared expert, expert choice, noisy gating), the
256x256-tile layers of the big-tile suite (dropless, shared expert, the capped
split pair), and the two largest full-size layers, whose matmuls run in the
launch configuration the bench times.
"""
import numpy as np
import pytest
import torch

import oracle as O
from synth import CONFIGS, make_inputs

from helpers import TOL_BF16, dx_terms_abs, host64, oracle_inputs, relerr, relerr_sum, run_backward, run_forward, \
    to_dev, y_terms_abs
from test_parity_big_tiles_gpu import CASES as BIG_CASES
from test_parity_gpu import CASES as SMALL_CASES

# outputs compared over all their elements; row-indexed ones over the kept rows
_FULL = ["probs", "topk_idx", "topk_w", "expert_counts", "expert_offsets", "slot", "y", "aux", "act_shared",
         "h_shared", "y_shared", "noisy_logits", "dx", "dw_router", "dw1", "dw2", "dws1", "dws2"]
_ROWS = ["row_token", "act_saved", "h_saved", "y_perm"]

CASES = {n: c for n, c in SMALL_CASES.items()}
CASES.update({n: c for n, (c, _) in BIG_CASES.items() if not n.startswith("router_big")})
FULL = ["finegrained_top8", "deepseek_v3"]


def _both_ways(c, dev):
    bwd = not c.fwd_only
    out = []
    for rows_in_place in (False, True):
        buf = run_forward(c, dev, backward=bwd, rows_in_place=rows_in_place)
        if bwd:
            run_backward(buf, dev)
        out.append(buf)
    torch.cuda.synchronize()
    a, b = out
    assert "x_perm" in a.t and "x_perm" not in b.t
    return a, b


def _assert_bitwise(c, a, b):
    n = int(a.t["expert_offsets"][-1].item())
    assert n == int(b.t["expert_offsets"][-1].item())
    checked = []
    for k in _FULL + _ROWS:
        if k not in a.t:
            continue
        if k == "topk_idx" and c.routing == "expert_choice":
            continue  # not written under expert choice (the column is the expert)
        x, y = a.t[k], b.t[k]
        if k in _ROWS:
            x, y = x[:n], y[:n]
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.uint8) if y.dtype == torch.bfloat16 else y), k
        checked.append(k)
    return checked


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(CASES))
def test_rows_in_place_bitwise(name):
    c = CASES[name]
    print(f"\n[rows in place] {name} T={c.T} d={c.d} f={c.f} E={c.E} k={c.k} {c.dtype}", flush=True)
    dev = to_dev(make_inputs(c, seed=0))
    a, b = _both_ways(c, dev)
    checked = _assert_bitwise(c, a, b)
    print(f"  bitwise equal: {', '.join(checked)}", flush=True)


@pytest.mark.gpu
@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", FULL)
def test_rows_in_place_bitwise_full_size(name):
    c = CONFIGS[name]
    print(f"\n[rows in place, full size] {name} T={c.T} d={c.d} f={c.f} E={c.E} k={c.k}", flush=True)
    dev = to_dev(make_inputs(c, seed=0, device="cuda"))
    a, b = _both_ways(c, dev)
    checked = _assert_bitwise(c, a, b)
    print(f"  bitwise equal: {', '.join(checked)}", flush=True)


@pytest.mark.gpu
def test_rows_in_place_matches_oracle():
    """End to end against the oracle without the permuted copy (deepseek-shaped
    reduced layer: sigmoid gate with bias, shared expert, SwiGLU)."""
    c = SMALL_CASES["deepseek_v3_s"] if "deepseek_v3_s" in SMALL_CASES else SMALL_CASES["deepseek_v3"]
    inp = make_inputs(c, seed=0)
    dev = to_dev(inp)
    buf = run_forward(c, dev, backward=True, rows_in_place=True)
    run_backward(buf, dev)
    torch.cuda.synchronize()
    spec = O.Spec.of(c)
    inp64 = oracle_inputs(inp)
    fw = O.forward(spec, inp64)
    bw = O.backward(spec, inp64, fw, inp64["dy"])
    t = buf.t
    n = int(fw["n_rows"])
    np.testing.assert_array_equal(t["row_token"][:n].cpu().numpy(), fw["row_token"][:n])
    assert relerr(host64(t["y_perm"][:n]), fw["y_perm"]) <= TOL_BF16
    assert relerr_sum(host64(t["y"]), fw["y"], y_terms_abs(fw, inp64["x"])) <= TOL_BF16
    dy64 = inp64["dy"]
    assert relerr_sum(host64(t["dx"]), bw["dx"], dx_terms_abs(fw, bw, dy64)) <= TOL_BF16
    assert relerr(host64(t["dw1"]), bw["dw1"]) <= TOL_BF16
    assert relerr(host64(t["dw2"]), bw["dw2"]) <= TOL_BF16
