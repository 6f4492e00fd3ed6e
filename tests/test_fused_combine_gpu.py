"""GPU: the top-1 combine fused into the down projection's epilogue
(moe_expert_ffn_combine) gives bitwise the outputs of moe_expert_ffn_rows
followed by moe_combine ([SW] eq. (2) plus the residual; [WIKI], cross-cutting
findings on fused dispatch / expert matmul / combine pipelines).

With one choice per token, the routed row r = slot[t] is token t's only expert
row, so the tile that computes y_perm[r] owns y[t]. Tokens whose choice was
dropped are copied by extra workgroups of the same launch. The epilogue takes
the same bf16 y_perm value and applies the combine's fp32 multiply-add in the
same order, so y must match bit for bit. The separate path is compared with
the oracle element by element in test_parity_gpu.py and test_full_size_gpu.py;
three reduced cases are compared with the oracle here as well.

Cases, with the instantiation each one reaches under the launcher's tile rule
(256x256 tiles when the average group has at least 256 rows and there are at
least 256 such tiles; layers capped at C <= 512 rows split into a 256x256
launch for groups of 64 rows or more and a 128x128 launch for the rest, which
also runs the copy workgroups):
  * capped_drops_small_tiles: gemm_bf16_kernel<128, 128, 64, 2, 0, 1, 7, 2, 0>
  * capped_split_pair: <256, 256, 64, 2, 0, 1, 7, 4, 0> then the 128x128 one
  * dropless_big_tiles: <256, 256, 64, 2, 0, 1, 7, 4, 0> alone (copy workgroups
    with nothing to copy)
  * ragged_swiglu: SwiGLU, d and f off the tile sizes, T not a multiple of 64
  * most_dropped: three quarters of the tokens dropped (most of y is copied)
  * noisy_top1, sigmoid_bias_top1: noisy top-1 and sigmoid gating with a
    selection bias (the routing differs; the fused step is the same)
  * switch_base at full size: the layer the fused bench forward times
"""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_mixture_experts_25_amd as M
from synth import CONFIGS, LayerConfig, make_inputs

from helpers import TOL_BF16, cfg_of, host64, oracle_inputs, relerr, relerr_sum, run_forward, to_dev, y_terms_abs

pytestmark = pytest.mark.gpu

CASES = {
    "capped_drops_small_tiles": LayerConfig("capped_drops_small_tiles", T=4096, d=512, f=1024, E=16, k=1,
                                            cf=1.0, alpha=0.01, logit_offset="normal", fwd_only=True),
    "capped_split_pair": LayerConfig("capped_split_pair", T=16384, d=1024, f=256, E=64, k=1, cf=2.0,
                                     logit_offset="logzipf", fwd_only=True),
    "dropless_big_tiles": LayerConfig("dropless_big_tiles", T=16384, d=1024, f=256, E=8, k=1, cf=0.0,
                                      fwd_only=True),
    "ragged_swiglu": LayerConfig("ragged_swiglu", T=1000, d=200, f=72, E=5, k=1, act="swiglu", cf=1.25,
                                 logit_offset="normal", fwd_only=True),
    "most_dropped": LayerConfig("most_dropped", T=2048, d=264, f=128, E=16, k=1, cf=0.25,
                                logit_offset="logzipf", fwd_only=True),
    # the other gates the entry point accepts with one choice per token
    "noisy_top1": LayerConfig("noisy_top1", T=1536, d=192, f=320, E=8, k=1, gate="noisy_topk", renorm=True,
                              cf=1.0, alpha=0.01, fwd_only=True),
    "sigmoid_bias_top1": LayerConfig("sigmoid_bias_top1", T=1536, d=192, f=320, E=8, k=1, gate="sigmoid_bias",
                                     sel_bias="uniform", cf=1.0, logit_offset="normal", fwd_only=True),
}
ORACLE = ["ragged_swiglu", "most_dropped", "sigmoid_bias_top1"]
NAN_BF16 = -1  # 0xFFFF: a bf16 NaN, so any output element left unwritten fails the comparison


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _fused_and_separate(c, dev):
    sep = run_forward(c, dev, backward=False, rows_in_place=True)
    fus = M.LayerBuffers.allocate(cfg_of(c), backward=False, rows_in_place=True)
    for k in ("y", "y_perm", "h_saved", "act_saved"):
        if k in fus.t:
            fus.t[k].view(torch.int16).fill_(NAN_BF16)
    M.forward(fus, dev, aux=True, fused_combine=True)
    torch.cuda.synchronize()
    return sep, fus


def _assert_bitwise(sep, fus, x):
    a, b = sep.t, fus.t
    n = int(a["expert_offsets"][-1].item())
    for k in ("slot", "expert_offsets", "topk_w"):
        assert torch.equal(a[k], b[k]), k
    for k in ("row_token", "y_perm", "h_saved", "act_saved"):  # written for the kept rows only
        if k in a:
            assert torch.equal(_bits(a[k][:n]), _bits(b[k][:n])), k
    assert torch.equal(_bits(a["y"]), _bits(b["y"])), "y"
    dropped = (a["slot"][:, 0] < 0)
    nd = int(dropped.sum().item())
    if nd:
        assert torch.equal(_bits(b["y"][dropped]), _bits(x[dropped])), "dropped tokens: y = x"
    return n, nd


@pytest.mark.parametrize("name", list(CASES))
def test_fused_combine_bitwise(name):
    c = CASES[name]
    print(f"\n[fused combine] {name} T={c.T} d={c.d} f={c.f} E={c.E} cf={c.cf} {c.act}", flush=True)
    dev = to_dev(make_inputs(c, seed=0, with_dy=False))
    sep, fus = _fused_and_separate(c, dev)
    n, nd = _assert_bitwise(sep, fus, dev["x"])
    print(f"  kept rows {n}, dropped tokens {nd}: y, y_perm, h bitwise equal", flush=True)
    if c.cf > 0 and name != "dropless_big_tiles":
        assert nd > 0, "the case is meant to drop tokens"
    if name == "most_dropped":
        assert nd > c.T // 2


@pytest.mark.parametrize("name", ORACLE)
def test_fused_combine_matches_oracle(name):
    c = CASES[name]
    inp = make_inputs(c, seed=1, with_dy=False)
    dev = to_dev(inp)
    _, fus = _fused_and_separate(c, dev)
    spec = O.Spec.of(c)
    inp64 = oracle_inputs(inp)
    fw = O.forward(spec, inp64)
    t = fus.t
    n = int(fw["n_rows"])
    np.testing.assert_array_equal(t["slot"].cpu().numpy(), fw["slot"])
    np.testing.assert_array_equal(t["row_token"][:n].cpu().numpy(), fw["row_token"][:n])
    assert relerr(host64(t["y_perm"][:n]), fw["y_perm"]) <= TOL_BF16
    assert relerr_sum(host64(t["y"]), fw["y"], y_terms_abs(fw, inp64["x"])) <= TOL_BF16


@pytest.mark.timeout(600)
def test_fused_combine_bitwise_full_size_switch_base():
    c = CONFIGS["switch_base"]
    assert c.k == 1 and c.shared == 0 and c.dtype == "bf16"
    print(f"\n[fused combine, full size] switch_base T={c.T} d={c.d} f={c.f} E={c.E}", flush=True)
    dev = to_dev(make_inputs(c, seed=0, device="cuda", with_dy=False))
    sep, fus = _fused_and_separate(c, dev)
    n, nd = _assert_bitwise(sep, fus, dev["x"])
    print(f"  kept rows {n}, dropped tokens {nd}: bitwise equal", flush=True)


def test_fused_combine_empty_batch():
    """T = 0: nothing to compute; the call succeeds and writes no rows."""
    c = CASES["most_dropped"].replace(name="empty", T=0)
    dev = to_dev(make_inputs(c, seed=0, with_dy=False))
    fus = M.LayerBuffers.allocate(cfg_of(c), backward=False, rows_in_place=True)
    M.forward(fus, dev, aux=True, fused_combine=True)
    torch.cuda.synchronize()
    assert int(fus.t["expert_offsets"][-1]) == 0
