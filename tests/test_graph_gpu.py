"""The whole layer step (forward, aux loss, selection-bias step, backward)
captured once in a HIP graph and replayed: every replay must give the same
bytes as the eager step. The library allocates nothing, synchronises nothing
and issues no memset, so its launches can be captured as they are. Between
replays the test does eager work of its own (restoring the bias state and
clearing every output), so a replay that skipped or reordered a kernel would
show up as stale or zero data."""
import pytest
import torch

import sparse_mixture_experts_25_amd as M
from synth import SMALL, LayerConfig, make_inputs

from helpers import cfg_of, to_dev

pytestmark = pytest.mark.gpu

BIAS_GAMMA = 1e-3

GRAPH_CASES = {
    "switch_base_s": SMALL["switch_base"],
    # the forward with the top-1 combine in the down projection (moe_expert_ffn_combine, no x_perm)
    "switch_base_s_fused": SMALL["switch_base"],
    "gshard_top2_s": SMALL["gshard_top2"],
    "deepseek_v3_s": SMALL["deepseek_v3"],
    "ec_relu": LayerConfig("ec_relu", T=777, d=192, f=320, E=8, k=8, act="relu", cf=2.0, gate="softmax",
                           renorm=False, alpha=0.0, routing="expert_choice"),
    "noisy_relu": LayerConfig("noisy_relu", T=777, d=192, f=320, E=8, k=2, act="relu", cf=1.25,
                              gate="noisy_topk", renorm=True, alpha=0.01),
}

# rows of these buffers at or past the kept count are never written
ROW_BUFFERS = ("row_token", "x_perm", "act_saved", "h_saved", "y_perm")


def _outputs(buf, c):
    n = int(buf.t["expert_offsets"][-1])
    out = {}
    for k, v in buf.t.items():
        if k == "ws" or (k == "topk_idx" and c.routing == "expert_choice"):
            continue
        out[k] = (v[:n] if k in ROW_BUFFERS else v).clone()
    return out


@pytest.mark.parametrize("name", list(GRAPH_CASES))
def test_graph_replay_matches_eager(name):
    c = GRAPH_CASES[name]
    inp = to_dev(make_inputs(c))
    cfg = cfg_of(c)
    fused = name.endswith("_fused")
    buf = M.LayerBuffers.allocate(cfg, rows_in_place=fused)
    biased = c.gate in ("sigmoid_bias", "sqrt_softplus_bias")
    bias0 = inp["sel_bias"].clone() if biased else None

    def step():
        M.forward(buf, inp, aux=True, fused_combine=fused)
        if biased:
            M.moe_bias_update(cfg, buf.t["expert_counts"], BIAS_GAMMA, inp["sel_bias"])
        M.backward(buf, inp, inp["dy"])

    def reset():
        if biased:
            inp["sel_bias"].copy_(bias0)
        for k, v in buf.t.items():
            v.zero_()

    reset()
    step()
    torch.cuda.synchronize()
    ref = _outputs(buf, c)
    ref_bias = inp["sel_bias"].clone() if biased else None

    # one eager pass on a side stream first, as torch asks before a capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        reset()
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _outputs(buf, c)
        for k in ref:
            assert torch.equal(got[k], ref[k]), (rep, k)
        if biased:
            assert torch.equal(inp["sel_bias"], ref_bias), rep
