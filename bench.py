"""Benchmark: MoE layer forward + backward tokens/s on one MI355X.

One step = the whole layer on one batch: moe_route, moe_dispatch,
moe_expert_ffn, moe_combine, moe_aux_loss, moe_backward (all through the C ABI,
inputs already resident in HBM), plus moe_bias_update for the gates that carry
a selection bias (the aux-loss-free balancing step, gamma = 1e-3, or with
--balance quantile the Quantile-Balancing step). Default workload: the
DeepSeek-V3-shaped layer, the largest of the five that fits one GPU (T=16384
tokens, d_model=7168, 256 routed SwiGLU experts 7168->2048->7168 plus one
always-on shared expert of the same shape, sigmoid gate with a per-expert
selection bias, top-8 renormalised, dropless, bf16 activations and weights, fp32
router). --config picks another (switch_base, gshard_top2, finegrained_top8,
tiny_f32). The dispatch is fused into the expert matmuls: moe_dispatch writes
only the positions and moe_expert_ffn_rows / moe_backward read the routed rows
of x through row_token; --x-perm times the layer with the permuted copy instead.

Prints one JSON line (see the keys below). Also measured and reported:
  roofline: the stage with the largest per-launch time, timed with HIP events on
    its own stream over the timed region, against its algorithmic bytes or flops;
  cpu_baseline: the oracle (plain C++ in double) on a bounded token sample of the
    same layer, on this host's cores (rank 0, N=1 only).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12          # B/s, MI355X HBM3E
PEAK_BF16 = 2.5e15         # flop/s, dense bf16 matrix cores
# flop/s, fp32 vector FMA without packed-fp32 instructions: 256 CUs x 64 FMA lanes
# per clock x 2 flop x 2.4 GHz (packed fp32 would double it; it is not generated)
PEAK_F32_VALU = 78.6e12

# step of the aux-loss-free selection-bias update (the pages give no value)
BIAS_GAMMA = 1e-3

# Kernel sources whose hash a measured HBM-traffic figure is tied to (all of them:
# the counter summaries cover every stage).
KERNEL_SOURCES = ("api.hip", "balance.hip", "common.h", "dispatch.hip", "ec_route.hip", "gate_math.h", "gemm_bf16.hip",
                  "gemm_common.h", "gemm_f32.hip", "internal.h", "mfma_tile.h", "noisy.hip", "router.hip",
                  "router_bwd.hip", "rows.hip")


def sources_sha(names):
    """Hash of the kernel sources with comments and blank space removed, so an
    edit to comments alone keeps a measured figure valid."""
    import hashlib
    import re
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "sparse_mixture_experts_25_amd", "csrc", n)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload, stage=None):
    """HBM bytes per launch of `stage` (or a dict of every stage's) from the
    committed counter summary profiles/hbm_traffic_<workload>.txt (FETCH_SIZE +
    WRITE_SIZE per dispatch, scaled by the same counters' reading for a plain copy
    of known size), or None when there is none or the kernel sources changed since
    it was taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    sha, vals = None, {}
    with open(path) as fh:
        for ln in fh:
            parts = ln.split()
            if len(parts) >= 2 and parts[0] == "sources_sha":
                sha = parts[1]
            if len(parts) >= 2 and parts[0].endswith("_bytes_per_launch"):
                vals[parts[0][:-len("_bytes_per_launch")]] = float(parts[1])
    if sha != sources_sha(KERNEL_SOURCES):
        return None
    return vals if stage is None else vals.get(stage)


def stage_roofline(stage, work, ms, dtype="bf16"):
    """Roofline of one launch of `stage` with (flops, bytes) = work taking `ms`:
    the exact fp32 router stages on the vector units (the logits always; the
    router gradients of fp32 layers) against the fp32 ALU, the grouped matmuls
    against the matrix cores when their arithmetic intensity is past the ridge
    point (else HBM), everything else against HBM (including the bf16 layers'
    router gradients, which run as split-operand matrix products)."""
    fl, by = work
    if stage in ("route", "route_ec") or (stage == "bwd_router_grads" and dtype != "bf16"):
        # exact fp32 router: sequential fp32 FMA on the vector units
        roof = {"bound": "alu", "achieved": fl / (ms * 1e-3) / 1e12, "peak": PEAK_F32_VALU / 1e12,
                "unit": "TFLOP/s"}
    elif fl and fl / max(by, 1) > PEAK_BF16 / PEAK_HBM and stage.startswith(("ffn", "bwd_dgrad", "bwd_wgrad")):
        roof = {"bound": "mfma", "achieved": fl / (ms * 1e-3) / 1e12, "peak": PEAK_BF16 / 1e12,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": by / (ms * 1e-3) / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    att = attainable_peak(roof["bound"])
    if att:
        roof["attainable_peak"] = att
        roof["frac_attainable"] = roof["achieved"] / att
    return roof


def attainable_peak(bound):
    """What the probe kernels of include/moe_peaks.h reach on MI355X
    (profiles/attainable_peaks.txt (JSON), from `bench.py --peaks`), in the roofline's
    unit: the higher of the streaming read and write rates for "hbm", the
    register-only MFMA loop for "mfma", the fp32 FMA loop for "alu"."""
    path = os.path.join(ROOT, "profiles", "attainable_peaks.txt")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        pk = json.load(fh)["peaks"]
    return {"hbm": max(pk["hbm_read_GBps"], pk["hbm_write_GBps"]), "mfma": pk["mfma_bf16_TFLOPs"],
            "alu": pk["fma_f32_TFLOPs"]}.get(bound)


class HipEvents:
    """Raw HIP events (for the library's stage timing hook)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            p = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(p)) == 0
            self.ev[i] = p
        self.n = n

    def elapsed_ms(self, a, b):
        self.hip.hipEventSynchronize(self.ev[b])
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), self.ev[a], self.ev[b]) == 0
        return ms.value


def stage_work(c, rows, ne_experts, permuted_copy=False):
    """Algorithmic (flops, bytes) of one launch of each stage, from the realised routing.
    rows: kept routed rows; ne_experts: experts with at least one row; permuted_copy:
    the dispatch writes x_perm (otherwise the matmuls read the rows of x in place)."""
    T, d, f, E, k = c.T, c.d, c.f, c.E, c.k
    ER = 2 * E if c.gate == "noisy_topk" else E  # router rows (clean + noise for noisy gating)
    f1 = 2 * f if c.act == "swiglu" else f
    eb = 2 if c.dtype == "bf16" else 4
    S = T if c.shared else 0
    R = rows + S
    W1 = (ne_experts + (1 if c.shared else 0)) * f1 * d * eb
    W2 = (ne_experts + (1 if c.shared else 0)) * d * f * eb
    W1all = (E + (1 if c.shared else 0)) * f1 * d * eb
    W2all = (E + (1 if c.shared else 0)) * d * f * eb
    return {
        "route": (2 * T * d * ER, T * d * eb + ER * d * 4 + T * ER * 4 + T * k * 8),
        # logits, softmax (probs + transposed copy), selection, token tables, gather
        "route_ec": (2 * T * d * E, T * d * eb + E * d * 4 + T * E * 4 * 6 + rows * 4 +
                     (rows * d * eb * 2 if permuted_copy else 0)),
        # token tables (indices read, positions written, slots written), row map; the copy
        "dispatch": (0, T * k * 4 * 3 + rows * 4 + ((T * d * eb + rows * d * eb) if permuted_copy else 0)),
        # SwiGLU stores the pre-activations and h; ReLU only h
        "ffn_gemm1": (2 * R * d * f1, W1 + R * d * eb + R * ((f1 if c.act == "swiglu" else 0) + f) * eb),
        "ffn_gemm2": (2 * R * f * d, W2 + R * f * eb + R * d * eb),
        "combine": (0, T * d * eb * (2 + (1 if c.shared else 0)) + rows * d * eb + T * k * 8),
        # top-1: the down projection with the combine in its epilogue (x read, y written, the token of
        # each row, the weight and slot of each token)
        "ffn_gemm2_combine": (2 * R * f * d, W2 + R * f * eb + R * d * eb + 2 * T * d * eb + rows * 4 + T * 8),
        "aux": (0, T * E * 4),
        "bwd_combine": (0, T * d * eb + rows * d * eb * 2 + T * k * 12),
        "bwd_dgrad2": (2 * R * d * f, W2 + R * d * eb + 2 * R * f1 * eb),
        "bwd_wgrad2": (2 * R * d * f, W2all + R * d * eb + R * f * eb),
        "bwd_dgrad1": (2 * R * f1 * d, W1 + R * f1 * eb + R * d * eb),
        "bwd_wgrad1": (2 * R * f1 * d, W1all + R * f1 * eb + R * d * eb),
        "bwd_dlogits": (0, T * E * 8 + T * k * 12),
        # bf16 with k <= 2: the dx_router product's epilogue also does the unpermute pass
        "bwd_router_grads": (4 * T * d * ER, T * ER * 4 + T * d * eb + ER * d * 4 * 2 +
                             (T * d * eb * 2 + rows * d * eb if (eb == 2 and k <= 2) else T * d * 4)),
        "bwd_unpermute": (0, T * d * eb * 2 + rows * d * eb + T * d * 4),
        "bias_update": (0, E * 4 * 3),
        # gate values read twice (cuts, margins), margins written and read twice (two selects)
        "bias_quantile": (0, T * E * 4 * 5 + T * 16 * 2),
    }


def check_determinism(buf, inp, step, c):
    """After the timed region: the step twice more from the same state (the
    selection bias restored between the two), with the routing tables, the
    output, the input gradient and every weight gradient compared bit for bit."""
    import torch
    keys = ["expert_counts", "expert_offsets", "slot", "topk_w", "y", "dx", "dw_router", "dw1", "dw2", "dws1", "dws2"]
    if c.routing != "expert_choice":
        keys.append("topk_idx")  # written by token-choice routing only
    keys = [k for k in keys if k in buf.t]
    bias0 = inp["sel_bias"].clone() if "sel_bias" in inp else None
    step()
    torch.cuda.synchronize()
    first = {k: buf.t[k].clone() for k in keys}
    if bias0 is not None:
        inp["sel_bias"].copy_(bias0)
    step()
    torch.cuda.synchronize()
    differ = [k for k in keys if not torch.equal(first[k].view(torch.uint8), buf.t[k].view(torch.uint8))]
    del first
    return {"runs": 2, "compared": keys, "bitwise_equal": not differ, "differ": differ}


def cpu_baseline_sized(c, inp, target_s=20.0, probe_tokens=16):
    """Oracle timing on a sample of about `target_s` seconds: start from
    `probe_tokens` tokens and grow the sample (at most 8x per try, scaled by the
    time the last try took) until a try takes at least half the target or covers
    the whole batch; the last try is the result. (The oracle's cost has a large
    per-expert part, so a small probe overstates the cost per token.)"""
    n = min(probe_tokens, c.T)
    while True:
        r = cpu_baseline(c, inp, n)
        if r["seconds"] >= 0.5 * target_s or n == c.T:
            return r
        n = min(c.T, max(n + 1, int(n * min(8.0, target_s / max(r["seconds"], 1e-3)))))


class _ExpertsF64:
    """Per-expert float64 view of a [E, ...] weight tensor, widened on first use
    (the oracle reads only the experts the sampled tokens reach, so the full
    expert weights are never widened at once)."""

    def __init__(self, t, f64):
        self.t, self.f64, self.cache = t, f64, {}
        self.shape = tuple(t.shape)

    def __len__(self):
        return self.shape[0]

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            self.cache[e] = self.f64(self.t[e])
        return self.cache[e]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(c, inp, budget_tokens):
    """Oracle forward+backward of the same layer on the first `budget_tokens` tokens
    (an independent batch of that size; capacity follows the formula for it)."""
    import oracle as O
    sub = c.replace(T=budget_tokens)
    oin = {}
    for k, v in inp.items():
        if k in ("w1", "w2"):
            oin[k] = _ExpertsF64(v, O.f64)
        else:
            oin[k] = O.f64(v[:budget_tokens] if k in ("x", "dy", "noise") else v)
    if os.environ.get("MOE_ORACLE_THREADS"):
        O.lib().orc_set_threads(int(os.environ["MOE_ORACLE_THREADS"]))
    spec = O.Spec.of(sub)
    fw = O.route(spec, oin["x"], oin["w_router"], oin.get("logit_offset"), oin.get("sel_bias"), oin.get("noise"))
    for e in np.unique(fw["idx"]):  # widen the reached experts' weights before the clock starts
        oin["w1"][e], oin["w2"][e]
    t0 = time.perf_counter()
    fw = O.forward(spec, oin)
    O.backward(spec, oin, fw, oin["dy"])
    dt = time.perf_counter() - t0
    threads = O.lib().orc_get_threads()  # what the oracle's OpenMP loops use
    return {"value": budget_tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(), "seconds": dt,
            "sample": f"{budget_tokens}-token batch of the same layer (same weights), forward+backward, "
                      f"{dt:.1f} s"}


def measure_peaks(torch, M, reps=10):
    """Attainable peaks from the probe kernels of include/moe_peaks.h (median of `reps` launches each)."""
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        ts.sort()
        return ts[len(ts) // 2]

    sink = torch.empty(M.moe_peak_sink_bytes() // 4, dtype=torch.float32, device="cuda")
    nb = 4 << 30  # far above the 256 MB last-level cache
    src = torch.empty(nb, dtype=torch.uint8, device="cuda")
    dst = torch.empty(nb, dtype=torch.uint8, device="cuda")
    M.moe_peak_write(src)  # touch every page before timing
    out = {}
    out["hbm_read_GBps"] = nb / timed(lambda: M.moe_peak_read(src, sink)) / 1e9
    out["hbm_write_GBps"] = nb / timed(lambda: M.moe_peak_write(dst)) / 1e9
    half = nb // 2
    out["hbm_copy_GBps"] = 2 * half / timed(lambda: M.moe_peak_copy(dst, src, nbytes=half)) / 1e9
    torch.cuda.synchronize()
    del src, dst
    it = 4000
    out["mfma_bf16_TFLOPs"] = M.MOE_PEAK_BLOCKS * 4 * it * 4 * 32768 / timed(
        lambda: M.moe_peak_mfma_bf16(sink, it)) / 1e12
    it = 5000
    out["fma_f32_TFLOPs"] = M.MOE_PEAK_BLOCKS * 256 * it * 64 * 2 / timed(lambda: M.moe_peak_fma_f32(sink, it)) / 1e12
    # library context: the vendor GEMM on a large square bf16 product (not one of the layer's kernels)
    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    out["torch_matmul_bf16_8192_TFLOPs"] = 2 * n ** 3 / timed(lambda: torch.matmul(a, b)) / 1e12
    return {"peaks": {k: round(v, 1) for k, v in out.items()},
            "published": {"hbm_GBps": PEAK_HBM / 1e9, "mfma_bf16_TFLOPs": PEAK_BF16 / 1e12,
                          "fma_f32_TFLOPs": PEAK_F32_VALU / 1e12},
            "probe": "include/moe_peaks.h kernels, median of %d launches; HBM buffers 4 GiB" % reps}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="deepseek_v3")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--balance", default="sign", choices=["sign", "quantile"],
                    help="selection-bias step of the bias-carrying gates: sign (fixed step) or quantile")
    ap.add_argument("--routing", default="token_choice", choices=["token_choice", "expert_choice"],
                    help="expert_choice: every expert takes its top tokens (k = E, capacity from cf)")
    ap.add_argument("--gate", default=None, choices=["softmax", "sigmoid_bias", "sqrt_softplus_bias", "noisy_topk"],
                    help="override the workload's gate (a bias-carrying gate draws the selection bias)")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="oracle sample size for cpu_baseline (default: sized from a 16-token probe for about "
                         "20 s of host work)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="OpenMP threads of the oracle timing (default: the host's setting); 1 gives the "
                         "single-thread baseline")
    ap.add_argument("--stages", action="store_true", help="also print per-stage times to stderr")
    ap.add_argument("--x-perm", action="store_true",
                    help="materialise the permuted copy of x (moe_dispatch writes x_perm, moe_expert_ffn reads "
                         "it); by default the expert matmuls read the routed rows of x in place")
    ap.add_argument("--separate-combine", action="store_true",
                    help="top-1 bf16 layers: run the combine as its own pass (moe_expert_ffn_rows + "
                         "moe_combine) instead of in the down projection's epilogue (moe_expert_ffn_combine)")
    ap.add_argument("--flush-mib", type=int, default=0,
                    help="write a scratch buffer of this many MiB before every timed step, so the 256 MB "
                         "last-level cache cannot serve the step's reads from the previous one; the per-step "
                         "median and min then exclude it (ms_per_step still brackets all K steps)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed region, run one plain device copy of this many MiB (a known-size "
                         "kernel to scale HBM counters against)")
    ap.add_argument("--peaks", action="store_true",
                    help="measure the attainable HBM, matrix-core and fp32-ALU peaks with the library's probe "
                         "kernels, print them as one JSON line and exit")
    args = ap.parse_args()
    if args.cpu_threads:
        # set in the oracle's OpenMP runtime itself when it is loaded
        os.environ["MOE_ORACLE_THREADS"] = str(args.cpu_threads)
    if args.gpus != 1:
        print(f"bench.py: the layer runs on one GPU; --gpus {args.gpus} is not supported "
              f"(there is no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_mixture_experts_25_amd as M
    from synth import CONFIGS, make_inputs

    if args.peaks:
        print(json.dumps(measure_peaks(torch, M)), flush=True)
        return

    c = CONFIGS[args.config]
    if c.fwd_only:
        c = c.replace(fwd_only=False)
    if args.gate and args.gate != c.gate:
        c = c.replace(gate=args.gate, sel_bias="uniform" if args.gate in ("sigmoid_bias", "sqrt_softplus_bias")
                      else "none")
        if args.gate == "noisy_topk":  # softmax over the top-k: renormalised; no per-expert logit offset
            c = c.replace(renorm=True, logit_offset="none")
    if args.routing == "expert_choice":
        # each expert takes C = ceil(T/E * cf) tokens: the same rows as top-k at cf = k
        c = c.replace(name=c.name + "_ec", routing="expert_choice", k=c.E, gate="softmax", renorm=False,
                      alpha=0.0, sel_bias="none", cf=c.cf if c.cf > 0 else float(c.k))
    torch.cuda.set_device(0)
    inp = make_inputs(c, seed=args.seed, device="cuda")
    cfg = M.make_config(c.T, c.d, c.f, c.E, c.k, cf=c.cf, renorm=c.renorm, gate=c.gate, act=c.act,
                        dtype=c.dtype, alpha=c.alpha, shared=c.shared, routing=c.routing)
    buf = M.LayerBuffers.allocate(cfg, rows_in_place=not args.x_perm)
    stream = torch.cuda.current_stream()
    # top-1 token choice in bf16 without a shared expert: the combine runs in the down projection's epilogue
    fused_combine = (not args.x_perm and not args.separate_combine and c.k == 1 and not c.shared and
                     c.dtype == "bf16" and c.routing == "token_choice")

    biased = c.gate in ("sigmoid_bias", "sqrt_softplus_bias")

    def step():
        M.forward(buf, inp, stream=stream, fused_combine=fused_combine)
        if biased and args.balance == "quantile":
            M.moe_bias_quantile(cfg, buf.t["probs"], inp["sel_bias"], buf.t["ws"], stream=stream)
        elif biased:
            M.moe_bias_update(cfg, buf.t["expert_counts"], BIAS_GAMMA, inp["sel_bias"], stream=stream)
        M.backward(buf, inp, inp["dy"], stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-stage times over a few steps (every stage armed) to find the dominant one
    nst = 32
    ev = HipEvents(2 * nst * 4)
    M.lib().moe_profile_arm.argtypes = [ctypes.c_char_p, ctypes.c_void_p, ctypes.c_int]
    M.lib().moe_profile_stage.restype = ctypes.c_char_p
    M.lib().moe_profile_arm(None, ctypes.cast(ev.ev, ctypes.c_void_p), nst * 4)
    for _ in range(3):
        step()
    npairs = M.lib().moe_profile_disarm()
    torch.cuda.synchronize()
    per_stage = {}
    for i in range(npairs):
        name = M.lib().moe_profile_stage(i).decode()
        per_stage.setdefault(name, []).append(ev.elapsed_ms(2 * i, 2 * i + 1))
    per_stage = {k: sum(v) / len(v) for k, v in per_stage.items()}
    dom = max(per_stage, key=per_stage.get)

    # timed region: K steps; the dominant stage's launches are bracketed by events,
    # and every step by a pair of its own (for the median and min)
    evd = HipEvents(2 * args.steps)
    M.lib().moe_profile_arm(dom.encode(), ctypes.cast(evd.ev, ctypes.c_void_p), args.steps)
    flush = torch.empty(args.flush_mib << 18, dtype=torch.float32, device="cuda") if args.flush_mib else None
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        if flush is not None:
            flush.fill_(float(i))
        sev[i][0].record(stream)
        step()
        sev[i][1].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    nd = M.lib().moe_profile_disarm()
    determinism = check_determinism(buf, inp, step, c)
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / args.steps
    per_step = sorted(a.elapsed_time(b) for a, b in sev)
    dom_ms = sum(evd.elapsed_ms(2 * i, 2 * i + 1) for i in range(nd)) / max(nd, 1)

    offs = buf.t["expert_offsets"].cpu()
    rows = int(offs[-1])
    ne = int(((offs[1:] - offs[:-1]) > 0).sum())
    work = stage_work(c, rows, ne, permuted_copy=args.x_perm)
    roof = stage_roofline(dom, work[dom], dom_ms, c.dtype)
    roof["traffic"] = measured_traffic(c.name, dom)
    roof["kernel"] = dom
    roof["launch_ms"] = dom_ms

    total_flops = sum(v[0] for v in work.values())
    # weight gradients are overwritten: experts without rows get zeros, written
    # inside the two weight-gradient launches (reported on its own line)
    f1 = 2 * c.f if c.act == "swiglu" else c.f
    eb = 2 if c.dtype == "bf16" else 4
    zero_bytes = (c.E - ne) * (f1 * c.d + c.d * c.f) * eb
    wr = attainable_peak("hbm")
    zero_fill = {"empty_experts": c.E - ne, "bytes": zero_bytes,
                 "ms_at_8TBps": zero_bytes / PEAK_HBM * 1e3,
                 "ms_at_measured_write_rate": (zero_bytes / (wr * 1e9) * 1e3) if wr else None,
                 "in_stages": ["bwd_wgrad1", "bwd_wgrad2"]}
    line = {
        "metric": "MoE layer fwd+bwd tokens/sec on 1 MI355X",
        "value": c.T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_median": per_step[len(per_step) // 2],
        "ms_per_step_min": per_step[0],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if c.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) inputs, random-init weights of the layer's shapes)",
        "config": {"workload": c.name, "T": c.T, "d_model": c.d, "d_ff": c.f, "experts": c.E, "top_k": c.k,
                   "capacity_factor": c.cf, "act": c.act, "gate": c.gate, "kept_rows": rows,
                   "nonempty_experts": ne, "tflops_algorithmic": total_flops / (ms_step * 1e-3) / 1e12,
                   "permuted_copy": bool(args.x_perm), "fused_combine": fused_combine},
        "roofline": roof,
        "zero_fill": zero_fill,
        "determinism": determinism,
        # every stage against its own roofline, from the per-stage pre-pass times
        "stage_roofline": {k: {kk: round(vv, 4) if isinstance(vv, float) else vv
                               for kk, vv in stage_roofline(k, work[k], v, c.dtype).items() if kk != "peak"}
                           for k, v in per_stage.items() if k in work},
    }
    # counted HBM bytes / algorithmic bytes per stage (committed counter summary)
    traffic = measured_traffic(c.name) or {}
    for k, v in line["stage_roofline"].items():
        if k in traffic and work[k][1]:
            v["traffic"] = traffic[k]
            v["traffic_over_algorithmic"] = round(traffic[k] / work[k][1], 3)
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.stages:
        print(json.dumps({"stage_ms": per_stage}), file=sys.stderr)
    line["stage_ms"] = {k: round(v, 4) for k, v in per_stage.items()}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = (cpu_baseline(c, inp, args.cpu_tokens) if args.cpu_tokens
                                else cpu_baseline_sized(c, inp))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
