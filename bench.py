"""Benchmark of the NVFP4-forward / MXFP8-backward expert-layer hot path on one MI355X.

Headline (`value`): NVFP4 forward grouped-GEMM TFLOPS on one GPU's expert
share (32768 tokens routed top-8 with Zipf(1.1) popularity over 384 experts,
experts 144..191 resident, d_model 4096, expert FFN 4096 -> 1536 -> 4096).
A step is both forward grouped GEMMs of that layer over its routed rows,

  moe_fwd_grouped_gemm(X_perm NVFP4 [M, 4096], W1 NVFP4 [48 x 1536, 4096])
  -> moe_fwd_grouped_gemm(H NVFP4 [M, 1536], W2 NVFP4 [48 x 4096, 1536]),

outputs in bf16, with the NVFP4 operands (per-token and per-expert outer
scales) already resident in HBM; value = 2 x 2 M F K flop / step time.
`extra` carries the rest of the path: the forward pass with its quantize and
permute, the weight quantizers, the small-MoE layer step (every stage of the
path forward and backward) with warm and cold per-stage rates, the SR bias
statistic of the backward re-quantization, the 1 GiB streaming quantize and
requant, the decode GEMMs, the routed FFN, the all-MXFP8 forward, the NVFP4
backward and the 16x16-tile ablation; plus the measured HBM copy ceiling and
the shader clock under load. `cpu_baseline` is the oracle on a sample of the
same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--cpu-seconds S]
       python bench.py --only {fwd-share,small-step,stream,ffn-share,ffn-small,nvfp4-bwd}
       python bench.py --calibrate-copy     (reference kernel for the HBM byte counters)
"""

import argparse
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 MoE grouped-GEMM fwd TFLOPS + quant/requant GB/s, % of MI355X peak"
PEAK = {"fp4": 10.1e15, "fp8": 5.0e15, "f16": 2.5e15, "hbm": 8.0e12}
# plain (non-packed) VALU lane operations per second: 256 CUs x 4 SIMDs x 16
# lanes per clock at 2.4 GHz; a wave64 VALU instruction is 64 lane operations
VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9

# algorithmic bytes per element
B_QUANT_BF16 = 2 + 0.5 + 1 / 16          # bf16 in, NVFP4 codes + scales out
B_REQUANT = 0.5 + 1 / 16 + 1 + 1 / 32    # NVFP4 in, MXFP8 out
B_DYQ = 2 + 1 + 1 / 32                   # bf16 in, MXFP8 out (one orientation)
B_NVFP4 = 0.5 + 1 / 16                   # NVFP4 codes + block scales
B_MXFP8 = 1 + 1 / 32                     # MXFP8 elements + block exponents

FLUSH_BYTES = 512 << 20                  # scratch written between cold timings
CLOCK_SETTLE_S = 0.3                     # untimed replays before the headline's warm-up


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the shader clock takes some 50 ms of load to settle: 100 warmup steps
    # of the headline (~80 ms), then 200 timed (~160 ms)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--only", choices=["fwd-share", "small-step", "stream", "ffn-share", "ffn-small",
                                       "nvfp4-bwd"], default=None,
                    help="time one workload alone and print its record (for profiling runs)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="0 skips the CPU oracle baseline")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run three 256 MiB device copies (the known-size reference for "
                         "HBM byte counters) and exit")
    return ap.parse_args()


def dev_tensor(a, torch):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


# kernel source each measured stage runs (a counter record is void once it changes)
STAGE_SOURCE = {
    "moe_fwd_grouped_gemm": "gemm_fwd.hip", "moe_fwd_grouped_gemm_expert_share": "gemm_fwd.hip",
    "moe_bwd_dgrad": "gemm_bwd.hip", "moe_bwd_wgrad": "gemm_bwd.hip",
    "moe_bwd_dgrad_expert_share": "gemm_bwd.hip", "moe_bwd_wgrad_expert_share": "gemm_bwd.hip",
    "nvfp4_quantize_x": "quant.hip", "nvfp4_quantize_w": "quant.hip",
    "mxfp8_requant_sr_x": "requant.hip", "mxfp8_requant_sr_w": "requant.hip",
    "mxfp8_quantize_dy": "requant.hip", "moe_permute": "permute.hip",
    "nvfp4_quantize_stream": "quant.hip", "mxfp8_requant_sr_stream": "requant.hip",
}


def profile_record(name, stage):
    """The JSON record of `stage` in profiles/<name> (written from rocprofv3
    counter runs), or None when there is none or the kernel source has
    changed since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", name)
    src = STAGE_SOURCE.get(stage)
    if not src or not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1)).get(stage)
    if not rec:
        return None
    code = os.path.join(ROOT, "precision_moe_numerics_nvfp4_amd", "csrc", src)
    digest = hashlib.sha256(open(code, "rb").read()).hexdigest()[:16]
    if rec.get("source_sha256_16") != digest:
        return None
    return rec


def measured_traffic(stage):
    """HBM bytes per launch of `stage` (rocprofv3 FETCH_SIZE and WRITE_SIZE
    runs scaled by a copy kernel's readings, profiles/hbm_traffic.md)."""
    rec = profile_record("hbm_traffic.md", stage)
    return rec.get("bytes_per_launch") if rec else None


def graph_time(torch, fn, reps):
    """Average GPU time of one fn() call: `reps` calls are captured into one
    HIP graph (one launch, no host overhead between kernels) and replayed
    between two HIP events on the current stream (the stream the library's
    kernels are launched on). Warm: a call's inputs may still sit in the L2
    and the Infinity Cache from the previous call."""
    fn()                                   # eager first call (kernel attributes)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    g.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


class Flusher:
    """Writes FLUSH_BYTES of scratch (twice the 256 MB Infinity Cache, and
    every XCD's L2 many times over) so that the next call reads its inputs
    from HBM."""

    def __init__(self, torch):
        self.buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        self.n = 0

    def __call__(self):
        self.n += 1
        self.buf.fill_(float(self.n))


def cold_time(torch, fn, reps, flush):
    """Average GPU time of one fn() call with cold caches: fn is captured
    once into a HIP graph; each of `reps` replays is preceded by a scratch
    write (outside the event pair) and timed alone between two HIP events on
    the current stream. The scratch write is queued first, so the GPU is
    still busy with it while the host queues the timed replay."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for s, e in ev:
        flush()
        s.record()
        g.replay()
        e.record()
    torch.cuda.synchronize()
    return sum(s.elapsed_time(e) for s, e in ev) / reps


def rate(kind, amount, ms):
    """Rate of `amount` algorithmic work in `ms` and its fraction of the peak."""
    sec = ms * 1e-3
    if kind == "hbm":
        return {"ms": round(ms, 4), "GB/s": round(amount / sec / 1e9, 1),
                "frac_hbm": round(amount / sec / PEAK["hbm"], 4)}
    r = amount / sec
    out = {"ms": round(ms, 4), "TFLOP/s": round(r / 1e12, 1), f"frac_{kind}_peak": round(r / PEAK[kind], 4)}
    if kind == "fp4":
        out["frac_f16_pipe"] = round(r / PEAK["f16"], 4)
    return out


def expert_share_forward(args, torch):
    """The headline: both NVFP4 forward grouped GEMMs of one GPU's expert
    share, plus the forward pass around them (quantize, permute) and the
    per-expert weight quantizers."""
    import precision_moe_numerics_nvfp4_amd as nv
    from workloads import gen
    w3 = gen.expert_share()
    T, K, F, E, k, e0 = w3["T"], w3["K"], w3["N"], w3["E"], w3["k"], w3["e0"]
    x = dev_tensor(w3["x"], torch)
    w1, w2 = dev_tensor(w3["w1"], torch), dev_tensor(w3["w2"], torch)
    topk = dev_tensor(w3["topk"], torch)
    w1q = nv.nvfp4_quantize(w1, rows_per_group=F)
    w2q = nv.nvfp4_quantize(w2, rows_per_group=K)
    xq = nv.nvfp4_quantize(x)
    perm = nv.moe_permute(topk, e0, E, *xq)
    torch.cuda.synchronize()
    M = int(perm["offsets"][-1].item())
    hid = dev_tensor(gen.expert_share_hidden(M, F), torch)     # stand-in for act(Y1), [M, F]
    hq = nv.nvfp4_quantize(hid)
    y1 = torch.empty((T * k, F), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    off = perm["offsets"]

    def gemm1():
        nv.moe_fwd_grouped_gemm(perm["codes"], perm["scales"], perm["outer"], *w1q, off, y=y1)

    def gemm2():
        nv.moe_fwd_grouped_gemm(*hq, *w2q, off, y=y2)

    def step():
        gemm1()
        gemm2()

    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    eager = (y1[:M].clone(), y2.clone())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(2):
        graph.replay()
        torch.cuda.synchronize()
        if not (torch.equal(eager[0], y1[:M]) and torch.equal(eager[1], y2)):
            raise RuntimeError("graph replay of the forward GEMMs differs from the eager call")
    # clock settling: the shader clock of a fresh process needs some 50 ms of
    # load to reach its loaded level (the first ~50 replays run ~7% slower),
    # so the graph replays for CLOCK_SETTLE_S before the W warm-up steps,
    # whatever W is; nothing of it is timed
    settle, t_s = 0, time.perf_counter()
    while time.perf_counter() - t_s < CLOCK_SETTLE_S:
        for _ in range(10):
            graph.replay()
        settle += 10
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    # timed region: exactly `steps` steps, bracketed by device syncs
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    fl = 2.0 * M * F * K                                # per GEMM
    value = 2 * fl / (ms_step * 1e-3) / 1e12
    # per-launch times on the launch stream (HIP events around graph replays)
    reps = max(min(args.steps, 50), 10)
    t1 = graph_time(torch, gemm1, reps)
    t2 = graph_time(torch, gemm2, reps)
    avg = 0.5 * (t1 + t2)
    ach = fl / (avg * 1e-3)
    traffic = measured_traffic("moe_fwd_grouped_gemm_expert_share")
    roof = {"kernel": "moe_fwd_grouped_gemm, 256x256 persistent tiles: k_fwd_lds4 (four "
                      "wavefronts of 128x128) for both GEMMs, k_fwd_stream for short tails",
            "bound": "mfma", "achieved": round(ach / 1e12, 2), "peak": PEAK["f16"] / 1e12,
            "unit": "TFLOP/s", "frac": round(ach / PEAK["f16"], 4), "traffic": traffic,
            "algorithmic_flop_per_launch": fl, "launch_ms_avg": round(avg, 4),
            "operands": "nvfp4", "mfma_pipe": "f16",
            "frac_of_fp4_peak": round(ach / PEAK["fp4"], 4),
            "algorithmic_bytes_per_launch_gemm1": int(M * K * B_NVFP4 + 4 * M + E * F * K * B_NVFP4
                                                      + 4 * E + 2 * M * F),
            "algorithmic_bytes_per_launch_gemm2": int(M * F * B_NVFP4 + 4 * M + E * K * F * B_NVFP4
                                                      + 4 * E + 2 * M * K)}
    rows = (off[1:] - off[:-1]).cpu().numpy()
    kernels = {"gemm1_4096x1536": rate("fp4", fl, t1), "gemm2_1536x4096": rate("fp4", fl, t2)}
    # the forward pass around the GEMMs: per-token quantize of X, permute and
    # gather, GEMM1, per-token quantize of the intermediate, GEMM2
    def fwd_pass():
        nv.nvfp4_quantize(x, None, *xq)
        nv.moe_permute(topk, e0, E, *xq, out=perm)
        gemm1()
        nv.nvfp4_quantize(hid, None, *hq)
        gemm2()
    rr = max(reps // 2, 5)
    t_pass = graph_time(torch, fwd_pass, rr)
    flush = Flusher(torch)
    tq = graph_time(torch, lambda: nv.nvfp4_quantize(x, None, *xq), rr)
    tq_c = cold_time(torch, lambda: nv.nvfp4_quantize(x, None, *xq), 5, flush)
    tw1 = cold_time(torch, lambda: nv.nvfp4_quantize(w1, F, *w1q), 3, flush)
    tw2 = cold_time(torch, lambda: nv.nvfp4_quantize(w2, K, *w2q), 3, flush)
    tp = graph_time(torch, lambda: nv.moe_permute(topk, e0, E, *xq, out=perm), rr)
    kernels.update({
        "nvfp4_quantize_x_32768x4096": {"warm": rate("hbm", T * K * B_QUANT_BF16 + 4 * T, tq),
                                        "cold": rate("hbm", T * K * B_QUANT_BF16 + 4 * T, tq_c)},
        "nvfp4_quantize_w1_per_expert_cold": rate("hbm", E * F * K * B_QUANT_BF16 + 4 * E, tw1),
        "nvfp4_quantize_w2_per_expert_cold": rate("hbm", E * F * K * B_QUANT_BF16 + 4 * E, tw2),
        "moe_permute_gather": {"ms": round(tp, 4), "pairs": T * k, "routed_rows": M},
        "forward_pass": {"ms": round(t_pass, 4),
                         "note": "quantize X, permute + gather, GEMM1, quantize H, GEMM2"},
    })
    cfg = {"workload": "one GPU's expert share, forward GEMMs: 32768 tokens routed top-8 with "
                       "Zipf(1.1) expert popularity over 384 experts, experts 144..191 resident "
                       "(48 local), d_model 4096, expert FFN 4096->1536 and 1536->4096; NVFP4 "
                       "operands with per-token and per-expert outer scales resident in HBM, "
                       "bf16 outputs; one step = both grouped GEMMs (one HIP-graph replay)",
           "tokens": T, "d_model": K, "ffn": F, "local_experts": E, "top_k": k,
           "routed_rows": M, "rows_per_expert_min_max": [int(rows.min()), int(rows.max())],
           "gemm_flop_per_step": 2 * fl}
    # (profiling runs, --only, skip the clock probe's seconds of replays)
    clock = None if args.only else clock_under_load(torch, graph.replay)
    return dict(value=value, ms_step=ms_step, roofline=roof, kernels=kernels, config=cfg, settle=settle,
                tensors=(x, w1, w2, topk, flush), host=w3, clock=clock)


def small_moe_step(args, torch, flush):
    """One pass of every stage of the path, forward and backward, on the small
    MoE layer (4096 tokens, d_model 1024, 8 experts, top-2 uniform, FFN
    1024 -> 2048; dY ~ N(0, std 1e-3)), replayed as a HIP graph; per-stage
    warm and cold rates, and the SR bias statistic of the backward
    re-quantization."""
    from precision_moe_numerics_nvfp4_amd.layer import ExpertLayerStep
    from workloads import gen

    w = gen.small_moe()
    T, K, N, E, k = w["T"], w["K"], w["N"], w["E"], w["k"]
    dy = gen.backward_dy(T * k, N)
    # production output types: Y and dX in bf16, dW in float32
    L = ExpertLayerStep(T, K, N, E, k, out_dtype=torch.bfloat16)
    x_d, w_d = dev_tensor(w["x"], torch), dev_tensor(w["w"], torch)
    t_d, dy_d = dev_tensor(w["topk"], torch), dev_tensor(dy, torch)

    stages = [
        ("nvfp4_quantize_x", lambda: L.quantize_x(x_d)),
        ("nvfp4_quantize_w", lambda: L.quantize_w(w_d)),
        ("moe_permute", lambda: L.permute(t_d)),
        ("moe_fwd_grouped_gemm", L.forward_gemm),
        ("mxfp8_requant_sr_x", L.requant_x),
        ("mxfp8_requant_sr_w", L.requant_w),
        ("mxfp8_quantize_dy", lambda: L.quantize_dy(dy_d)),
        ("moe_bwd_dgrad", L.dgrad),
        ("moe_bwd_wgrad", L.wgrad),
    ]
    for _ in range(max(args.warmup, 1)):
        L.step(x_d, w_d, t_d, dy_d)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (L.y, L.dx, L.dw, L.xT[0], L.dyT[0])]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        L.step(x_d, w_d, t_d, dy_d)
    for _ in range(2):
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(eager, (L.y, L.dx, L.dw, L.xT[0], L.dyT[0])):
            if not torch.equal(a, b):
                raise RuntimeError("graph replay of the step differs from the eager step")
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    steps = max(args.steps, 10)
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    reps = max(min(args.steps, 50), 10)
    warm = {name: graph_time(torch, fn, reps) for name, fn in stages}
    cold = {name: cold_time(torch, fn, 10, flush) for name, fn in stages}

    M = T * k   # top-k distinct experts, all local
    P = int(L.perm["padded_offsets"][-1].item())
    gemm_flop = 2.0 * M * N * K
    # wgrad's algorithmic bytes: both MXFP8 operands and the float32 dW
    wgrad_bytes = (N + K) * P * B_MXFP8 + 4.0 * E * N * K
    work = {
        "nvfp4_quantize_x": ("hbm", T * K * B_QUANT_BF16 + 4 * T),
        "nvfp4_quantize_w": ("hbm", E * N * K * B_QUANT_BF16 + 4 * E),
        "moe_permute": ("hbm", 4 * T * k + 8 * M + 2 * M * (K * B_NVFP4 + 4)),
        "moe_fwd_grouped_gemm": ("fp4", gemm_flop),
        "mxfp8_requant_sr_x": ("hbm", M * K * B_REQUANT),
        "mxfp8_requant_sr_w": ("hbm", E * N * K * B_REQUANT),
        "mxfp8_quantize_dy": ("hbm", 2 * M * N * B_DYQ),
        "moe_bwd_dgrad": ("fp8", gemm_flop),
        "moe_bwd_wgrad": ("fp8", gemm_flop),
    }
    kernels = {}
    for name, (kind, amount) in work.items():
        kernels[name] = {"warm": rate(kind, amount, warm[name]), "cold": rate(kind, amount, cold[name])}
        if name in ("moe_fwd_grouped_gemm", "moe_bwd_dgrad", "moe_bwd_wgrad"):
            kernels[name]["traffic_bytes_per_launch"] = measured_traffic(name)
    # wgrad is rated against the larger of its two bounds
    t_flop = gemm_flop / PEAK["fp8"]
    t_byte = wgrad_bytes / PEAK["hbm"]
    for mode, ms in (("warm", warm["moe_bwd_wgrad"]), ("cold", cold["moe_bwd_wgrad"])):
        kernels["moe_bwd_wgrad"][mode].update({
            "bound": "hbm" if t_byte > t_flop else "fp8", "algorithmic_bytes": wgrad_bytes,
            "bound_us": round(max(t_flop, t_byte) * 1e6, 2),
            "frac_of_bound": round(max(t_flop, t_byte) / (ms * 1e-3), 4)})
    bias = sr_bias_statistic(torch, L, N, E)
    return {"ms_per_step": round(ms_step, 4),
            "gemm_TFLOP/s_over_step": round(3 * gemm_flop / (ms_step * 1e-3) / 1e12, 1),
            "kernels": kernels, "sr_bias_check": bias,
            "workload": "4096 tokens, d_model 1024, 8 experts, top-2 uniform routing, FFN "
                        "1024->2048, bf16 inputs; backward with dY ~ N(0, std 1e-3); Y and dX "
                        "bf16, dW float32; one step = one HIP-graph replay of the ten calls",
            "cold_note": f"cold: {FLUSH_BYTES >> 20} MiB scratch written before each timed call"}


def _e4m3_to_f32(torch, codes):
    return codes.view(torch.float8_e4m3fn).to(torch.float32)


def sr_bias_statistic(torch, L, N, E):
    """Bias of the backward SR re-quantization on the small MoE layer
    (Philox seed 0x5EED0004): mean(SR outputs) - mean(inputs) over every
    re-quantized activation and weight element, next to the analytic
    standard deviation of that difference, sqrt(sum D (1 - D) gap^2) / n,
    where an input v sits a fraction D of the way across an E4M3 gap of
    width gap (scaled by its block exponent)."""
    torch.cuda.synchronize()
    off = L.perm["offsets"].tolist()
    pad = L.perm["padded_offsets"].tolist()
    p = L.perm
    X = _dequant_nvfp4(torch, p["codes"], p["scales"], p["outer"])       # [cap, K]
    W = _dequant_nvfp4(torch, L.wq[0], L.wq[1], L.wq[2].repeat_interleave(N))  # [E*N, K]
    pt = pad[-1]
    parts = []
    # activations: output column pad[g] + j holds token row off[g] + j
    sx = (_e4m3_to_f32(torch, L.xT[0][:, :pt]) *
          torch.pow(2.0, L.xT[1][:, :pt // 32].to(torch.float32) - 127).repeat_interleave(32, 1))
    vx = torch.zeros_like(sx)
    for g in range(len(off) - 1):
        a, b = off[g], off[g + 1]
        vx[:, pad[g]:pad[g] + (b - a)] = X[a:b].t()
    parts.append((vx, sx, L.xT[1][:, :pt // 32]))
    # weights: per-expert blocks [E, K, N] back to [K, E*N]
    K = W.shape[1]
    wq8, we8 = (t.reshape(E, K, -1).transpose(0, 1).reshape(K, -1) for t in L.wT)
    sw = (_e4m3_to_f32(torch, wq8) *
          torch.pow(2.0, we8.to(torch.float32) - 127).repeat_interleave(32, 1))
    parts.append((W.t().contiguous(), sw, we8))
    n = 0
    diff = 0.0
    var = 0.0
    for v, sr, e8 in parts:
        v = v.double()
        sc = torch.pow(2.0, e8.double() - 127).repeat_interleave(32, 1)
        y = (v / sc).abs()
        ex = torch.floor(torch.log2(torch.clamp(y, min=2.0 ** -6)))
        gap = torch.pow(2.0, ex - 3)
        lo = torch.floor(y / gap) * gap
        D = torch.where(y >= 448.0, torch.zeros_like(y), (y - lo) / gap)
        var += float((D * (1 - D) * (gap * sc) ** 2).sum())
        diff += float((sr.double() - v).sum())
        n += v.numel()
    bias = diff / n
    sd = var ** 0.5 / n
    return {"elements": n, "mean_sr_minus_mean_input": bias, "analytic_sd": sd,
            "bias_over_sd": round(bias / sd, 3) if sd > 0 else None,
            "inputs": "requantized X_perm (grouped transpose) and W of the small MoE layer, "
                      "seed 0x5EED0004"}


def _time(torch, fn, reps):
    return graph_time(torch, fn, reps)


def mxfp8_forward_compare(torch, reps):
    import precision_moe_numerics_nvfp4_amd as nv
    from workloads import gen
    w = gen.small_moe()
    T, K, N, E, k = w["T"], w["K"], w["N"], w["E"], w["k"]
    x, wt = dev_tensor(w["x"], torch), dev_tensor(w["w"], torch)
    topk = dev_tensor(w["topk"], torch)
    xq = nv.nvfp4_quantize(x)
    wq = nv.nvfp4_quantize(wt, rows_per_group=N)
    perm = nv.moe_permute(topk, 0, E, *xq)
    x8 = nv.mxfp8_quantize(x, "rowwise")
    w8 = nv.mxfp8_quantize(wt, "rowwise")
    g8 = nv.mxfp8_gather_rows(perm["row_token"], perm["offsets"], *x8)
    y = torch.empty((T * k, N), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    M = int(perm["offsets"][-1].item())
    t_nv = _time(torch, lambda: nv.moe_fwd_grouped_gemm(perm["codes"], perm["scales"], perm["outer"],
                                                        *wq, perm["offsets"], y=y), reps)
    t_mx = _time(torch, lambda: nv.moe_fwd_grouped_gemm_mxfp8(*g8, *w8, perm["offsets"], y=y), reps)
    t_nv_path = _time(torch, lambda: (nv.nvfp4_quantize(x, None, *xq),
                                      nv.moe_permute(topk, 0, E, *xq, out=perm),
                                      nv.moe_fwd_grouped_gemm(perm["codes"], perm["scales"],
                                                              perm["outer"], *wq, perm["offsets"],
                                                              y=y)), reps)
    t_mx_path = _time(torch, lambda: (nv.mxfp8_quantize(x, "rowwise", out=x8[0], out_e8=x8[1]),
                                      nv.mxfp8_gather_rows(perm["row_token"], perm["offsets"], *x8,
                                                           out=g8),
                                      nv.moe_fwd_grouped_gemm_mxfp8(*g8, *w8, perm["offsets"], y=y)),
                      reps)
    fl = 2.0 * M * N * K
    return {"routed_rows": M,
            "gemm_nvfp4": {"ms": round(t_nv, 4), "TFLOP/s": round(fl / t_nv / 1e9, 1)},
            "gemm_mxfp8": {"ms": round(t_mx, 4), "TFLOP/s": round(fl / t_mx / 1e9, 1),
                           "frac_fp8_peak": round(fl / t_mx / 1e-3 / PEAK["fp8"], 4)},
            "forward_nvfp4_quantize_permute_gemm": {"ms": round(t_nv_path, 4)},
            "forward_mxfp8_quantize_gather_gemm": {"ms": round(t_mx_path, 4)},
            "note": "weights quantized once outside the timed paths"}


def ffn_step_bench(torch, reps, x, w1, w2, topk, gate, dout, E, F, e0):
    """The routed expert FFN (up-projection, per-token re-quantization of the
    intermediate, down-projection, combine) forward and backward through both
    projections: per-step, forward and backward times and the rate of its six
    grouped GEMMs."""
    from precision_moe_numerics_nvfp4_amd.layer import ExpertFFNStep
    T, K = x.shape
    k = topk.shape[1]
    L = ExpertFFNStep(T, K, F, E, k, e0=e0)
    L.quantize_weights(w1, w2)
    L.forward(x, topk, gate)
    torch.cuda.synchronize()
    M = int(L.perm["offsets"][-1].item())
    t_step = _time(torch, lambda: L.step(x, w1, w2, topk, gate, dout), reps)
    t_fwd = _time(torch, lambda: L.forward(x, topk, gate), reps)
    t_bwd = _time(torch, lambda: L.backward(dout, gate), reps)
    fl = 6 * 2.0 * M * F * K
    # the four MXFP8 backward GEMMs one by one (inputs as the step left them);
    # wgrad rated against the larger of its flop and byte bounds (the float32
    # dW it writes: E F K 4 bytes)
    from precision_moe_numerics_nvfp4_amd import binding as B
    off, poff = L.perm["offsets"], L.perm["padded_offsets"]
    P = int(poff[-1].item())             # the padded token count (the buffers hold capacity)
    gemms = {
        "dgrad_down_4096": lambda: B.moe_bwd_dgrad(*L.dy2_8, *L.w2T, off, K, F, dx=L.dh),
        "wgrad_down": lambda: B.moe_bwd_wgrad(*L.dy2T, *L.hT, poff, K, F, dw=L.dw2),
        "dgrad_up_1536": lambda: B.moe_bwd_dgrad(*L.dh8, *L.w1T, off, F, K, dx=L.dxp),
        "wgrad_up": lambda: B.moe_bwd_wgrad(*L.dhT, *L.xT, poff, F, K, dw=L.dw1),
    }
    g_fl = 2.0 * M * F * K
    w_bytes = (K + F) * P * B_MXFP8 + 4.0 * E * F * K
    per = {}
    for name, fn in gemms.items():
        ms = graph_time(torch, fn, reps)
        r = rate("fp8", g_fl, ms)
        if name.startswith("wgrad"):
            t_bound = max(g_fl / PEAK["fp8"], w_bytes / PEAK["hbm"])
            r.update({"bound": "hbm" if w_bytes / PEAK["hbm"] > g_fl / PEAK["fp8"] else "fp8",
                      "algorithmic_bytes": w_bytes, "bound_us": round(t_bound * 1e6, 1),
                      "frac_of_bound": round(t_bound / (ms * 1e-3), 4)})
        per[name] = r
    if (E, F, K) == (48, 1536, 4096):     # the expert share: its counter records
        stage = "moe_bwd_dgrad_expert_share", "moe_bwd_wgrad_expert_share"
        per["traffic_bytes_per_launch"] = {s_: measured_traffic(s_) for s_ in stage}
    del L
    return {"routed_rows": M, "ms_per_step": round(t_step, 4), "ms_forward": round(t_fwd, 4),
            "ms_backward": round(t_bwd, 4), "gemm_TFLOP": round(fl / 1e12, 3),
            "TFLOP/s": round(fl / t_step / 1e9, 1), "backward_gemms": per,
            "note": "step = weight quantize + forward + backward; six grouped GEMMs"}


def ffn_workload(torch, name, reps):
    """ffn_step_bench on the expert share ("ffn-share": 48 of 384 experts,
    32768 tokens top-8 Zipf, 4096 -> 1536 -> 4096) or on the small MoE layer's
    shapes ("ffn-small": 4096 tokens top-2 over 8, 1024 -> 2048 -> 1024)."""
    from workloads import gen
    if name == "ffn-share":
        w3 = gen.expert_share()
        T, K, F, E = w3["T"], w3["K"], w3["N"], w3["E"]
        args = (dev_tensor(w3["x"], torch), dev_tensor(w3["w1"], torch),
                dev_tensor(w3["w2"], torch), dev_tensor(w3["topk"], torch),
                dev_tensor(gen.gates(3, T, 8), torch),
                dev_tensor(gen.to_bf16_bits(gen.normal(3, 3, (T, K), std=1e-3)), torch))
        return ffn_step_bench(torch, reps, *args, E, F, 144)
    c = gen.ffn_case(2, T=4096, K=1024, F=2048, E=8, k=2)
    return ffn_step_bench(
        torch, reps, dev_tensor(c["x"], torch), dev_tensor(c["w1"].reshape(8 * 2048, 1024), torch),
        dev_tensor(c["w2"].reshape(8 * 1024, 2048), torch), dev_tensor(c["topk"], torch),
        dev_tensor(c["gate"], torch), dev_tensor(c["dout"], torch), 8, 2048, 0)


def _dequant_nvfp4(torch, codes, scales, outer):
    """NVFP4 rows -> float32 (codes [R, C/2], scales [R, C/16], outer [R]) with
    plain torch ops, for the error measurement only."""
    e2m1 = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                         -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0],
                        dtype=torch.float32, device=codes.device)
    c = codes.to(torch.int64)
    v = torch.stack([e2m1[c & 15], e2m1[c >> 4]], dim=2).reshape(codes.shape[0], -1)
    sc = scales.to(torch.int64)
    e, m = (sc >> 3) & 15, (sc & 7).to(torch.float32)
    S = torch.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * torch.pow(2.0, (e - 7).to(torch.float32)))
    return v * S.repeat_interleave(16, dim=1) * outer[:, None]


def nvfp4_backward_compare(torch, reps, n_seeds=8):
    """The NVFP4 backward next to the MXFP8 backward on the small MoE layer:
    time of each path (requant of the saved activations and weights, dY in
    both orientations, dgrad, wgrad) and, against the exact gradients of the
    forward's dequantized operands (float32 matmuls), the relative error of
    one step and the relative bias (error of the mean over n_seeds seeds)."""
    from precision_moe_numerics_nvfp4_amd.layer import ExpertLayerStep, NVFP4BackwardStep
    from workloads import gen
    w = gen.small_moe()
    T, K, N, E, k = w["T"], w["K"], w["N"], w["E"], w["k"]
    dy = dev_tensor(gen.backward_dy(T * k, N), torch)
    L = ExpertLayerStep(T, K, N, E, k, out_dtype=torch.float32)
    x, wt, topk = dev_tensor(w["x"], torch), dev_tensor(w["w"], torch), dev_tensor(w["topk"], torch)
    L.quantize_x(x)
    L.quantize_w(wt)
    L.permute(topk)
    L.forward_gemm()
    NB = NVFP4BackwardStep(L)
    t_mx = _time(torch, lambda: (L.requant_x(), L.requant_w(), L.quantize_dy(dy), L.dgrad(),
                                 L.wgrad()), reps)
    t_nv = _time(torch, lambda: NB.backward(dy), reps)
    stages = {"requant_x_w": lambda: NB.requant(), "quantize_dy_both": lambda: NB.quantize_dy(dy),
              "dgrad": NB.dgrad, "wgrad": NB.wgrad}
    t_st = {n: round(_time(torch, f, reps), 4) for n, f in stages.items()}
    # exact gradients of the dequantized forward operands
    torch.cuda.synchronize()
    off = L.perm["offsets"].tolist()
    p = L.perm
    X = _dequant_nvfp4(torch, p["codes"], p["scales"], p["outer"])                  # [cap, K]
    W = _dequant_nvfp4(torch, L.wq[0], L.wq[1], L.wq[2].repeat_interleave(N))       # [E*N, K]
    dyf = dy.float()
    dx_ex = torch.zeros((T * k, K), dtype=torch.float32, device="cuda")
    dw_ex = torch.zeros((E, N, K), dtype=torch.float32, device="cuda")
    for g in range(E):
        a, b = off[g], off[g + 1]
        dx_ex[a:b] = dyf[a:b] @ W[g * N:(g + 1) * N]
        dw_ex[g] = dyf[a:b].t() @ X[a:b]
    M = off[-1]
    rel = lambda a, ref: float((a - ref).norm() / ref.norm())
    out = {}
    for name, run, dxb, dwb in (("mxfp8", lambda: (L.requant_x(), L.requant_w(), L.quantize_dy(dy),
                                                   L.dgrad(), L.wgrad()), L.dx, L.dw),
                                ("nvfp4", lambda: NB.backward(dy), NB.dx, NB.dw)):
        sdx = torch.zeros_like(dx_ex)
        sdw = torch.zeros_like(dw_ex)
        first = None
        seed0 = L.seed
        for i in range(n_seeds):
            L.seed = seed0 + i
            run()
            sdx += dxb.float()
            sdw += dwb
            if first is None:
                torch.cuda.synchronize()
                first = (rel(dxb[:M].float(), dx_ex[:M]), rel(dwb, dw_ex))
        L.seed = seed0
        out[name] = {"rel_err_dx": round(first[0], 5), "rel_err_dw": round(first[1], 5),
                     "rel_bias_dx": round(rel(sdx[:M] / n_seeds, dx_ex[:M]), 5),
                     "rel_bias_dw": round(rel(sdw / n_seeds, dw_ex), 5)}
    out["mxfp8"]["ms_backward"] = round(t_mx, 4)
    out["nvfp4"]["ms_backward"] = round(t_nv, 4)
    out["nvfp4"]["stages_ms"] = t_st
    out["seeds_for_bias"] = n_seeds
    out["note"] = ("error: one step against the exact gradient of the dequantized forward operands; "
                   "bias: the mean over the seeds against it (includes the seeds' noise / sqrt(n))")
    return out


def tile16_compare(torch, reps):
    import precision_moe_numerics_nvfp4_amd as nv
    from workloads import gen
    w = gen.small_moe()
    N, E, K = w["N"], w["E"], w["K"]
    wt = dev_tensor(w["w"], torch)
    q1 = nv.nvfp4_quantize(wt, rows_per_group=N)
    qt = nv.nvfp4_quantize_tile16(wt, rows_per_group=N)
    t1 = _time(torch, lambda: nv.nvfp4_quantize(wt, N, *q1), reps)
    tt = _time(torch, lambda: nv.nvfp4_quantize_tile16(wt, N, *qt), reps)
    n = E * N * K
    tbytes = n * (2 + 0.5) + n / 256        # bf16 in, codes out, one scale per 256 elements
    return {"weights": f"{E}x{N}x{K} bf16",
            "blocks_1x16": {"ms": round(t1, 4), "GB/s": round(n * B_QUANT_BF16 / t1 / 1e6, 1)},
            "tiles_16x16": {"ms": round(tt, 4), "GB/s": round(tbytes / tt / 1e6, 1)}}


def streaming_bench(torch, reps, flush):
    """1 GiB bf16 [262144 x 2048] per-token NVFP4 quantize, then the SR
    re-quantization of its transpose (one segment, P = 262144, tag 2). The
    working sets (1.4 GB and 0.86 GB) exceed the Infinity Cache; each call is
    also timed after a scratch write. The requant's VALU fraction comes from
    the counter record in profiles/valu_counters.md."""
    import precision_moe_numerics_nvfp4_amd as nv
    from workloads import gen
    rows, cols = 262144, 2048
    xs = dev_tensor(gen.streaming(rows, cols), torch)
    q = nv.nvfp4_quantize(xs)
    off = torch.tensor([0, rows], dtype=torch.int64, device="cuda")
    o8 = torch.empty((cols, rows), dtype=torch.uint8, device="cuda")
    e8 = torch.empty((cols, rows // 32), dtype=torch.uint8, device="cuda")
    fq = lambda: nv.nvfp4_quantize(xs, None, *q)
    fr = lambda: nv.mxfp8_requant_sr(*q, off, off, rows, 0x5EED0005, 2, out=o8, out_e8=e8)
    n = rows * cols
    bq, br = n * B_QUANT_BF16 + 4 * rows, n * B_REQUANT + 4 * rows
    tq, tr = graph_time(torch, fq, reps), graph_time(torch, fr, reps)
    tq_c, tr_c = cold_time(torch, fq, 5, flush), cold_time(torch, fr, 5, flush)
    out = {"quantize": {"back_to_back": rate("hbm", bq, tq), "cold": rate("hbm", bq, tq_c)},
           "requant_sr": {"back_to_back": rate("hbm", br, tr), "cold": rate("hbm", br, tr_c)}}
    for key, stage, ms in (("quantize", "nvfp4_quantize_stream", tq_c),
                           ("requant_sr", "mxfp8_requant_sr_stream", tr_c)):
        rec = profile_record("valu_counters.md", stage)
        if rec:
            ops = 64.0 * rec["valu_insts_per_launch"]
            out[key]["valu"] = {"lane_ops_per_element": round(ops / n, 2),
                                "lane_ops_per_s": ops / (ms * 1e-3),
                                "frac_valu_roofline": round(ops / (ms * 1e-3) / VALU_LANE_OPS, 4),
                                "valu_roofline_lane_ops_per_s": VALU_LANE_OPS}
            if "valu_busy_frac" in rec:
                out[key]["valu"]["valu_busy_frac_counter"] = rec["valu_busy_frac"]
        else:
            out[key]["valu"] = None
    del xs, q, o8, e8
    return out


def hbm_copy_ceiling(torch, flush):
    """Measured device-to-device copy rate of 1 GiB (2 GiB moved), the
    practical HBM ceiling next to the 8 TB/s spec."""
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    src.fill_(1.0)
    dst = torch.empty_like(src)
    t = cold_time(torch, lambda: dst.copy_(src), 5, flush)
    acc = torch.empty((), dtype=torch.float32, device="cuda")
    tr = cold_time(torch, lambda: torch.sum(src, dim=0, out=acc), 5, flush)
    del src, dst
    return {"copy": {"bytes_moved": 2 << 30, "ms": round(t, 4), "GB/s": round((2 << 30) / t / 1e6, 1),
                     "frac_of_8TB/s": round((2 << 30) / t / 1e-3 / PEAK["hbm"], 4)},
            "read_sum": {"bytes_read": 1 << 30, "ms": round(tr, 4), "GB/s": round((1 << 30) / tr / 1e6, 1),
                         "frac_of_8TB/s": round((1 << 30) / tr / 1e-3 / PEAK["hbm"], 4)},
            "note": "torch's device copy and sum of a 1 GiB float32 tensor, cold"}


def clock_under_load(torch, fn, seconds=8.0, samples=3):
    """Shader clock read with amd-smi while `fn` replays keep the GPU busy:
    about `seconds` of replays are queued first, then amd-smi is sampled up
    to `samples` times; the sample with the highest mean is kept (a sample
    taken after the queue drained reads the idle clock). None where amd-smi
    is unavailable or prints nothing usable."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    per = max(time.perf_counter() - t0, 1e-4)
    for _ in range(int(seconds / per) + 1):
        fn()                                 # queued; the GPU stays busy meanwhile

    def parse(rec):
        data = json.loads(rec)
        if isinstance(data, dict) and "gpu_data" in data:
            data = data["gpu_data"]
        d = data[0] if isinstance(data, list) else data
        clk = d.get("clock", d)
        return [v["clk"]["value"] for k, v in sorted(clk.items())
                if k.lower().startswith("gfx_") and isinstance(v, dict)
                and isinstance(v.get("clk"), dict) and isinstance(v["clk"].get("value"), (int, float))]

    best, raw = None, None
    for _ in range(samples):
        try:
            r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "--json"], capture_output=True,
                               text=True, timeout=20)
            rec = r.stdout.strip() if r.returncode == 0 else None
        except Exception:
            rec = None
        if not rec:
            continue
        raw = rec
        try:
            mhz = parse(rec)
        except Exception:
            continue
        if mhz and (best is None or sum(mhz) / len(mhz) > sum(best) / len(best)):
            best = mhz
    torch.cuda.synchronize()
    if best is None:
        return {"raw": raw[:400]} if raw else None
    return {"gfx_clk_mhz": best, "mean_mhz": round(sum(best) / len(best), 1),
            "source": f"amd-smi metric -c during forward-GEMM replays (highest of {samples} samples)"}


def extras(torch, reps, tensors):
    import precision_moe_numerics_nvfp4_amd as nv
    from workloads import gen
    out = {}
    x, w1, w2, topk, flush = tensors
    T, K = x.shape
    F, E = w1.shape[0] // 48, 48
    # the routed FFN at the expert share, forward and backward
    gate = dev_tensor(gen.gates(3, T, 8), torch)
    dout = dev_tensor(gen.to_bf16_bits(gen.normal(3, 3, (T, K), std=1e-3)), torch)
    out["expert_share_ffn_step"] = ffn_step_bench(torch, reps, x, w1, w2, topk, gate, dout, E, F,
                                                  144)
    del gate, dout
    torch.cuda.empty_cache()
    # the same on the small MoE layer's shapes (1024 -> 2048 -> 1024, 8 experts, top-2)
    c = gen.ffn_case(2, T=4096, K=1024, F=2048, E=8, k=2)
    out["small_moe_ffn_step"] = ffn_step_bench(
        torch, reps, dev_tensor(c["x"], torch), dev_tensor(c["w1"].reshape(8 * 2048, 1024), torch),
        dev_tensor(c["w2"].reshape(8 * 1024, 2048), torch), dev_tensor(c["topk"], torch),
        dev_tensor(c["gate"], torch), dev_tensor(c["dout"], torch), 8, 2048, 0)
    del c
    torch.cuda.empty_cache()
    # decode: 512 tokens top-8 uniform over 384, 48 local, weights pre-quantized
    w5 = gen.decode()
    x5 = dev_tensor(w5["x"], torch)
    topk5 = dev_tensor(w5["topk"], torch)
    w1q = nv.nvfp4_quantize(dev_tensor(w5["w1"], torch), rows_per_group=F)
    w2q5 = nv.nvfp4_quantize(dev_tensor(w5["w2"], torch), rows_per_group=K)
    xq5 = nv.nvfp4_quantize(x5)
    perm5 = nv.moe_permute(topk5, 144, E, *xq5)
    torch.cuda.synchronize()
    M5 = int(perm5["offsets"][-1].item())
    hq5 = nv.nvfp4_quantize(dev_tensor(gen.expert_share_hidden(M5, F, cfg=5), torch))
    yd1 = torch.empty((512 * 8, F), dtype=torch.bfloat16, device="cuda")
    yd2 = torch.empty((M5, K), dtype=torch.bfloat16, device="cuda")
    fd = lambda: (nv.moe_fwd_grouped_gemm(perm5["codes"], perm5["scales"], perm5["outer"],
                                          *w1q, perm5["offsets"], y=yd1),
                  nv.moe_fwd_grouped_gemm(*hq5, *w2q5, perm5["offsets"], y=yd2))
    td = graph_time(torch, fd, reps)
    td_c = cold_time(torch, fd, 5, flush)
    wbytes = 2 * E * F * K * B_NVFP4
    out["decode_fwd"] = {"routed_rows_local": M5,
                         "back_to_back": {"ms_both_gemms": round(td, 4),
                                          "weight_GB/s": round(wbytes / td / 1e6, 1),
                                          "frac_hbm": round(wbytes / td / 1e-3 / PEAK["hbm"], 4)},
                         "cold": {"ms_both_gemms": round(td_c, 4),
                                  "weight_GB/s": round(wbytes / td_c / 1e6, 1),
                                  "frac_hbm": round(wbytes / td_c / 1e-3 / PEAK["hbm"], 4)},
                         "flop": 2 * 2.0 * M5 * F * K}
    del w1q, w2q5, hq5, yd1, yd2, perm5, xq5, x5
    torch.cuda.empty_cache()
    # the all-MXFP8 forward (the reference the NVFP4 forward is compared against)
    out["mxfp8_forward_small_moe"] = mxfp8_forward_compare(torch, reps)
    torch.cuda.empty_cache()
    # the NVFP4 backward next to the MXFP8 one: time, error, bias
    out["nvfp4_backward_small_moe"] = nvfp4_backward_compare(torch, reps)
    torch.cuda.empty_cache()
    # the rejected 16x16-tile scaling (ablation)
    out["tile16_weight_quantize"] = tile16_compare(torch, reps)
    torch.cuda.empty_cache()
    out["streaming_1GiB"] = streaming_bench(torch, reps, flush)
    torch.cuda.empty_cache()
    return out


def _host_info():
    import platform
    info = {"os_cpu_count": os.cpu_count(), "numpy": np.__version__, "python": platform.python_version()}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        info["blas"] = [{k: i.get(k) for k in ("internal_api", "version", "num_threads",
                                                "threading_layer")} for i in threadpool_info()]
    except Exception:
        info["blas"] = None
    try:
        info["affinity_cores"] = len(os.sched_getaffinity(0))
    except Exception:
        pass
    return info


def cpu_baseline(w3, budget_s):
    """The oracle, as it stands, on a bounded sample of the headline workload:
    the whole forward of the expert share restricted to its first local
    experts (taken in order until about budget_s of work), every stage timed
    on its own. Elementwise stages (quantizers, gather) run in numpy on one
    core; the GEMMs' float32 matmuls run on the BLAS threads. `value` is the
    oracle's forward-GEMM rate (dequantize + float32 matmul) in TFLOP/s."""
    from oracle import gemm as GM
    from oracle import nvfp4 as Q
    from oracle import permute as PM
    from workloads import gen
    T, K, F, E, k, e0 = w3["T"], w3["K"], w3["N"], w3["E"], w3["k"], w3["e0"]
    info = _host_info()
    blas_threads = max([b.get("num_threads") or 1 for b in (info.get("blas") or [])] + [1])
    t0 = time.perf_counter()
    off, pad, rt, rs = PM.permute(w3["topk"], e0, E)
    t_perm = time.perf_counter() - t0
    M = int(off[-1])
    hid = gen.expert_share_hidden(M, F)
    tt = {"quantize_x": 0.0, "quantize_w": 0.0, "gather": 0.0, "gemm1": 0.0, "quantize_h": 0.0,
          "gemm2": 0.0}
    n_tok = n_rows = n_exp = 0
    start = time.perf_counter()
    for g in range(E):
        a, b = int(off[g]), int(off[g + 1])
        if b == a:
            continue
        toks = rt[a:b]
        t = time.perf_counter()
        xq = Q.quantize(w3["x"][toks])                    # rows of this expert's tokens
        tt["quantize_x"] += time.perf_counter() - t
        t = time.perf_counter()
        w1q = Q.quantize(w3["w1"][g * F:(g + 1) * F], rows_per_group=F)
        w2q = Q.quantize(w3["w2"][g * K:(g + 1) * K], rows_per_group=K)
        tt["quantize_w"] += time.perf_counter() - t
        t = time.perf_counter()
        ga = PM.gather_rows(np.arange(b - a), *xq)
        tt["gather"] += time.perf_counter() - t
        o1 = np.array([0, b - a])
        t = time.perf_counter()
        GM.fwd_grouped(*ga, *w1q, o1, F)
        tt["gemm1"] += time.perf_counter() - t
        t = time.perf_counter()
        hq = Q.quantize(hid[a:b])
        tt["quantize_h"] += time.perf_counter() - t
        t = time.perf_counter()
        GM.fwd_grouped(*hq, *w2q, o1, K)
        tt["gemm2"] += time.perf_counter() - t
        n_tok += b - a
        n_rows += b - a
        n_exp += 1
        if time.perf_counter() - start >= budget_s:
            break
    fl = 2.0 * n_rows * F * K
    t_g = tt["gemm1"] + tt["gemm2"]
    stages = {
        "permute_whole": {"s": round(t_perm, 3), "pairs": T * k, "cores": 1},
        "quantize_x": {"s": round(tt["quantize_x"], 3), "cores": 1,
                       "GB/s": round(n_tok * K * B_QUANT_BF16 / tt["quantize_x"] / 1e9, 4)},
        "quantize_w1_w2": {"s": round(tt["quantize_w"], 3), "cores": 1,
                           "GB/s": round(2 * n_exp * F * K * B_QUANT_BF16 / tt["quantize_w"] / 1e9, 4)},
        "gather": {"s": round(tt["gather"], 3), "cores": 1},
        "gemm1_4096x1536": {"s": round(tt["gemm1"], 3), "cores": blas_threads,
                            "TFLOP/s": round(fl / tt["gemm1"] / 1e12, 5)},
        "quantize_h": {"s": round(tt["quantize_h"], 3), "cores": 1,
                       "GB/s": round(n_rows * F * B_QUANT_BF16 / tt["quantize_h"] / 1e9, 4)},
        "gemm2_1536x4096": {"s": round(tt["gemm2"], 3), "cores": blas_threads,
                            "TFLOP/s": round(fl / tt["gemm2"] / 1e12, 5)},
    }
    return {"value": round(2 * fl / t_g / 1e12, 5), "unit": "TFLOPS", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"the expert-share forward restricted to its first {n_exp} of {E} local experts "
                      f"({n_rows} of {M} routed rows): per-token quantize of their tokens, per-expert "
                      f"quantize of their W1 and W2, gather, GEMM1, per-token quantize of H, GEMM2; "
                      f"value = both GEMMs' flops / their oracle time (dequantize + float32 BLAS "
                      f"matmul); elementwise stages on one core",
            "seconds": round(sum(tt.values()) + t_perm, 2), "stages": stages, "host": info}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus above 1 is not supported "
                                   "(the expert-parallel design is described, not built)"}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)                     # 256 MiB read, 256 MiB written
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": 256 << 20, "copies": 3}))
        return
    from precision_moe_numerics_nvfp4_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        raise RuntimeError(f"{binding.LIB_PATH} is not built; run python -m "
                           "precision_moe_numerics_nvfp4_amd.build first")
    reps = max(min(args.steps, 50), 10)          # graph replays per kernel timing
    if args.only in ("ffn-share", "ffn-small", "nvfp4-bwd"):
        rec = (nvfp4_backward_compare(torch, reps) if args.only == "nvfp4-bwd"
               else ffn_workload(torch, args.only, reps))
        print(json.dumps({args.only: rec}))
        return
    if args.only == "small-step":
        print(json.dumps({"small-step": small_moe_step(args, torch, Flusher(torch))}))
        return
    if args.only == "stream":
        print(json.dumps({"stream": streaming_bench(torch, reps, Flusher(torch))}))
        return
    print("bench: expert-share forward GEMMs", file=sys.stderr, flush=True)
    r = expert_share_forward(args, torch)
    line = {
        "metric": METRIC, "value": round(r["value"], 3), "unit": "TFLOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "nvfp4 operands, f16 MFMA with exact products, f32 accumulate", "data": "synthetic",
        "config": r["config"], "clock_settle_replays": r["settle"], "roofline": r["roofline"],
        "kernels": r["kernels"],
    }
    if args.only == "fwd-share":
        print(json.dumps(line))
        return
    x, w1, w2, topk, flush = r["tensors"]
    if not args.no_extra:
        print("bench: clock, copy ceiling, small-MoE step and extras", file=sys.stderr, flush=True)
        extra = {"sclk_under_load": r["clock"]}
        extra["hbm_copy_ceiling"] = hbm_copy_ceiling(torch, flush)
        extra["small_moe_step"] = small_moe_step(args, torch, flush)
        torch.cuda.empty_cache()
        extra.update(extras(torch, reps, r["tensors"]))
        line["extra"] = extra
    del x, w1, w2, topk
    torch.cuda.empty_cache()
    if args.cpu_seconds > 0:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(r["host"], args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line))


if __name__ == "__main__":
    main()
