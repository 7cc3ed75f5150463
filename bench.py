"""Benchmark of the MI355X retention library on one GPU.

Headline (`value`): chunkwise retention tokens/s on the long-context workload
(B1 H8 L32768 dk128 dv256, chunk 256, bf16 in and out, final state written),
inputs resident in HBM.  One step = one retention_chunkwise call.  The same JSON
line also carries the recurrent decode rate (B128 H16 dk128 dv256, 1024 steps
after a 512-token prefill), the parallel-form and MSR-layer rates, each with its
roofline, and the fp64 CPU oracle timed on a bounded sample of the headline
workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "chunkwise retention tokens/s @L=32K; recurrent decode tokens/s; % roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


SETTLE_S = 0.25  # untimed back-to-back calls before the warmup, so the GPU clocks reach steady state


def _settle(fn, seconds=SETTLE_S):
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


_LAST_CALLS = []  # per-call seconds of the latest _time_calls (event pairs between consecutive calls)


def _time_calls(fn, steps, warmup):
    """Seconds for `steps` back-to-back calls, between two events on the stream the
    calls run on (torch's current stream, which the library is given), with nothing
    else enqueued between the calls.  A second loop of `steps` calls with an event
    after every call gives per-call times (_LAST_CALLS) for the median and min; an
    event between two calls costs the GPU a few microseconds (the next launch waits
    for it), so those times run slightly above the back-to-back mean."""
    import torch
    _settle(fn)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    total = e0.elapsed_time(e1) / 1000.0  # seconds for all steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    _LAST_CALLS[:] = [ev[i].elapsed_time(ev[i + 1]) / 1000.0 for i in range(steps)]
    return total


def _spread():
    """Median and min per-call milliseconds of the latest timed loop."""
    import statistics
    c = _LAST_CALLS
    return {"median_ms": statistics.median(c) * 1e3, "min_ms": min(c) * 1e3, "calls_timed": len(c)} if c else {}


def _read_traffic(name):
    """HBM bytes per call from a committed rocprofv3 PMC summary, or None if it
    is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    try:
        if kv.get("src_sha") != _src_sha():
            return None
        return float(kv["hbm_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def _src_sha():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "retentive_network_scale_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def _alg_bytes_chunkwise():
    """Q, K, V read once, O (bf16) and the final fp32 state written once."""
    from workloads import CHUNKWISE_32K as wl
    return 2 * (2 * wl.B * wl.H * wl.L * wl.dk) + 2 * wl.B * wl.H * wl.L * wl.dv * 2 + 4 * wl.B * wl.H * wl.dk * wl.dv


def _alg_bytes_decode():
    """fp32 state read and written, bf16 q, k, v read and o written, per step."""
    from workloads import DECODE as wl
    return 2 * 4 * wl.B * wl.H * wl.dk * wl.dv + 2 * 2 * wl.B * wl.H * wl.dk + 2 * 2 * wl.B * wl.H * wl.dv


def _alg_bytes_parallel():
    """Q, K, V read once, O (bf16) written once."""
    from workloads import PARALLEL_2K as wl
    return 2 * 2 * wl.B * wl.H * wl.L * wl.dk + 2 * 2 * wl.B * wl.H * wl.L * wl.dv


def bench_chunkwise(steps, warmup):
    import torch
    import retentive_network_scale_amd as rn
    from workloads import CHUNKWISE_32K as wl
    q, k, v = (t.cuda() for t in wl.qkv())
    g, th = wl.gamma(), wl.theta()
    out = torch.empty((wl.B, wl.H, wl.L, wl.dv), dtype=torch.bfloat16, device="cuda")
    state = torch.empty((wl.B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device="cuda")
    ws = torch.empty(rn.retention_chunkwise_workspace_bytes(wl.B, wl.H, wl.L, wl.dk, wl.dv, wl.chunk),
                     dtype=torch.uint8, device="cuda")

    def call():
        rn.retention_chunkwise(q, k, v, g, wl.chunk, th, state_out=state, out=out, workspace=ws)
    t = _time_calls(call, steps, warmup)
    per_call = t / steps
    tokens = wl.B * wl.L
    bytes_alg = _alg_bytes_chunkwise()
    C = wl.chunk
    flops_alg = wl.B * wl.H * (wl.L / C) * 2 * (C * (C + 1) / 2 * (wl.dk + wl.dv) + 2 * C * wl.dk * wl.dv)
    achieved = bytes_alg / per_call / 1e9
    traffic = _read_traffic("chunkwise_32k")
    spread = _spread()
    return {
        "tokens_per_s": tokens / per_call, "ms_per_step": per_call * 1e3, "tokens": tokens, **spread,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "retention_chunkwise call: seg_state_kernel + seg_scan_kernel + seg_out_kernel (durations summed)",
                     "algorithmic_bytes_per_call": bytes_alg},
        "mfma": {"algorithmic_tflop_per_call": flops_alg / 1e12,
                 "achieved_tflops": flops_alg / per_call / 1e12,
                 "frac_of_bf16_peak": flops_alg / per_call / 1e12 / BF16_PEAK_TFLOPS},
    }


def bench_chunkwise_bwd(steps, warmup, with_saved=True):
    """Gradients of retention (dq, dk, dv) on the long-context workload (B1 H8
    L32768 dk128 dv256, chunk 256, bf16 in and out) for a seeded output gradient.
    with_saved: also the backward on the forward call's segment states, and the
    forward + backward step (left out of the counter runs, which count the
    self-contained backward's calls)."""
    import torch
    import retentive_network_scale_amd as rn
    from workloads import CHUNKWISE_32K as wl, randn
    q, k, v = (t.cuda() for t in wl.qkv())
    do = randn((wl.B, wl.H, wl.L, wl.dv), 3009, 1.0, torch.bfloat16).cuda()
    g, th = wl.gamma(), wl.theta()
    outs = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    ws = torch.empty(rn.retention_chunkwise_bwd_workspace_bytes(wl.B, wl.H, wl.L, wl.dk, wl.dv, wl.chunk),
                     dtype=torch.uint8, device="cuda")
    t = _time_calls(lambda: rn.retention_chunkwise_bwd(q, k, v, do, g, wl.chunk, th, out=outs, workspace=ws),
                    steps, warmup)
    per_call = t / steps
    spread = _spread()
    bytes_alg = _alg_bytes_bwd()
    achieved = bytes_alg / per_call / 1e9
    roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": _read_traffic("chunkwise_bwd"),
            "kernel": "retention_chunkwise_bwd call: one rotation pass, three chunkwise retentions "
                      "(64-token chunks inside the chunk-256 segments) writing the gradients through "
                      "an un-rotating, reversing epilogue",
            "algorithmic_bytes_per_call": bytes_alg}
    res = {"tokens_per_s": wl.B * wl.L / per_call, "ms_per_step": per_call * 1e3, **spread, "roofline": roof}
    if not with_saved:
        return res
    # The same gradients with the forward call's segment states handed over (as a
    # training step keeps them): the forward runs once, untimed, into its
    # workspace; then the backward alone, and forward + backward as one step.
    fo = torch.empty_like(v)
    fws = torch.empty(rn.retention_chunkwise_workspace_bytes(wl.B, wl.H, wl.L, wl.dk, wl.dv, wl.chunk),
                      dtype=torch.uint8, device="cuda")
    rn.retention_chunkwise(q, k, v, g, wl.chunk, th, out=fo, workspace=fws)
    t_s = _time_calls(lambda: rn.retention_chunkwise_bwd(q, k, v, do, g, wl.chunk, th, out=outs, workspace=ws,
                                                         fwd_workspace=fws), steps, warmup)
    saved = {"ms_per_step": t_s / steps * 1e3, "tokens_per_s": wl.B * wl.L * steps / t_s, **_spread(),
             "hbm_frac": bytes_alg / (t_s / steps) / 1e9 / HBM_PEAK_GBS,
             "what": "retention_chunkwise_bwd_saved: the dq sum reads the forward call's segment states "
                     "(no state pass or scan of its own)"}

    def train_step():
        rn.retention_chunkwise(q, k, v, g, wl.chunk, th, out=fo, workspace=fws)
        rn.retention_chunkwise_bwd(q, k, v, do, g, wl.chunk, th, out=outs, workspace=ws, fwd_workspace=fws)
    t_t = _time_calls(train_step, steps, warmup)
    train = {"ms_per_step": t_t / steps * 1e3, "tokens_per_s": wl.B * wl.L * steps / t_t, **_spread(),
             "what": "forward (retention_chunkwise, bf16 out) then the backward with its segment states"}
    return {**res, "with_forward_states": saved, "forward_plus_backward": train}


SWEEP_CHUNKS = (64, 128, 256, 512, 1024, 2048)


def bench_chunk_sweep(steps, warmup):
    """Chunkwise tokens/s on the L=32768 workload for each chunk size (same inputs,
    same outputs up to rounding; the chunk only moves work between the direct
    intra-chunk sums and the state)."""
    import torch
    import retentive_network_scale_amd as rn
    from workloads import CHUNKWISE_32K as wl
    q, k, v = (t.cuda() for t in wl.qkv())
    g, th = wl.gamma(), wl.theta()
    out = torch.empty((wl.B, wl.H, wl.L, wl.dv), dtype=torch.bfloat16, device="cuda")
    state = torch.empty((wl.B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device="cuda")
    res = {}
    for chunk in SWEEP_CHUNKS:
        ws = torch.empty(rn.retention_chunkwise_workspace_bytes(wl.B, wl.H, wl.L, wl.dk, wl.dv, chunk),
                         dtype=torch.uint8, device="cuda")
        t = _time_calls(lambda: rn.retention_chunkwise(q, k, v, g, chunk, th, state_out=state, out=out,
                                                       workspace=ws), steps, warmup)
        res[str(chunk)] = {"tokens_per_s": wl.B * wl.L * steps / t, "ms_per_step": t / steps * 1e3, **_spread()}
    return res


def bench_decode(warmup_loops=1):
    import torch
    import retentive_network_scale_amd as rn
    from workloads import DECODE as wl
    g, th = wl.gamma(), wl.theta()
    pq, pk, pv = (t.cuda() for t in wl.prefill_qkv())
    sq, sk, sv = (t.cuda() for t in wl.step_qkv())
    state = torch.empty((wl.B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device="cuda")
    pos_all = (torch.arange(wl.steps, dtype=torch.int32) + wl.prefill).reshape(-1, 1).expand(-1, wl.B)
    pos_all = pos_all.contiguous().cuda()
    outs = torch.empty((wl.steps, wl.B, wl.H, wl.dv), dtype=torch.bfloat16, device="cuda")
    qs, ks, vs, ps, os_ = ([x[t] for t in range(wl.steps)] for x in (sq, sk, sv, pos_all, outs))

    def prefill():
        rn.retention_chunkwise(pq, pk, pv, g, wl.chunk, th, state_out=state)

    def loop():
        for t in range(wl.steps):
            rn.retention_recurrent_step(qs[t], ks[t], vs[t], state, ps[t], g, th, out=os_[t])
    for _ in range(warmup_loops):
        prefill()
        loop()
    prefill()
    torch.cuda.synchronize()
    t = _time_calls(loop, 1, 0)
    per_step = t / wl.steps
    bytes_step = _alg_bytes_decode()
    achieved = bytes_step / per_step / 1e9
    return {"tokens_per_s": wl.B * wl.steps / t, "ms_per_step": per_step * 1e3, "steps": wl.steps,
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "traffic": _read_traffic("decode_step"),
                         "kernel": "vec_step_kernel (one launch per step; launch gaps included)",
                         "algorithmic_bytes_per_call": bytes_step}}


def bench_parallel(steps, warmup):
    import torch
    import retentive_network_scale_amd as rn
    from workloads import PARALLEL_2K as wl
    q, k, v = (t.cuda() for t in wl.qkv())
    g, th = wl.gamma(), wl.theta()
    out = torch.empty((wl.B, wl.H, wl.L, wl.dv), dtype=torch.bfloat16, device="cuda")
    t = _time_calls(lambda: rn.retention_parallel(q, k, v, g, th, gn_eps=wl.gn_eps, out=out), steps, warmup)
    per_call = t / steps
    flops = 2 * wl.B * wl.H * wl.L * (wl.L + 1) / 2 * (wl.dk + wl.dv)
    tf = flops / per_call / 1e12
    return {"tokens_per_s": wl.B * wl.L / per_call, "ms_per_step": per_call * 1e3, **_spread(),
            "roofline": {"bound": "mfma", "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf / BF16_PEAK_TFLOPS, "traffic": _read_traffic("parallel_2k"),
                         "kernel": "retention_parallel call: rotate_keys_kernel (keys rotated once) + qblock_kernel<256,512,parallel> (hi+lo scores for the first query block of each sequence; keys by LDS-DMA, bf16 scores for the rest)",
                         "algorithmic_tflop_per_call": flops / 1e12}}


def bench_msr(steps, warmup):
    import torch
    import retentive_network_scale_amd as rn
    from workloads import MSR_LAYER as wl
    x, wq, wk, wv, wg, wo = wl.inputs()
    x, wo = x.cuda(), wo.cuda()
    wq, wk, wv, wg = _fused_qkvg(wq, wk, wv, wg)
    g, th = wl.gamma(), wl.theta()
    y = torch.empty((wl.B, wl.L, wl.d_model), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(rn.msr_layer_fwd_workspace_bytes(wl.B, wl.L, wl.d_model, wl.H, wl.dk, wl.dv, wl.chunk),
                     dtype=torch.uint8, device="cuda")
    t = _time_calls(lambda: rn.msr_layer_fwd(x, wq, wk, wv, wg, wo, wl.H, wl.dk, wl.dv, wl.chunk, g, th,
                                             gn_eps=wl.gn_eps, out=y, workspace=ws), steps, warmup)
    per_call = t / steps
    T = wl.B * wl.L
    C = wl.chunk
    gemm = 2 * T * wl.d_model * (2 * wl.H * wl.dk + 2 * wl.H * wl.dv) + 2 * T * wl.H * wl.dv * wl.d_model
    ret = T * wl.H * ((C + 1) * (wl.dk + wl.dv) + 4 * wl.dk * wl.dv)
    tf = (gemm + ret) / per_call / 1e12
    return {"tokens_per_s": T / per_call, "ms_per_step": per_call * 1e3, **_spread(),
            "roofline": {"bound": "mfma", "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf / BF16_PEAK_TFLOPS, "traffic": _read_traffic("msr_layer"),
                         "kernel": "msr_layer_fwd (GEMM, chunkwise retention, GroupNorm+gate, GEMM)",
                         "algorithmic_tflop_per_call": (gemm + ret) / 1e12}}


COPY_BYTES = 1 << 29  # 512 MiB: the plain streaming kernel that calibrates FETCH_SIZE / WRITE_SIZE


def copy_calibration(reps=3):
    """A plain elementwise copy (torch.neg, bf16) of COPY_BYTES read + COPY_BYTES
    written, larger than the last-level cache, so that a rocprofv3 PMC run of this
    command can convert the TCC FETCH_SIZE / WRITE_SIZE counters to HBM bytes."""
    import torch
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


# Which dispatches make one call of each workload, for the PMC summary:
# (kernels summed per call, kernel that occurs exactly once per call).  The
# parallel form launches two query-block kernels per call (its hi+lo first
# blocks, SPLIT = true, and the rest): only the second counts the calls.
# The gated layer's legs also count the hipBLASLt GEMM kernels (names start with
# Cijk / Custom_Cijk); the backward counts calls by its one (dk, dv) = (128, 256)
# retention.
_PMC_GROUPS = {
    "chunkwise_32k": (("ret::",), ("seg_out_kernel",)),
    "decode_step": (("vec_step_kernel",), ("vec_step_kernel",)),
    "parallel_2k": (("qblock_kernel", "rotate_keys_kernel"), ("qblock_kernel<256, 512, true, false, true>",)),
    "chunkwise_bwd": (("ret::",), ("seg_state_kernel<128, 256>",)),
    "msr_layer": (("ret::", "Cijk"), ("seg_scan_t_kernel",)),
    "msr_decode": (("ret::", "Cijk"), ("vec_step_kernel",)),
    "retnet_block": (("ret::", "Cijk"), ("gelu_bf16_kernel",)),
}


def _alg_bytes_bwd():
    """q, k, v, dO read once; dq, dk, dv written once (bf16)."""
    from workloads import CHUNKWISE_32K as wl
    return 2 * wl.B * wl.H * wl.L * (2 * wl.dk + 2 * wl.dv) + 2 * wl.B * wl.H * wl.L * (2 * wl.dk + wl.dv)


def _alg_bytes_msr():
    """The gated layer's minimum: X and the five weights read once, Y written once."""
    from workloads import MSR_LAYER as wl
    T = wl.B * wl.L
    return 2 * (2 * T * wl.d_model + wl.d_model * (2 * wl.H * wl.dk + 3 * wl.H * wl.dv))


def _alg_bytes_block():
    """The residual block's minimum: X and the seven weights read once, the block's
    output written once (FFN width 2 d_model, as bench_block runs it)."""
    from workloads import MSR_LAYER as wl
    T, dff = wl.B * wl.L, 2 * wl.d_model
    return 2 * (2 * T * wl.d_model + wl.d_model * (2 * wl.H * wl.dk + 3 * wl.H * wl.dv) + 2 * wl.d_model * dff)


def _alg_bytes_msr_decode():
    """Per step of 64 sequences: the five weights, the fp32 state read and written,
    the step's input and output rows."""
    from workloads import MSR_LAYER as wl
    B = MSR_DECODE_B
    return 2 * wl.d_model * (2 * wl.H * wl.dk + 3 * wl.H * wl.dv) + 2 * 4 * B * wl.H * wl.dk * wl.dv + 2 * 2 * B * wl.d_model


def pmc_summary(name, fetch_csv, write_csv, command, out_dir=None):
    """Turns two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, then
    WRITE_SIZE, in KiB per dispatch) of a `bench.py --only ... --copy-calibration`
    run into profiles/traffic_<name>.txt: HBM bytes per call, scaled by the
    counters' reading for the calibration copy."""
    import csv
    import collections
    incl, once = _PMC_GROUPS[name]

    def read(path, counter):
        per_kernel = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                per_kernel[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        copy = [v for k, lst in per_kernel.items() if "neg_kernel" in k for v in lst]
        calls = sum(len(lst) for k, lst in per_kernel.items() if any(o in k for o in once))
        total = sum(sum(lst) for k, lst in per_kernel.items() if any(i in k for i in incl))
        names = sorted(k for k in per_kernel if any(i in k for i in incl))
        if not copy or not calls:
            raise SystemExit(f"{path}: no calibration copy or no {once} dispatches")
        copy_kib = sum(copy) / len(copy)
        return total / calls, copy_kib, calls, names
    f_kib, f_copy, calls, names = read(fetch_csv, "FETCH_SIZE")
    w_kib, w_copy, _, _ = read(write_csv, "WRITE_SIZE")
    f_fac, w_fac = COPY_BYTES / (f_copy * 1024), COPY_BYTES / (w_copy * 1024)
    hbm = f_kib * 1024 * f_fac + w_kib * 1024 * w_fac
    alg = {"chunkwise_32k": _alg_bytes_chunkwise, "decode_step": _alg_bytes_decode,
           "parallel_2k": _alg_bytes_parallel, "chunkwise_bwd": _alg_bytes_bwd, "msr_layer": _alg_bytes_msr,
           "msr_decode": _alg_bytes_msr_decode, "retnet_block": _alg_bytes_block}[name]()
    out = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"traffic_{name}.txt")
    with open(out, "w") as fh:
        fh.write(f"# HBM traffic per call of {name}: rocprofv3 PMC FETCH_SIZE and WRITE_SIZE (KiB per dispatch),\n"
                 f"# summed over the dispatches of one call ({calls} calls), each scaled by the factor that maps\n"
                 f"# the counter's reading for a plain bf16 copy of {COPY_BYTES} bytes (torch.neg) to those bytes.\n")
        for c in command:
            fh.write(f"# command: {c}\n")
        fh.write("# kernels: " + "; ".join(n[:90] for n in names) + "\n")
        fh.write(f"fetch_kib_per_call = {f_kib:.1f}\nwrite_kib_per_call = {w_kib:.1f}\n"
                 f"copy_fetch_kib = {f_copy:.1f}\ncopy_write_kib = {w_copy:.1f}\n"
                 f"fetch_factor = {f_fac:.4f}\nwrite_factor = {w_fac:.4f}\n"
                 f"hbm_bytes_per_call = {hbm:.0f}\nalgorithmic_bytes_per_call = {alg}\n"
                 f"traffic_over_algorithmic = {hbm / alg:.3f}\nsrc_sha = {_src_sha()}\n")
    print(open(out).read())


# MI355X layout the utilisation counters are normalised by: SQ counters are summed
# over all CUs (and SIMDs), GRBM_GUI_ACTIVE over the XCDs.
N_XCD, N_CU, SIMD_PER_CU = 8, 256, 4
UTIL_COUNTERS = ("SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_WAVE_CYCLES SQ_WAIT_INST_LDS SQ_INSTS_LDS_LOAD_BANDWIDTH "
                 "SQ_INSTS_LDS_STORE_BANDWIDTH SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE")


def util_summary(name, counters_csv, command, out_dir=None):
    """Turns one rocprofv3 --pmc counter_collection.csv (the UTIL_COUNTERS set) of a
    `bench.py --only ...` run into profiles/util_<name>.txt: per kernel, the
    dispatch-averaged counters and the fractions derived from them.
      active cycles per XCD = GRBM_GUI_ACTIVE / N_XCD
      MFMA busy  = SQ_VALU_MFMA_BUSY_CYCLES / (cycles * N_CU * SIMD_PER_CU)
      LDS busy   = SQ_LDS_IDX_ACTIVE / (cycles * N_CU)
      bank conflicts = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE
      LDS wait   = SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES"""
    import csv
    import collections
    sums = collections.defaultdict(lambda: collections.defaultdict(float))
    counts = collections.defaultdict(lambda: collections.defaultdict(int))
    for r in csv.DictReader(open(counters_csv)):
        k = r["Kernel_Name"]
        if not k.startswith(("ret::", "void ret::")):
            continue
        sums[k][r["Counter_Name"]] += float(r["Counter_Value"])
        counts[k][r["Counter_Name"]] += 1
    if not sums:
        raise SystemExit(f"{counters_csv}: no kernels of this library")
    out = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"util_{name}.txt")
    with open(out, "w") as fh:
        fh.write(f"# MFMA and LDS utilisation of the {name} kernels: rocprofv3 PMC counters, averaged per dispatch.\n"
                 f"# Normalised for {N_XCD} XCDs, {N_CU} CUs, {SIMD_PER_CU} SIMDs per CU:\n"
                 "#   cycles = GRBM_GUI_ACTIVE / XCDs; mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles * SIMDs);\n"
                 "#   lds_busy = SQ_LDS_IDX_ACTIVE / (cycles * CUs); lds_bank_conflict = SQ_LDS_BANK_CONFLICT /\n"
                 "#   SQ_LDS_IDX_ACTIVE; lds_wait = SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES\n")
        for c in command:
            fh.write(f"# command: {c}\n")
        for k in sorted(sums, key=lambda k: -sums[k].get("GRBM_GUI_ACTIVE", 0.0)):
            avg = {c: sums[k][c] / counts[k][c] for c in sums[k]}
            cyc = avg.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD
            if cyc <= 0:
                continue
            mfma = avg.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (cyc * N_CU * SIMD_PER_CU)
            lds = avg.get("SQ_LDS_IDX_ACTIVE", 0.0) / (cyc * N_CU)
            conf = avg.get("SQ_LDS_BANK_CONFLICT", 0.0) / max(avg.get("SQ_LDS_IDX_ACTIVE", 0.0), 1.0)
            wait = avg.get("SQ_WAIT_INST_LDS", 0.0) / max(avg.get("SQ_WAVE_CYCLES", 0.0), 1.0)
            n = max(counts[k].values())
            fh.write(f"\nkernel = {k[:110]}\ndispatches = {n}\ncycles_per_xcd = {cyc:.0f}\n"
                     f"mfma_busy = {mfma:.3f}\nlds_busy = {lds:.3f}\nlds_bank_conflict = {conf:.3f}\n"
                     f"lds_wait = {wait:.3f}\n")
        fh.write(f"\nsrc_sha = {_src_sha()}\n")
    print(open(out).read())


def stats_summary(trace_dir, command):
    """Markdown tables of a rocprofv3 --kernel-trace --stats run: the kernel_stats.csv
    as written, then the kernel_trace.csv grouped by kernel and grid size (one
    group per workload shape)."""
    import csv
    import glob
    import collections
    stats = glob.glob(os.path.join(trace_dir, "*_kernel_stats.csv"))[0]
    trace = glob.glob(os.path.join(trace_dir, "*_kernel_trace.csv"))[0]
    print(f"command: `{command}`\n")
    print("| kernel | calls | avg us | min us | max us | % of GPU time |\n|---|---|---|---|---|---|")
    for r in csv.DictReader(open(stats)):
        print(f"| `{r['Name'][:100]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
              f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |")
    groups = collections.OrderedDict()
    for r in csv.DictReader(open(trace)):
        key = (r["Kernel_Name"][:80], int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]), r["VGPR_Count"],
               r["Accum_VGPR_Count"], r["Scratch_Size"], r["LDS_Block_Size"])
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print("\n| kernel | workgroups | arch VGPR | acc VGPR | scratch B | LDS B | calls | avg us | min us |\n"
          "|---|---|---|---|---|---|---|---|---|")
    for (name, wg, vg, ag, sc, lds), d in groups.items():
        print(f"| `{name}` | {wg} | {vg} | {ag} | {sc} | {lds} | {len(d)} | {sum(d) / len(d):.1f} | {min(d):.1f} |")


def bench_block(steps, warmup):
    """The pre-LN residual block around the gated layer at the layer workload's
    dimensions, FFN width 2 d_model (the pages give none): one retnet_block_fwd."""
    import torch
    import retentive_network_scale_amd as rn
    from workloads import MSR_LAYER as wl, randn
    x, wq, wk, wv, wg, wo = wl.inputs()
    dff = 2 * wl.d_model
    w1 = randn((dff, wl.d_model), 5008, wl.w_std, torch.bfloat16).cuda()
    w2 = randn((wl.d_model, dff), 5009, wl.w_std, torch.bfloat16).cuda()
    x, wo = x.cuda(), wo.cuda()
    wq, wk, wv, wg = _fused_qkvg(wq, wk, wv, wg)
    g, th = wl.gamma(), wl.theta()
    out = torch.empty_like(x)
    ws = torch.empty(rn.retnet_block_fwd_workspace_bytes(wl.B, wl.L, wl.d_model, wl.H, wl.dk, wl.dv, dff,
                                                         wl.chunk), dtype=torch.uint8, device="cuda")
    t = _time_calls(lambda: rn.retnet_block_fwd(x, wq, wk, wv, wg, wo, w1, w2, wl.H, wl.dk, wl.dv, wl.chunk, g, th,
                                                gn_eps=wl.gn_eps, out=out, workspace=ws), steps, warmup)
    per_call = t / steps
    T, C = wl.B * wl.L, wl.chunk
    gemm = 2 * T * wl.d_model * (2 * wl.H * wl.dk + 2 * wl.H * wl.dv) + 2 * T * wl.H * wl.dv * wl.d_model
    ret = T * wl.H * ((C + 1) * (wl.dk + wl.dv) + 4 * wl.dk * wl.dv)
    ffn = 4 * T * wl.d_model * dff
    tf = (gemm + ret + ffn) / per_call / 1e12
    return {"tokens_per_s": T / per_call, "ms_per_step": per_call * 1e3, "d_ffn": dff, **_spread(),
            "roofline": {"bound": "mfma", "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf / BF16_PEAK_TFLOPS, "traffic": _read_traffic("retnet_block"),
                         "kernel": "retnet_block_fwd (LayerNorm, gated layer, residual GEMM, LayerNorm, FFN GEMMs "
                                   "with gelu, residual GEMM)",
                         "algorithmic_tflop_per_call": (gemm + ret + ffn) / 1e12}}


MSR_DECODE_B, MSR_DECODE_STEPS = 64, 1024


def _fused_qkvg(wq, wk, wv, wg):
    """The four projection weights in one device buffer, rows [W_Q; W_K; W_V; W_G]
    (as a model stores them), returned as views."""
    import torch
    cat = torch.cat([wq, wk, wv, wg], 0).cuda()
    n = [wq.shape[0], wk.shape[0], wv.shape[0], wg.shape[0]]
    return list(torch.split(cat, n, 0))


def bench_msr_decode(steps=MSR_DECODE_STEPS):
    """Decode with the gated layer (d_model 2048, 8 heads, dk 256, dv 512) for 64
    sequences: one captured msr_layer_step (positions advanced on the device)
    replayed once per token.  The step's input rows stay in one static buffer;
    every replay does the whole step's work."""
    import torch
    import retentive_network_scale_amd as rn
    from workloads import MSR_LAYER as wl, randn
    B = MSR_DECODE_B
    _, wq, wk, wv, wg, wo = wl.inputs()
    wd = [*_fused_qkvg(wq, wk, wv, wg), wo.cuda()]
    g, th = wl.gamma(), wl.theta()
    x = randn((B, wl.d_model), 5000, 1.0, torch.bfloat16).cuda()
    y = torch.empty((B, wl.d_model), dtype=torch.bfloat16, device="cuda")
    state = torch.zeros((B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device="cuda")
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    ws = torch.empty(rn.msr_layer_step_workspace_bytes(B, wl.d_model, wl.H, wl.dk, wl.dv), dtype=torch.uint8,
                     device="cuda")

    def step(adv):
        rn.msr_layer_step(x, *wd, state, pos, wl.H, wl.dk, wl.dv, g, th, gn_eps=wl.gn_eps, advance_pos=adv,
                          out=y, workspace=ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(True)
    for _ in range(8):
        graph.replay()
    torch.cuda.synchronize()
    t = _time_calls(graph.replay, steps, 0)
    per_step = t / steps
    weights = 2 * wl.d_model * (2 * wl.H * wl.dk + 3 * wl.H * wl.dv)
    bytes_step = weights + 2 * 4 * B * wl.H * wl.dk * wl.dv + 2 * 2 * B * wl.d_model
    achieved = bytes_step / per_step / 1e9
    return {"tokens_per_s": B * steps / t, "ms_per_step": per_step * 1e3, "steps": steps, "batch": B,
            **{k: v for k, v in _spread().items() if k != "calls_timed"},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "traffic": _read_traffic("msr_decode"),
                         "kernel": "msr_layer_step graph replay (fused projection GEMM, vec_step_kernel with "
                                   "GroupNorm and gate, output GEMM, position advance)",
                         "algorithmic_bytes_per_call": bytes_step}}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _omp_threads():
    """Threads the oracle's OpenMP loops run with: OMP_NUM_THREADS when set (the
    process's CPU share), else the CPUs this process may run on."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    return int(env) if env.isdigit() and int(env) > 0 else len(os.sched_getaffinity(0))


def _set_omp_threads(n):
    import ctypes
    ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))


def _recurrent_column_blocks(q, k, v, g, th, ncb):
    """The oracle's recurrent form with V split into ncb column blocks, each block a
    head of its own: an output column depends only on the same column of V, so the
    blocks are independent units for the oracle's OpenMP loop (the rotation of q and
    k is repeated per block; everything else is the same arithmetic)."""
    import numpy as np
    import oracle
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    qq, kk = (np.ascontiguousarray(np.repeat(x, ncb, axis=1)) for x in (q, k))
    vv = np.ascontiguousarray(v.reshape(B, H, L, ncb, dv // ncb).transpose(0, 1, 3, 2, 4).reshape(B, H * ncb, L, -1))
    gg = np.repeat(np.asarray(g, dtype=np.float64), ncb)

    def run():
        return oracle.recurrent(qq, kk, vv, gg, th)
    return run


def cpu_baseline(seconds=10.0):
    """The fp64 oracle timed on this host's CPUs, after the GPU legs.  Main figure:
    the recurrent form (the reference form for the long-context workload) over the
    whole B1 H8 L32768 dk128 dv256 workload, V split into column blocks so that the
    OpenMP loop has a unit per thread, whole passes until `seconds` have elapsed.
    Context: one-thread runs of the tiny workload (all three forms), of one (b, h)
    slice of the parallel workload (the literal double sum) and of the first 4096
    tokens of the long-context workload (recurrent form)."""
    import numpy as np
    import oracle
    from workloads import CHUNKWISE_32K as wl, PARALLEL_2K, TINY
    threads = _omp_threads()
    q, k, v = (oracle.as_f64(t) for t in wl.qkv())
    g, th = wl.gamma().double().numpy(), wl.theta()
    ncb = 1
    while wl.B * wl.H * ncb < threads and wl.dv // (2 * ncb) >= 8:
        ncb *= 2
    run = _recurrent_column_blocks(q, k, v, g, th, ncb)
    _set_omp_threads(threads)
    reps, t0 = 0, time.perf_counter()
    while True:
        run()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= seconds or reps >= 50:
            break
    units = wl.B * wl.H * ncb
    res = {"value": reps * wl.B * wl.L / dt, "unit": "tokens/s", "cores": min(threads, units), "kind": "oracle",
           "nproc": os.cpu_count(), "cpus_allowed": len(os.sched_getaffinity(0)), "cpu_model": _cpu_model(),
           "sample": f"fp64 recurrent oracle over the whole chunkwise workload (B1 H8 L32768 dk128 dv256, all 32768 "
                     f"tokens of all {wl.H} heads), V in {ncb} column blocks: {units} OpenMP units on {threads} "
                     f"threads, {reps} passes in {dt:.1f} s"}
    # one-thread context runs
    _set_omp_threads(1)
    one = {}
    try:
        tq, tk, tv = TINY.qkv()
        tg, tt = TINY.gamma(), TINY.theta()
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 0.5:
            oracle.parallel(tq, tk, tv, tg, tt)
            oracle.recurrent(tq, tk, tv, tg, tt)
            oracle.chunkwise(tq, tk, tv, tg, TINY.chunk, tt)
            n += 1
        one["tiny"] = {"tokens_per_s": n * TINY.B * TINY.L / (time.perf_counter() - t0),
                       "form": "parallel + recurrent + chunkwise, whole workload"}
        pw = PARALLEL_2K
        pq, pk, pv = (oracle.as_f64(x[:1, :1]) for x in pw.qkv())
        t0 = time.perf_counter()
        oracle.parallel(pq, pk, pv, pw.gamma()[:1], pw.theta())
        dt1 = time.perf_counter() - t0
        one["parallel"] = {"tokens_per_s": pw.L / pw.H / dt1, "seconds": dt1,
                           "form": "literal double sum on one (b, h) slice (a token counts once over its 8 heads)"}
        m = 4096
        t0 = time.perf_counter()
        oracle.recurrent(q[:, :, :m], k[:, :, :m], v[:, :, :m], g, th)
        dt1 = time.perf_counter() - t0
        one["chunkwise"] = {"tokens_per_s": wl.B * m / dt1, "seconds": dt1,
                            "form": f"recurrent form on tokens 0..{m - 1} of all {wl.H} heads"}
    finally:
        _set_omp_threads(threads)
    res["one_thread"] = one
    return res


def probe_peaks():
    """Rates this GPU attains beside the spec peaks: a plain HBM copy (torch.neg over
    1 GiB of bf16: 1 GiB read + 1 GiB written) and a large dense bf16 GEMM
    (torch.matmul, 8192 x 8192 x 8192, the vendor library)."""
    import torch
    n = 1 << 29
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    t = _time_calls(lambda: torch.neg(src, out=dst), 20, 3)
    copy = 2 * 2 * n * 20 / t / 1e9
    del src, dst
    a = torch.randn(8192, 8192, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(8192, 8192, dtype=torch.bfloat16, device="cuda")
    c = torch.empty_like(a)
    t = _time_calls(lambda: torch.matmul(a, b, out=c), 20, 3)
    gemm = 2 * 8192 ** 3 * 20 / t / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    return {"hbm_copy_gbs": copy, "bf16_gemm_tflops": gemm,
            "what": "torch.neg over 1 GiB bf16 (bytes read + written); torch.matmul 8192^3 bf16"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-extra", action="store_true", help="headline chunkwise workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="wall time of the CPU oracle's main figure")
    ap.add_argument("--only", choices=["chunkwise", "decode", "parallel", "msr", "msr_decode", "sweep", "bwd",
                                       "block"],
                    help="run one workload and print its figures (for profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run the plain copy that calibrates the PMC byte counters")
    ap.add_argument("--pmc-summary", nargs=3, metavar=("NAME", "FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_NAME.txt from two rocprofv3 PMC runs (no GPU needed)")
    ap.add_argument("--pmc-command", action="append", default=[], help="command line recorded in the summary")
    ap.add_argument("--util-summary", nargs=2, metavar=("NAME", "COUNTERS_CSV"),
                    help="write profiles/util_NAME.txt from one rocprofv3 PMC run of UTIL_COUNTERS (no GPU needed)")
    ap.add_argument("--stats-summary", nargs=2, metavar=("TRACE_DIR", "COMMAND"),
                    help="print a rocprofv3 --kernel-trace --stats output folder as tables (no GPU needed)")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, args.pmc_command)
        return
    if args.stats_summary:
        stats_summary(*args.stats_summary)
        return
    if args.util_summary:
        util_summary(*args.util_summary, args.pmc_command)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import retentive_network_scale_amd as rn
    rn.lib()  # fails loudly if the HIP library is not built
    if args.copy_calibration:
        _log(f"calibration copy of {COPY_BYTES} bytes")
        copy_calibration()
    if args.only and args.only != "chunkwise":
        _log(args.only)
        res = {"decode": lambda: bench_decode(), "parallel": lambda: bench_parallel(args.steps, args.warmup),
               "msr": lambda: bench_msr(args.steps, args.warmup),
               "msr_decode": lambda: bench_msr_decode(),
               "bwd": lambda: bench_chunkwise_bwd(args.steps, args.warmup, with_saved=False),
               "block": lambda: bench_block(args.steps, args.warmup),
               "sweep": lambda: {"chunk_sweep": bench_chunk_sweep(args.steps, args.warmup)}}[args.only]()
        print(json.dumps({"workload": args.only, **res}), flush=True)
        return
    from workloads import CHUNKWISE_32K
    _log("chunkwise L=32768")
    ch = bench_chunkwise(args.steps, args.warmup)
    line = {
        "metric": METRIC, "value": ch["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ch["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": CHUNKWISE_32K.name, "batch": CHUNKWISE_32K.B, "seq_len": CHUNKWISE_32K.L,
                   "heads": CHUNKWISE_32K.H, "dk": CHUNKWISE_32K.dk, "dv": CHUNKWISE_32K.dv,
                   "chunk": CHUNKWISE_32K.chunk},
        "roofline": ch["roofline"], "chunkwise_mfma": ch["mfma"],
        "median_ms_per_step": ch.get("median_ms"), "min_ms_per_step": ch.get("min_ms"),
    }
    if not (args.no_extra or args.only):
        _log("decode B128 H16, 1024 steps")
        line["decode"] = bench_decode()
        _log("parallel B8 H8 L2048")
        line["parallel"] = bench_parallel(max(3, args.steps // 2), args.warmup)
        _log("msr layer B4 L4096")
        line["msr_layer"] = bench_msr(max(3, args.steps // 4), args.warmup)
        _log("retnet block B4 L4096")
        line["retnet_block"] = bench_block(max(3, args.steps // 4), args.warmup)
        _log("chunkwise backward L=32768")
        line["chunkwise_bwd"] = bench_chunkwise_bwd(max(3, args.steps // 4), args.warmup)
        _log("msr decode B64, 1024 graph replays")
        line["msr_decode"] = bench_msr_decode()
        _log("chunk-size sweep")
        line["chunk_sweep"] = bench_chunk_sweep(max(5, args.steps // 2), args.warmup)
    if not args.only:
        _log("probe peaks (HBM copy, bf16 GEMM)")
        pk = line["probe_peaks"] = probe_peaks()
        for leg in [line] + [v for v in line.values() if isinstance(v, dict) and "roofline" in v]:
            r = leg["roofline"]
            att = pk["hbm_copy_gbs"] if r["bound"] == "hbm" else pk["bf16_gemm_tflops"]
            r["attainable"] = att
            r["frac_of_attainable"] = r["achieved"] / att
    if not (args.no_cpu or args.only):
        _log("cpu baseline")
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
