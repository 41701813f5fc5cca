"""Benchmark: packed CTC loss + gradient on one MI355X.

One step = one packed_ctc_loss call (loss, mean reduction and the full (T_total, D) gradient) over
the large-vocabulary batch: B=16 utterances, T_i uniform in [500, 3000], D=8193 (blank 0),
U_i = round(T_i/6), float16 log probabilities, reduction mean.  Inputs are generated with a fixed
seed and are resident in HBM before the timed region.

The calls run on the streamed pipeline (one persistent launch for the recursions and the gradient
rows) unless --pipeline grouped is given; the other pipeline is timed too, for context.

Prints one JSON line with frames/s, the whole-call HBM rate over the counted bytes
T_total * D * (2 bytes read + 2 bytes written), the per-kernel breakdown from HIP events recorded
around each kernel during a second pass of the same number of steps (the timed pass records no
events of its own), the roofline of the dominant kernel, and the float64 CPU oracle timed on
this host's cores on the same batch.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "packed CTC loss+grad frames/s and achieved HBM GB/s (% of MI355X peak)"
HBM_PEAK_GBPS = 8000.0
# fp32 vector peak without packed FP32 instructions (the library is built without them): 256 compute
# units x 4 SIMDs x 16 lanes x 2 flops (FMA) x 2.4 GHz = 78.6 TFLOP/s (the packed rate is twice that)
FP32_VECTOR_PEAK_TFLOPS = 78.6
WORKLOADS = ["tiny", "small", "asr_bpe", "large_vocab", "char_level"]
DTYPE_BYTES = {"f32": 4, "bf16": 2, "f16": 2}

# fp32 operations charged per state and frame of one recursion (alpha or beta): a 3-way max/med/min,
# two subtractions, two exp2, two adds, one log2, two adds (shift and emission) -- 12 ops, each
# transcendental counted once.  Used only when the recursion kernel is the dominant one.
OPS_PER_STATE_STEP = 12


PHASE_KERNELS = {"chains": "chain_workers", "dense": "dense_kernel", "gather": "gather_kernel", "stream": "stream_workers"}


def kernel_sources_sha() -> str:
    import glob
    import hashlib

    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "ctc_forward_backward_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(workload: str, phase: str):
    """HBM bytes per call of a kernel (summed over its launches, one per utterance group) from the
    committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary (already scaled by the copy calibration);
    None when there is no summary or the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_bytes_{workload}.txt")
    if not os.path.exists(path) or phase not in PHASE_KERNELS:
        return None
    sha, rows = None, {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("source_sha = "):
                sha = line.split("=", 1)[1].strip()
            parts = line.split()
            if len(parts) >= 5 and parts[0].startswith(PHASE_KERNELS[phase]):
                try:
                    rows[parts[0]] = (float(parts[3]) + float(parts[4])) * 1e6
                except ValueError:
                    pass
    if sha != kernel_sources_sha() or len(rows) != 1:
        return None
    return next(iter(rows.values()))


def _median_ms(stream, fn, n, warm=2):
    import torch

    for _ in range(warm):
        fn()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for e0, e1 in evs:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    return t[len(t) // 2]


def all_configs(api, lib, dev, stream):
    """Every workload: median call time on the default (streamed) pipeline, frames/s, counted GB/s and
    its fraction of 8 TB/s, the longest utterance's frames and ns per frame of the call; the
    recursion floor (the longest utterance alone, loss only: its recursion kernel time) and the
    critical-path fraction (that floor over the call); alpha checkpointing at K = 8 and 32 (grouped
    pipeline): workspace and call time."""
    import ctypes

    import torch

    from ctc_forward_backward_amd import workloads as W

    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    sh = ctypes.c_void_p(stream.cuda_stream)
    res = {}
    for name in WORKLOADS:
        b = W.make_workload(name)
        lp, cu, ln, tg, tl = (x.to(dev) for x in (b.log_probs, b.cu_seqlens, b.lengths, b.targets, b.target_lengths))
        Umax, Wd = int(b.target_lengths.max()), int(b.targets.shape[1])
        flags = 1 * (cu.dtype == torch.int64) | 2 * (ln.dtype == torch.int64) | 4 * (tg.dtype == torch.int64) \
            | 8 * (tl.dtype == torch.int64)
        losses = torch.empty(b.B, dtype=torch.float32, device=dev)
        reduced = torch.empty((), dtype=torch.float32, device=dev)
        grad = torch.empty((b.T_total, b.D), dtype=lp.dtype, device=dev)
        bpe = lp.element_size()
        counted = b.T_total * b.D * 2 * bpe
        t_max = int(b.lengths.max())
        entry = {"B": b.B, "T_total": b.T_total, "D": b.D, "input_dtype": str(lp.dtype).replace("torch.", ""),
                 "T_max": t_max}
        for K in (1, 8, 32):
            ws_bytes = api.packed_ctc_workspace_size(b.T_total, b.D, b.B, Umax, K)
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
            args = (P(lp), api.DTYPE_CODES[lp.dtype], b.T_total, b.D, P(cu), P(ln), b.B, P(tg), Wd, P(tl), flags, Umax,
                    b.blank, int(b.zero_infinity), api.REDUCTIONS[b.reduction], None, P(losses), P(reduced), P(grad),
                    K, P(ws), ws_bytes, sh)

            def call():
                rc = lib.packed_ctc_loss(*args)
                if rc != 0:
                    raise RuntimeError(lib.packed_ctc_last_error().decode())

            ms = _median_ms(stream, call, 10 if K == 1 else 5)
            if K == 1:
                gbps = counted / (ms * 1e-3) / 1e9
                entry.update({"ms_per_call": ms, "frames_per_s": b.T_total / (ms * 1e-3), "counted_gbps": gbps,
                              "hbm_frac": gbps / HBM_PEAK_GBPS, "ns_per_frame_of_T_max": ms * 1e6 / t_max,
                              "workspace_bytes": ws_bytes})
            else:
                entry[f"checkpoint_K{K}"] = {"ms_per_call": ms, "workspace_bytes": ws_bytes}
            del ws
        # the recursion floor: the longest utterance alone, loss only, its recursion kernel's time
        i = int(b.lengths.argmax())
        r0, T0, U0 = int(b.cu_seqlens[i]), int(b.lengths[i]), int(b.target_lengths[i])
        lp1 = lp[r0:r0 + T0].contiguous()
        one = (torch.tensor([0, T0], dtype=torch.int32, device=dev), torch.tensor([T0], device=dev),
               tg[i:i + 1].contiguous(), torch.tensor([U0], device=dev))
        api.packed_ctc_loss(lp1, *one, blank=b.blank, need_grad=False, max_target_length=U0)
        torch.cuda.synchronize()
        api.set_phase_timing(True)
        for _ in range(5):
            api.packed_ctc_loss(lp1, *one, blank=b.blank, need_grad=False, max_target_length=U0)
        torch.cuda.synchronize()
        ph = api.phase_times()
        api.set_phase_timing(False)
        floor_ms = ph.get("chains@0", float("nan"))
        entry["critical_path"] = {"frames": t_max, "labels": U0, "floor_us": floor_ms * 1e3,
                                  "floor_ns_per_frame": floor_ms * 1e6 / t_max,
                                  "call_frac": floor_ms / entry["ms_per_call"]}
        res[name] = entry
        del lp, grad
        torch.cuda.empty_cache()
    return res


def extras(api, dev, stream):
    """The autograd forward + backward on the large-vocabulary batch, and float64 inputs (computed in
    float64) on a 13-utterance, 1025-class batch: median times."""
    import numpy as np
    import torch

    from ctc_forward_backward_amd import workloads as W

    out = {}
    b = W.make_workload("large_vocab")
    lp = b.log_probs.to(dev).requires_grad_(True)
    args = tuple(x.to(dev) for x in (b.cu_seqlens, b.lengths, b.targets, b.target_lengths))
    kw = dict(blank=b.blank, reduction=b.reduction, max_target_length=int(b.target_lengths.max()))

    half = torch.tensor(0.5, device=dev)

    def fwd_bwd():
        lp.grad = None
        api.ctc_loss(lp, *args, **kw).backward()

    def fwd_bwd_scaled():
        lp.grad = None
        api.ctc_loss(lp, *args, **kw).backward(half)

    out["autograd_large_vocab"] = {
        "ms_forward_backward": _median_ms(stream, fwd_bwd, 10),
        "ms_forward_backward_upstream_0.5": _median_ms(stream, fwd_bwd_scaled, 10),
        "note": "ctc_loss(...).backward(): packed_ctc_forward_grad writes the rows for a unit upstream gradient, "
                "packed_ctc_backward_update keeps them (upstream 1) or rewrites them (upstream 0.5)"}
    del lp
    rng = np.random.default_rng(31)
    lengths = [int(x) for x in rng.integers(1, 400, size=11)] + [0, 3]
    tl = [int(rng.integers(0, max(1, T // 3) + 1)) for T in lengths]
    targets = [[int(x) for x in rng.integers(1, 1025, size=u)] for u in tl]
    b64 = W.make_batch(lengths, targets, 1025, seed=9, sigma=3.0, dtype="f64", reduction="mean")
    a64 = tuple(x.to(dev) for x in (b64.log_probs, b64.cu_seqlens, b64.lengths, b64.targets, b64.target_lengths))
    ms64 = _median_ms(stream, lambda: api.packed_ctc_loss(*a64, blank=0, reduction="mean",
                                                          max_target_length=max(tl)), 10)
    out["float64"] = {"workload": f"B={b64.B} T_total={b64.T_total} D=1025 float64, computed in float64",
                      "ms_per_call": ms64, "frames_per_s": b64.T_total / (ms64 * 1e-3)}
    return out


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large_vocab",
                    choices=["tiny", "small", "asr_bpe", "large_vocab", "char_level"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle CPU-baseline leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-run", action="store_true",
                    help="only the warmup, timed and phase-timed steps (no call medians, other pipeline or HMM "
                         "leg): the run a profiler traces")
    ap.add_argument("--pipeline", default="streamed", choices=["streamed", "grouped"],
                    help="pipeline of the timed calls (the other one is timed too, for context)")
    ap.add_argument("--checkpoint-interval", type=int, default=1,
                    help="alpha checkpoint interval K of the timed calls (K > 1 runs the grouped pipeline); "
                         "for profiling that path, not the headline line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run one device copy of 512 MiB (a known-size kernel for "
                         "scaling hardware byte counters)")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (utterances would shard across "
              "GPUs with no exchange but a scalar all-reduce for sum/mean; see DESIGN.md). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from ctc_forward_backward_amd import api
    from ctc_forward_backward_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    lib = api._load()
    api.set_pipeline(args.pipeline)

    b = W.make_workload(args.workload)
    T_total, D, B = b.T_total, b.D, b.B
    dname = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}[b.log_probs.dtype]
    lp = b.log_probs.to(dev)
    cu = b.cu_seqlens.to(dev)
    ln = b.lengths.to(dev)
    tg = b.targets.to(dev)
    tl = b.target_lengths.to(dev)
    Umax = int(b.target_lengths.max())
    W_ = int(b.targets.shape[1])
    flags = 1 * (cu.dtype == torch.int64) | 2 * (ln.dtype == torch.int64) | 4 * (tg.dtype == torch.int64) \
        | 8 * (tl.dtype == torch.int64)
    K = args.checkpoint_interval
    ws_bytes = api.packed_ctc_workspace_size(T_total, D, B, Umax, K)
    if ws_bytes == 0:
        print(f"checkpoint interval {K} is not a power of two in [1, 32]", file=sys.stderr)
        sys.exit(2)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    losses = torch.empty(B, dtype=torch.float32, device=dev)
    reduced = torch.empty((), dtype=torch.float32, device=dev)
    grad = torch.empty((T_total, D), dtype=lp.dtype, device=dev)
    red_code = api.REDUCTIONS[b.reduction]
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    call_args = (P(lp), api.DTYPE_CODES[lp.dtype], T_total, D, P(cu), P(ln), B, P(tg), W_, P(tl), flags, Umax,
                 b.blank, int(b.zero_infinity), red_code, None, P(losses), P(reduced), P(grad), K, P(ws), ws_bytes, sh)

    def step():
        rc = lib.packed_ctc_loss(*call_args)
        if rc != 0:
            raise RuntimeError(lib.packed_ctc_last_error().decode())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the timed steps carry no events of the library's own (recording about twenty per call costs
    # tens of microseconds); the per-kernel times come from the same number of steps right after,
    # with HIP events recorded on each group's stream around every kernel
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    api.set_phase_timing(True)
    torch.cuda.synchronize()
    tp0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    tp1 = time.perf_counter()
    phases = api.phase_times()
    api.set_phase_timing(False)

    elapsed = t1 - t0
    ms_per_step = elapsed * 1e3 / args.steps
    frames_per_s = T_total * args.steps / elapsed
    bpe = DTYPE_BYTES[dname]
    bytes_call = T_total * D * (bpe + bpe)
    call_gbps = bytes_call / (ms_per_step * 1e-3) / 1e9

    lengths = b.lengths.numpy().astype(np.int64)
    S = 2 * b.target_lengths.numpy().astype(np.int64) + 1
    state_steps = int((lengths * S).sum())
    # kernels that run once per utterance group ("chains@0" is the group of the longest utterances)
    # are summed over their launches: kernel time per call
    by_kernel = {}
    for name, ms in phases.items():
        base = name.split("@")[0]
        if base != "join":
            by_kernel[base] = by_kernel.get(base, 0.0) + ms
    dominant = max(by_kernel, key=by_kernel.get) if by_kernel else None
    if dominant == "chains":
        t = by_kernel["chains"] * 1e-3
        achieved = 2 * state_steps * OPS_PER_STATE_STEP / t / 1e12
        t_max = int(lengths.max())
        t_crit = phases.get("chains@0", by_kernel["chains"]) * 1e-3
        roofline = {"bound": "alu", "kernel": "chains", "achieved": achieved, "peak": FP32_VECTOR_PEAK_TFLOPS,
                    "peak_note": "fp32 vector, non-packed (the library is built without packed FP32)",
                    "unit": "TFLOP/s", "frac": achieved / FP32_VECTOR_PEAK_TFLOPS,
                    "traffic": profiled_traffic(b.name, "chains"),
                    "work_per_call": f"2 recursions x {state_steps} state-steps x {OPS_PER_STATE_STEP} fp32 ops",
                    "critical_path": {"frames": t_max, "ns_per_frame": t_crit * 1e9 / t_max}}
    elif dominant is not None:
        t = by_kernel[dominant] * 1e-3
        achieved = bytes_call / t / 1e9
        roofline = {"bound": "hbm", "kernel": dominant, "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBPS, "traffic": profiled_traffic(b.name, dominant),
                    "work_per_call": f"{T_total} rows x {D} x ({bpe} B read + {bpe} B written)"}
    else:
        roofline = None
    # the HBM-bound kernel beside it: the gradient rows, counted bytes over their summed launch
    # time per call (a time-weighted average over the group launches, which share the device with
    # the other groups' kernels)
    roofline_rows = None
    if "dense" in by_kernel and by_kernel["dense"] > 0:
        t_rows = by_kernel["dense"] * 1e-3
        a_rows = bytes_call / t_rows / 1e9
        roofline_rows = {"bound": "hbm", "kernel": "dense", "achieved": a_rows, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": a_rows / HBM_PEAK_GBPS, "traffic": profiled_traffic(b.name, "dense"),
                         "work_per_call": f"{T_total} rows x {D} x ({bpe} B read + {bpe} B written)"}

    out = {
        "metric": METRIC,
        "value": frames_per_s,
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": b.name, "B": B, "T_total": T_total, "D": D, "input_dtype": dname,
                   "max_target_length": Umax, "reduction": b.reduction, "zero_infinity": b.zero_infinity,
                   "seed": "fixed", **({"checkpoint_interval": K} if K > 1 else {})},
        "call_hbm": {"achieved": call_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": call_gbps / HBM_PEAK_GBPS,
                     "counted_bytes": bytes_call},
        "phases_ms": phases,
        "ms_per_step_with_phase_events": (tp1 - tp0) * 1e3 / args.steps,
        "kernel_ms_per_call": by_kernel,
        "roofline": roofline,
        "roofline_rows": roofline_rows,
    }

    if not args.profile_run:
        # per-call medians with HIP events around single calls: warm (back to back) and cold (L2 and
        # MALL flushed by writing a 512 MB buffer before each call); and the attainable rate, a 1 GB
        # device-to-device copy
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        nmed = 20
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(2 * nmed)]
        for k, (e0, e1) in enumerate(evs):
            if k >= nmed:
                flush.fill_(k & 0xff)
            e0.record(stream)
            step()
            e1.record(stream)
        torch.cuda.synchronize()
        warm = sorted(e0.elapsed_time(e1) for e0, e1 in evs[:nmed])
        cold = sorted(e0.elapsed_time(e1) for e0, e1 in evs[nmed:])
        del flush
        csrc_ = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cdst_ = torch.empty_like(csrc_)
        cdst_.copy_(csrc_)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(5):
            cdst_.copy_(csrc_)
        c1.record(stream)
        torch.cuda.synchronize()
        copy_gbps = 5 * 2 * (1 << 30) / (c0.elapsed_time(c1) * 1e-3) / 1e9
        del csrc_, cdst_
        out["call_medians_ms"] = {"warm": warm[len(warm) // 2], "cold_l2_mall_flushed": cold[len(cold) // 2],
                                  "calls": nmed, "pipeline": args.pipeline}
        # the other pipeline, same calls (warm median), for context
        other = "grouped" if args.pipeline == "streamed" else "streamed"
        api.set_pipeline(other)
        for _ in range(3):
            step()
        oth = []
        for e0, e1 in evs[:nmed]:
            e0.record(stream)
            step()
            e1.record(stream)
        torch.cuda.synchronize()
        oth = sorted(e0.elapsed_time(e1) for e0, e1 in evs[:nmed])
        api.set_pipeline(args.pipeline)
        step()  # (the gradient left in grad is the timed pipeline's, for the parity check below)
        torch.cuda.synchronize()
        out["call_medians_ms"]["other_pipeline"] = {"pipeline": other, "warm": oth[len(oth) // 2]}
        out["call_hbm"]["device_copy_gbps"] = copy_gbps
        out["call_hbm"]["frac_of_device_copy"] = call_gbps / copy_gbps

        # the second workload of the library: the dense HMM forward at the HMM page's size
        # (S = 16 states, T = 128 frames, B = 64 sequences, O = 64 symbols), HIP events on the stream
        hrng = np.random.default_rng(16)
        hS, hT, hB, hO = 16, 128, 64, 64
        h_in = [torch.from_numpy(hrng.normal(0, 1, size=sh).astype(np.float32)).to(dev) for sh in ((hS,), (hS, hS), (hS, hO))]
        h_obs = torch.from_numpy(hrng.integers(0, hO, size=(hB, hT)).astype(np.int32)).to(dev)
        for _ in range(5):
            api.hmm_forward(*h_in, h_obs)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        hreps = 200
        ev0.record(stream)
        for _ in range(hreps):
            api.hmm_forward(*h_in, h_obs)
        ev1.record(stream)
        torch.cuda.synchronize()
        h_us = ev0.elapsed_time(ev1) * 1e3 / hreps
        out["hmm_forward"] = {"workload": f"S={hS} T={hT} B={hB} O={hO} float32", "us_per_call": h_us,
                              "sequences_per_s": hB / (h_us * 1e-6), "frames_per_s": hB * hT / (h_us * 1e-6),
                              "bound": "latency of T dependent log-semiring matrix-vector steps"}

        out["configs"] = all_configs(api, lib, dev, stream)
        out["extras"] = extras(api, dev, stream)
        crit = out["configs"]["large_vocab"]["critical_path"] if b.name == "large_vocab" else None
        if crit is not None and out["roofline"] is not None and "stream" in by_kernel:
            # the launch's own floor: the longest recursion alone (loss-only call on that utterance)
            out["roofline"]["critical_path"] = dict(crit, launch_us=by_kernel["stream"] * 1e3,
                                                   frac=crit["floor_us"] / (by_kernel["stream"] * 1e3))

    if args.copy_calibration:  # last device work of the run
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    if not args.no_cpu_baseline:
        from oracle import oracle

        gpu_losses = losses.cpu().double().numpy()
        gpu_grad = grad.cpu()
        runs, t_cpu, ref = 0, 0.0, None
        while runs == 0 or t_cpu < args.cpu_seconds:
            c0 = time.perf_counter()
            ref = oracle.ctc_batch(b)
            t_cpu += time.perf_counter() - c0
            runs += 1
        c0 = time.perf_counter()
        oracle.ctc_batch(b, nthreads=1)
        t_one = time.perf_counter() - c0
        cpu_model = ""
        try:
            with open("/proc/cpuinfo") as fh:
                cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
        except OSError:
            pass
        out["cpu_baseline"] = {
            "value": T_total * runs / t_cpu, "unit": "frames/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"the whole {b.name} batch ({T_total} frames, D={D}), loss + gradient in float64, {runs} run(s)",
            "one_thread_value": T_total / t_one, "cpu_model": cpu_model,
            "gbps_over_counted_bytes": bytes_call * runs / t_cpu / 1e9,
        }
        fin = np.isfinite(ref["loss"])
        rel = np.abs(gpu_losses[fin] - ref["loss"][fin]) / np.maximum(np.abs(ref["loss"][fin]), 1e-30)
        gerr = 0.0
        for r0 in range(0, T_total, 4096):
            g = gpu_grad[r0:r0 + 4096].double().numpy()
            rg = ref["grad"][r0:r0 + 4096]
            ok = ~np.isnan(rg)
            if ok.any():
                gerr = max(gerr, float(np.max(np.abs(g[ok] - rg[ok]))))
        out["parity_vs_oracle"] = {"loss_max_rel_err": float(rel.max()) if rel.size else 0.0,
                                   "grad_max_abs_err": gerr}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
