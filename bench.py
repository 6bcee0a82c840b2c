#!/usr/bin/env python3
"""Throughput of the decayed-recurrence hot path on one MI355X.

Default workload (one "step"): retention with a scalar per-head decay,
B=8, H=8, T=2048, Dk=Dv=64, bf16 q/k/v, fp32 state -- one forward and one
reverse la_forward call over the same batch.  Throughput counts B*H*T tokens
per la_forward call.  Inputs are resident in HBM before the timed region;
R rotating copies of every input and output (R * working set >= 512 MB) keep
the 256 MB Infinity Cache from serving repeated steps.

Prints one JSON line with the throughput, a roofline object for the dominant
kernel and the fp64 oracle's CPU throughput on a bounded sample.  The K timed
steps run back to back between one pair of HIP events (no events in between):
that gives ms_per_step and value.  The kernel's own duration for the roofline
is timed separately: the same calls captured into one HIP graph and replayed,
so the launches follow each other on the device with no host in the loop,
between one event pair on the launch stream.

Other workloads (--config normalized_bf16 | step_decay_bf16 | decode_bf16 |
elem_decay_bf16 | bidir_retention_bf16 | backward_retention_bf16 | wkv_f32 | backward_wkv_f32 |
ema_bf16 | bidir_ema_bf16) exist for profiling; the default is the headline
configuration.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "fwd tokens/s (B·H·T) at T=2048,D=64 bf16; % of MFMA / HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFS = 2500.0    # dense bf16
ROTATE_BYTES = 512 << 20
TRAFFIC_FILE = ROOT / "profiles" / "traffic.json"
KERNEL_SOURCES = {
    "la": ["la_fwd_impl.h", "la_fwd_launch.h", "la_bf16_dk64.hip", "la_bf16_dk128.hip", "common.h", "lookback.h"],
    "wkv": ["wkv.hip", "wkv.h", "common.h", "lookback.h"],
    "wkv_bwd": ["wkv_bwd.hip", "wkv.h", "common.h"],
    "ema": ["ema.hip", "ema.h", "common.h", "lookback.h"],
    "la_rec": ["la_rec.hip", "la_rec.h", "common.h"],
    "la_elem": ["la_elem.hip", "la_elem.h", "common.h"],
    "la_bwd": ["la_fwd_impl.h", "la_fwd_launch.h", "la_bf16_dk64.hip", "la_bwd.hip", "common.h", "lookback.h"],
    "la_rbwd": ["la_rec_bwd.hip", "la_rec_bwd.h", "common.h"],
    "la_nbwd": ["la_fwd_impl.h", "la_fwd_launch.h", "la_f32_dk16.hip", "la_f32_dk128.hip", "la_bwd.hip", "common.h",
                "lookback.h"],
    "bidir": ["la_fwd_impl.h", "la_fwd_launch.h", "la_bidir_bf16_dk64.hip", "common.h", "lookback.h"],
    "ema_bidir": ["ema.hip", "ema.h", "combine.hip", "common.h", "lookback.h"],
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="retention_bf16")
    ap.add_argument("--rotate", type=int, default=0, help="buffer copies (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--wkv-path", choices=["auto", "seq", "scan", "chain", "rows"], default="auto",
                    help="pin the WKV path (profiling)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="only run a plain device copy of MB megabytes (counter calibration)")
    return ap.parse_args()


def source_digest(kind):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        h.update((ROOT / "decayed_recurrence_scans_amd" / "csrc" / name).read_bytes())
    return h.hexdigest()


def traffic_for(kind, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when the
    kernel sources changed since the counters were taken."""
    if not TRAFFIC_FILE.exists():
        return None
    data = json.loads(TRAFFIC_FILE.read_text())
    rec = data.get(workload)
    if not rec or rec.get("source_sha256") != source_digest(kind):
        return None
    return rec.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def la_algorithmic_bytes(cfg, with_state_in, esize):
    """Bytes one call must move: q, k, v in, y out, the states, the factors.  A
    bidirectional call reads its inputs once and writes y once (no states)."""
    B, H, T, Dk, Dv = cfg.B, cfg.H, cfg.T, cfg.Dk, cfg.Dv
    if cfg.backward:
        # q, k, v, dy in; dq, dk, dv out; the initial-state gradient and the factor gradient
        n = B * H * T * (2 * Dk + Dv) * esize * 2 + B * H * T * Dv * esize
        n += B * H * Dk * Dv * 4 + ({"head": H * 8, "step": B * H * T * 8,
                                     "elem": B * H * T * Dk * 8}.get(cfg.mode, 0))
        if with_state_in:
            n += B * H * Dk * Dv * 4                                  # the initial state, read
        if cfg.normalize:
            n += B * H * Dk * 4 * 2 + B * H * Dk * Dv * 4 + B * H * Dk * 4   # z0 in, dz0 out; dS_final, dz_final in
        return n
    n = B * H * T * (2 * Dk + Dv) * esize + B * H * T * Dv * esize   # q, k, v in; y out
    if not cfg.bidirectional:
        n += B * H * Dk * Dv * 4 * (2 if with_state_in else 1)       # state out (+ in)
        if cfg.normalize:
            n += B * H * Dk * 4 * (2 if with_state_in else 1)        # key sum out (+ in)
    if cfg.mode == "step":
        n += B * H * T * 4
    elif cfg.mode == "elem":
        n += B * H * T * Dk * 4
    elif cfg.mode == "head":
        n += H * 4
    return n


def la_kernel_name(cfg):
    if cfg.backward and cfg.normalize and cfg.mode != "elem" and cfg.dtype == "bf16" and cfg.T > 16:
        return "la_backward (normalized form as seven fp32 la_fwd_kernel scans, casts, norm_terms)"
    if cfg.backward and (cfg.normalize or cfg.mode == "elem"):
        return "la_backward (step-by-step: la_rbwd_fwd + la_rbwd_rev)"
    if cfg.backward:
        return "la_backward (three la_fwd_kernel gradient scans, decay_terms_cast, decay_grad)"
    if cfg.bidirectional:
        if cfg.mode in ("none", "head") and not cfg.normalize and cfg.Dk <= 64 and cfg.Dv <= 64 and cfg.T > 16:
            return "la_fwd_kernel, fused bidirectional (both scan orders in one pass: la_bidirectional)"
        return "la_bidirectional (la_fwd_kernel forward + reverse, add_bf16)"
    if cfg.T <= 16 or (cfg.mode == "elem" and (cfg.dtype != "bf16" or cfg.normalize)):
        return "la_rec_kernel"
    return "la_elem_kernel (summary + output passes)" if cfg.mode == "elem" else "la_fwd_kernel"


def la_algorithmic_flops(cfg):
    # recurrent form: k v^T update and q^T S read-out, 2*Dk*Dv flops each per token
    return 4 * cfg.B * cfg.H * cfg.T * cfg.Dk * cfg.Dv


def setup_la(cfg, rotate, dev):
    import torch
    from decayed_recurrence_scans_amd import workloads as wl
    inp = wl.la_config_inputs(cfg)
    if cfg.backward:
        inp["dy"], inp["dsf"] = wl.output_gradients(cfg.B, cfg.H, cfg.T, cfg.Dk, cfg.Dv, dtype=cfg.dtype,
                                                    seed=cfg.seed, with_state=cfg.normalize)
        if cfg.normalize:
            inp["dzf"] = torch.randn(cfg.B, cfg.H, cfg.Dk, generator=torch.Generator().manual_seed(cfg.seed + 31))
    esize = 2 if cfg.dtype == "bf16" else 4
    ws = la_algorithmic_bytes(cfg, inp["state_in"] is not None, esize) * len(cfg.reverse)
    R = rotate or max(1, -(-ROTATE_BYTES // ws))
    sets = []
    for r in range(R):
        d = {n: (None if x is None else x.to(dev).clone()) for n, x in inp.items()}
        B, H, T, Dk, Dv = cfg.B, cfg.H, cfg.T, cfg.Dk, cfg.Dv
        d["y"] = [torch.empty((B, H, T, Dv), dtype=d["q"].dtype, device=dev) for _ in cfg.reverse]
        if cfg.backward:
            d["grads"] = [(torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"]))
                          for _ in cfg.reverse]
        if cfg.in_place:   # a decode step: the carried state and key sum are updated where they are
            d["s"] = [d["state_in"] for _ in cfg.reverse]
            d["z"] = [d["cum_k_in"] for _ in cfg.reverse]
        else:
            d["s"] = [torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev) for _ in cfg.reverse]
            d["z"] = [torch.empty((B, H, Dk), dtype=torch.float32, device=dev) if cfg.normalize else None
                      for _ in cfg.reverse]
        sets.append(d)
    return inp, sets, R


def la_grouped(cfg):
    """Forward scans in several directions over the same sequences run as one
    la_forward_group call (one launch of the chunked kernel)."""
    return not cfg.backward and not cfg.bidirectional and len(cfg.reverse) > 1 and la_kernel_name(cfg) == "la_fwd_kernel"


def run_la_step(drs, cfg, d):
    if la_grouped(cfg):
        drs.la_forward_group([dict(q=d["q"], k=d["k"], v=d["v"], decay=d["decay"], mode=cfg.mode,
                                   state_in=d["state_in"], cum_k_in=d["cum_k_in"] if cfg.normalize else None,
                                   reverse=rev, normalize=cfg.normalize, y=d["y"][i], state_out=d["s"][i],
                                   cum_k_out=d["z"][i]) for i, rev in enumerate(cfg.reverse)],
                             chunk=cfg.chunk if cfg.chunk != 64 else 0)
        return
    for i, rev in enumerate(cfg.reverse):
        if cfg.backward:
            dq, dk, dv = d["grads"][i]
            drs.la_backward(d["q"], d["k"], d["v"], d["dy"], d["decay"], cfg.mode, d["state_in"], None,
                            d.get("dsf"), reverse=rev, normalize=cfg.normalize,
                            cum_k_in=d["cum_k_in"] if cfg.normalize else None, dcum_k_out=d.get("dzf"),
                            dq=dq, dk=dk, dv=dv)
        elif cfg.bidirectional:
            drs.la_bidirectional(d["q"], d["k"], d["v"], d["decay"], cfg.mode, normalize=cfg.normalize,
                                 y=d["y"][i])
        else:
            drs.la_forward(d["q"], d["k"], d["v"], d["decay"], cfg.mode, d["state_in"],
                           d["cum_k_in"] if cfg.normalize else None, reverse=rev, normalize=cfg.normalize,
                           chunk=cfg.chunk if cfg.chunk != 64 else 0, y=d["y"][i], state_out=d["s"][i],
                           cum_k_out=d["z"][i])


def setup_wkv(cfg, rotate, dev):
    import torch
    from decayed_recurrence_scans_amd import workloads as wl
    inp = wl.wkv_config_inputs(cfg)
    if cfg.backward:
        g = torch.Generator().manual_seed(cfg.seed + 7919)
        inp["dy"] = torch.randn(cfg.B, cfg.T, cfg.C, generator=g)
    ws = wkv_algorithmic_bytes(cfg)
    R = rotate or max(1, -(-ROTATE_BYTES // ws))
    sets = []
    for r in range(R):
        d = {n: (None if x is None else x.to(dev).clone()) for n, x in inp.items()}
        d["y"] = torch.empty_like(d["k"])
        d["s"] = torch.empty((3, cfg.B, cfg.C), dtype=torch.float32, device=dev)
        if cfg.backward:
            d["dk"] = torch.empty_like(d["k"])
            d["dv"] = torch.empty_like(d["v"])
        sets.append(d)
    return inp, sets, R


def setup_ema(cfg, rotate, dev):
    import torch
    from decayed_recurrence_scans_amd import workloads as wl
    inp = wl.ema_config_inputs(cfg)
    ws = ema_algorithmic_bytes(cfg) * len(cfg.reverse)
    R = rotate or max(1, -(-ROTATE_BYTES // ws))
    sets = []
    for r in range(R):
        d = {n: (None if x is None else x.to(dev).clone()) for n, x in inp.items()}
        d["y"] = [torch.empty_like(d["x"]) for _ in cfg.reverse]
        d["s"] = [torch.empty((cfg.B, cfg.C), dtype=torch.float32, device=dev) for _ in cfg.reverse]
        sets.append(d)
    return inp, sets, R


def ema_algorithmic_bytes(cfg):
    esize = 2 if cfg.dtype == "bf16" else 4
    n = cfg.B * cfg.T * cfg.C * 3 * esize                          # x, f in; y out
    return n if cfg.bidirectional else n + cfg.B * cfg.C * 4      # state out


def run_ema_step(drs, cfg, d):
    for i, rev in enumerate(cfg.reverse):
        if cfg.bidirectional:
            drs.ema_bidirectional(d["x"], d["f"], y=d["y"][i])
        else:
            drs.ema_forward(d["x"], d["f"], d["state_in"], reverse=rev, y=d["y"][i], state_out=d["s"][i])


def wkv_path_name(drs, cfg, flags):
    """Which WKV kernel the library runs for these sizes and flags (from the
    workspace it asks for: none for the sequential kernel)."""
    if flags & drs.DRS_FORCE_SEQ:
        return "seq"
    if flags & drs.DRS_FORCE_SCAN:
        return "scan"
    if flags & drs.DRS_FORCE_CHAIN:
        return "chain"
    if flags & drs.DRS_FORCE_ROWS:
        return "rows"
    if drs.wkv_workspace_bytes(cfg.B, cfg.T, cfg.C, 0) == 0:
        return "seq"
    chain = drs.wkv_workspace_bytes(cfg.B, cfg.T, cfg.C, drs.DRS_FORCE_CHAIN)
    return "chain" if drs.wkv_workspace_bytes(cfg.B, cfg.T, cfg.C, 0) == chain else "scan"


def wkv_algorithmic_bytes(cfg):
    steps = cfg.B * cfg.T * cfg.C
    if cfg.backward:
        return steps * 20 + cfg.C * 16                     # k, v, dy in, dk, dv out; w, u in, dw, du out
    return steps * 12 + cfg.C * 8 + 3 * cfg.B * cfg.C * 4   # k, v in, y out; w, u; state out


def run_wkv_step(drs, cfg, d, force=None):
    if cfg.backward:
        drs.wkv_backward(d["w"], d["u"], d["k"], d["v"], d["dy"], d["state_in"], dk=d["dk"], dv=d["dv"])
        return
    drs.wkv_forward(d["w"], d["u"], d["k"], d["v"], d["state_in"], y=d["y"], state_out=d["s"],
                    force=force, workspace=d.get("ws"))


def events_pair():
    import torch
    return (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))


def kernel_time_us(step, sets, R, launches_per_step, min_launches=32, replays=4):
    """Average duration of one launch of the step's call(s): whole rotations of the
    buffer sets, at least `min_launches` launches, captured into one HIP graph on a
    stream of their own and replayed between one event pair on that stream.  The
    launches then follow each other on the device (the host is not in the loop), so
    the time is the kernels' own.  If capture fails, the same launches run eagerly
    back to back.  Returns (microseconds per launch, how it was timed)."""
    import torch
    n_steps = R * max(1, -(-min_launches // (R * launches_per_step)))
    n_launch = n_steps * launches_per_step
    s = torch.cuda.Stream()   # default priority
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        for i in range(n_steps):          # the library's cached workspace for this stream
            step(sets[i % R])
        s.synchronize()
        how = f"HIP graph of {n_launch} launches, {replays} replays, one event pair on the launch stream"
        try:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for i in range(n_steps):
                    step(sets[i % R])
            g.replay()
            s.synchronize()
            run = g.replay
        except Exception as e:   # pragma: no cover - capture unsupported here
            how = f"eager, {n_launch} launches back to back per repeat ({type(e).__name__} in capture)"
            def run():
                for i in range(n_steps):
                    step(sets[i % R])
        a, b = events_pair()
        a.record()
        for _ in range(replays):
            run()
        b.record()
        b.synchronize()
    torch.cuda.synchronize()
    return 1000.0 * a.elapsed_time(b) / (replays * n_launch), how


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle, unchanged, on a bounded sample
# ---------------------------------------------------------------------------

def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def first_batch_row(kind, cfg, f64):
    """The inputs of batch row 0 only (the per-core sample)."""
    out = {}
    for n, x in f64.items():
        if x is None or n in ("w", "u") or (n == "decay" and cfg.mode == "head"):
            out[n] = x
        elif kind == "wkv" and n == "state_in":
            out[n] = x[:, :1].copy()
        else:
            out[n] = x[:1].copy()
    return out


def cpu_baseline(kind, cfg, inp, seconds):
    """Whole-batch oracle calls (the workload's own shapes) on every core this
    process may use, repeated until the time budget is used; then the oracle on one
    thread over batch row 0 only, for a per-core rate.  Inputs are converted to
    fp64 once, outside the timing."""
    import numpy as np
    import oracle
    threads = oracle.default_threads()
    f64 = {n: (None if x is None else np.ascontiguousarray(x.double().numpy())) for n, x in inp.items()}
    rate, what, el = _oracle_rate(kind, cfg, f64, threads, seconds, cfg.B)
    rate1, what1, el1 = _oracle_rate(kind, cfg, first_batch_row(kind, cfg, f64), 1, max(1.0, seconds / 4), 1)
    return {"value": round(rate, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{what}; fp64 C oracle, OpenMP over independent units; {el:.1f} s wall",
            "cpu_model": cpu_model(),
            "per_core": {"value": round(rate1, 1), "unit": "tokens/s", "threads": 1,
                         "sample": f"{what1}; one thread; {el1:.1f} s wall"}}


def _oracle_rate(kind, cfg, f64, threads, seconds, B):
    import oracle
    calls = 0
    t0 = time.perf_counter()
    while True:
        if kind == "la" and cfg.backward:
            rev = cfg.reverse[calls % len(cfg.reverse)]
            oracle.la_backward(f64["q"], f64["k"], f64["v"], f64["dy"], f64["decay"], cfg.mode, f64["state_in"],
                               f64.get("dsf"), reverse=rev, threads=threads, normalize=cfg.normalize,
                               cum_k_in=f64["cum_k_in"] if cfg.normalize else None, dcum_k_out=f64.get("dzf"))
        elif kind == "la" and cfg.bidirectional:
            oracle.la_bidirectional(f64["q"], f64["k"], f64["v"], f64["decay"], cfg.mode,
                                    normalize=cfg.normalize, threads=threads)
        elif kind == "la":
            rev = cfg.reverse[calls % len(cfg.reverse)]
            oracle.la(f64["q"], f64["k"], f64["v"], f64["decay"], cfg.mode, f64["state_in"],
                      f64["cum_k_in"] if cfg.normalize else None, reverse=rev,
                      normalize=cfg.normalize, threads=threads)
        elif kind == "ema" and cfg.bidirectional:
            oracle.ema_bidirectional(f64["x"], f64["f"], threads=threads)
        elif kind == "ema":
            oracle.ema(f64["x"], f64["f"], f64["state_in"], reverse=cfg.reverse[calls % len(cfg.reverse)],
                       threads=threads)
        elif cfg.backward:
            oracle.wkv_backward(f64["w"], f64["u"], f64["k"], f64["v"], f64["dy"], f64["state_in"], threads=threads)
        else:
            oracle.wkv(f64["w"], f64["u"], f64["k"], f64["v"], f64["state_in"], threads=threads)
        calls += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    if kind == "la":
        tokens = calls * B * cfg.H * cfg.T
        dirs = "bidirectional (forward + reverse summed)" if cfg.bidirectional else \
            f"directions alternating {['fwd', 'rev'][:len(cfg.reverse)]}"
        if cfg.backward:
            dirs = "backward, " + dirs
        what = f"{calls} la calls (B={B} H={cfg.H} T={cfg.T} Dk={cfg.Dk} Dv={cfg.Dv}, {dirs})"
    elif kind == "ema":
        tokens = calls * B * cfg.T
        dirs = "bidirectional" if cfg.bidirectional else "directions alternating"
        what = f"{calls} ema calls (B={B} T={cfg.T} C={cfg.C}, {dirs})"
    else:
        tokens = calls * B * cfg.T
        what = f"{calls} wkv{' backward' if cfg.backward else ''} calls (B={B} T={cfg.T} C={cfg.C})"
    return tokens / el, what, el


# ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the (b,h) and (b,c) units are independent, so more GPUs would each run "
              "this same kernel on their share).", file=sys.stderr)
        sys.exit(2)
    import torch
    import decayed_recurrence_scans_amd as drs
    from decayed_recurrence_scans_amd import workloads as wl

    dev = torch.device("cuda:0")
    drs.load_library()

    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))
        return

    if args.config in wl.LA_CONFIGS:
        kind, cfg = "la", wl.LA_CONFIGS[args.config]
        inp, sets, R = setup_la(cfg, args.rotate, dev)
        step = lambda d: run_la_step(drs, cfg, d)
        launches_per_step = len(cfg.reverse)
        tokens_per_launch = cfg.B * cfg.H * cfg.T
        bytes_per_launch = la_algorithmic_bytes(cfg, inp["state_in"] is not None, 2 if cfg.dtype == "bf16" else 4)
        flops_per_launch = la_algorithmic_flops(cfg) * (2 if cfg.bidirectional else 1)
        if cfg.backward:
            flops_per_launch = la_algorithmic_flops(cfg) * 3 // 2 * 2   # three scans of 2 products each
        kernel = la_kernel_name(cfg)
        if la_grouped(cfg):   # every direction in one launch
            n = len(cfg.reverse)
            launches_per_step, tokens_per_launch = 1, tokens_per_launch * n
            bytes_per_launch, flops_per_launch = bytes_per_launch * n, flops_per_launch * n
            kernel = f"la_fwd_kernel ({n} scans in one launch: la_forward_group)"
        if kernel.startswith(("la_rec_kernel", "la_backward (step-by-step", "la_backward (normalized form")):
            flops_per_launch = None   # vector ALU or fp32 matrix cores, not the bf16 ones
        if cfg.backward:
            kind = ("la_rbwd" if kernel.startswith("la_backward (step-by-step") else
                    "la_nbwd" if kernel.startswith("la_backward (normalized form") else "la_bwd")
        elif cfg.bidirectional:
            kind = "bidir"
        elif kernel == "la_rec_kernel":
            kind = "la_rec"
        elif kernel.startswith("la_elem_kernel"):
            kind = "la_elem"
        workload_cfg = {"workload": f"{cfg.name}: {cfg.description}", "B": cfg.B, "H": cfg.H, "T": cfg.T,
                        "Dk": cfg.Dk, "Dv": cfg.Dv, "decay": cfg.mode, "normalize": cfg.normalize,
                        "scans_per_step": len(cfg.reverse) * (2 if cfg.bidirectional else 1),
                        "directions": (["forward + reverse, summed"] if cfg.bidirectional else
                                       ["reverse" if r else "forward" for r in cfg.reverse])}
        if cfg.in_place:
            workload_cfg["state"] = "carried state and key sum updated in place"
        dtype = cfg.dtype
    elif args.config in wl.WKV_CONFIGS:
        kind, cfg = "wkv", wl.WKV_CONFIGS[args.config]
        inp, sets, R = setup_wkv(cfg, args.rotate, dev)
        force = None if args.wkv_path == "auto" else args.wkv_path
        flags = {None: 0, "seq": drs.DRS_FORCE_SEQ, "scan": drs.DRS_FORCE_SCAN,
                 "chain": drs.DRS_FORCE_CHAIN, "rows": drs.DRS_FORCE_ROWS}[force]
        need = drs.wkv_workspace_bytes(cfg.B, cfg.T, cfg.C, flags)
        for d in sets:   # zero-filled: the look-back counters must start at zero
            d["ws"] = torch.zeros(need, dtype=torch.uint8, device=dev) if need else None
        step = lambda d: run_wkv_step(drs, cfg, d, force)
        launches_per_step = 1
        tokens_per_launch = cfg.B * cfg.T
        bytes_per_launch = wkv_algorithmic_bytes(cfg)
        flops_per_launch = None
        path = wkv_path_name(drs, cfg, flags)
        # the chained path walks the time blocks in one workgroup (wkv_walk_fwd) when there
        # are enough 64-channel units to fill the GPU, else exchanges them (wkv_chain_fwd)
        walk = cfg.B * -(-cfg.C // 64) >= 512
        kernel = {"chain": "wkv_walk_fwd" if walk else "wkv_chain_fwd",
                  "scan": "wkv_seg_summary+wkv_seg_output", "seq": "wkv_seq_fwd", "rows": "wkv_rows_fwd"}[path]
        if cfg.backward:
            kernel, path, kind = "wkv_bwd", "backward", "wkv_bwd"
        workload_cfg = {"workload": f"{cfg.name}: {cfg.description}", "B": cfg.B, "T": cfg.T, "C": cfg.C,
                        "path": {"chain": "chained single-pass time-parallel scan",
                                 "scan": "two-pass time-parallel segment scan", "seq": "sequential",
                                 "rows": "row-owning sweep (spans of 1 KB row pieces, look-back)",
                                 "backward": "backward: forward pass then reverse pass per channel"}[path]}
        dtype = "f32"
    elif args.config in wl.EMA_CONFIGS:
        kind, cfg = "ema", wl.EMA_CONFIGS[args.config]
        inp, sets, R = setup_ema(cfg, args.rotate, dev)
        step = lambda d: run_ema_step(drs, cfg, d)
        launches_per_step = len(cfg.reverse)
        tokens_per_launch = cfg.B * cfg.T
        bytes_per_launch = ema_algorithmic_bytes(cfg)
        flops_per_launch = None
        if cfg.bidirectional:
            fused = cfg.B * -(-cfg.C // 64) >= 512   # enough channels: one fused kernel
            kernel = "ema_bidir (fused)" if fused else "ema_bidirectional (ema_fwd forward + reverse, add_bf16)"
        else:
            kernel = "ema_fwd"
        if cfg.bidirectional:
            kind = "ema_bidir"
        workload_cfg = {"workload": f"{cfg.name}: {cfg.description}", "B": cfg.B, "T": cfg.T, "C": cfg.C,
                        "scans_per_step": len(cfg.reverse) * (2 if cfg.bidirectional else 1),
                        "directions": (["forward + reverse, summed"] if cfg.bidirectional else
                                       ["reverse" if r else "forward" for r in cfg.reverse])}
        dtype = cfg.dtype
    else:
        raise SystemExit(f"unknown config {args.config}")
    workload_cfg["rotating_buffer_sets"] = R

    for i in range(args.warmup):
        step(sets[i % R])
    torch.cuda.synchronize()

    # throughput: K steps back to back between one event pair
    t_start, t_end = events_pair()
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(sets[i % R])
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps

    # the kernel's own duration (separately: graph replays, no host in the loop)
    avg_launch_us, how = kernel_time_us(step, sets, R, launches_per_step)

    tokens_per_step = tokens_per_launch * launches_per_step
    value = tokens_per_step / (ms_per_step / 1000.0)
    achieved_gbs = bytes_per_launch / (avg_launch_us * 1e-6) / 1e9
    step_gbs = bytes_per_launch * launches_per_step / (ms_per_step * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": traffic_for(kind, args.config),
                "kernel": kernel, "avg_launch_us": round(avg_launch_us, 2), "kernel_timing": how,
                "algorithmic_bytes_per_launch": bytes_per_launch,
                "step_achieved": round(step_gbs, 1), "step_frac": round(step_gbs / HBM_PEAK_GBS, 4)}
    if flops_per_launch:
        tfs = flops_per_launch / (avg_launch_us * 1e-6) / 1e12
        roofline["mfma_bf16_algorithmic_tflops"] = round(tfs, 2)
        roofline["mfma_bf16_frac"] = round(tfs / MFMA_BF16_PEAK_TFS, 4)

    out = {"metric": METRIC if args.config == "retention_bf16" else f"tokens/s ({args.config})",
           "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
           "config": workload_cfg, "roofline": roofline}
    if not args.no_cpu_baseline:
        base_kind = {"la_rec": "la", "la_elem": "la", "bidir": "la", "la_bwd": "la", "la_rbwd": "la", "la_nbwd": "la",
                     "ema_bidir": "ema",
                     "wkv_bwd": "wkv"}.get(kind, kind)
        out["cpu_baseline"] = cpu_baseline(base_kind, cfg, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
