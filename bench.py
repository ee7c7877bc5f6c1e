"""Benchmark of the Matryoshka-sliced conv1d + selective-scan hot path on one GPU.

One step = the prefill path of the 1.4B-scale block on one batch of seeded
synthetic input resident in HBM: causal conv1d (kernel 4) + SiLU over the
[x | B | C] stream (b=4, l=8192, 4352 channels, bf16), then the chunked
selective scan on strided views of the conv output (64 heads of 64, d_state
128, chunk 256, full width m=2048).  ``value`` is tokens/s of that step.

Also reported on the same JSON line:
  - ``roofline``: the scan call's algorithmic HBM bytes divided by its own
    duration (HIP events around each scan call inside the timed steps, on the
    stream it runs on), against MI355X's 8 TB/s.  A scan call is two kernels:
    tile_prep_kernel (per-tile C.B^T, B^T and C fragments and head-major dt,
    shared by the heads) and ssd_bf16_kernel (the scan itself);
  - ``fused``: the same step as one fused call (mm_ssd_forward_fused: the conv
    runs inside the scan kernels, its output never reaches HBM), with its own
    HBM fraction and measured traffic;
  - ``slices``: the scan call's tokens/s, HBM and MFMA fractions at every
    Matryoshka width: 5 warmup calls, then 50 calls timed one by one with HIP
    events, each after a 512 MiB write that evicts the caches; median, p10,
    p90; ``fused_slices``: the same for the fused call;
  - ``configs``: the same for the 130M-scale and long-context workloads;
  - ``mixed``: the scan with a width per sequence (mm_ssd_forward_mixed),
    widths round-robin {512, 1024, 2048} over the 4 sequences, against the
    same batch run at the widest width;
  - ``gated_rmsnorm``: the gated RMSNorm epilogue (y * SiLU(z), RMSNorm over
    d_i) on the 1.4B-scale rows at every width, timed as the slices are;
  - ``backward``: the scan's backward pass (mm_ssd_backward: dx, ddt, dA,
    dB, dC, dD from the cotangent of y) on the same inputs at every width,
    and the conv's backward (mm_conv1d_silu_backward) at full width, timed as
    the slices are, with their HBM fractions;
  - ``decode``: the recurrent decode step (conv state roll + scan step) for a
    batch of 256 sequences at mixed widths, 1024 tokens captured in a HIP graph;
    ``decode.fused_vs_two_launches``: microseconds per token of those two
    launches against the one-launch mm_ssd_step_fused at batch 1, 16, 64, 256;
  - ``cpu_baseline``: the fp64 oracle on the host cores over a bounded sample
    of the same workload, scaled to the step.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_FILES = {"scan": os.path.join(ROOT, "profiles", "traffic_ssd_scan_1p4b_m2048.json"),
                 "fused": os.path.join(ROOT, "profiles", "traffic_fused_prefill_1p4b_m2048.json")}


def traffic_file(which: str, workload: str = "1.4b", m: int = 0) -> str:
    """Record of the measured HBM bytes of one scan (or fused) call of a
    workload at width m (0 = the 1.4B full-width records above)."""
    if not m or (workload == "1.4b" and m == 2048):
        return TRAFFIC_FILES[which]
    return os.path.join(ROOT, "profiles", f"traffic_ssd_scan_{workload.replace('.', 'p')}_m{m}.json")
SCAN_SRCS = [os.path.join(ROOT, "selective_state_space_12_amd", "csrc", f)
             for f in ("ssd_fwd_bf16.hip", "device_common.h")]
# the kernels of one call: tile prep, and with the sequences split the
# state-only pass and the combine, then the scan (absent ones are skipped)
SCAN_KERNELS = ("tile_prep_kernel", "ssd_bf16_seg_kernel", "ssd_bf16_seg2_kernel", "seg_combine_bf16_kernel",
                "ssd_bf16_kernel")


COPY_BYTES = 1 << 30


def _pmc_per_dispatch(dirname: str, counter: str, kernel_substr: str, min_grid: int = 0):
    """Mean value (KiB) of a counter over the dispatches of one kernel, from a
    rocprofv3 --output-format csv counter_collection file."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(dirname, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            if row.get("Counter_Name") != counter or kernel_substr not in row.get("Kernel_Name", ""):
                continue
            if int(row.get("Grid_Size", 0)) < min_grid:
                continue
            key = (f, row.get("Dispatch_Id"))
            vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} rows for kernel '{kernel_substr}' under {dirname}")
    return sum(vals.values()) / len(vals), len(vals)


def summarize_pmc(which, scan_fetch, scan_write, copy_fetch, copy_write, workload="1.4b", heads=0):
    """HBM bytes per scan call or fused prefill call (``which``: counter runs
    of ``--mode scan`` / ``--mode fused``, with ``--workload`` / ``--heads``):
    FETCH_SIZE + WRITE_SIZE of its kernels (mean per dispatch of each,
    summed), each counter scaled by what it reads for a copy of known size."""
    import synth
    w = synth.WORKLOADS[workload]
    h = heads or w.n_heads
    m = next(mm for mm in w.slices if w.heads(mm) == h)
    sf = sw = 0.0
    nsf, nsw, per = [], [], {}
    for kname in SCAN_KERNELS:
        try:
            f1, n1 = _pmc_per_dispatch(scan_fetch, "FETCH_SIZE", kname)
            w1, n2 = _pmc_per_dispatch(scan_write, "WRITE_SIZE", kname)
        except SystemExit:
            continue
        sf += f1
        sw += w1
        nsf.append(n1)
        nsw.append(n2)
        per[kname] = {"fetch_kib": f1, "write_kib": w1}
    # the calibration copy is the only large copy dispatch of its run
    cf, _ = _pmc_per_dispatch(copy_fetch, "FETCH_SIZE", "copyBuffer", min_grid=1 << 16)
    cw, _ = _pmc_per_dispatch(copy_write, "WRITE_SIZE", "copyBuffer", min_grid=1 << 16)
    kf = COPY_BYTES / (cf * 1024.0)
    kw = COPY_BYTES / (cw * 1024.0)
    total = sf * 1024.0 * kf + sw * 1024.0 * kw
    alg = scan_bytes(w.batch * w.seqlen, h, w.d_head, w.d_state, 2)
    for v in per.values():
        v["hbm_bytes"] = v["fetch_kib"] * 1024.0 * kf + v["write_kib"] * 1024.0 * kw
    rec = {"kernel": ("fused prefill call (conv + scan" if which == "fused" else "scan call (scan") +
                     ", bf16, d_head 64, d_state 128, 128-token tiles): " + " + ".join(per),
           "workload": f"{workload} prefill, b={w.batch} l={w.seqlen}, {h} of {w.n_heads} heads "
                       f"(m={m}), chunk {w.chunk}, inputs as in bench.py",
           "kernel_source_sha256_16": src_hash(),
           "fetch_kib_per_dispatch": sf, "write_kib_per_dispatch": sw,
           "per_kernel": per,
           "copy_calibration": {"bytes": COPY_BYTES, "fetch_kib": cf, "write_kib": cw,
                                "fetch_scale": kf, "write_scale": kw},
           "hbm_bytes_per_launch": total, "alg_bytes_per_launch": alg,
           "traffic_over_alg": total / alg, "dispatches": [nsf, nsw]}
    path = traffic_file(which, workload, m)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    json.dump(rec, open(path, "w"), indent=1)
    print(json.dumps(rec))


def scan_bytes(tokens: int, heads: int, P: int, N: int, elem: int) -> int:
    """Algorithmic HBM bytes of one scan call: x and y of the active heads,
    B and C, and dt of the active heads (A, D negligible)."""
    return tokens * (2 * heads * P * elem + 2 * N * elem + heads * elem)


def bwd_bytes(tokens: int, heads: int, P: int, N: int, elem: int) -> int:
    """Algorithmic HBM bytes of one scan backward call: x, dy read and dx
    written for the active heads, dt read and ddt written, B and C read, the
    fp32 dB and dC written (A, D, dA, dD negligible)."""
    return tokens * (3 * heads * P * elem + 2 * heads * elem + 2 * N * elem + 2 * N * 4)


def scan_flops(tokens: int, heads: int, P: int, N: int, Q: int) -> int:
    """Algorithmic flops of one scan call, causal-counted chunked form at chunk
    Q with one B/C group: (Q+1) N for the shared C.B^T blocks, and per head
    (Q+1) P for the masked product with x plus 4 P N for the chunk state and
    the inter-chunk output term."""
    return tokens * ((Q + 1) * N + heads * ((Q + 1) * P + 4 * P * N))


MFMA_PEAK_TFLOPS = 2500.0  # dense bf16
FLUSH_BYTES = 512 << 20


def timed_calls(torch, fn, flush, iters: int = 50, warmup: int = 5):
    """Per-call HIP-event timing: ``warmup`` untimed calls, then ``iters``
    calls each preceded by a write of ``flush`` (512 MiB, larger than the L2s
    and the 256 MB Infinity Cache together) so that every call starts cold.
    Returns the median, p10 and p90 in ms."""
    for _ in range(warmup):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    torch.cuda.synchronize()
    for i in range(iters):
        flush.fill_(i & 0x7F)
        ev[i][0].record()
        fn()
        ev[i][1].record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(z) for a, z in ev)
    q = lambda f: t[min(len(t) - 1, int(round(f * (len(t) - 1))))]
    return {"median": q(0.5), "p10": q(0.1), "p90": q(0.9)}


def scan_entry(tokens, h, P, N, Q, t, elem=2, traffic=None):
    """JSON fields of one scan timing ``t`` (median/p10/p90 in ms); ``traffic``:
    the measured HBM bytes of the call (rocprofv3 record), if any."""
    ms = t["median"]
    ab = scan_bytes(tokens, h, P, N, elem)
    fl = scan_flops(tokens, h, P, N, Q)
    e = {"heads": h, "scan_ms": ms, "scan_ms_p10": t["p10"], "scan_ms_p90": t["p90"],
         "tokens_per_s": tokens / (ms * 1e-3), "alg_bytes": ab,
         "hbm_frac": ab / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
         "mfma_frac": fl / (ms * 1e-3) / (MFMA_PEAK_TFLOPS * 1e12)}
    if traffic:
        e["traffic"] = traffic
        e["traffic_over_alg"] = traffic / ab
    return e


def conv_bytes(tokens: int, channels: int, elem: int) -> int:
    return tokens * channels * elem * 2


def decode_bytes(heads_per_seq, P: int, N: int, d_inner: int) -> int:
    """Per decode step: fp32 state read+write of active heads, conv state
    read+write and xbc input of active channels, dt and y (fp32)."""
    tot = 0
    for h in heads_per_seq:
        ch = h * P + 2 * N
        tot += h * P * N * 4 * 2 + ch * 3 * 4 * 2 + ch * 4 * 2 + h * 4 + h * P * 4
    return tot


def src_hash() -> str:
    """Hash of the scan kernel sources with comments and blank space removed,
    so a record of measured traffic stays valid across comment-only edits."""
    import re
    text = "".join(open(f).read() for f in SCAN_SRCS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"\s+", " ", text)
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def load_traffic(which, workload="1.4b", m=0):
    """HBM bytes per scan / fused call measured with rocprofv3 (FETCH_SIZE and
    WRITE_SIZE, calibrated on a copy kernel), if taken on this kernel source."""
    try:
        d = json.load(open(traffic_file(which, workload, m)))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256_16") != src_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-slices", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the scan-only timings of the 130M and long-context workloads")
    ap.add_argument("--mode", choices=["step", "fused", "scan", "backward", "conv_backward", "copy"],
                    default="step",
                    help="fused / scan / backward / conv_backward: only the full-width fused "
                         "call / scan call / scan backward / conv backward (for counter and "
                         "trace runs); copy: a 1 GiB device copy that calibrates the HBM "
                         "byte counters")
    ap.add_argument("--workload", choices=["1.4b", "long", "130m", "tiny"], default="1.4b",
                    help="with --mode scan: the workload whose scan call is repeated")
    ap.add_argument("--heads", type=int, default=0,
                    help="with --mode scan or backward: active heads (default: all)")
    ap.add_argument("--summarize-pmc", nargs=5,
                    metavar=("WHICH", "FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="WHICH = scan or fused, then rocprofv3 --pmc output dirs (csv); writes "
                         "the traffic record under profiles/")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, workload=args.workload, heads=args.heads)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the scan shards by batch and head with no exchange; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch
    import selective_state_space_12_amd as mm
    import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.mode == "scan":
        scan_only(torch, mm, synth, dev, synth.WORKLOADS[args.workload], args)
        return
    w = synth.WORKLOADS["1.4b"]
    b, l, H, P, N = w.batch, w.seqlen, w.n_heads, w.d_head, w.d_state
    tokens = b * l
    elem = 2
    print(f"# generating inputs for {w.name}: b={b} l={l} conv_dim={w.conv_dim}", file=sys.stderr, flush=True)
    xi = synth.xbc_inputs(w)
    xbc_raw = xi["xbc"].to(dev)
    conv_w = xi["w"].to(dev)
    dt = synth.pipeline_dt(w).to(dev)
    A = synth.draw_A(w).to(dev)
    D = synth.draw_D(w).to(dev)
    del xi
    xbc = torch.empty_like(xbc_raw)
    y = torch.empty((b, l, H, P), dtype=w.dtype, device=dev)
    xv = xbc[..., :w.d_inner].view(b, l, H, P)
    Bv = xbc[..., w.d_inner:w.d_inner + N].unsqueeze(2)
    Cv = xbc[..., w.d_inner + N:].unsqueeze(2)
    ws_bytes = mm.ssd_forward_workspace_size(b, l, H, P, N, 1, H, w.chunk, w.dtype)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    wsf_bytes = mm.ssd_forward_fused_workspace_size(b, l, H, P, N, 1, H, w.chunk, w.dtype)
    wsf = torch.empty(max(wsf_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def fused(heads):
        # dt is the workload's step size as given (after softplus), so no
        # bias and no softplus here
        mm.ssd_forward_fused(xbc_raw, conv_w, dt, A, D, d_head=P, d_state=N,
                             n_heads_active=heads, chunk=w.chunk, y=y, workspace=wsf)

    def scan(heads):
        mm.ssd_forward(xv, dt, A, Bv, Cv, D, n_heads_active=heads, chunk=w.chunk, y=y,
                       workspace=ws)

    def conv(heads):
        mm.conv1d_silu(xbc_raw, conv_w, None, None, d_inner=w.d_inner, d_head=P,
                       d_state=N, n_heads_active=heads, out=xbc)

    if args.mode == "fused":  # counter runs: the full-width fused call alone
        for _ in range(args.warmup + args.steps):
            fused(H)
        torch.cuda.synchronize()
        print(f"# fused-only: {args.warmup + args.steps} launches", file=sys.stderr)
        return
    if args.mode == "backward":  # counter runs: the scan backward alone (full width by default)
        conv(H)
        hb = args.heads or H
        dy = synth.cotangents(w)["dy"].to(dev)
        g = {"dx": torch.empty((b, l, H, P), dtype=w.dtype, device=dev),
             "ddt": torch.empty((b, l, H), dtype=w.dtype, device=dev)}
        bws = torch.empty(mm.ssd_backward_workspace_size(b, l, H, P, N, 1, hb, w.dtype),
                          dtype=torch.uint8, device=dev)
        for _ in range(args.warmup + args.steps):
            g = mm.ssd_backward(xv, dt, A, Bv, Cv, D, dy, n_heads_active=hb, grads=g, workspace=bws)
        torch.cuda.synchronize()
        print(f"# backward-only: {args.warmup + args.steps} launches", file=sys.stderr)
        return
    if args.mode == "conv_backward":  # trace runs: the full-width conv backward alone
        dout = synth.conv_cotangent(w).to(dev)
        cg = {"dxbc": torch.empty_like(xbc_raw), "dw": torch.empty((w.conv_dim, 4), device=dev)}
        for _ in range(args.warmup + args.steps):
            mm.conv1d_silu_backward(xbc_raw, conv_w, dout, d_inner=w.d_inner, d_head=P, d_state=N,
                                    grads=cg)
        torch.cuda.synchronize()
        print(f"# conv-backward-only: {args.warmup + args.steps} launches", file=sys.stderr)
        return
    if args.mode == "copy":  # counter calibration: a plain copy of known size
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"# copy: {args.warmup + args.steps} x {COPY_BYTES} bytes", file=sys.stderr)
        return

    def timed_steps(step, inner=None):
        """W warmup steps, then K steps back to back between two events;
        with ``inner``, HIP events also bracket that part of each step."""
        for _ in range(args.warmup):
            step(inner)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(args.steps):
            step(ev[i])
        t1.record(stream)
        torch.cuda.synchronize()
        part = [a.elapsed_time(z) for a, z in ev]
        return t0.elapsed_time(t1) / args.steps, sum(part) / len(part)

    def fused_step(evs):
        if evs:
            evs[0].record(stream)
        fused(H)
        if evs:
            evs[1].record(stream)

    def two_call_step(evs):
        conv(H)
        if evs:
            evs[0].record(stream)
        scan(H)
        if evs:
            evs[1].record(stream)

    # ---- the step: conv + scan at full width ------------------------------------
    ms_step, scan_avg_ms = timed_steps(two_call_step)
    value = tokens / (ms_step * 1e-3)
    # ---- the same step as one fused call ------------------------------------------
    ms_fused, fused_avg_ms = timed_steps(fused_step)

    alg = scan_bytes(tokens, H, P, N, elem)
    achieved = alg / (scan_avg_ms * 1e-3) / 1e9
    traffic = load_traffic("scan")

    out = {
        "metric": "SSD scan tokens/s per Matryoshka slice; % of MI355X MFMA/HBM roofline",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) xBC stream, log-uniform dt in [1e-3, 1e-1]; no dataset)",
        "config": {"workload": "1.4B-scale MatMamba block prefill: conv1d(k=4)+SiLU then chunked "
                               "selective scan, b=4 l=8192 d_model=2048 d_inner=4096 64 heads x 64, "
                               "d_state=128, chunk=256 (evaluated as two 128-token tiles), "
                               "slice m=2048 (64 heads)",
                   "global_batch": b, "seq_len": l, "parallelism": "single GPU"},
        "roofline": {"kernel": "scan call (tile_prep_kernel + ssd_bf16_kernel)", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "alg_bytes_per_launch": alg, "avg_launch_ms": scan_avg_ms},
        "fused": {"ms_per_step": ms_fused, "tokens_per_s": tokens / (ms_fused * 1e-3),
                  "call_ms": fused_avg_ms,
                  "hbm_frac": alg / (fused_avg_ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
                  "traffic": load_traffic("fused")},
    }

    # ---- every Matryoshka width, scan only -----------------------------------
    flush = None
    if not (args.no_slices and args.no_configs and args.no_backward):
        flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    if not args.no_slices:
        slices, fused_slices = {}, {}
        conv(H)
        for m in w.slices:
            h = w.heads(m)
            slices[str(m)] = scan_entry(tokens, h, P, N, w.chunk,
                                        timed_calls(torch, lambda: scan(h), flush),
                                        traffic=load_traffic("scan", "1.4b", m))
            fused_slices[str(m)] = scan_entry(tokens, h, P, N, w.chunk,
                                              timed_calls(torch, lambda: fused(h), flush))
        # conv alone at full width, and a plain device copy of the same bytes
        # (the practical ceiling for that read + write traffic)
        tcv = timed_calls(torch, lambda: conv(H), flush)
        cpy = torch.empty_like(xbc_raw)
        tcp = timed_calls(torch, lambda: cpy.copy_(xbc_raw), flush)
        del cpy
        tc, tcopy = tcv["median"], tcp["median"]
        cb = conv_bytes(tokens, w.conv_dim, elem)
        out["slices"] = slices
        out["fused_slices"] = fused_slices
        out["conv"] = {"ms": tc, "ms_p10": tcv["p10"], "ms_p90": tcv["p90"],
                       "tokens_per_s": tokens / (tc * 1e-3), "gb_per_s": cb / (tc * 1e-3) / 1e9,
                       "hbm_frac": cb / (tc * 1e-3) / (HBM_PEAK_GBS * 1e9),
                       "copy_same_bytes_ms": tcopy, "vs_copy": tcopy / tc}

    # ---- a width per sequence: widths round-robin {512, 1024, 2048} ----------------
    if not args.no_slices:
        hps = [w.heads(w.slices[1 + (i % 3)]) for i in range(b)]
        wsm = torch.empty(max(mm.ssd_forward_mixed_workspace_size(b, l, H, P, N, 1, hps, w.chunk,
                                                                  w.dtype), 1),
                          dtype=torch.uint8, device=dev)
        tmix = timed_calls(torch, lambda: mm.ssd_forward_mixed(
            xv, dt, A, Bv, Cv, D, heads_per_seq=hps, chunk=w.chunk, y=y, workspace=wsm), flush)
        tmax = timed_calls(torch, lambda: scan(max(hps)), flush)
        mb = sum(scan_bytes(l, h, P, N, elem) for h in hps)
        out["mixed"] = {"heads_per_seq": hps, "scan_ms": tmix["median"],
                        "scan_ms_p10": tmix["p10"], "scan_ms_p90": tmix["p90"],
                        "tokens_per_s": tokens / (tmix["median"] * 1e-3),
                        "hbm_frac": mb / (tmix["median"] * 1e-3) / (HBM_PEAK_GBS * 1e9),
                        "widest_for_all_ms": tmax["median"]}
        del wsm

    # ---- gated RMSNorm epilogue on the same rows, every width -------------------
    if not args.no_slices:
        gi = synth.gate_inputs(w)
        gy, gz, gw = gi["y"].to(dev), gi["z"].to(dev), gi["w"].to(dev)
        del gi
        gout = torch.empty_like(gy)
        norm = {}
        for m in w.slices:
            d_i = w.heads(m) * P
            t = timed_calls(torch, lambda: mm.gated_rmsnorm(gy, gz, gw, 1e-5, d=d_i, out=gout[..., :d_i]),
                            flush)
            nb = 3 * tokens * d_i * elem
            norm[str(m)] = {"d": d_i, "ms": t["median"], "ms_p10": t["p10"], "ms_p90": t["p90"],
                            "gb_per_s": nb / (t["median"] * 1e-3) / 1e9,
                            "hbm_frac": nb / (t["median"] * 1e-3) / (HBM_PEAK_GBS * 1e9)}
        out["gated_rmsnorm"] = norm
        del gy, gz, gw, gout

    # ---- scan backward on the same inputs, every width ------------------------
    if not args.no_backward:
        out["backward"] = bench_backward(torch, mm, synth, w, dev, flush, xv, dt, A, Bv, Cv, D)

    # ---- the other bf16 workloads, scan only, every slice ----------------------
    if not args.no_configs:
        del xbc_raw, xbc, xv, Bv, Cv, y, ws, wsf
        torch.cuda.empty_cache()
        out["configs"] = bench_configs(torch, mm, synth, dev, flush)

    # ---- decode: conv state roll + scan step, 1024 tokens in a HIP graph -----
    if not args.no_decode:
        out["decode"] = bench_decode(torch, mm, synth, dev)

    # ---- CPU baseline: the oracle on a bounded sample --------------------------
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w)

    print(json.dumps(out), flush=True)


def scan_only(torch, mm, synth, dev, w, args):
    """Trace and counter runs: the scan call of one workload at one width,
    repeated, on inputs as in the timings: the 1.4B scan reads strided views
    of the conv output (as in the step), the others dense seeded tensors."""
    h = args.heads or w.n_heads
    b, l = w.batch, w.seqlen
    if w.name == "1.4b":
        P, N = w.d_head, w.d_state
        xi = synth.xbc_inputs(w)
        raw, cw = xi["xbc"].to(dev), xi["w"].to(dev)
        del xi
        xbc = torch.empty_like(raw)
        mm.conv1d_silu(raw, cw, None, None, d_inner=w.d_inner, d_head=P, d_state=N,
                       n_heads_active=w.n_heads, out=xbc)
        del raw
        d = {"x": xbc[..., :w.d_inner].view(b, l, w.n_heads, P),
             "B": xbc[..., w.d_inner:w.d_inner + N].unsqueeze(2),
             "C": xbc[..., w.d_inner + N:].unsqueeze(2),
             "dt": synth.pipeline_dt(w).to(dev), "A": synth.draw_A(w).to(dev),
             "D": synth.draw_D(w).to(dev)}
    else:
        inp = synth.forward_inputs(w)
        d = {k: v.to(dev) for k, v in inp.items()}
    y = torch.empty((b, l, w.n_heads, w.d_head), dtype=w.dtype, device=dev)
    ws = torch.empty(max(mm.ssd_forward_workspace_size(b, l, w.n_heads, w.d_head, w.d_state, 1,
                                                       h, w.chunk, w.dtype), 1),
                     dtype=torch.uint8, device=dev)
    for _ in range(args.warmup + args.steps):
        mm.ssd_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], n_heads_active=h,
                       chunk=w.chunk, y=y, workspace=ws)
    torch.cuda.synchronize()
    print(f"# scan-only {w.name} heads={h}: {args.warmup + args.steps} launches", file=sys.stderr)


def bench_backward(torch, mm, synth, w, dev, flush, xv, dt, A, Bv, Cv, D, slices=None):
    """mm_ssd_backward at every width of the 1.4B-scale workload (dy from the
    seeded cotangents, no final-state cotangent, gradients overwritten)."""
    b, l, H, P, N = w.batch, w.seqlen, w.n_heads, w.d_head, w.d_state
    tokens = b * l
    dy = synth.cotangents(w)["dy"].to(dev)
    g = {"dx": torch.empty((b, l, H, P), dtype=w.dtype, device=dev),
         "ddt": torch.empty((b, l, H), dtype=w.dtype, device=dev),
         "dA": torch.empty(H, device=dev), "dD": torch.empty(H, device=dev),
         "dB": torch.empty((b, l, 1, N), device=dev), "dC": torch.empty((b, l, 1, N), device=dev)}
    ws = torch.empty(mm.ssd_backward_workspace_size(b, l, H, P, N, 1, H, w.dtype),
                     dtype=torch.uint8, device=dev)
    res = {}
    for m in (slices or w.slices):
        h = w.heads(m)
        t = timed_calls(torch, lambda: mm.ssd_backward(xv, dt, A, Bv, Cv, D, dy, n_heads_active=h,
                                                        grads=g, workspace=ws), flush)
        ab = bwd_bytes(tokens, h, P, N, 2)
        res[str(m)] = {"heads": h, "ms": t["median"], "ms_p10": t["p10"], "ms_p90": t["p90"],
                       "tokens_per_s": tokens / (t["median"] * 1e-3),
                       "hbm_frac": ab / (t["median"] * 1e-3) / (HBM_PEAK_GBS * 1e9)}
    del dy, g, ws
    # the conv's backward on the 1.4B-scale rows at full width
    xi = synth.xbc_inputs(w)
    xbc, cw = xi["xbc"].to(dev), xi["w"].to(dev)
    del xi
    dout = synth.conv_cotangent(w).to(dev)
    cg = {"dxbc": torch.empty_like(xbc), "dw": torch.empty((w.conv_dim, 4), device=dev)}
    t = timed_calls(torch, lambda: mm.conv1d_silu_backward(
        xbc, cw, dout, d_inner=w.d_inner, d_head=P, d_state=N, grads=cg), flush)
    cb = 3 * tokens * w.conv_dim * 2
    res["conv"] = {"ms": t["median"], "ms_p10": t["p10"], "ms_p90": t["p90"],
                   "tokens_per_s": tokens / (t["median"] * 1e-3),
                   "gb_per_s": cb / (t["median"] * 1e-3) / 1e9,
                   "hbm_frac": cb / (t["median"] * 1e-3) / (HBM_PEAK_GBS * 1e9)}
    del xbc, cw, dout, cg
    return res


def bench_configs(torch, mm, synth, dev, flush):
    """Scan-only tokens/s, HBM and MFMA fractions at every slice of the tiny
    fp32 (b=1, l=256, 4 heads of 32, d_state 16, chunk 64), 130M-scale (b=8,
    l=2048, 24 heads) and long-context (b=1, l=131072, 32 heads) workloads:
    dense seeded inputs (x, dt, B, C as separate tensors), no initial state,
    timed as the 1.4B slices are (``timed_calls``)."""
    res = {}
    for name in ("tiny", "130m", "long"):
        w = synth.WORKLOADS[name]
        print(f"# generating inputs for {name}: b={w.batch} l={w.seqlen}", file=sys.stderr, flush=True)
        inp = synth.forward_inputs(w)
        d = {k: v.to(dev) for k, v in inp.items()}
        del inp
        y = torch.empty_like(d["x"])
        tokens = w.batch * w.seqlen
        per = {}
        for m in w.slices:
            h = w.heads(m)
            need = mm.ssd_forward_workspace_size(w.batch, w.seqlen, w.n_heads, w.d_head, w.d_state,
                                                 1, h, w.chunk, w.dtype)
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

            def call():
                mm.ssd_forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], n_heads_active=h,
                               chunk=w.chunk, y=y, workspace=ws)
            per[str(m)] = scan_entry(tokens, h, w.d_head, w.d_state, w.chunk,
                                     timed_calls(torch, call, flush),
                                     elem=torch.finfo(w.dtype).bits // 8,
                                     traffic=load_traffic("scan", name, m))
            del ws
        res[name] = {"batch": w.batch, "seq_len": w.seqlen, "n_heads": w.n_heads,
                     "dtype": str(w.dtype).replace("torch.", ""), "slices": per}
        del d, y
        torch.cuda.empty_cache()
    return res


def decode_batch_sweep(torch, mm, synth, dev, batches=(1, 16, 64, 256)):
    """Decode step of the decode workload's model (mixed widths) at several
    batch sizes: the conv step and mm_ssd_step as two launches per token
    against mm_ssd_step_fused (one launch, two conv-state buffers in turn),
    each in HIP graphs of 64 tokens, best of two timings of 16 replays;
    microseconds per token."""
    d = synth.WORKLOADS["decode"]
    H, P, N, cd = d.n_heads, d.d_head, d.d_state, d.conv_dim
    out = {}
    for bsz in batches:
        pool = synth.decode_pool(d, pool=64, batch=bsz)
        xbc_t, dt_t = pool["xbc_t"].to(dev), pool["dt_t"].to(dev)
        hv = synth.decode_heads(d, batch=bsz).to(dev)
        A, D, cw = synth.draw_A(d).to(dev), synth.draw_D(d).to(dev), synth.draw_conv_w(d).to(dev)
        state = torch.zeros((bsz, H, P, N), device=dev)
        csb = (torch.zeros((bsz, 3, cd), device=dev), torch.zeros((bsz, 3, cd), device=dev))
        u = torch.empty((bsz, 1, cd), device=dev)
        yt = torch.empty((bsz, H, P), device=dev)

        def two(k):
            mm.conv1d_silu(xbc_t[k].unsqueeze(1), cw, None, csb[0], d_inner=d.d_inner, d_head=P,
                           d_state=N, n_heads_active=H, heads_per_seq=hv, out=u)
            u2 = u[:, 0]
            mm.ssd_step(state, u2[:, :d.d_inner].view(bsz, H, P), dt_t[k], A,
                        u2[:, d.d_inner:d.d_inner + N], u2[:, d.d_inner + N:], D,
                        n_heads_active=H, heads_per_seq=hv, y=yt)

        def fused(k):
            mm.ssd_step_fused(state, csb[k % 2], csb[(k + 1) % 2], xbc_t[k], cw, dt_t[k], A, D,
                              n_heads_active=H, heads_per_seq=hv, y=yt)

        best = {}
        for name, fn in (("two_launches_us", two), ("fused_us", fused)) * 2:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                for k in range(4):
                    fn(k)
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for k in range(64):
                    fn(k)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(16):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            best[name] = min(best.get(name, 1e30), e0.elapsed_time(e1) * 1e3 / (16 * 64))
            del g
        out[str(bsz)] = best
    return out


def bench_decode(torch, mm, synth, dev):
    d = synth.WORKLOADS["decode"]
    bsz, H, P, N, cd = d.batch, d.n_heads, d.d_head, d.d_state, d.conv_dim
    pool = synth.decode_pool(d, pool=64)
    xbc_t = pool["xbc_t"].to(dev)          # (64, b, cd) fp32
    dt_t = pool["dt_t"].to(dev)            # (64, b, H)
    hv_cpu = synth.decode_heads(d)
    hv = hv_cpu.to(dev)
    A = synth.draw_A(d).to(dev)
    D = synth.draw_D(d).to(dev)
    cw = synth.draw_conv_w(d).to(dev)
    state = torch.zeros((bsz, H, P, N), device=dev)
    cstate = torch.zeros((bsz, 3, cd), device=dev)
    u = torch.empty((bsz, 1, cd), device=dev)
    yt = torch.empty((bsz, H, P), device=dev)

    def one(k):
        mm.conv1d_silu(xbc_t[k].unsqueeze(1), cw, None, cstate, d_inner=d.d_inner, d_head=P,
                       d_state=N, n_heads_active=H, heads_per_seq=hv, out=u)
        u2 = u[:, 0]
        mm.ssd_step(state, u2[:, :d.d_inner].view(bsz, H, P), dt_t[k], A,
                    u2[:, d.d_inner:d.d_inner + N], u2[:, d.d_inner + N:], D,
                    n_heads_active=H, heads_per_seq=hv, y=yt)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for k in range(4):
            one(k)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(64):
            one(k)
    g.replay()
    torch.cuda.synchronize()
    reps = d.steps // 64
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    steps = reps * 64
    per_step_us = ms * 1e3 / steps
    by = decode_bytes(hv_cpu.tolist(), P, N, d.d_inner)
    sweep = decode_batch_sweep(torch, mm, synth, dev)
    # speculative decoding at full width (64 heads, every sequence): verify 4
    # draft tokens in one pass over the states (conv of the 4 tokens on a copy
    # of the conv state, then mm_ssd_step_multi with no state write), commit
    # each sequence's accepted prefix (mm_ssd_step_multi in place with the
    # accepted counts, mm_conv_state_advance), against 4 single steps
    kd = 4
    xk = xbc_t[:kd].permute(1, 0, 2).contiguous()
    dk = dt_t[:kd].permute(1, 0, 2).contiguous()
    uk = torch.empty_like(xk)
    yk = torch.empty((bsz, kd, H, P), device=dev)
    cs_v = cstate.clone()
    acc = torch.randint(0, kd + 1, (bsz,), generator=torch.Generator().manual_seed(5),
                        dtype=torch.int32).to(dev)
    di = d.d_inner

    def verify():
        cs_v.copy_(cstate)
        mm.conv1d_silu(xk, cw, None, cs_v, d_inner=di, d_head=P, d_state=N, n_heads_active=H,
                       out=uk)
        mm.ssd_step_multi(state, uk[..., :di].view(bsz, kd, H, P), dk, A, uk[..., di:di + N],
                          uk[..., di + N:], D, state_out=None, y=yk)

    def commit():
        mm.ssd_step_multi(state, uk[..., :di].view(bsz, kd, H, P), dk, A, uk[..., di:di + N],
                          uk[..., di + N:], D, state_out=state, tokens_per_seq=acc, y=yk)
        mm.conv_state_advance(cstate, xk, d_inner=di, d_head=P, d_state=N, tokens_per_seq=acc)

    def four_steps():
        for t in range(kd):
            mm.ssd_step(state, uk[:, t, :di].view(bsz, H, P), dk[:, t], A, uk[:, t, di:di + N],
                        uk[:, t, di + N:], D, y=yt)

    def timed(fn, reps=20):
        for _ in range(3):
            fn()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    v_us, c_us, s_us = timed(verify), timed(commit), timed(four_steps)
    return {"workload": "decode: batch 256, 64 heads x 64 x 128 fp32 state, slices "
                        "round-robin {16,32,64} heads, 1024 tokens in a HIP graph",
            "tokens_per_s": bsz * steps / (ms * 1e-3), "us_per_step": per_step_us,
            "bytes_per_step": by, "hbm_frac": by / (per_step_us * 1e-6) / (HBM_PEAK_GBS * 1e9),
            "fused_vs_two_launches": sweep,
            "spec_decode": {"draft_tokens": kd, "heads": H, "verify_us": v_us, "commit_us": c_us,
                            "four_single_steps_us": s_us,
                            "verify_plus_commit_vs_steps": s_us / (v_us + c_us)}}


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w):
    """The fp64 oracle as it stands, on the host cores.  ``value``: one full
    step of the benchmarked workload (conv over all 4352 channels, then the
    scan for all 64 heads of the 4 sequences of 8192 tokens; ~86 GFLOP of
    fp64 work).  ``per_config``: the oracle's scan alone at the smallest and
    the full slice of every forward workload (the long-context one on its
    first 32768 tokens: the oracle's time is linear in them), and 64 decode
    steps (conv state roll + state update) of 32 of the decode batch's 256
    sequences at its mixed widths, each on that workload's seeded inputs."""
    import oracle
    import synth

    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    b, l, H, P, N = w.batch, w.seqlen, w.n_heads, w.d_head, w.d_state
    xi = synth.xbc_inputs(w)
    u = xi["xbc"].double().numpy()
    cw = xi["w"].double().numpy()
    dt = synth.pipeline_dt(w).double().numpy()
    A = synth.draw_A(w).double().numpy()
    D = synth.draw_D(w).double().numpy()
    del xi
    oracle.build()
    t0 = time.perf_counter()
    xo, _ = oracle.conv1d_silu(u, cw, None, None, d_inner=w.d_inner, d_head=P)
    t1 = time.perf_counter()
    del u
    x = xo[..., :w.d_inner].reshape(b, l, H, P)
    Bm = xo[..., w.d_inner:w.d_inner + N]
    Cm = xo[..., w.d_inner + N:]
    oracle.ssd_forward(x, dt, A, Bm, Cm, D, return_state=False)
    t2 = time.perf_counter()
    del xo, x, Bm, Cm
    per = {}
    for name in ("tiny", "130m", "1.4b", "long"):
        wl = synth.WORKLOADS[name]
        sl = min(wl.seqlen, 32768)
        inp = {k: v.double().numpy() for k, v in synth.forward_inputs(wl, seqlen=sl).items()}
        toks = wl.batch * sl
        for m in (wl.slices[0], wl.slices[-1]):
            h = wl.heads(m)
            ta = time.perf_counter()
            oracle.ssd_forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                               heads_active=h, return_state=False)
            tb = time.perf_counter()
            per[f"{name} m={m}"] = {"heads": h, "tokens": toks, "seconds": tb - ta,
                                    "tokens_per_s": toks / (tb - ta)}
            if sl < wl.seqlen:
                per[f"{name} m={m}"]["sample"] = f"first {sl} of {wl.seqlen} tokens"
        del inp
    dw = synth.WORKLOADS["decode"]
    nb = 32  # sequences of the decode batch timed
    pool = synth.decode_pool(dw, pool=64, batch=nb)
    xs = pool["xbc_t"].double().numpy()
    dts = pool["dt_t"].double().numpy()
    hv = synth.decode_heads(dw, batch=nb).numpy()
    Ad, Dd = synth.draw_A(dw).double().numpy(), synth.draw_D(dw).double().numpy()
    cwd = synth.draw_conv_w(dw).double().numpy()
    import numpy as np
    st = np.zeros((nb, dw.n_heads, dw.d_head, dw.d_state))
    cst = np.zeros((nb, dw.conv_dim, 3))
    di, Nd = dw.d_inner, dw.d_state
    ta = time.perf_counter()
    for k in range(64):
        uo, cst = oracle.conv1d_silu(xs[k][:, None, :], cwd, None, cst, d_inner=di, d_head=dw.d_head,
                                     heads_active=hv)
        uo = uo[:, 0]
        _, st = oracle.ssd_step(st, uo[:, :di].reshape(nb, dw.n_heads, dw.d_head), dts[k], Ad,
                                uo[:, di:di + Nd], uo[:, di + Nd:], Dd, heads_active=hv)
    tb = time.perf_counter()
    per["decode 64 steps"] = {"sequences": nb, "seconds": tb - ta,
                              "tokens_per_s": nb * 64 / (tb - ta),
                              "sample": f"{nb} of the {dw.batch} sequences, widths round-robin"}
    nthr = int(os.environ["OMP_NUM_THREADS"])
    return {"value": b * l / (t2 - t0), "unit": "tokens/s", "cores": nthr,
            "kind": "oracle", "cpu_model": _cpu_model(), "omp_num_threads": nthr,
            "sample": f"one full step (b={b}, l={l}): fp64 conv {t1 - t0:.1f}s + scan {t2 - t1:.1f}s "
                      f"on {nthr} threads",
            "per_config": per}


if __name__ == "__main__":
    main()
