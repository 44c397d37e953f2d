"""Benchmark of the hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step is one pass of the whole hot path over synthetic inputs already
resident in HBM: a causal GQA prefill (attn_fwd, Llama-3-8B shape:
B=1, Hq=32, Hkv=8, N=8192, d=128, bf16) followed by a GQA split-K decode
(attn_decode, B=64, Hq=32, Hkv=8, d=128, bf16 cache of 32768 rows, lengths
uniform in [1024, 32768]). Each part is timed with HIP events on the stream
the library launches on (torch's current stream).

Printed (one JSON line):
  value      prefill forward throughput, TFLOP/s of algorithmic work
             (4 d per attended query-key pair) over the prefill part of the steps
  decode     KV-read GB/s of the decode part (sum of lengths x Hkv x d x 2 x 2 B)
  roofline   prefill kernel against the dense bf16 MFMA peak (and against that peak
             scaled to the engine clock measured under the kernel in this run)
  clock      the engine clock the main kernel ran at, measured in this run: a
             probe (libmiclock.so) on a second stream reads the shader-clock
             cycle counter against the 100 MHz real-time counter on every XCD
             while the back-to-back calls of the main part run (mean, min and
             max over the XCDs); next to it the bracket from a stored counter
             pass of the same command (profiles/clock.json, gated by a hash of
             the kernel sources)
  roofline_decode  decode against the HBM peak
  cpu_baseline  the fp64 oracle on the host cores, on a bounded sample
  ms_parts_back_to_back  per part, the average of --back-to-back calls (200)
             issued back to back after the timed steps (warm, no host gaps)

--workload runs a single named workload instead (one call per step):
gpt2-causal, gpt2-medium-causal, llama3-8b-gqa-causal-8k, gqa-decode-b64,
video-frames-16x880 (online), video-frames-16x880-fixed,
video-frames-16x880-centered, tiny-f32, and the backward pass (attn_bwd, with
O and the LSE from one attn_fwd call made before the timed steps; 10 d FLOPs
per attended pair): llama3-8b-gqa-causal-8k-bwd, gpt2-medium-causal-bwd,
video-frames-16x880-bwd; and gqa-decode-b64-4tok (attn_decode_multi, 4 new
tokens per sequence against the cache, KV-read GB/s), gqa-decode-b64-paged
(attn_decode_paged, the decode cache in 64-row pages placed at random).
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK = 2516.6   # TFLOP/s, 256 CU x 4096 FLOP/clk x 2.4 GHz (dense)
FP32_PEAK = 157.3         # TFLOP/s
HBM_PEAK = 8000.0         # GB/s

# Counter-derived HBM bytes per launch of the kernels timed by the default step
# (rocprofv3 FETCH_SIZE and WRITE_SIZE, each scaled by what it reads for a plain
# device copy of known size). They describe the kernel sources whose hash is
# stored with them and are reported only while those sources are unchanged.
DEFAULT = ("llama3-8b-gqa-causal-8k", "gqa-decode-b64")   # the default step
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
TRAFFIC_NOTE = ("stored, not measured in this run: HBM bytes per launch from two rocprofv3 "
                "counter passes (FETCH_SIZE, WRITE_SIZE, scaled by a plain copy) kept in "
                "profiles/hbm_traffic.json; null whenever the kernel sources no longer match "
                "the hash stored with them")


def measured_traffic(part):
    """HBM bytes per launch for this kernel from the stored counters, or None."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_FILE))[part]
    except (OSError, KeyError, ValueError):
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:
        with open(os.path.join(ROOT, "exact_io_aware_attn_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != rec["source_sha256_16"]:
        return None
    return rec["bytes"]


CLOCK_FILE = os.path.join(ROOT, "profiles", "clock.json")


def _sources_match(rec):
    import hashlib
    h = hashlib.sha256()
    for f in rec["sources"]:
        with open(os.path.join(ROOT, "exact_io_aware_attn_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16] == rec["source_sha256_16"]


def stored_clock(workload):
    """The main kernel's sustained engine clock for this workload, from the
    stored counter pass, or None (no record, or the sources changed since)."""
    try:
        rec = json.load(open(CLOCK_FILE))[workload]
    except (OSError, KeyError, ValueError):
        return None
    if not _sources_match(rec):
        return None
    return {"mhz_low": rec["mhz_low"], "mhz_high": rec["mhz_high"], "kernel": rec["kernel"],
            "source": "stored, not measured in this run: a rocprofv3 counter pass of the same "
                      "bench command over the kernel's duration; low = SQ_BUSY_CYCLES / 32 "
                      "shader engines (an engine out of work stops counting), high = "
                      "GRBM_GUI_ACTIVE / 8 XCDs (includes the counter window); null whenever "
                      "the kernel sources no longer match the hash stored with it "
                      "(profiles/clock.json)"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="default")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--back-to-back", type=int, default=200,
                    help="after the timed steps, time this many calls of each part back "
                         "to back between one pair of events (ms_parts_back_to_back)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="before the steps, copy this many MiB device-to-device once "
                         "(a plain copy of known size that scales HBM byte counters)")
    return ap.parse_args()


class Part:
    """One call of a workload with pre-allocated inputs/outputs/workspace."""

    def __init__(self, name, dev):
        import torch
        from exact_io_aware_attn_amd import accounting as acc
        from exact_io_aware_attn_amd import binding as bd
        from exact_io_aware_attn_amd.inputs import WORKLOADS, workload_inputs

        base = name.replace("-fixed", "").replace("-centered", "")
        self.softmax = "fixed_max" if name.endswith("-fixed") else (
            "fixed_max_centered" if name.endswith("-centered") else "online")
        self.name = name
        self.w = w = WORKLOADS[base]
        self.ins = ins = workload_inputs(w, device=dev)
        self.kind = w.kind
        if w.kind == "prefill":
            q, k, v = ins["q"], ins["k"], ins["v"]
            self.o = torch.empty_like(q)
            self.lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=dev)
            bm = ins.get("block_mask")
            self.bm = None if bm is None else torch.from_numpy(bm).to(dev)
            mode = bd.SOFTMAX_MODES[self.softmax]
            kind = (bd.MIATTN_MASK_CAUSAL if w.causal else 0) | (
                bd.MIATTN_MASK_BLOCK if self.bm is not None else 0)
            need = bd.attn_fwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, kind, w.block, w.block, mode)
            self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev) if need else None
            self.flops, self.bytes = acc.workload_work(w, block_mask=bm)
            # arguments marshalled once; each step is one call into the library
            self.call, _, _ = bd.prepare_fwd(
                q, k, v, causal=w.causal, block_mask=self.bm,
                block=(w.block, w.block) if self.bm is not None else None,
                softmax=self.softmax, out=self.o, lse_out=self.lse, workspace=self.ws)
        elif w.kind == "backward":
            q, k, v, do = ins["q"], ins["k"], ins["v"], ins["dout"]
            bm = ins.get("block_mask")
            self.bm = None if bm is None else torch.from_numpy(bm).to(dev)
            blk = (w.block, w.block) if bm is not None else None
            self.o, self.lse = bd.attn_fwd(q, k, v, causal=w.causal, block_mask=self.bm, block=blk)
            self.flops, self.bytes = acc.workload_work(w, block_mask=bm)
            self.call, _ = bd.prepare_bwd(q, k, v, self.o, self.lse, do, causal=w.causal,
                                          block_mask=self.bm, block=blk)
        else:
            sl = ins["seqlens"]
            self.o = torch.empty_like(ins["q"])
            self.lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)
            need = bd.attn_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nk, w.d, 0)
            self.ws = torch.empty(need, dtype=torch.uint8, device=dev)
            self.seqlens_host = sl.cpu().numpy()
            self.flops, self.bytes = acc.workload_work(w, seqlens=self.seqlens_host)
            if w.page_size:
                self.lse = torch.empty((w.B, 1, w.Hq), dtype=torch.float32, device=dev)
                self.call, _, _ = bd.prepare_decode_paged(ins["q"], ins["k_pages"], ins["v_pages"],
                                                          ins["block_table"], sl, lse_out=self.lse,
                                                          workspace=self.ws)
            elif w.n_new > 1:
                self.lse = torch.empty((w.B, w.n_new, w.Hq), dtype=torch.float32, device=dev)
                need = bd.attn_decode_multi_workspace_bytes(w.B, w.n_new, w.Hq, w.Hkv, w.Nk, w.d, 0)
                self.ws = torch.empty(need, dtype=torch.uint8, device=dev)
                self.call, _, _ = bd.prepare_decode_multi(ins["q"], ins["k_cache"], ins["v_cache"],
                                                          sl, out=self.o, lse_out=self.lse,
                                                          workspace=self.ws)
            else:
                self.call, _, _ = bd.prepare_decode(ins["q"], ins["k_cache"], ins["v_cache"], sl,
                                                    out=self.o, lse_out=self.lse, workspace=self.ws)


def cpu_baseline(part, budget_s):
    """The oracle, as it is, on a bounded sample of the prefill workload: whole
    query heads of batch 0, one at a time, until the time budget is spent."""
    import numpy as np
    import oracle
    from exact_io_aware_attn_amd import accounting as acc

    w = part.w
    ins = part.ins
    f64 = lambda t: t.to("cpu").double().numpy()
    q, k, v = f64(ins["q"][:1]), f64(ins["k"][:1]), f64(ins["v"][:1])
    bm = ins.get("block_mask")
    kw = dict(causal=w.causal)
    if bm is not None:
        kw.update(block_mask=bm, block_q=w.block, block_k=w.block)
    pairs = acc.attended_pairs(w.Nq, w.Nk, causal=w.causal, block_mask=bm,
                               block_q=w.block or None, block_k=w.block or None)
    heads = 0
    t0 = time.perf_counter()
    while heads < w.Hq and (heads == 0 or time.perf_counter() - t0 < budget_s):
        oracle.attention(q, k, v, w.scale, heads=[heads], **kw)
        heads += 1
    dt = time.perf_counter() - t0
    flops = 4 * w.d * pairs * heads
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _threads(), "kind": "oracle",
            "sample": f"{w.name}: batch 0, {heads} of {w.Hq} query heads, all {w.Nq} rows "
                      f"(fp64 NumPy, S and P materialised), {dt:.1f} s",
            "seconds": dt}


def cpu_baseline_bwd(part, budget_s):
    """The gradient oracle, as it is, on a bounded sample of a backward
    workload: one query head (with its KV head) of batch 0 at a time, until the
    time budget is spent."""
    import oracle
    from exact_io_aware_attn_amd import accounting as acc

    w = part.w
    ins = part.ins
    f64 = lambda t: t.to("cpu").double().numpy()
    G = w.Hq // w.Hkv
    bm = ins.get("block_mask")
    kw = dict(causal=w.causal)
    if bm is not None:
        kw.update(block_mask=bm, block_q=w.block, block_k=w.block)
    pairs = acc.attended_pairs(w.Nq, w.Nk, causal=w.causal, block_mask=bm,
                               block_q=w.block or None, block_k=w.block or None)
    heads = 0
    t0 = time.perf_counter()
    while heads < w.Hq and (heads == 0 or time.perf_counter() - t0 < budget_s):
        h, hk = heads, heads // G
        oracle.attention_backward(f64(ins["q"][:1, :, h:h + 1]), f64(ins["k"][:1, :, hk:hk + 1]),
                                  f64(ins["v"][:1, :, hk:hk + 1]), f64(ins["dout"][:1, :, h:h + 1]),
                                  w.scale, **kw)
        heads += 1
    dt = time.perf_counter() - t0
    flops = 10 * w.d * pairs * heads
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _threads(), "kind": "oracle",
            "sample": f"{w.name}: batch 0, {heads} of {w.Hq} query heads, all {w.Nq} rows "
                      f"(fp64 NumPy, S, P, dP and dS materialised), {dt:.1f} s",
            "seconds": dt}


def _threads():
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads") or 0) for i in threadpool_info()) or None
    except Exception:
        pass
    return threads or len(os.sched_getaffinity(0))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = "cuda:0"
    torch.cuda.set_device(0)

    if args.workload == "default":
        names = list(DEFAULT)
    else:
        names = [args.workload]
    parts = [Part(n, dev) for n in names]
    torch.cuda.synchronize()
    if args.calibration_copy_mib:
        n = args.calibration_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # bring the GPU out of its idle clocks before the warm-up steps (a short
    # matrix-multiply burst, ~0.3 s; not part of any step)
    x = torch.randn(4096, 4096, device=dev)
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < 0.3:
        for _ in range(10):
            x = (x @ x) * 1e-4
        torch.cuda.synchronize()
    del x

    for _ in range(args.warmup):
        for p in parts:
            p.call()
    torch.cuda.synchronize()

    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in parts] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        for i, p in enumerate(parts):
            ev[s][i][0].record()
            p.call()
            ev[s][i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [[ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)]
          for i in range(len(parts))]
    # after the timed steps: each part's average over back-to-back calls
    # between one pair of events (warm; no gap for the host between calls)
    ms_avg = [sum(m) / len(m) for m in ms]
    b2b = {}
    live_clock = None
    for i, p in enumerate(parts):
        probe = None
        # the main part's engine clock: a probe on a second stream (default
        # priority) spans these calls but the first and last 0.5 ms
        window_s = (args.back_to_back * ms_avg[i] - 1.0) * 1e-3
        if i == 0 and window_s >= 1e-3:
            from exact_io_aware_attn_amd import clock as clk_mod
            probe = clk_mod.ClockProbe(device=dev)
            side = torch.cuda.Stream()
            torch.cuda.synchronize()
            probe.start(window_s, warm_s=0.5e-3, stream=side)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.back_to_back):
            p.call()
        e1.record()
        torch.cuda.synchronize()
        b2b[p.name] = e0.elapsed_time(e1) / args.back_to_back if args.back_to_back > 0 else None
        if probe is not None:
            live_clock = clk_mod.summary(probe.result())
            live_clock.update(window_ms=window_s * 1e3, calls=args.back_to_back,
                              source="measured in this run: shader-clock cycles (s_memtime) over "
                                     "the 100 MHz real-time counter, one probe wave per XCD "
                                     "(two rounds of 8) on a second stream, across the "
                                     "back-to-back calls of the main part that follow the "
                                     "timed steps")
    ms_step = wall * 1e3 / args.steps

    main_p = parts[0]
    out = {"metric": "fwd attn TFLOP/s & %MFMA peak (prefill); KV-read GB/s & %HBM peak (decode)"}
    if main_p.kind == "backward":
        out["metric"] = "bwd attn TFLOP/s (10 d FLOPs per attended pair) & %MFMA peak"
    if main_p.kind in ("prefill", "backward"):
        tflops = main_p.flops / (ms_avg[0] * 1e-3) / 1e12
        peak = MFMA_BF16_PEAK if main_p.w.dtype == "bf16" else FP32_PEAK
        out.update(value=tflops, unit="TFLOP/s")
        roof = {"bound": "mfma", "achieved": tflops, "peak": peak, "unit": "TFLOP/s",
                "frac": tflops / peak,
                "traffic": measured_traffic("prefill") if main_p.name == DEFAULT[0] else None,
                "traffic_source": TRAFFIC_NOTE}
    else:
        gbs = main_p.bytes / (ms_avg[0] * 1e-3) / 1e9
        out.update(value=gbs, unit="GB/s")
        roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK, "unit": "GB/s",
                "frac": gbs / HBM_PEAK,
                "traffic": measured_traffic("decode") if main_p.name == DEFAULT[1] else None,
                "traffic_source": TRAFFIC_NOTE}
    out.update(n_gpus=1, steps=args.steps, warmup=args.warmup, ms_per_step=ms_step,
               higher_is_better=True, scaling="weak", vs_baseline=None,
               dtype="bf16" if main_p.w.dtype == "bf16" else "f32",
               data="synthetic (seeded N(0,1) inputs, generated on the GPU)")
    cfg = {"workload": " + ".join(p.name for p in parts)}
    for p in parts:
        w = p.w
        cfg[p.name] = {"B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                       "causal": w.causal, "softmax": p.softmax,
                       "flops": p.flops, "bytes": p.bytes}
    out["config"] = cfg
    out["ms_parts"] = {p.name: m for p, m in zip(parts, ms_avg)}
    # per-call spread over the timed steps (warm: inputs resident, GPU clocks up)
    out["ms_parts_median"] = {p.name: sorted(m)[len(m) // 2] for p, m in zip(parts, ms)}
    out["ms_parts_min"] = {p.name: min(m) for p, m in zip(parts, ms)}
    out["ms_parts_back_to_back"] = b2b
    out["clock"] = {"measured": live_clock, "counter_bracket": stored_clock(main_p.name)}
    if live_clock is not None and roof["bound"] == "mfma":
        # the same peak at the engine clock the kernel held (the 2516.6
        # TFLOP/s figure assumes 2.4 GHz): at the mean over the XCDs, and at
        # the slowest and fastest XCD's clock
        pk = roof["peak"] * live_clock["mhz_mean"] / 2400.0
        roof["peak_at_measured_clock"] = pk
        roof["frac_at_measured_clock"] = roof["achieved"] / pk
        rng = [roof["peak"] * live_clock[m] / 2400.0 for m in ("mhz_min", "mhz_max")]
        roof["peak_at_xcd_clock_range"] = rng
        roof["frac_at_xcd_clock_range"] = [roof["achieved"] / rng[1], roof["achieved"] / rng[0]]
    out["roofline"] = roof
    if len(parts) > 1 and parts[1].kind == "decode":
        d = parts[1]
        gbs = d.bytes / (ms_avg[1] * 1e-3) / 1e9
        out["decode"] = {"value": gbs, "unit": "GB/s", "ms": ms_avg[1]}
        out["roofline_decode"] = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK,
                                  "unit": "GB/s", "frac": gbs / HBM_PEAK,
                                  "traffic": measured_traffic("decode"),
                                  "traffic_source": TRAFFIC_NOTE}
    if not args.no_cpu_baseline and main_p.kind == "prefill":
        out["cpu_baseline"] = cpu_baseline(main_p, args.cpu_seconds)
    elif not args.no_cpu_baseline and main_p.kind == "backward":
        out["cpu_baseline"] = cpu_baseline_bwd(main_p, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
