#!/usr/bin/env python3
"""Benchmark of the FA-quantization hot path on one MI355X.

One step = quantize Q, K and V with the workload's mode (each configured
branch), then quantized attention on the codes (the whole hot path;
calibration of static per-head scales is offline - done once before timing -
as the scales are frozen).
Inputs are seeded synthetic tensors already resident in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config N]

prints one JSON line.  The default workload is the largest configuration
that fits one GPU: FP8 E4M3 per-token dynamic on the video-DiT shape (bf16
[1,40,32760,128], non-causal).  `value` is attention operations (4*D per
unmasked query-key pair) per second of the whole step (mean over the timed
steps), in TFLOPS (TOPS for INT8); the median and minimum step times are
reported beside it.  `roofline` reports the attention call (K/V re-layout +
fused kernel) against the mode's dense MFMA peak; `cpu_baseline` times the
CPU oracle on a bounded sample of the same workload; `clocks` records the
GPU's shader and memory clocks, read with amd-smi while attention calls
run back to back after the timed steps.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantized-attention TFLOPS/TOPS (% MFMA peak) + quantize GB/s, 1 MI355X"
PEAK_HBM_GBS = 8000.0
PEAK_TOPS = {"int8_head": 5000.0, "fp8_token": 5000.0, "rot_fp8_block": 5000.0, "mxfp4": 10100.0,
             "fp8_head": 5000.0, "int8_token": 5000.0, "mxfp8": 5000.0}
DTYPE = {"int8_head": "int8", "fp8_token": "fp8_e4m3", "rot_fp8_block": "fp8_e4m3", "mxfp4": "mxfp4",
         "fp8_head": "fp8_e4m3", "int8_token": "int8", "mxfp8": "mxfp8"}
MODE_TEXT = {"int8_head": "INT8 per-head static", "fp8_token": "FP8 E4M3 per-token dynamic",
             "mxfp4": "MXFP4 per-32 block dynamic", "rot_fp8_block": "rotate + FP8 E4M3 token-block",
             "fp8_head": "FP8 E4M3 per-head static", "int8_token": "INT8 per-token dynamic",
             "mxfp8": "MXFP8 per-32 block dynamic"}
P_RULE = {"int8_head": "int8", "fp8_token": "fp8", "mxfp4": "mxfp4", "rot_fp8_block": "fp8",
          "fp8_head": "fp8", "int8_token": "int8", "mxfp8": "mxfp8", "float": "bf16"}
BF16_PEAK = 2500.0
STATIC = {"int8_head": "int8", "fp8_head": "fp8_e4m3"}  # per-head static modes -> scale dtype


def attention_ops(w):
    """4 D operations per unmasked (query, key) pair."""
    B, H, S, D = w.shape
    Sq = int(w.q.shape[2])
    pairs = S * (S + 1) // 2 if w.spec["causal"] else Sq * S
    return 4 * D * B * H * pairs


def is_decode(w):
    return "q_len" in w.spec


def attention_bytes(w):
    """Algorithmic HBM bytes of one decode attention call: the Q, K and V
    codes and scales once, and the bf16 output."""
    B, H, S, D = w.shape
    Sq = int(w.q.shape[2])
    tot = 0
    for br, mode in enumerate(branch_modes(w)):
        n = B * H * (Sq if br == 0 else S)
        if mode == "float":
            tot += 2 * n * D
        elif mode == "mxfp4":
            tot += n * D // 2 + n * D // 32
        elif mode == "mxfp8":
            tot += n * D + n * D // 32
        elif mode in STATIC:
            tot += n * D + H * 4
        else:
            tot += n * D + n * 4
    return tot + 2 * B * H * Sq * D


def branch_modes(w):
    """The mode of each branch (Q, K, V); "float" = not quantized."""
    return tuple(w.spec.get("modes", (w.spec["mode"],) * 3))


def peak_of(w):
    """Dense MFMA peak the attention is quoted against: the mode's; with an
    unquantized side, the harmonic combination of the two products' peaks
    (each product is half the operations)."""
    mq, _, mv = branch_modes(w)
    pk = lambda m: BF16_PEAK if m == "float" else PEAK_TOPS[m]
    a, b = pk(mq), pk(mv)
    return a if a == b else round(2.0 / (1.0 / a + 1.0 / b), 1)


def quantize_bytes(w):
    """Algorithmic bytes of quantizing the configured branches: input read +
    codes + scales (an unquantized branch moves nothing)."""
    B, H, S, D = w.shape
    inb = 4 if w.spec["dtype"] == "f32" else 2
    tot = 0
    for br, mode in enumerate(branch_modes(w)):
        if mode == "float" or (br > 0 and is_decode(w)):
            continue  # decode: the K/V cache is quantized once, outside the step
        n = B * H * (int(w.q.shape[2]) if br == 0 else S) * D
        if mode in STATIC:
            tot += n * inb + n + H * 4
        elif mode in ("fp8_token", "int8_token"):
            tot += n * inb + n + B * H * S * 4
        elif mode == "mxfp4":
            tot += n * inb + n // 2 + n // 32
        elif mode == "mxfp8":
            tot += n * inb + n + n // 32
        else:
            bt = w.spec["q_block"] if br == 0 else w.spec["kv_block"]
            tot += n * inb + n + B * H * (-(-S // bt)) * 4 + (D * D * 2 if br < 2 else 0)
    return tot


def make_step(w, dev, layout="bnsd"):
    """Pre-allocates every output and returns (step_fn, attention_fn).  With
    layout "bsnd" the inputs, codes and output are BSND."""
    import torch
    import quantized_attention_fa_amd as faq

    modes = branch_modes(w)
    xs = [t.to(dev) for t in (w.q, w.k, w.v)]
    if layout == "bsnd":
        xs = [x.permute(0, 2, 1, 3).contiguous() for x in xs]
    rot = w.rot.to(dev) if w.rot is not None else None
    cfgs, statics, outs = [], [None] * 3, []
    for br in range(3):
        mode = modes[br]
        if mode == "float":
            cfgs.append(None)
            outs.append(faq.float_branch(xs[br], layout=layout))
            continue
        if mode in STATIC:
            cfg = faq.QConfig(STATIC[mode], "per_head")
            amax = torch.zeros(w.shape[1], dtype=torch.float32, device=dev)
            for c in w.calib[br]:
                faq.fa_quant_calibrate(c.to(dev), amax)  # calibration data stays BNSD
            statics[br] = faq.fa_quant_scales_from_amax(amax, STATIC[mode])
        elif mode == "fp8_token":
            cfg = faq.QConfig("fp8_e4m3", "per_token")
        elif mode == "int8_token":
            cfg = faq.QConfig("int8", "per_token")
        elif mode in ("mxfp4", "mxfp8"):
            cfg = faq.QConfig(mode, "per_block")
        else:
            cfg = faq.QConfig("fp8_e4m3", "per_token_block",
                              block_tokens=w.spec["q_block"] if br == 0 else w.spec["kv_block"])
        cfgs.append(cfg)
        qt = faq.fa_quantize(xs[br], cfg, static_scale=statics[br], rot=rot if br < 2 else None, layout=layout)
        if mode in STATIC:
            qt.scales = statics[br]  # per-head scales are used in place
        outs.append(qt)
    ws = torch.empty(max(faq.fa_quant_attention_workspace_bytes(*outs), 1), dtype=torch.uint8, device=dev)
    B_, H_, S_, D_ = outs[0].shape
    out = torch.empty((B_, H_, S_, D_) if layout == "bnsd" else (B_, S_, H_, D_), dtype=torch.bfloat16, device=dev)

    def quantize():
        for br in range(1 if is_decode(w) else 3):
            if cfgs[br] is not None:
                faq.fa_quantize(xs[br], cfgs[br], static_scale=statics[br], rot=rot if br < 2 else None,
                                out=outs[br], layout=layout)

    def attention():
        faq.fa_quant_attention(*outs, causal=w.spec["causal"], out=out, workspace=ws)

    return quantize, attention


def cpu_baseline(w, budget_s=20.0):
    """The oracle (as it stands) on a bounded sample of the workload: whole
    (b,h) heads, quantize + attention, until about `budget_s` seconds."""
    import numpy as np
    import torch
    from oracle import attention as OA
    from oracle import formats as F
    from oracle import quantize as OQ

    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    cores = len(os.sched_getaffinity(0))
    B, H, S, D = w.shape
    modes = branch_modes(w)
    causal = w.spec["causal"]
    rule = P_RULE[modes[2]]
    t0 = time.perf_counter()
    ops = 0
    heads = 0
    rows = None
    # a single head can exceed the budget at long sequence lengths: sample rows
    Sq = int(w.q.shape[2])
    full_pairs = S * (S + 1) // 2 if causal else Sq * S
    if full_pairs > 4096 * 4096:
        rows = np.arange(0, Sq, max(1, Sq // 1024))
    blocks = (w.spec.get("q_block"), w.spec.get("kv_block"), w.spec.get("kv_block"))
    for h in range(H):
        if time.perf_counter() - t0 > budget_s:
            break
        x = [t[0:1, h:h + 1].to(torch.float32).numpy() for t in (w.q, w.k, w.v)]
        deq, scl = [], []
        for br in range(3):
            mode = modes[br]
            sv = None
            if mode == "float":
                d = x[br].astype(np.float64)
            elif mode in STATIC:
                amax = None
                for c in w.calib[br]:
                    amax = OQ.calibrate_amax(c[:, h:h + 1].to(torch.float32).numpy(), amax)
                if mode == "int8_head":
                    s = OQ.int8_scales(amax)
                    d = OQ.dequantize_per_head(OQ.quantize_int8_per_head(x[br], s), s)
                else:
                    s = OQ.fp8_scales(amax)
                    d = OQ.dequantize_per_head(OQ.quantize_fp8_per_head(x[br], s), s, F.e4m3_decode)
                sv = np.full((1, 1, S), s[0])
            elif mode == "fp8_token":
                c, sv = OQ.quantize_fp8_per_token(x[br])
                d = OQ.dequantize_per_token(c, sv, F.e4m3_decode)
            elif mode == "int8_token":
                c, sv = OQ.quantize_int8_per_token(x[br])
                d = OQ.dequantize_per_token(c, sv, lambda a: a.astype(np.float64))
            elif mode == "mxfp4":
                d = OQ.dequantize_mxfp4(*OQ.quantize_mxfp4(x[br]))
            elif mode == "mxfp8":
                d = OQ.dequantize_mxfp8(*OQ.quantize_mxfp8(x[br]))
            else:
                y = OQ.rotate(x[br], w.rot.to(torch.float32).numpy()) if br < 2 else x[br]
                c, s = OQ.quantize_fp8_block(y, blocks[br])
                sv = OQ.block_scales_per_token(s, blocks[br], S)
                d = OQ.dequantize_per_token(c, sv, F.e4m3_decode)
            deq.append(d)
            scl.append(sv)
        vs = scl[2]
        OA.attention(*deq, rule, v_scale=vs, causal=causal, rows=rows)
        r = np.arange(Sq) if rows is None else rows
        ops += 4 * D * int(np.sum(np.minimum(r + 1, S) if causal else np.full(r.size, S)))
        heads += 1
    dt = time.perf_counter() - t0
    sample = f"{heads} of {B * H} (b,h) heads" + ("" if rows is None else f", {rows.size} of {Sq} query rows each")
    sample += ", quantize + attention"
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": cores, "blas_threads": blas, "kind": "oracle",
            "sample": sample, "seconds": round(dt, 2)}


def source_digest():
    """sha256 of the attention kernel source with its comments and
    whitespace removed: HBM traffic counted by the profiler is only reported
    for the kernel code it was counted on."""
    import hashlib
    import re
    src = os.path.join(ROOT, "quantized_attention_fa_amd", "csrc", "attention.hip")
    with open(src, encoding="utf-8") as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)  # block comments
    text = re.sub(r"//[^\n]*", " ", text)                # line comments
    code = " ".join(text.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def recorded_traffic(workload):
    """HBM bytes per attention launch from the profiler counter runs stored
    in profiles/traffic.json (FETCH_SIZE + WRITE_SIZE, scaled by the factor
    a plain copy of known size reads), or None when there is no record for
    this workload or the kernel source has changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload)
    if not rec or rec.get("attention_source") != source_digest():
        return None
    return rec.get("attention_bytes_per_launch")


def _amd_smi_clocks(text):
    """Shader clocks of the 8 XCDs (gfx_0..gfx_7) and the memory clock, MHz,
    from the output of `amd-smi metric -c --json`."""
    try:
        clk = json.loads(text)["gpu_data"][0]["clock"]
        gfx = [clk[k]["clk"]["value"] for k in sorted(clk) if k.startswith("gfx_")]
        return {"sclk_mhz_per_xcd": gfx, "sclk_mhz_mean": round(sum(gfx) / len(gfx), 1),
                "mclk_mhz": clk["mem_0"]["clk"]["value"]}
    except Exception as e:  # pragma: no cover - depends on the host's tools
        return {"error": f"amd-smi: {type(e).__name__}: {e}"[:200]}


def copy_reference(dev, nbytes, flush, flush_out, reps=10):
    """HBM rate of a plain device-to-device copy moving `nbytes` in total
    (nbytes / 2 read, nbytes / 2 written), timed like the quantize step
    (cache flushed before each copy): the practical ceiling the quantize
    fraction is read against on this machine."""
    import torch
    n = max(nbytes // 2, 1)
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    st = torch.cuda.current_stream()
    ms = []
    for _ in range(reps):
        if flush is not None:
            torch.sum(flush, dim=0, out=flush_out)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        dst.copy_(src)
        b.record(st)
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    ms.sort()
    return 2 * n / (ms[len(ms) // 2] * 1e-3) / 1e9


def clocks_under_load(fn, ms_per_call, warm_s=1.0, limit_s=30.0):
    """GPU clocks read while `fn` calls keep the GPU busy (an idle GPU drops
    its clocks within milliseconds).  The calls are issued for `warm_s`
    seconds first, then for as long as amd-smi runs, never more than about
    40 ms of work ahead of the GPU: a deep queue would leave the host done
    (and amd-smi reading an idle GPU) while the work still drains."""
    import collections
    import subprocess
    import tempfile
    import torch
    depth = max(2, int(40.0 / max(ms_per_call, 1e-3)) + 1)
    pending = collections.deque()
    calls = 0

    def pump(done):
        nonlocal calls
        while not done():
            fn()
            calls += 1
            e = torch.cuda.Event()
            e.record(torch.cuda.current_stream())
            pending.append(e)
            if len(pending) > depth:
                pending.popleft().synchronize()

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    pump(lambda: time.perf_counter() - t0 > warm_s)
    with tempfile.TemporaryFile(mode="w+") as out:
        try:
            proc = subprocess.Popen(["amd-smi", "metric", "-g", "0", "-c", "--json"], stdout=out,
                                    stderr=subprocess.DEVNULL, text=True)
        except Exception as e:  # pragma: no cover - depends on the host's tools
            torch.cuda.synchronize()
            return {"error": f"amd-smi: {type(e).__name__}"}
        t1 = time.perf_counter()
        pump(lambda: proc.poll() is not None or time.perf_counter() - t1 > limit_s)
        torch.cuda.synchronize()
        if proc.poll() is None:  # pragma: no cover
            proc.kill()
            proc.wait()
            return {"error": "amd-smi did not finish", "calls_issued": calls}
        out.seek(0)
        res = _amd_smi_clocks(out.read())
    res["calls_issued"] = calls
    res["seconds_sampled_under"] = round(time.perf_counter() - t1, 2)
    return res


def copy_calibration(dev, nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of known size, for scaling the
    profiler's FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3,
                    help="workload 1..11 (default 3, FP8 per-token on the video-DiT shape: the largest of the "
                         "metric's configurations; 1-5 are the metric's configurations, 6-8 the sibling FA "
                         "modes, 9-10 per-branch configurations, 11 decode over a quantized cache)")
    ap.add_argument("--no-clocks", action="store_true", help="do not read the GPU clocks with amd-smi")
    ap.add_argument("--no-flush", action="store_true", help="skip the cache flush between steps")
    ap.add_argument("--layout", choices=("bnsd", "bsnd"), default="bnsd",
                    help="memory layout of Q/K/V, their codes and the output")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (scale reference for the profiler's byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the hot path shards over (batch, head) with no communication - see the design notes.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from synth import make_inputs

    dev = "cuda:0"
    if args.copy_calibration:
        copy_calibration(dev)
        return
    w = make_inputs(args.config)
    modes = branch_modes(w)
    quantize, attention = make_step(w, dev, args.layout)
    flush = None
    if not args.no_flush:
        # read (not write) 512 MB between steps: evicts the inputs from L2
        # and the Infinity Cache and leaves only clean lines, so no
        # write-back of the flush's own data lands inside the timed step
        flush = torch.zeros(64 << 20, dtype=torch.int64, device=dev)
        flush_out = torch.empty((), dtype=torch.int64, device=dev)

    for _ in range(args.warmup):
        quantize()
        attention()
    torch.cuda.synchronize()

    st = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(args.steps):
        if flush is not None:
            torch.sum(flush, dim=0, out=flush_out)  # evict the inputs from the caches (outside the step's events)
        ev[i][0].record(st)
        quantize()
        ev[i][1].record(st)
        attention()
        ev[i][2].record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    q_ms = [e[0].elapsed_time(e[1]) for e in ev]
    a_ms = [e[1].elapsed_time(e[2]) for e in ev]
    step_ms = [q + a for q, a in zip(q_ms, a_ms)]
    mean = lambda v: sum(v) / len(v)
    median = lambda v: sorted(v)[len(v) // 2] if len(v) % 2 else 0.5 * sum(sorted(v)[len(v) // 2 - 1:len(v) // 2 + 1])
    ms_step = mean(step_ms)
    ops = attention_ops(w)
    qbytes = quantize_bytes(w)
    att_ms = mean(a_ms)
    att_tops = ops / (att_ms * 1e-3) / 1e12
    q_gbs = qbytes / (mean(q_ms) * 1e-3) / 1e9 if qbytes else 0.0
    peak = peak_of(w)
    dtypes = [DTYPE.get(m, "bf16") for m in (modes[0], modes[2])]
    dtype = dtypes[0] if dtypes[0] == dtypes[1] else "+".join(dtypes)
    mode_text = (MODE_TEXT[modes[0]] if len(set(modes)) == 1 and modes[0] != "float" else
                 "Q/K " + MODE_TEXT.get(modes[0], "bf16 (not quantized)") + ", V " +
                 MODE_TEXT.get(modes[2], "bf16 (not quantized)"))
    B, H, S, D = w.shape
    line_workload = w.spec["name"] + ("" if args.layout == "bnsd" else "_bsnd")
    kernel = "fa_quant_attention: k_prep (V / K re-layout) + k_attn (fused attention)"
    if is_decode(w):
        # a few queries against a long cache: bound by reading the cache
        abytes = attention_bytes(w)
        a_gbs = abytes / (att_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(a_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(a_gbs / PEAK_HBM_GBS, 4), "traffic": recorded_traffic(line_workload),
                    "kernel": kernel + " + k_combine (key-split merge)", "attention_source": source_digest(),
                    "bytes_per_launch": abytes, "ops_per_launch": ops, "ms_per_launch": round(att_ms, 4),
                    "tops": round(att_tops, 2)}
    else:
        roofline = {"bound": "mfma", "achieved": round(att_tops, 2), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(att_tops / peak, 4), "traffic": recorded_traffic(line_workload),
                    "kernel": kernel, "attention_source": source_digest(),
                    "ops_per_launch": ops, "ms_per_launch": round(att_ms, 4)}
    line = {
        "metric": METRIC,
        "value": round(ops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TOPS" if dtype == "int8" else "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": line_workload, "mode": mode_text,
                   "layout": args.layout.upper(), "B": B, "H": H, "S": S, "D": D,
                   **({"q_len": int(w.q.shape[2]), "cache": "quantized once, outside the step"}
                      if is_decode(w) else {}),
                   "causal": w.spec["causal"], "input_dtype": w.spec["dtype"]},
        "roofline": roofline,
        "quantize": ({"bound": "hbm", "achieved": round(q_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                      "frac": round(q_gbs / PEAK_HBM_GBS, 4), "bytes_per_step": qbytes,
                      "ms_per_step": round(mean(q_ms), 4),
                      "copy_same_bytes_gbs": round(copy_reference(dev, qbytes, flush, flush_out if flush is not None
                                                                  else None), 1)} if qbytes else None),
        "timing": {"method": "hip events on the compute stream, per step", "mean_step_ms": round(ms_step, 4),
                   "median_step_ms": round(median(step_ms), 4), "min_step_ms": round(min(step_ms), 4),
                   "attention_median_ms": round(median(a_ms), 4), "attention_min_ms": round(min(a_ms), 4),
                   "quantize_median_ms": round(median(q_ms), 4), "quantize_min_ms": round(min(q_ms), 4),
                   "wall_s_incl_flush": round(wall, 3), "cache_flush_between_steps": flush is not None},
    }
    if not args.no_clocks:
        line["clocks"] = {"attention_under_load": clocks_under_load(attention, att_ms)}
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
