"""Benchmark of the relative-position-bias attention hot path on one MI355X.

One step = one relbias_attn_fwd call over the local-layer prefill workload
(B2 S4096 Hq32/Hkv8 D128, window 512, r.E bias R=8 over distances < 512, bf16),
inputs resident in HBM before timing.  Prints ONE JSON line with the useful
TFLOP/s (4*D flops per visible (query head, key) pair), the roofline of the
prefill kernel and the float64 oracle timed on this host as a CPU baseline.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
  (default warmup: as many steps as fill 0.3 s, so that the clocks have settled)
                  [--no-cpu-baseline] [--cpu-seconds T]

Other workloads (--workload): global_prefill, long_global_prefill,
decode_global, decode_local, tiny_local_f32, decode_global_paged /
decode_local_paged (the decode steps over a paged cache, 64-row pages),
decode_global_fp4 / decode_local_fp4 (over MXFP4 caches: 68 bytes per row and kv
head for each of K and V; GB/s counts those bytes), and
local_prefill_bwd / global_prefill_bwd / long_global_prefill_bwd (one
relbias_attn_bwd call per step, the forward's o and lse computed before timing;
10*D algorithmic flops per visible pair: the five products of the backward).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "relbias-attn TFLOP/s + % bf16 MFMA peak (prefill); decode HBM GB/s %peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
KERNEL_SOURCES = {
    "prefill": ["fwd_bf16.hip", "fwd_bf16_split.hip"],
    "decode": ["decode_bf16.hip"],
    "f32": ["attn_f32.hip"],
    "backward": ["bwd_bf16.hip"],
}


def visible_pairs_prefill(S: int, window: int) -> int:
    """Number of (query, key) pairs with 0 <= i - j < window (window 0: i >= j)."""
    if window == 0 or window >= S:
        return S * (S + 1) // 2
    return window * (window + 1) // 2 + (S - window) * window


def visible_keys_decode(kv_len: int, window: int) -> int:
    return kv_len if window == 0 else min(kv_len, window)


def kernel_hash(kind: str) -> str:
    """sha256 of the kernel sources with comments and blank lines removed (first 16 hex digits)."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind] + ["rba_device.h", "rba_internal.h"]:
        with open(os.path.join(ROOT, "transformer_attention_learned_amd", "csrc", name)) as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        for line in text.splitlines():
            code = re.sub(r"//.*", "", line).strip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def profiled_traffic(workload: str, kind: str):
    """HBM bytes per launch from the committed counter summary, if it matches this kernel."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_hash(kind):
        return None
    return float(m_bytes.group(1))


def cpu_baseline(w, inp, seconds: float):
    """Time the float64 oracle on whole (batch, kv-group) slices of the workload."""
    import numpy as np
    import torch

    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    G = w.Hq // w.Hkv
    done_flops, t_total, n_slices = 0.0, 0.0, 0
    if w.kind == "backward":
        # one (batch, kv-group) slice over a causal prefix of the sequence (a prefix is an
        # exact sub-problem): the float64 score matrices of the whole sequence do not fit
        Sp = min(w.S, 4096)
        pairs = visible_pairs_prefill(Sp, w.window)
        for g in range(w.Hkv):
            hs = slice(g * G, (g + 1) * G)
            cut = lambda t: None if t is None else t[:1, :Sp, hs].contiguous().cpu()
            k = inp["k"][:1, :Sp, g:g + 1].contiguous().cpu()
            v = inp["v"][:1, :Sp, g:g + 1].contiguous().cpu()
            tab = None if inp["table"] is None else inp["table"][hs].cpu()
            E = None if inp["E"] is None else inp["E"][hs].cpu()
            t0 = time.perf_counter()
            oracle.prefill_backward(cut(inp["q"]), k, v, cut(inp["dout"]), scale=w.scale,
                                    window=w.window, bias_range=w.bias_range, mode=w.mode,
                                    table=tab, r=cut(inp["r"]), E=E, temp_len=w.temp_len)
            t_total += time.perf_counter() - t0
            done_flops += 10.0 * w.D * G * pairs
            n_slices += 1
            if t_total >= seconds:
                break
        sample = (f"{n_slices} of {w.Hkv} kv-group slices of batch 0, first {Sp} rows, "
                  f"{G} query heads each")
    elif w.kind == "prefill":
        pairs = visible_pairs_prefill(w.S, w.window)
        for b in range(w.B):
            for g in range(w.Hkv):
                hs = slice(g * G, (g + 1) * G)
                q = inp["q"][b:b + 1, :, hs].contiguous().cpu()
                k = inp["k"][b:b + 1, :, g:g + 1].contiguous().cpu()
                v = inp["v"][b:b + 1, :, g:g + 1].contiguous().cpu()
                r = None if inp["r"] is None else inp["r"][b:b + 1, :, hs].contiguous().cpu()
                tab = None if inp["table"] is None else inp["table"][hs].cpu()
                E = None if inp["E"] is None else inp["E"][hs].cpu()
                t0 = time.perf_counter()
                oracle.prefill(q, k, v, scale=w.scale, temp_len=w.temp_len, window=w.window,
                               bias_range=w.bias_range, mode=w.mode, table=tab, r=r, E=E)
                t_total += time.perf_counter() - t0
                done_flops += 4.0 * w.D * G * pairs
                n_slices += 1
                if t_total >= seconds:
                    break
            if t_total >= seconds:
                break
        sample = (f"{n_slices} of {w.B * w.Hkv} (batch, kv-group) slices, all {w.S} rows, "
                  f"{G} query heads each")
    else:
        nvis = visible_keys_decode(w.S, w.window)
        for b in range(w.B):
            t0 = time.perf_counter()
            oracle.decode(inp["q"][b:b + 1], inp["k"][b:b + 1], inp["v"][b:b + 1], w.S,
                          scale=w.scale, temp_len=w.temp_len, window=w.window,
                          bias_range=w.bias_range, mode=w.mode,
                          table=inp["table"], r=None if inp["r"] is None else inp["r"][b:b + 1],
                          E=inp["E"])
            t_total += time.perf_counter() - t0
            done_flops += 4.0 * w.D * w.Hq * nvis
            n_slices += 1
            if t_total >= seconds:
                break
        sample = f"{n_slices} of {w.B} sequences, all heads"
    return {"value": done_flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "sample": sample, "seconds": round(t_total, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps; default: as many as fill 0.3 s (at least 10), "
                         "long enough for the GPU clocks to settle at their sustained level")
    ap.add_argument("--workload", default="local_prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this hot path has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read_per_copy": n, "bytes_written_per_copy": n}))
        return

    import transformer_attention_learned_amd as rba
    from transformer_attention_learned_amd.workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    rba.load_library()
    inp = make_inputs(w, device=dev)
    torch.cuda.synchronize()

    if w.kind == "backward":
        o, lse = rba.fwd(inp["q"], inp["k"], inp["v"], window=w.window, bias_range=w.bias_range,
                         mode=w.mode, table=inp["table"], r=inp["r"], E=inp["E"], scale=w.scale,
                         temp_len=w.temp_len, return_lse=True)
        need = rba.load_library().relbias_attn_bwd_workspace_size(w.B, w.S, w.Hq, rba.MODES[w.mode],
                                                                  w.bias_range)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

        def step():
            rba.bwd(inp["q"], inp["k"], inp["v"], o, lse, inp["dout"], window=w.window,
                    bias_range=w.bias_range, mode=w.mode, table=inp["table"], r=inp["r"],
                    E=inp["E"], scale=w.scale, temp_len=w.temp_len, workspace=ws)

        flops = 10.0 * w.D * w.Hq * w.B * visible_pairs_prefill(w.S, w.window)
        tokens = w.B * w.S
        hbm_bytes = None
        kind = "backward"
    elif w.kind == "prefill":
        out = torch.empty_like(inp["q"])
        need = rba.fwd_workspace_size(w.B, w.S, w.Hq, w.Hkv, w.D, dtype=w.dtype, window=w.window,
                                      bias_range=w.bias_range, mode=w.mode, R=w.R, scale=w.scale)
        fws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None

        def step():
            rba.fwd(inp["q"], inp["k"], inp["v"], window=w.window, bias_range=w.bias_range,
                    mode=w.mode, table=inp["table"], r=inp["r"], E=inp["E"], scale=w.scale,
                    temp_len=w.temp_len, out=out, workspace=fws)

        flops = 4.0 * w.D * w.Hq * w.B * visible_pairs_prefill(w.S, w.window)
        tokens = w.B * w.S
        hbm_bytes = None
        kind = "prefill" if w.dtype == "bf16" else "f32"
    else:
        out = torch.empty_like(inp["q"])
        need = rba.decode_workspace_size(w.B, w.Hq, w.Hkv, w.D, w.S, w.window)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

        # A windowed step touches only window rows per sequence (134 MB for the local decode),
        # which would stay in the 256 MB Infinity Cache across steps; rotating over 4 cache
        # lengths makes consecutive steps read 4 disjoint windows, so the bytes come from HBM.
        kv_lens = [w.S - j * w.window for j in range(4)] if (w.window and 4 * w.window <= w.S) else [w.S]
        it = [0]

        if w.extra.get("kv") == "fp4":
            # MXFP4 caches: 64 code bytes + 4 scale bytes per row and kv head, quantised once
            kc, ks = rba.kv_quantize_fp4(inp["k"])
            vc, vs = rba.kv_quantize_fp4(inp["v"])
            torch.cuda.synchronize()

            def step():
                kv_len = kv_lens[it[0] % len(kv_lens)]
                it[0] += 1
                rba.decode_fp4(inp["q"], kc, ks, vc, vs, kv_len, window=w.window,
                               bias_range=w.bias_range, mode=w.mode, table=inp["table"],
                               r=inp["r"], E=inp["E"], scale=w.scale, temp_len=w.temp_len,
                               out=out, workspace=ws)
        elif w.extra.get("page_size"):
            # paged cache: the table scatters each sequence over a page pool; every sequence
            # has the step's cache length
            from transformer_attention_learned_amd.workloads import paged_view
            kp, vp, bt = paged_view(w, inp["k"], inp["v"])
            lens_t = [torch.full((w.B,), L, dtype=torch.int32, device=dev) for L in kv_lens]

            def step():
                j = it[0] % len(kv_lens)
                it[0] += 1
                rba.decode_paged(inp["q"], kp, vp, bt, lens_t[j], kv_lens[j], window=w.window,
                                 bias_range=w.bias_range, mode=w.mode, table=inp["table"],
                                 r=inp["r"], E=inp["E"], scale=w.scale, temp_len=w.temp_len,
                                 out=out, workspace=ws)
        else:
            def step():
                kv_len = kv_lens[it[0] % len(kv_lens)]
                it[0] += 1
                rba.decode(inp["q"], inp["k"], inp["v"], kv_len, window=w.window,
                           bias_range=w.bias_range, mode=w.mode, table=inp["table"], r=inp["r"],
                           E=inp["E"], scale=w.scale, temp_len=w.temp_len, out=out, workspace=ws)

        nvis = visible_keys_decode(w.S, w.window)
        flops = 4.0 * w.D * w.Hq * w.B * nvis
        tokens = w.B
        hbm_bytes = 2.0 * w.B * nvis * w.Hkv * w.D * 2   # K + V over visible rows
        if w.extra.get("kv") == "fp4":
            hbm_bytes = 2.0 * w.B * nvis * w.Hkv * (w.D // 2 + w.D // 32)
        kind = "decode"

    if args.warmup is None:
        # The GPU raises its clocks only under sustained load: a few milliseconds of warmup
        # times the kernels well below their steady-state speed (about 15 % slower for the
        # local prefill).  Warm up for 0.3 s, synchronising every 10 steps so that wall time
        # tracks GPU time.
        t0, n = time.perf_counter(), 0
        while n < 10 or time.perf_counter() - t0 < 0.3:
            step()
            n += 1
            if n % 10 == 0:
                torch.cuda.synchronize()
        args.warmup = n
    else:
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()
    # one event before every step and one after the last: the whole span gives ms_per_step, the
    # gaps give the median and minimum step
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record()
    for i in range(args.steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    timing = {"median_ms": round(per_step[len(per_step) // 2], 5), "min_ms": round(per_step[0], 5)}

    tflops = flops / (ms * 1e-3) / 1e12
    if w.kind in ("prefill", "backward"):
        value, unit = tflops, "TFLOP/s"
        if w.dtype == "bf16":
            roof = {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 5)}
        else:
            roof = {"bound": "alu", "achieved": round(tflops, 5), "peak": PEAK_FP32_VALU_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(tflops / PEAK_FP32_VALU_TFLOPS, 7)}
    else:
        gbs = hbm_bytes / (ms * 1e-3) / 1e9
        value, unit = gbs, "GB/s"
        roof = {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 5)}
    roof["traffic"] = profiled_traffic(w.name, kind)

    cfg = {"workload": w.name, "B": w.B, "kv_len" if w.kind == "decode" else "S": w.S,
           "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "window": w.window, "bias_range": w.bias_range,
           "bias": w.mode, "R": w.R if w.mode == "rproj" else None,
           "useful_gflop_per_step": round(flops / 1e9, 4), "tokens_per_step": tokens,
           "tokens_per_s": round(tokens / (ms * 1e-3), 1), "tflops": round(tflops, 3),
           "parallelism": "single-gpu"}
    if w.extra.get("page_size"):
        cfg["page_size"] = w.extra["page_size"]
    if w.temp_len:
        cfg["temp_len"] = w.temp_len
    if w.extra.get("kv"):
        cfg["kv_cache"] = "mxfp4"
    line = {"metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": w.dtype, "data": "synthetic (seeded, drawn on the GPU)", "config": cfg,
            "timing": timing, "roofline": roof}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
