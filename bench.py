"""Benchmark of the relative-position-bias attention hot path on one MI355X.

Default run: ONE JSON line whose headline is the long-context global prefill
(B1 S131072 Hq16/Hkv4 D128, full causal, table bias over distances < 1024,
NoPE beyond, bf16), the largest of the workloads, with the useful TFLOP/s
(4*D flops per visible (query head, key) pair), its MFMA roofline fraction and
the float64 oracle timed on this host's cores as a CPU baseline.  Under
"workloads" the same line carries every workload of the set, each timed in the
same run with its own roofline, tokens/s, oracle baseline and parity figures:

  tiny_local_f32       B1 H1 S256 D32, window 64, table bias (fp32)
  local_prefill        B2 S4096 H32/8 D128, window 512, r.E bias R=8
  global_prefill       B1 S32768 H32/8 D128, full causal, r.E bias below 1024
  long_global_prefill  (the headline)
  decode_global        B64 H32/8 D128, cache 65536, r.E bias below 1024
  decode_local         the same cache, window 512

Inputs are resident in HBM before the timed region; a step is one library call
(every kernel it launches), timed with events on the stream the kernels run on.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--no-cpu-baseline] [--cpu-seconds T]

--workload NAME times one workload alone (the profiling runs use this), also
the paged and MXFP4 decode variants (decode_global_paged, decode_local_paged,
decode_global_fp4, decode_local_fp4, decode_global_paged_fp4, decode_local_paged_fp4;
GB/s then counts the MXFP4 bytes) and the
backward passes (local_prefill_bwd, global_prefill_bwd,
long_global_prefill_bwd; 10*D algorithmic flops per visible pair).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "relbias-attn TFLOP/s + % bf16 MFMA peak (prefill); decode HBM GB/s %peak"
# MI355X published peaks: dense bf16 MFMA, fp32 vector, HBM3E
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_VALU_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
HEADLINE = "long_global_prefill"
WORKLOAD_SET = ["long_global_prefill", "tiny_local_f32", "local_prefill", "global_prefill",
                "decode_global", "decode_local"]
KERNEL_SOURCES = {
    "prefill": ["fwd_bf16.hip", "fwd_bf16_split.hip"],
    "decode": ["decode_bf16.hip"],
    "f32": ["attn_f32.hip"],
    "backward": ["bwd_bf16.hip"],
}
BF16_MAX_ABS, BF16_REL_L2, F32_TOL = 2e-2, 5e-3, 1e-5


def visible_pairs_prefill(S: int, window: int) -> int:
    """Number of (query, key) pairs with 0 <= i - j < window (window 0: i >= j)."""
    if window == 0 or window >= S:
        return S * (S + 1) // 2
    return window * (window + 1) // 2 + (S - window) * window


def visible_keys_row(i: int, window: int) -> int:
    return i + 1 if window == 0 else min(i + 1, window)


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


def device_info():
    """Name, compute units and peak clocks of cuda:0, read at run time."""
    import ctypes

    import torch
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "hbm_gib": round(p.total_memory / 2**30, 1)}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        val = ctypes.c_int(0)
        # hipDeviceAttributeClockRate (5) and hipDeviceAttributeMemoryClockRate (60), in kHz
        if hip.hipDeviceGetAttribute(ctypes.byref(val), 5, 0) == 0:
            info["peak_sclk_mhz"] = val.value // 1000
        if hip.hipDeviceGetAttribute(ctypes.byref(val), 60, 0) == 0:
            info["peak_mclk_mhz"] = val.value // 1000
    except OSError:
        pass
    if "peak_sclk_mhz" in info:
        # dense bf16 MFMA: 4 SIMDs x 1024 flops per clock per CU
        info["bf16_peak_from_clock_tflops"] = round(info["compute_units"] * 4096 * info["peak_sclk_mhz"] / 1e6, 1)
    return info


def host_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# ---------------------------------------------------------------------------------------------
# One workload: its step, its algorithmic work, its timing
# ---------------------------------------------------------------------------------------------

def setup(w, dev):
    """Inputs in HBM and a step function (one library call); returns (step, work dict)."""
    import torch

    import transformer_attention_learned_amd as rba
    from transformer_attention_learned_amd.workloads import make_inputs

    inp = make_inputs(w, device=dev)
    torch.cuda.synchronize()
    work = {"inputs": inp}
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

        work.update(flops=10.0 * w.D * w.Hq * w.B * visible_pairs_prefill(w.S, w.window),
                    tokens=w.B * w.S, hbm_bytes=None, kind="backward")
    elif w.kind == "prefill":
        out = torch.empty_like(inp["q"])
        lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=dev)
        need = rba.fwd_workspace_size(w.B, w.S, w.Hq, w.Hkv, w.D, dtype=w.dtype, window=w.window,
                                      bias_range=w.bias_range, mode=w.mode, R=w.R, scale=w.scale)
        fws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None

        def step():
            rba.fwd(inp["q"], inp["k"], inp["v"], window=w.window, bias_range=w.bias_range,
                    mode=w.mode, table=inp["table"], r=inp["r"], E=inp["E"], scale=w.scale,
                    temp_len=w.temp_len, out=out, lse=lse, workspace=fws)

        work.update(flops=4.0 * w.D * w.Hq * w.B * visible_pairs_prefill(w.S, w.window),
                    tokens=w.B * w.S, hbm_bytes=None, kind="prefill" if w.dtype == "bf16" else "f32",
                    out=out, lse=lse)
    else:
        out = torch.empty_like(inp["q"])
        need = rba.decode_workspace_size(w.B, w.Hq, w.Hkv, w.D, w.S, w.window)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        # A windowed step touches only window rows per sequence (134 MB for the local decode),
        # which would stay in the 256 MB Infinity Cache across steps; rotating over 4 cache
        # lengths makes consecutive steps read 4 disjoint windows, so the bytes come from HBM.
        kv_lens = [w.S - j * w.window for j in range(4)] if (w.window and 4 * w.window <= w.S) else [w.S]
        it = [0]
        if w.extra.get("kv") == "fp4" and w.extra.get("page_size"):
            # MXFP4 page pools: the quantised caches viewed as pages, scattered by the table
            from transformer_attention_learned_amd.workloads import paged_view
            kc, ks = rba.kv_quantize_fp4(inp["k"])
            vc, vs = rba.kv_quantize_fp4(inp["v"])
            kcp, vcp, bt = paged_view(w, kc, vc)
            ksp, vsp, bt2 = paged_view(w, ks, vs)
            torch.cuda.synchronize()
            assert torch.equal(bt, bt2)
            lens_t = [torch.full((w.B,), L, dtype=torch.int32, device=dev) for L in kv_lens]

            def step():
                j = it[0] % len(kv_lens)
                it[0] += 1
                rba.decode_fp4_paged(inp["q"], kcp, ksp, vcp, vsp, bt, lens_t[j], kv_lens[j],
                                     window=w.window, bias_range=w.bias_range, mode=w.mode,
                                     table=inp["table"], r=inp["r"], E=inp["E"], scale=w.scale,
                                     temp_len=w.temp_len, out=out, workspace=ws)
        elif w.extra.get("kv") == "fp4":
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
        hbm = 2.0 * w.B * nvis * w.Hkv * w.D * 2   # K + V over visible rows
        if w.extra.get("kv") == "fp4":
            hbm = 2.0 * w.B * nvis * w.Hkv * (w.D // 2 + w.D // 32)
        work.update(flops=4.0 * w.D * w.Hq * w.B * nvis, tokens=w.B, hbm_bytes=hbm, kind="decode",
                    out=out, kv_lens=kv_lens)
    return step, work


def time_steps(step, steps, warmup, min_warm_s=0.0):
    """W untimed steps (and, when min_warm_s > 0, more until that long has passed), then
    exactly `steps` timed steps between two events on the current stream.  A second pass of
    `steps` steps with an event after every step gives the per-step median and minimum (those
    events cost about 2 us per step, which shows only on the short decode steps, so the
    headline time comes from the first pass)."""
    import torch
    t0, n = time.perf_counter(), 0
    while n < warmup or time.perf_counter() - t0 < min_warm_s:
        step()
        n += 1
        if n % 10 == 0:
            torch.cuda.synchronize()   # keep wall time tracking GPU time
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return ms, n, {"median_ms": round(per[len(per) // 2], 5), "min_ms": round(per[0], 5),
                   "per_step_pass": "a second pass of the same number of steps, an event after each"}


def roofline(w, work, ms):
    if work["kind"] == "decode":
        gbs = work["hbm_bytes"] / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 5)}
        value, unit = gbs, "GB/s"
    else:
        tf = work["flops"] / (ms * 1e-3) / 1e12
        if w.dtype == "bf16":
            roof = {"bound": "mfma", "achieved": round(tf, 3), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 5)}
        else:
            roof = {"bound": "alu", "achieved": round(tf, 5), "peak": PEAK_FP32_VALU_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(tf / PEAK_FP32_VALU_TFLOPS, 7)}
        value, unit = tf, "TFLOP/s"
    roof["traffic"] = profiled_traffic(w.name, work["kind"])
    return value, unit, roof


def config_of(w, work, ms):
    cfg = {"workload": w.name, "B": w.B, "kv_len" if w.kind == "decode" else "S": w.S,
           "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "window": w.window, "bias_range": w.bias_range,
           "bias": w.mode, "R": w.R if w.mode in ("rproj", "rproj_shared") else None,
           "useful_gflop_per_step": round(work["flops"] / 1e9, 4),
           "tokens_per_step": work["tokens"],
           "tokens_per_s": round(work["tokens"] / (ms * 1e-3), 1),
           "tflops": round(work["flops"] / (ms * 1e-3) / 1e12, 3),
           "parallelism": "single-gpu"}
    if work["hbm_bytes"]:
        cfg["hbm_gb_per_step"] = round(work["hbm_bytes"] / 1e9, 5)
    if w.extra.get("page_size"):
        cfg["page_size"] = w.extra["page_size"]
    if w.temp_len:
        cfg["temp_len"] = w.temp_len
    if w.extra.get("kv"):
        cfg["kv_cache"] = "mxfp4"
    return cfg


# ---------------------------------------------------------------------------------------------
# The float64 oracle on a bounded sample of the same workload (CPU baseline + parity)
# ---------------------------------------------------------------------------------------------

def _sample_rows(S, Rb, seed, n_edge, n_rand):
    """First rows, rows around the bias range, last rows and seeded random rows, in an order that
    interleaves the four groups (a time-bounded prefix still covers all of them)."""
    import numpy as np
    rng = np.random.default_rng(seed)
    groups = [list(range(min(S, n_edge))),
              list(range(max(0, Rb - n_edge // 2), min(S, Rb + n_edge // 2))),
              list(range(max(0, S - n_edge), S)),
              sorted(rng.choice(S, size=min(S, n_rand), replace=False).tolist())]
    out, seen = [], set()
    for k in range(max(len(g) for g in groups)):
        for g in groups:
            if k < len(g) and g[k] not in seen:
                seen.add(g[k])
                out.append(g[k])
    return out


def _host64(t):
    """A device or host tensor as a float64 numpy array (copied to the host in its own dtype first)."""
    import torch
    return None if t is None else t.detach().cpu().to(torch.float64).numpy()


def cpu_baseline(w, work, seconds: float):
    """Time the float64 oracle (as it is) on a bounded sample of the workload, on a pool of host
    threads (one per core of this process's affinity mask, BLAS at one thread each), and compare
    the GPU output of the sampled rows with it.

    Prefill: items of (batch, kv group, row chunk) over all rows (small workloads) or over a fixed
    row sample (first rows, rows around the bias range, last rows, seeded random rows); decode:
    one item per sequence.  Items run until the time budget is spent; the rate counts the useful
    flops (4 D per visible pair) of the items done, and the time of the whole workload at that
    rate is labelled as extrapolated when the sample is not the whole workload.  Inputs reach the
    oracle as host float64 arrays converted before the clock starts."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle

    inp = work["inputs"]
    cores = host_cores()
    G = w.Hq // w.Hkv
    items = []          # (useful flops, fn); fn() -> (max |err|, sum err^2, sum ref^2, rows)
    if w.kind == "prefill":
        whole = w.B * w.S <= 8192
        rows = list(range(w.S)) if whole else _sample_rows(w.S, w.bias_range, w.seed, 512, 2048)
        chunk = 128 if whole else 8
        ridx = torch.as_tensor(rows, device=work["out"].device)
        o_gpu = _host64(work["out"][:, ridx])                      # [B, n_rows, Hq, D]
        pos = {r: n for n, r in enumerate(rows)}
        tab, E = _host64(inp["table"]), _host64(inp["E"])
        sl = {}
        for b in range(w.B):
            for g in range(w.Hkv):
                hs = slice(g * G, (g + 1) * G)
                sl[b, g] = (_host64(inp["q"][b:b + 1, :, hs]), _host64(inp["k"][b:b + 1, :, g:g + 1]),
                            _host64(inp["v"][b:b + 1, :, g:g + 1]),
                            None if inp["r"] is None else _host64(inp["r"][b:b + 1, :, hs]),
                            None if tab is None else tab[hs],
                            None if E is None else (E if w.mode == "rproj_shared" else E[hs]))

        def make(b, g, rr):
            def fn():
                q, k, v, r, t, e = sl[b, g]
                o, _ = oracle.prefill(q, k, v, scale=w.scale, temp_len=w.temp_len, window=w.window,
                                      bias_range=w.bias_range, mode=w.mode, table=t, r=r, E=e,
                                      rows=rr)
                got = o_gpu[b][[pos[int(i)] for i in rr]][:, g * G:(g + 1) * G]
                d = got - o[0]
                return float(np.abs(d).max()), float((d * d).sum()), float((o[0] ** 2).sum()), len(rr)
            return fn

        for c0 in range(0, len(rows), chunk):
            rr = np.array(rows[c0:c0 + chunk])
            fl = 4.0 * w.D * G * sum(visible_keys_row(int(i), w.window) for i in rr)
            for b in range(w.B):
                for g in range(w.Hkv):
                    items.append((fl, make(b, g, rr)))
    else:
        import transformer_attention_learned_amd as rba
        kv_len = w.S
        nvis = visible_keys_decode(kv_len, w.window)
        k0 = kv_len - nvis
        # the GPU output the sample is compared with: one more step at the full cache length
        o_gpu = _host64(rba.decode(inp["q"], inp["k"], inp["v"], kv_len, window=w.window,
                                   bias_range=w.bias_range, mode=w.mode, table=inp["table"],
                                   r=inp["r"], E=inp["E"], scale=w.scale, temp_len=w.temp_len))
        q64, r64 = _host64(inp["q"]), _host64(inp["r"])
        tab, E = _host64(inp["table"]), _host64(inp["E"])
        kpos = np.arange(k0, kv_len)

        def make(b):
            def fn():
                # the sequence's visible cache rows, converted inside the item (they are large)
                kb = _host64(inp["k"][b:b + 1, k0:kv_len])
                vb = _host64(inp["v"][b:b + 1, k0:kv_len])
                o, _ = oracle.attention(q64[b:b + 1][:, None], kb, vb, qpos=[kv_len - 1], kpos=kpos,
                                        scale=w.scale, temp_len=w.temp_len, window=w.window,
                                        bias_range=w.bias_range, mode=w.mode, table=tab,
                                        r=None if r64 is None else r64[b:b + 1][:, None], E=E)
                d = o_gpu[b] - o[0, 0]
                return float(np.abs(d).max()), float((d * d).sum()), float((o[0, 0] ** 2).sum()), 1
            return fn

        order = list(range(0, w.B, 2)) + list(range(1, w.B, 2))
        items = [(4.0 * w.D * w.Hq * nvis, make(b)) for b in order]

    done_fl, mx, se, sr, n_units, n_items = 0.0, 0.0, 0.0, 0.0, 0, 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=cores) as ex:
        pending, k = [], 0
        while True:
            while k < len(items) and len(pending) < 2 * cores and time.perf_counter() - t0 < seconds:
                pending.append((items[k][0], ex.submit(items[k][1])))
                k += 1
            if not pending:
                break
            fl, fut = pending.pop(0)
            a, b_, c_, n = fut.result()
            mx, se, sr = max(mx, a), se + b_, sr + c_
            done_fl += fl
            n_units += n
            n_items += 1
    t_total = time.perf_counter() - t0
    rate = done_fl / t_total
    complete = n_items == len(items)
    if w.kind == "prefill":
        if complete and whole:
            sample = f"the whole workload: all {w.S} rows of {w.B} x {w.Hkv} (batch, kv group) slices"
        else:
            sample = (f"{n_items} of {len(items)} (batch, kv group, {chunk}-row) items over a "
                      f"{len(rows)}-row sample (first rows, rows around the bias range, last rows, "
                      f"seeded random rows), {G} query heads each")
    else:
        sample = f"{n_items} of {w.B} sequences (even indices first), all heads, every visible key"
    res = {"value": rate / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
           "sample": sample, "seconds": round(t_total, 2),
           "threads": "one host thread per core of the affinity mask, BLAS at 1 thread each"}
    if not (complete and (w.kind != "prefill" or whole)):
        res["extrapolated_full_workload_s"] = round(work["flops"] / rate, 1)
    tol = (F32_TOL, F32_TOL) if w.dtype == "f32" else (BF16_MAX_ABS, BF16_REL_L2)
    rel = math.sqrt(se / sr) if sr > 0 else 0.0
    parity = {"max_abs": float(f"{mx:.3e}"), "rel_l2": float(f"{rel:.3e}"),
              "bar": {"max_abs": tol[0], "rel_l2": tol[1]},
              "pass": bool(mx <= tol[0] and rel <= tol[1]), "over": "the oracle's sample above"}
    return res, parity


def measure(w, dev, steps, warmup, min_warm_s, cpu_seconds):
    step, work = setup(w, dev)
    ms, nwarm, timing = time_steps(step, steps, warmup, min_warm_s)
    value, unit, roof = roofline(w, work, ms)
    entry = {"value": round(value, 3), "unit": unit, "ms_per_step": round(ms, 5), "steps": steps,
             "warmup": nwarm, "dtype": w.dtype, "config": config_of(w, work, ms), "timing": timing,
             "roofline": roof}
    if cpu_seconds > 0 and w.kind in ("prefill", "decode") and not w.extra:
        entry["cpu_baseline"], entry["parity"] = cpu_baseline(w, work, cpu_seconds)
    del work
    import torch
    torch.cuda.empty_cache()
    return entry


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps; default: as many as fill 0.3 s (at least 5), "
                         "long enough for the GPU clocks to settle at their sustained level")
    ap.add_argument("--workload", default=None,
                    help="time this workload alone (default: the headline plus the whole set)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU time budget of each workload's oracle sample")
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
    from transformer_attention_learned_amd.workloads import WORKLOADS

    dev = torch.device("cuda:0")
    rba.load_library()
    cpu_s = 0.0 if args.no_cpu_baseline else args.cpu_seconds
    warm = args.warmup if args.warmup is not None else 5
    min_warm = 0.3 if args.warmup is None else 0.0

    name = args.workload or HEADLINE
    w = WORKLOADS[name]
    head = measure(w, dev, args.steps, warm, min_warm, cpu_s)
    line = {"metric": METRIC, "value": head["value"], "unit": head["unit"], "n_gpus": 1,
            "steps": args.steps, "warmup": head["warmup"], "ms_per_step": head["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": w.dtype, "data": "synthetic (seeded, drawn on the GPU)",
            "config": head["config"], "timing": head["timing"], "roofline": head["roofline"]}
    for k in ("cpu_baseline", "parity"):
        if k in head:
            line[k] = head[k]
    if args.workload is None:
        # every workload of the set, timed after the headline (the clocks are settled by then);
        # each with at least the requested steps and warmup, more for the short ones
        entries = {HEADLINE: head}
        for nm in WORKLOAD_SET:
            if nm == HEADLINE:
                continue
            print(f"[bench] {nm}", file=sys.stderr, flush=True)
            wk = WORKLOADS[nm]
            entries[nm] = measure(wk, dev, max(args.steps, 50), warm, 0.2, cpu_s)
        line["workloads"] = entries
    line["device"] = device_info()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
