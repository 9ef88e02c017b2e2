#!/usr/bin/env python3
"""Benchmark of weight-absorbed MLA decode on one MI355X.

One step = one layer's decode attention over one batch: the split-KV decode
kernel and the log-sum-exp combine kernel, on a plan made once per decode step
(the plan is reused by every layer; its host time is reported as plan_ms).
Inputs are seeded synthetic bf16 tensors of the named workload, resident in HBM
before timing starts.  To measure HBM rather than the 256 MB last-level cache,
every step reads its own copy of the cache and queries (copies rotate, together
larger than 1 GB).

Prints ONE JSON line (value = algorithmic TFLOP/s of the whole step).

    python bench.py [--config mixed] [--steps 200] [--warmup 20] [--kv bf16|fp8]

With --kv fp8 the same workload runs over an FP8 cache (E4M3 codes with
per-token E8M0 scales; seeded codes of the same N(0, 1) draw) on the FP8
kernel, against the FP8 matrix peak.

With --layer a step is the whole attention of one decode layer around the
cache: the prolog (absorbed-query projection, RoPE, RMSNorm and the new rows
appended to the cache), the decode, the combine, the value up-projection and
the output projection (to DeepSeek-V3's 7168-wide hidden state);
value stays the attention's algorithmic TFLOP/s, now over the longer step, and
the prolog and up-projection report their own HBM rooflines (their weights
rotate over copies larger than the last-level cache, as each layer has its own).

HBM traffic evidence (roofline.traffic): rocprofv3 counter passes over this
script, one counter per pass, for the decode workload and for a plain device
copy of known size (--calibrate-copy), turned into profiles/traffic_<config>.json
by --traffic-from; the commands are listed in the profile summaries under
profiles/ (decode_<workload>_profile.md, decode_fp8_traffic_profile.md).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode attention TFLOP/s + HBM GB/s (% of roofline), H=128, 576-d latent"


#: the sources each decode kernel is built from (its file and what it includes)
KERNEL_SOURCES = {
    "bf16": ["mla_decode.hip", "device_common.h", "agpr_tiles.inc", "plan_internal.h", "decode_fp8.h"],
    "fp8": ["mla_decode_fp8.hip", "device_common.h", "agpr_tiles.inc", "agpr_tiles_fp8.inc", "plan_internal.h",
            "decode_fp8.h"],
}


def kernel_sha(kv: str = "bf16") -> str:
    """Hash of one decode kernel's sources: counters taken for another build are stale."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kv]:
        h.update(open(os.path.join(ROOT, "decode_attention_absorbed_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def traffic_name(config: str, kv: str) -> str:
    return config if kv == "bf16" else f"{config}_{kv}"


def load_traffic(config: str, kv: str):
    """HBM bytes per decode launch measured with rocprofv3 counters (see
    profiles/), or None if missing or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{traffic_name(config, kv)}.json")
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    if t.get("kernel_sha") != kernel_sha(kv):
        return None
    return t.get("decode_bytes_per_launch")


COPY_BYTES = 1 << 30  # calibration copy: 1 GiB read + 1 GiB written per launch
COPY_LAUNCHES = 5


def calibrate_copy() -> int:
    """Plain device-to-device copies of COPY_BYTES, the counters' yardstick."""
    import torch

    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(COPY_LAUNCHES):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": COPY_LAUNCHES}), flush=True)
    return 0


def _counter_per_dispatch(directory: str, counter: str, kernel_part: str) -> list:
    """Per-dispatch values (KiB) of one counter for kernels whose name contains kernel_part."""
    import csv

    vals = {}
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and kernel_part in r["Kernel_Name"]:
                key = (r.get("Agent_Id"), r["Dispatch_Id"])
                vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    return [vals[k] for k in sorted(vals, key=lambda k: int(k[1]))]


def traffic_from(config: str, fetch_dir: str, write_dir: str, copy_fetch_dir: str, copy_write_dir: str) -> int:
    """Turns the four counter passes into profiles/traffic_<config>.json."""
    import statistics

    def med(xs):
        if not xs:
            raise SystemExit("no counter rows found")
        return statistics.median(xs)

    # the copy kernel is the only kernel in the calibration run besides torch's fill
    cf = [v for v in _counter_per_dispatch(copy_fetch_dir, "FETCH_SIZE", "") if v > 0]
    cw = [v for v in _counter_per_dispatch(copy_write_dir, "WRITE_SIZE", "") if v > 0]
    cf_k, cw_k = max(cf), max(cw)
    f_fetch = COPY_BYTES / (cf_k * 1024.0)
    f_write = COPY_BYTES / (cw_k * 1024.0)
    kname = "decode_fp8_kernel" if config.endswith("_fp8") else "decode_kernel<"
    fetch = med(_counter_per_dispatch(fetch_dir, "FETCH_SIZE", kname))
    write = med(_counter_per_dispatch(write_dir, "WRITE_SIZE", kname))
    # both combine kernels (combine_kernel and combine_small_kernel)
    cfetch = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", "combine")
    cwrite = _counter_per_dispatch(write_dir, "WRITE_SIZE", "combine")
    res = {
        "config": config,
        "kernel_sha": kernel_sha("fp8" if config.endswith("_fp8") else "bf16"),
        "copy_bytes": COPY_BYTES,
        "copy_fetch_kib": cf_k,
        "copy_write_kib": cw_k,
        "fetch_factor": f_fetch,
        "write_factor": f_write,
        "decode_fetch_kib": fetch,
        "decode_write_kib": write,
        "decode_bytes_per_launch": fetch * 1024.0 * f_fetch + write * 1024.0 * f_write,
        "combine_bytes_per_launch": (med(cfetch) * 1024.0 * f_fetch + med(cwrite) * 1024.0 * f_write)
        if cfetch and cwrite else None,
    }
    path = os.path.join(ROOT, "profiles", f"traffic_{config}.json")
    with open(path, "w") as fh:
        json.dump(res, fh, indent=1)
        fh.write("\n")
    print(json.dumps(res), flush=True)
    return 0


def _oracle_threads() -> int:
    try:
        from threadpoolctl import threadpool_info

        return max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:
        return os.cpu_count() or 1


def _oracle_sample(x, arrays, seconds: float) -> tuple:
    """Runs the fp64 oracle on whole requests (longest first) until `seconds`
    of wall time are spent; returns (FLOPs done, seconds, requests done)."""
    import numpy as np

    from decode_attention_absorbed_amd import accounting as acc
    from oracle import mla_decode_ref

    cache, qn, qp = arrays
    done, flops, t0 = 0, 0, time.perf_counter()
    order = np.argsort(-x.seq_lens, kind="stable") if x.batch > 1 else np.arange(1)
    # whole passes over the workload repeat until the time is spent (a small
    # workload takes a fraction of a second per pass)
    while time.perf_counter() - t0 < seconds:
        for b in order:
            mla_decode_ref(qn[b : b + 1], qp[b : b + 1], cache, x.block_table[b : b + 1], x.seq_lens[b : b + 1],
                           x.softmax_scale)
            done += 1
            flops += acc.flops([int(x.seq_lens[b])], x.heads, x.q_len)
            if time.perf_counter() - t0 >= seconds:
                break
    return flops, time.perf_counter() - t0, done


def cpu_baseline(x, seconds: float, single_thread_seconds: float = 0.0) -> dict:
    """The fp64 oracle as it stands, timed on this host on a bounded sample of
    whole requests of the same workload, with every BLAS thread and (when
    single_thread_seconds > 0) with one."""
    arrays = (x.cache_f64(), x.q_nope_f64(), x.q_pe_f64())  # widened once, outside the timed samples
    flops, dt, done = _oracle_sample(x, arrays, seconds)
    res = {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(_oracle_threads()),
        "kind": "oracle",
        "sample": f"{done} requests of the {x.batch}-request workload, longest first, whole passes repeated "
                  f"(fp64 numpy, {dt:.1f} s)",
    }
    if single_thread_seconds > 0:
        try:
            from threadpoolctl import threadpool_limits

            with threadpool_limits(limits=1):
                f1, d1, n1 = _oracle_sample(x, arrays, single_thread_seconds)
            res["single_thread"] = {"value": f1 / d1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                                    "sample": f"{n1} requests, same order ({d1:.1f} s)"}
        except Exception as e:  # threadpoolctl missing: report why, keep the all-core figure
            res["single_thread"] = {"error": str(e)}
    return res


def _quantiles(xs: list) -> dict:
    xs = sorted(xs)
    q = lambda p: xs[min(len(xs) - 1, int(p * len(xs)))]
    return {"p10": q(0.1), "p50": q(0.5), "p90": q(0.9), "n": len(xs)}


def run(config: str, steps: int, warmup: int, cpu_seconds: float, kv: str = "bf16", diag: int = 100,
        cpu_single_seconds: float = 0.0, rescale: str = "lazy") -> dict:
    """One workload: `steps` decode steps (decode kernel + combine kernel)
    timed as one region between two HIP events on the launch stream, then
    diagnostics (`diag` individually timed steps, and bursts of each kernel
    alone) outside that region.  rescale = "pow2" runs the bf16 decode's
    power-of-two rescale form (mla_decode_variant) instead of mla_decode's."""
    import torch

    import decode_attention_absorbed_amd as mla
    from decode_attention_absorbed_amd import accounting as acc
    from decode_attention_absorbed_amd import binding as bnd
    from workloads import make_config, make_config_fp8

    dev = torch.device("cuda:0")
    fp8 = kv == "fp8"
    x = make_config_fp8(config) if fp8 else make_config(config)
    lens = [int(v) for v in x.seq_lens]
    roof = acc.roofline_seconds(lens, x.heads, x.q_len, x.page, kv)

    t = x.to_torch(dev)
    cache_t = t["cache_codes"] if fp8 else t["cache"]
    kv_bytes = cache_t.numel() * cache_t.element_size()
    # every step reads its own copy of the cache and queries: the copies
    # together exceed 1 GB, so repeats are not served by the 256 MB last-level cache
    copies = max(1, min(16, -(-(1 << 30) // max(kv_bytes, 1))))
    caches = [cache_t] + [cache_t.clone() for _ in range(copies - 1)]
    scales = ([t["cache_exps"]] + [t["cache_exps"].clone() for _ in range(copies - 1)]) if fp8 else None
    qns = [t["q_nope"]] + [t["q_nope"].clone() for _ in range(copies - 1)]
    qps = [t["q_pe"]] + [t["q_pe"].clone() for _ in range(copies - 1)]
    bt, sl = t["block_table"], t["seq_lens"]

    tp0 = time.perf_counter()
    plan = (bnd.mla_decode_fp8_plan if fp8 else mla.mla_decode_plan)(x.seq_lens, x.q_len, x.heads, x.page)
    plan_ms = (time.perf_counter() - tp0) * 1e3
    # re-planning in place (the per-step path of a serving loop), host time per call
    tp0 = time.perf_counter()
    for _ in range(20):
        plan.update(x.seq_lens)
    plan_update_ms = (time.perf_counter() - tp0) * 1e3 / 20
    torch.cuda.synchronize()
    B, H, q = x.batch, x.heads, x.q_len
    out = torch.empty((B, q, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((B, q, H), dtype=torch.float32, device=dev)
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=dev)
    L = mla.lib()
    stream = torch.cuda.current_stream(dev)
    variant = bnd.MLA_RESCALE_POW2 if rescale == "pow2" else bnd.MLA_RESCALE_LAZY
    if fp8 and variant != bnd.MLA_RESCALE_LAZY:
        raise ValueError("the power-of-two rescale form is a bf16 decode variant")

    def decode_variant(i, events_ptr=None):
        """decode + combine through mla_decode_variant"""
        c = i % copies
        bnd._check(L.mla_decode_variant(plan.handle, qns[c].data_ptr(), qps[c].data_ptr(), caches[c].data_ptr(),
                                        int(caches[c].shape[0]), bt.data_ptr(), int(bt.shape[1]), sl.data_ptr(),
                                        float(x.softmax_scale), out.data_ptr(), lse.data_ptr(), ws.data_ptr(),
                                        plan.workspace_bytes, variant, events_ptr, stream.cuda_stream))

    def partials(i):
        c = i % copies
        tail = (bt.data_ptr(), int(bt.shape[1]), sl.data_ptr(), float(x.softmax_scale), out.data_ptr(),
                lse.data_ptr(), ws.data_ptr(), plan.workspace_bytes, stream.cuda_stream)
        if fp8:
            bnd._check(L.mla_decode_fp8_partials(plan.handle, qns[c].data_ptr(), qps[c].data_ptr(), caches[c].data_ptr(),
                                                 scales[c].data_ptr(), int(caches[c].shape[0]), *tail))
        else:
            bnd._check(L.mla_decode_partials(plan.handle, qns[c].data_ptr(), qps[c].data_ptr(), caches[c].data_ptr(),
                                             int(caches[c].shape[0]), *tail))

    def combine(i=0, st=None):
        bnd._check(L.mla_decode_combine(plan.handle, out.data_ptr(), lse.data_ptr(), ws.data_ptr(), plan.workspace_bytes,
                                        (st or stream).cuda_stream))

    def step(i):
        if variant != bnd.MLA_RESCALE_LAZY:
            decode_variant(i)
            return
        partials(i)
        combine(i)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def graph_burst(fn, n):
        """n launches of fn captured once in a HIP graph, then one replay
        between two events on the launch stream: ms per launch."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cap = torch.cuda.current_stream()
            for i in range(n):
                fn(i, cap)
        torch.cuda.synchronize()
        g.replay()  # first replay uploads the graph
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        del g
        return a.elapsed_time(b) / n

    def burst(fn, n, offset=0):
        """n launches back to back between one pair of events: ms per launch."""
        a, b = ev(), ev()
        a.record(stream)
        for i in range(n):
            fn(offset + i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # The timed region: exactly `steps` steps between two events, nothing else
    # on the stream (markers between the kernels would add idle gaps).
    split = variant == bnd.MLA_RESCALE_LAZY
    w0 = time.perf_counter()
    ms_step = burst(step, steps)
    wall = time.perf_counter() - w0

    # Diagnostics, outside the timed region.
    # (1) `diag` steps timed one by one (each between its own events), for the spread;
    per_step = []
    for i in range(diag):
        a, b = ev(), ev()
        a.record(stream)
        step(i)
        b.record(stream)
        per_step.append((a, b))
    torch.cuda.synchronize()
    step_q = _quantiles([a.elapsed_time(b) for a, b in per_step])
    # (2) the combine kernel alone: `diag` launches captured in a HIP graph
    # and replayed between two events (a host-side burst of launches would be
    # bound by the launch rate, not by the kernel); and the decode kernel
    # alone, back to back.
    cmb_ms = graph_burst(combine, diag) if split and plan.workspace_bytes else 0.0
    dec_burst = burst(partials, diag) if split else None
    # (3) how often the online softmax rescaled O: one untimed call with the
    # rescale counter, against the (wave, tile) pairs the plan runs.
    rescale_rec = None
    if not fp8:
        events = torch.zeros(1, dtype=torch.int32, device=dev)
        decode_variant(0, events.data_ptr())
        torch.cuda.synchronize()
        seg = plan.segments()
        nrb = plan.query(bnd.MLA_Q_NUM_ROW_BLOCKS)
        wave_tiles = int(sum(-(-(int(e) - int(s0)) // 32) for s0, e in zip(seg[:, 1], seg[:, 2]))) * 4 * nrb
        ev_n = int(events.item())
        rescale_rec = {"form": rescale, "events": ev_n, "wave_tiles": wave_tiles,
                       "per_1000_wave_tiles": 1000.0 * ev_n / max(wave_tiles, 1)}
    # The decode kernel's duration for the roofline: the timed step minus the
    # combine kernel's time, so that decode + combine never exceeds the step
    # (rocprofv3's kernel trace of the same command gives the decode duration
    # to compare with).  The variant entry point runs both kernels in one
    # call: there the whole step stands in.
    if split:
        dec_ms = max(ms_step - cmb_ms, 1e-9)
    else:
        dec_ms, cmb_ms = ms_step, None

    flops = roof["flops"]
    nbytes = roof["bytes"]
    bound = roof["bound"]
    if bound == "hbm":
        achieved = nbytes / (dec_ms * 1e-3) / 1e9
        peak, unit = acc.PEAK_HBM_BYTES_PER_S / 1e9, "GB/s"
    else:
        achieved = flops / (dec_ms * 1e-3) / 1e12
        peak, unit = (acc.PEAK_FP8_FLOPS if fp8 else acc.PEAK_BF16_FLOPS) / 1e12, "TFLOP/s"
    traffic = load_traffic(config, kv)
    res = {
        "metric": METRIC,
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if fp8 else "bf16",
        "data": ("synthetic (seeded N(0,1) bf16 queries, E4M3 cache codes of N(0,1) draws with per-token E8M0 "
                 "scales, random page permutation)") if fp8 else "synthetic (seeded N(0,1) bf16, random page permutation)",
        "config": {
            "workload": config if not fp8 else f"{config}-fp8",
            "kv_dtype": kv,
            "batch": B,
            "heads": H,
            "q_len": q,
            "page": x.page,
            "seq_len": lens[0] if len(set(lens)) == 1 else f"{min(lens)}..{max(lens)}",
            "kv_tokens": int(sum(lens)),
        },
        "hbm_gbps": nbytes / (ms_step * 1e-3) / 1e9,
        "tflops": flops / (ms_step * 1e-3) / 1e12,
        "roofline": {
            "bound": bound,
            "achieved": achieved,
            "peak": peak,
            "unit": unit,
            "frac": achieved / peak,
            "traffic": traffic,
            "kernel": "decode_fp8_kernel" if fp8 else "decode_kernel",
            "duration_ms": dec_ms,
            "duration_source": ("timed step minus the combine kernel's time (HIP graph replay of back-to-back "
                                "combine launches)" if split else "whole timed step (decode and combine in one call)"),
        },
        "step_roofline_frac": roof["t_bound"] / (ms_step * 1e-3),
        "step_ms_quantiles": step_q,
        "decode_kernel_ms": dec_ms,
        "decode_kernel_burst_ms": dec_burst,
        "combine_kernel_ms": cmb_ms,
        "plan_ms": plan_ms,
        "plan_update_ms": plan_update_ms,
        "wall_ms_per_step": wall * 1e3 / steps,
        "algorithmic_flops": flops,
        "algorithmic_bytes": nbytes,
        "roofline_ms": roof["t_bound"] * 1e3,
        "input_copies": copies,
        "num_workgroups": plan.query(bnd.MLA_Q_NUM_WORKGROUPS),
        "num_partials": plan.query(bnd.MLA_Q_NUM_PARTIALS),
        "rescale": rescale_rec,
        "kernel_sha": kernel_sha(kv),
    }
    res["cpu_baseline"] = cpu_baseline(x, cpu_seconds, cpu_single_seconds) if cpu_seconds > 0 else None
    del caches, qns, qps, scales, t
    torch.cuda.empty_cache()
    return res


#: keys of a workload record that a sub-record repeats (the rest is headline-only)
SUB_KEYS = ["value", "unit", "ms_per_step", "dtype", "config", "hbm_gbps", "tflops", "roofline", "step_roofline_frac",
            "step_ms_quantiles", "decode_kernel_ms", "decode_kernel_burst_ms", "combine_kernel_ms", "plan_ms", "plan_update_ms",
            "roofline_ms", "algorithmic_flops", "algorithmic_bytes", "num_workgroups", "num_partials", "rescale",
            "cpu_baseline"]


def run_layer(config: str, steps: int, warmup: int, kv: str = "bf16") -> dict:
    """The prolog + decode + combine + up-projection + output projection step (see the module notes)."""
    import torch

    import decode_attention_absorbed_amd as mla
    from decode_attention_absorbed_amd import accounting as acc
    from decode_attention_absorbed_amd import binding as bnd
    from workloads import CONFIGS, make_config, make_config_fp8, make_prolog_inputs

    dev = torch.device("cuda:0")
    fp8 = kv == "fp8"
    x = make_config_fp8(config) if fp8 else make_config(config)
    pi = make_prolog_inputs(x.batch, x.q_len, x.heads, x.seq_lens, seed=CONFIGS[config]["seed"] + 100,
                            hidden=acc.HIDDEN)
    lens = [int(v) for v in x.seq_lens]
    roof = acc.roofline_seconds(lens, x.heads, x.q_len, x.page, kv)
    B, H, q = x.batch, x.heads, x.q_len
    M = B * q

    def bf16(a):
        return torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)

    t = x.to_torch(dev)
    cache_t = t["cache_codes"] if fp8 else t["cache"]
    copies = max(1, min(16, -(-(1 << 30) // (cache_t.numel() * cache_t.element_size()))))
    caches = [cache_t] + [cache_t.clone() for _ in range(copies - 1)]
    scales = ([t["cache_exps"]] + [t["cache_exps"].clone() for _ in range(copies - 1)]) if fp8 else None
    wcopies = 16  # 16 x 16.8 MB per weight: past the 256 MB last-level cache
    wuk = [bf16(pi.w_uk_t)] + [None] * (wcopies - 1)
    wuv = [bf16(pi.w_uv)] + [None] * (wcopies - 1)
    for i in range(1, wcopies):
        wuk[i], wuv[i] = wuk[0].clone(), wuv[0].clone()
    ocopies = 4  # 4 x 235 MB of W_O
    wo = [bf16(pi.w_o)]
    wo += [wo[0].clone() for _ in range(ocopies - 1)]
    N_o, K_o = int(pi.w_o.shape[0]), int(pi.w_o.shape[1])
    y = torch.empty((B, q, N_o), dtype=torch.bfloat16, device=dev)
    ows_bytes = bnd.mla_o_project_workspace_bytes(B, q, K_o, N_o)
    ows = torch.empty(max(ows_bytes, 16), dtype=torch.uint8, device=dev)
    qn128, qpr, ckv, nw, kpe = (bf16(a) for a in (pi.q_nope128, pi.q_pe_raw, pi.c_kv_raw, pi.kv_norm_w, pi.k_pe_raw))
    table = torch.from_numpy(pi.rope_cos_sin).to(dev)
    bt, sl = t["block_table"], t["seq_lens"]
    plan = (bnd.mla_decode_fp8_plan if fp8 else mla.mla_decode_plan)(x.seq_lens, q, H, x.page)
    q_abs = torch.empty((B, q, H, 512), dtype=torch.bfloat16, device=dev)
    q_pe = torch.empty((B, q, H, 64), dtype=torch.bfloat16, device=dev)
    out = torch.empty((B, q, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((B, q, H), dtype=torch.float32, device=dev)
    o = torch.empty((B, q, H, 128), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=dev)
    L = mla.lib()
    stream = torch.cuda.current_stream(dev)
    s = stream.cuda_stream

    def prolog(i):
        c = i % copies
        bnd._check(L.mla_prolog(B, q, H, qn128.data_ptr(), qpr.data_ptr(), wuk[i % wcopies].data_ptr(), ckv.data_ptr(),
                                nw.data_ptr(), pi.rms_eps, kpe.data_ptr(), table.data_ptr(), int(table.shape[0]),
                                sl.data_ptr(), bt.data_ptr(), int(bt.shape[1]), int(caches[c].shape[0]), x.page,
                                bnd.MLA_KV_FP8 if fp8 else bnd.MLA_KV_BF16, caches[c].data_ptr(),
                                scales[c].data_ptr() if fp8 else None, q_abs.data_ptr(), q_pe.data_ptr(), s))

    def attend(i):
        c = i % copies
        tail = (bt.data_ptr(), int(bt.shape[1]), sl.data_ptr(), float(x.softmax_scale), out.data_ptr(),
                lse.data_ptr(), ws.data_ptr(), plan.workspace_bytes, s)
        if fp8:
            bnd._check(L.mla_decode_fp8(plan.handle, q_abs.data_ptr(), q_pe.data_ptr(), caches[c].data_ptr(),
                                        scales[c].data_ptr(), int(caches[c].shape[0]), *tail))
        else:
            bnd._check(L.mla_decode(plan.handle, q_abs.data_ptr(), q_pe.data_ptr(), caches[c].data_ptr(),
                                    int(caches[c].shape[0]), *tail))

    def up(i):
        bnd._check(L.mla_up_project(B, q, H, out.data_ptr(), wuv[i % wcopies].data_ptr(), o.data_ptr(), s))

    def oproj(i):
        bnd._check(L.mla_o_project(B, q, K_o, N_o, o.data_ptr(), wo[i % ocopies].data_ptr(), y.data_ptr(),
                                   ows.data_ptr(), ows_bytes, s))

    for i in range(warmup):
        prolog(i)
        attend(i)
        up(i)
        oproj(i)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(steps):
        prolog(i)
        attend(i)
        up(i)
        oproj(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps

    def burst(fn):
        n = max(steps, 20)
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record(stream)
        for i in range(n):
            fn(i)
        b1.record(stream)
        torch.cuda.synchronize()
        return b0.elapsed_time(b1) / n

    pro_ms, att_ms, up_ms, op_ms = burst(prolog), burst(attend), burst(up), burst(oproj)

    def hbm(nbytes, ms):
        a = nbytes / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": a, "peak": acc.PEAK_HBM_BYTES_PER_S / 1e9, "unit": "GB/s",
                "frac": a / (acc.PEAK_HBM_BYTES_PER_S / 1e9), "bytes": nbytes, "duration_ms": ms}

    return {
        "metric": METRIC,
        "value": roof["flops"] / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if fp8 else "bf16",
        "data": "synthetic (seeded N(0,1) bf16 activations, N(0, 1/fan-in) bf16 weights, random page permutation)",
        "config": {"workload": f"{config}{'-fp8' if fp8 else ''}-layer", "kv_dtype": kv, "batch": B, "heads": H,
                   "q_len": q, "page": x.page, "kv_tokens": int(sum(lens)),
                   "hidden": N_o, "steps_in_step": "prolog + decode + combine + up-projection + output projection"},
        "prolog_ms": pro_ms,
        "attention_ms": att_ms,
        "up_project_ms": up_ms,
        "prolog_roofline": hbm(acc.prolog_bytes(M, H, kv), pro_ms),
        "up_project_roofline": hbm(acc.up_project_bytes(M, H), up_ms),
        "o_project_ms": op_ms,
        "o_project_roofline": hbm(acc.o_project_bytes(M, H, N_o), op_ms),
        "attention_share": att_ms / (pro_ms + att_ms + up_ms + op_ms),
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="mixed", help="headline workload: tiny | dsv3 | mtp | mixed | long | mtp4 | mtp8")
    ap.add_argument("--subrecords", default="tiny,dsv3,mtp,long,mtp4,mtp8",
                    help="other workloads measured into the same JSON line (comma list; empty for none)")
    ap.add_argument("--diag", type=int, default=100, help="individually timed steps and kernel bursts per workload")
    ap.add_argument("--kv", default="bf16", choices=["bf16", "fp8"], help="cache format (bf16: the headline; fp8: E4M3 + E8M0)")
    ap.add_argument("--layer", action="store_true",
                    help="time prolog + decode + combine + up-projection + output projection per step")
    ap.add_argument("--rescale", default="lazy", choices=["lazy", "pow2"],
                    help="bf16 O-rescale form: lazy (mla_decode) or pow2 (the power-of-two variant)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle sample of the headline workload (all cores)")
    ap.add_argument("--cpu-single-seconds", type=float, default=5.0, help="same sample with one BLAS thread")
    ap.add_argument("--sub-cpu-seconds", type=float, default=2.0, help="oracle sample per sub-record (each thread setting)")
    ap.add_argument("--calibrate-copy", action="store_true", help="run the plain copy the traffic counters are scaled by")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write profiles/traffic_<config>.json from rocprofv3 counter output (no GPU needed)")
    args = ap.parse_args()
    if args.traffic_from:
        return traffic_from(traffic_name(args.config, args.kv), *args.traffic_from)
    if args.calibrate_copy:
        return calibrate_copy()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the decode shards by request; "
              "see the design notes). Run with --gpus 1.", file=sys.stderr)
        return 2
    if args.layer:
        print(json.dumps(run_layer(args.config, args.steps, args.warmup, args.kv)), flush=True)
        return 0
    cpu = not args.no_cpu_baseline and args.kv == "bf16"
    subs = {}
    for name in [n for n in args.subrecords.split(",") if n and n != args.config]:
        r = run(name, max(20, args.steps // 4), args.warmup, args.sub_cpu_seconds if cpu else 0.0, args.kv, args.diag,
                args.sub_cpu_seconds if cpu else 0.0, args.rescale)
        subs[name] = {k: r[k] for k in SUB_KEYS}
        print(f"# {name}: {r['ms_per_step'] * 1e3:.2f} us/step, decode {r['decode_kernel_ms'] * 1e3:.2f} us, "
              f"roofline frac {r['roofline']['frac']:.3f}", file=sys.stderr, flush=True)
    res = run(args.config, args.steps, args.warmup, args.cpu_seconds if cpu else 0.0, args.kv, args.diag,
              args.cpu_single_seconds if cpu else 0.0, args.rescale)
    res["configs"] = subs
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
