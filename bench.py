"""Benchmark of the verify pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config qwen3-4b] ...

Workload (default): one Qwen3-4B-shaped decoder layer (q 4096x2560, k/v
1024x2560, o 2560x4096, gate/up 9728x2560, down 2560x9728) plus the
151936x2560 vocabulary head, 8-bit affine group-64 weights, bf16 N(0,1) rows,
greedy acceptance of drafts that match the target's token with probability
0.7 per position.  One step = one verify round at each width
M = 1, 2, 4, 6, 8, 12, 16 (the verify-cost curve); each round is
  4 projection launches per layer + head/argmax with the greedy acceptance in
  its last workgroup (one launch; sampling rounds launch the accept kernels
  after the head), which write the result to pinned host memory directly;
  the host waits for the result words themselves (no copy launch, no stream
  sync),
launched from the host with arguments marshalled once per width and weight
copy (--graph replays HIP graphs of the same calls instead).

Other workloads of the same path:
  --config dense-27b --layers 64 --sweep 17 --copies 1 --accept sample
        64 resident 27B-shaped layers, M = 17, speculative sampling at T = 1
        against draft distributions q = softmax(target logits + N(0, 0.5));
        add --top-k 50 --top-p 0.9 --presence 0.5 --frequency 0.1 for the
        truncated, penalised rule (history counts of a seeded 4096-token
        Zipf-like history; drafts drawn from the untruncated q);
  --config ornith-9b --bits 2|3|4|8|16 --sweep 1,2,...,16
        the 9B-shaped layer and 151936x4096 head per weight format;
  --config qwen3-8b --batch 4 --sweep 6 --alpha 0.3,0.5,0.7,0.9
        four requests of six rows in one launch, greedy accept per request.

  --prefill 2048 [--bits 4]
        the prefill workload: one layer's seven projections over 2048 prompt
        rows (dspk_qgemm_prefill) plus the head on the last row, in TFLOP/s
        against the bf16 matrix-core peak.

Printed: one JSON line with the whole-job weight-GB/s (weight bytes of every
round / wall time of the timed steps, which run with no timing events), the
per-width curve t(M)/t(1) and the roofline of the dominant kernel (the
vocabulary head) from a second, event-instrumented pass over the same steps,
and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published
SWEEP = (1, 2, 4, 6, 8, 12, 16)


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="qwen3-4b", choices=["qwen3-4b", "qwen3-8b", "ornith-9b", "dense-27b"])
    ap.add_argument("--bits", type=int, default=8, choices=[2, 3, 4, 8, 16])
    ap.add_argument("--layers", type=int, default=1)
    ap.add_argument("--copies", type=int, default=3, help="rotating weight copies (defeat the 256 MB MALL)")
    ap.add_argument("--sweep", default=",".join(map(str, SWEEP)), help="rows per request, one round each")
    ap.add_argument("--batch", type=int, default=1, help="requests verified together in one launch")
    ap.add_argument("--alpha", default="0.7", help="per-position draft match rate (one per request)")
    ap.add_argument("--accept", default="greedy", choices=["greedy", "sample"])
    ap.add_argument("--temperature", type=float, default=1.0)
    ap.add_argument("--noise", type=float, default=0.5, help="std of the drafter's logit noise (sampling)")
    ap.add_argument("--top-k", type=int, default=0, help="sampling: top-k truncation of target and draft (0: off)")
    ap.add_argument("--top-p", type=float, default=1.0, help="sampling: nucleus truncation (1: off)")
    ap.add_argument("--presence", type=float, default=0.0, help="sampling: presence penalty")
    ap.add_argument("--frequency", type=float, default=0.0, help="sampling: frequency penalty")
    ap.add_argument("--history", type=int, default=4096, help="sampling with penalties: history length (tokens)")
    ap.add_argument("--prefill", type=int, default=0,
                    help="prefill workload instead: one layer's projections over this many prompt rows "
                         "(dspk_qgemm_prefill) plus the head on the last row")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--variant-curves", action="store_true",
                    help="instead: t(M) of each Qwen3-4B projection launch under each forced decomposition "
                         "(stream-K and slab on the matrix cores, slab with vector-ALU dot products)")
    ap.add_argument("--draft-sets", type=int, default=8,
                    help="independent draft sets per (width, weight copy); rounds cycle through them")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the streaming probe and the 27B-shaped layer + head section")
    ap.add_argument("--cpu-sample-s", type=float, default=20.0)
    ap.add_argument("--graph", action="store_true",
                    help="replay each round as HIP graphs (layers, head, accept) captured once per width and "
                         "weight copy, instead of host launches with pre-marshalled arguments")
    ap.add_argument("--calibrate", action="store_true",
                    help="after the timed region, run one plain device copy of 256 MiB (the reference "
                         "dispatch for scaling hardware byte counters)")
    return ap.parse_args(argv)


def host_cpu() -> dict:
    """The host's CPU model and numpy's BLAS library, for the CPU baseline."""
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = ""
    try:
        cfg = np.show_config(mode="dicts")
        blas = cfg.get("Build Dependencies", {}).get("blas", {}).get("name", "")
    except Exception:     # older numpy: no dict form
        pass
    return {"cpu_model": model, "blas": blas}


def device_info() -> dict:
    """What the numbers were measured on: the device's name, architecture,
    compute units, clock and memory, the HIP runtime torch was built with,
    and the library's version."""
    import torch
    from speculative_decoding_verify_dspk_amd import binding
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2 ** 30, 1), "hip": torch.version.hip,
            "torch": torch.__version__, "dspk_version": binding.version()}
    clock = getattr(p, "clock_rate", None)
    if clock:
        info["clock_mhz"] = round(clock / 1000)
    return info


def cpu_baseline(model: str, bits: int, m: int, budget_s: float):
    """The oracle, as it stands, on one verify round of the same workload:
    every projection of one layer at width m, then as many 8192-entry slices
    of the vocabulary head as fit the time budget.  Reported in weight-GB/s."""
    import oracle
    from speculative_decoding_verify_dspk_amd import inputs
    shapes = inputs.LAYER_SHAPES[model]
    threads = len(os.sched_getaffinity(0))
    done_bytes, t_total = 0, 0.0
    projs = inputs.layer_projections(model)
    acts = {}
    for name, n, k, src in projs:
        w = inputs.make_qweight(n, k, bits, "cpu-baseline", model, name, keep_codes=False)
        x = acts.setdefault((src, k), inputs.make_activations(m, k, "cpu-baseline", src))
        t0 = time.perf_counter()
        oracle.qlinear(x, w.codes, w.scales, w.biases, bits, n, k)
        t_total += time.perf_counter() - t0
        done_bytes += inputs.weight_bytes(n, k, bits)
    v, h = shapes["vocab"], shapes["hidden"]
    hx = inputs.make_activations(m, h, "cpu-baseline", "h")
    slices = 0
    sl = 8192
    while t_total < budget_s and slices * sl < v:
        n = min(sl, v - slices * sl)
        w = inputs.make_qweight(n, h, bits, "cpu-baseline", "head", slices, keep_codes=False)
        t0 = time.perf_counter()
        z = oracle.qlinear(hx, w.codes, w.scales, w.biases, bits, n, h)
        oracle.argmax_lowest(z)
        t_total += time.perf_counter() - t0
        done_bytes += inputs.weight_bytes(n, h, bits)
        slices += 1
    return {"value": round(done_bytes / t_total / 1e9, 4), "unit": "weight-GB/s", "cores": threads,
            "kind": "oracle", **host_cpu(),
            "sample": f"one {model} layer (7 projections) + {slices} x {sl}-row slices of the {v}x{h} head, "
                      f"{bits}-bit, M={m}; {done_bytes / 1e6:.1f} MB of weights in {t_total:.1f} s "
                      f"(numpy fp64, {threads} threads)"}


def measured_traffic():
    """HBM bytes per launch of the head kernel from the committed hardware-
    counter summary, if it was taken on the current kernel sources (else None)."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    summary = os.path.join(here, "profiles", "vocab_head_traffic.txt")
    csrc = os.path.join(here, "speculative_decoding_verify_dspk_amd", "csrc")
    srcs = [os.path.join(csrc, f) for f in ("qgemm.hip", "decode.h", "dspk_internal.h")]
    if not os.path.exists(summary):
        return None
    kv = {}
    for line in open(summary):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            kv[k.strip()] = v.strip()
    sha = hashlib.sha256(b"".join(open(f, "rb").read() for f in srcs)).hexdigest()
    if kv.get("kernel_source_sha256") != sha:
        return None
    try:
        return int(float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


MFMA_BF16_PEAK_TFS = 2500.0   # MI355X dense bf16 matrix peak, published

PENDING = -12345   # no accept_len or committed entry ever takes this value


def wait_result(res_np, stream, spin_s: float = 2.0):
    """Wait for a round's result by watching its pinned buffer: the
    acceptance writes every accept_len and committed entry exactly once, so
    the round is complete (for the host) once no entry still holds PENDING,
    whatever order the writes arrive in.  After spin_s of spinning, fall back
    to a stream sync and fail if an entry is still missing."""
    t0 = time.perf_counter()
    while (res_np == PENDING).any():
        if time.perf_counter() - t0 > spin_s:
            stream.synchronize()
            if (res_np == PENDING).any():
                raise RuntimeError("bench.py: a round's result never arrived in host memory")
            break


def prefill_bench(args):
    """Prefill workload: one decoder layer's seven projections over P prompt
    rows through dspk_qgemm_prefill, then the vocabulary head on the last row
    only (dspk_lmhead_argmax with m = 1).  One step = one such pass; the
    metric is MFMA throughput (the wide-row regime is bound by the matrix
    cores, not by HBM)."""
    import gc
    import torch
    from speculative_decoding_verify_dspk_amd import binding, inputs
    binding.lib()
    P = args.prefill
    s = inputs.LAYER_SHAPES[args.config]
    H, Q, KV, F, V = s["hidden"], s["q"], s["kv"], s["inter"], s["vocab"]
    projs = [("q", Q, H), ("k", KV, H), ("v", KV, H), ("o", H, Q), ("gate", F, H), ("up", F, H), ("down", H, F)]
    calls, ev_pairs, flops = [], [], 0
    keep = []
    # one workspace for every projection (calls ordered on one stream): the
    # launches with few output blocks split K through it
    wsp = binding.alloc_workspace(max(binding.prefill_workspace_bytes(n, k, P, args.bits) for _, n, k in projs))
    for name, n, k in projs:
        c, sc, bi = inputs.make_qweight_device(n, k, args.bits, args.config, "prefill", name)
        w = binding.DeviceQWeight(n, k, args.bits, c, sc, bi)
        x = inputs.make_activations_rowmajor_device(P, k, args.config, "prefill", name)
        y = torch.empty((P, n), dtype=torch.float32, device="cuda")
        calls.append((name, binding.prepare_qgemm_prefill(w, x, P, y, wsp)))
        keep += [w, x, y, c, sc, bi]
        flops += 2 * P * n * k
    c, sc, bi = inputs.make_qweight_device(V, H, args.bits, args.config, "prefill", "head")
    head = binding.DeviceQWeight(V, H, args.bits, c, sc, bi)
    hlast = inputs.make_activations_device(1, H, args.config, "prefill", "last")
    am = torch.empty((1,), dtype=torch.int32, device="cuda")
    wsh = binding.alloc_workspace(binding.lmhead_workspace_bytes(V, 1))
    head_call = binding.prepare_lmhead(head, hlast, 1, am, None, wsh)
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)   # noqa: E731

    def step(rec):
        e = [ev() for _ in range(len(calls) + 2)] if rec is not None else None
        if e: e[0].record(stream)
        for i, (_, f) in enumerate(calls):
            f()
            if e: e[i + 1].record(stream)
        head_call()
        if e:
            e[-1].record(stream)
            rec.append(e)

    for _ in range(args.warmup):
        step(None)
    gc.collect()
    gc.freeze()
    torch.cuda.synchronize()
    recs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(recs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {name: float(np.median([r[i].elapsed_time(r[i + 1]) for r in recs])) * 1e3
           for i, (name, _) in enumerate(calls)}
    head_us = float(np.median([r[-2].elapsed_time(r[-1]) for r in recs])) * 1e3
    proj_us = sum(per.values())
    # dominant kernel: the gate projection (largest), algorithmic flops / its mean launch time
    gate_us = float(np.mean([r[4].elapsed_time(r[5]) for r in recs])) * 1e3
    gate_flops = 2 * P * F * H
    achieved = gate_flops / (gate_us * 1e-6) / 1e12
    value = flops * args.steps / wall / 1e12
    lib_tfs = library_bf16_gemm_tflops(P, F, H)
    out = {
        "metric": "prefill projection throughput (TFLOP/s) over a prompt",
        "value": round(value, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.config} layer (7 projections) over {P} prompt rows + lm_head {V}x{H} "
                               f"on the last row, {'bf16' if args.bits == 16 else str(args.bits) + '-bit g64'}"},
        "per_projection_us": {k2: round(v2, 1) for k2, v2 in per.items()},
        "projections_us": round(proj_us, 1), "last_row_head_us": round(head_us, 1),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFS, 4), "traffic": None,
                     "kernel": f"prefill_kernel<{args.bits}> (gate projection {F}x{H})",
                     "avg_launch_us": round(gate_us, 2), "flops_per_launch": gate_flops},
        # context: the box's own library GEMM (torch.matmul, bf16 in and out)
        # on the gate shape; the quantised kernel's share of it is the
        # figure comparable with a wide-GEMM's fraction of a bf16 GEMM
        "library_bf16_gemm": {"tflops": round(lib_tfs, 1), "shape": f"{P}x{H} @ {H}x{F}",
                              "gate_fraction": round(achieved / lib_tfs, 3)},
        "cpu_baseline": None if args.no_cpu_baseline else prefill_cpu_baseline(args.config, args.bits, P),
        "device": torch.cuda.get_device_name(0), "device_info": device_info(), "host": platform.node(),
    }
    print(json.dumps(out))


def library_bf16_gemm_tflops(p: int, n: int, k: int, reps: int = 20) -> float:
    """TFLOP/s of torch.matmul (the ROCm BLAS library) on a plain bf16
    [p, k] x [k, n] product, both operands contiguous, timed with events."""
    import torch
    a = torch.randn(p, k, device="cuda").to(torch.bfloat16)
    b = torch.randn(k, n, device="cuda").to(torch.bfloat16).contiguous()
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    return 2.0 * p * n * k * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12


def prefill_cpu_baseline(model: str, bits: int, rows: int, budget_s: float = 15.0):
    """The oracle's x . deq(W)^T on the gate projection's shape, on as many
    32-row slices of the prompt as fit the budget, in TFLOP/s."""
    import oracle
    from speculative_decoding_verify_dspk_amd import inputs
    s = inputs.LAYER_SHAPES[model]
    n, k = s["inter"], s["hidden"]
    w = inputs.make_qweight(n, k, bits, "cpu-baseline", model, "prefill-gate", keep_codes=False)
    done = 0
    t0 = time.perf_counter()
    while done < rows and time.perf_counter() - t0 < budget_s:
        x = inputs.make_activations(32, k, "cpu-baseline", model, "prefill", done)
        oracle.qlinear(x, w.codes, w.scales, w.biases, bits, n, k)
        done += 32
    t = time.perf_counter() - t0
    return {"value": round(2 * done * n * k / t / 1e12, 6), "unit": "TFLOP/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle", "sample": f"{done} of {rows} prompt rows through the {n}x{k} gate projection, "
                                        f"{bits}-bit, in {t:.1f} s"}


def achievable_bandwidth(nbytes: int, reps: int = 12):
    """In-process streaming-read probe (libdspk_probe.so): the best rate at
    which this device streams `nbytes` from HBM with the projection kernels'
    access pattern (16 B per lane, 1 KiB per wave instruction, non-temporal),
    rotating three buffers so the 256 MB MALL cannot serve a repeat.  Timed
    with HIP events on the launch stream; best over a few grid sizes."""
    import ctypes
    import torch
    from speculative_decoding_verify_dspk_amd import build as _b
    if not os.path.exists(_b.PROBE_LIB):
        return None
    lib = ctypes.CDLL(_b.PROBE_LIB)
    f = lib.dspk_probe_stream_read
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    nb = (nbytes + 1023) // 1024 * 1024
    bufs = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(3)]
    for b in bufs:
        b.fill_(1)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(8 * cus, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    best = None
    for grid in (2 * cus, 4 * cus, 8 * cus):
        times = []
        for r in range(reps + 2):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            if f(bufs[r % 3].data_ptr(), nb, grid, sink.data_ptr(), stream.cuda_stream) != 0:
                return None
            e1.record(stream)
            e1.synchronize()
            if r >= 2:
                times.append(e0.elapsed_time(e1) * 1e-3)
        gbs = nb / float(np.median(times)) / 1e9
        if best is None or gbs > best["GBps"]:
            best = {"GBps": round(gbs, 1), "grid": grid, "median_us": round(float(np.median(times)) * 1e6, 2)}
    del bufs
    best["bytes"] = nb
    best["frac_of_peak"] = round(best["GBps"] / HBM_PEAK_GBS, 4)
    return best


def dense27b_section(steps: int, warmup: int, widths=(1, 8, 16), copies: int = 2):
    """One 27B-shaped 8-bit layer (q/k/v, o, gate/up, down in 4 launches) and
    the 151936 x 5120 head with the greedy acceptance, rotating `copies`
    weight copies: per-launch device times from HIP events on the launch
    stream (median over steps), and the weight bytes of layer + head over the
    round's device time."""
    import torch
    from speculative_decoding_verify_dspk_amd import binding, inputs
    from speculative_decoding_verify_dspk_amd.verify_round import VerifyStack
    st = VerifyStack("dense-27b", 1, 8, max(widths), copies=copies, seed="bench-27b")
    stream = torch.cuda.current_stream()
    out = {"workload": "dense-27b layer x1 (5120 hidden, q 5120, kv 1024, inter 17408) + lm_head 151936x5120, "
                       f"8-bit g64, greedy, {copies} rotating copies",
           "weight_bytes_per_round": st.round_weight_bytes(), "widths": {}}
    names = ["qkv", "o", "gate_up", "down", "head"]
    for m in widths:
        calls = {}
        for cp in range(copies):
            t = None
            st.launch_head(m, cp, stream=stream)
            t = st.argmax[:m].cpu().numpy().reshape(1, m)
            d = inputs.drafts_match_rate(t, 0.7, st.vocab, "bench-27b", m, cp) if m > 1 else None
            dd = torch.from_numpy(np.ascontiguousarray(d, dtype=np.int32)).cuda() if m > 1 else None
            res = torch.empty((1 + m,), dtype=torch.int32, pin_memory=True)
            layers, _ = st.prepare_round(m, cp, stream=stream)
            head = binding.prepare_lmhead_accept_greedy(st.heads[cp], st.h, 1, m, st.argmax, None, dd, res[:1],
                                                        res[1:].view(1, m), st.ws_head, stream)
            calls[cp] = (layers + [head], dd, res)
        recs = []
        for it in range(warmup + steps):
            cp = it % copies
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
            ev[0].record(stream)
            for i, f in enumerate(calls[cp][0]):
                f()
                ev[i + 1].record(stream)
            stream.synchronize()
            if it >= warmup:
                recs.append([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(5)])
        med = np.median(np.array(recs), axis=0)
        layer_us, head_us = float(med[:4].sum()), float(med[4])
        lb, hb = st.layer_weight_bytes(), st.head_weight_bytes()
        out["widths"][str(m)] = {
            "launch_us": {n: round(float(v), 2) for n, v in zip(names, med)},
            "layer_us": round(layer_us, 2), "head_us": round(head_us, 2),
            "layer_hbm_frac": round(lb / (layer_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "head_hbm_frac": round(hb / (head_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "round_hbm_frac": round((lb + hb) / ((layer_us + head_us) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    first = out["widths"][str(widths[0])]
    for k in out["widths"]:
        w = out["widths"][k]
        w["t_over_t1"] = round((w["layer_us"] + w["head_us"]) / (first["layer_us"] + first["head_us"]), 4)
    del st
    torch.cuda.empty_cache()
    return out


def single_linear_section(steps: int, warmup: int, copies: int = 24):
    """The correctness-sized workload: one 2048 x 2048 8-bit linear over 6
    rows, then the 8192 x 2048 8-bit head with the greedy acceptance of 5
    drafts (the first 3 equal to the head's own tokens, the rest uniform),
    rotating `copies` weight copies (22 MB per round, so the copies exceed the
    MALL).  Device time per round from events around the two launches; its
    weight-GB/s is reported, but launch latency bounds it."""
    import torch
    from speculative_decoding_verify_dspk_amd import binding, inputs
    m, k, n, v = 6, 2048, 2048, 8192
    stream = torch.cuda.current_stream()

    def qw(rows, *lab):
        c, sc, bi = inputs.make_qweight_device(rows, k, 8, "bench-c1", *lab)
        return binding.DeviceQWeight(rows, k, 8, c, sc, bi)
    lins = [qw(n, "linear", cp) for cp in range(copies)]
    heads = [qw(v, "head", cp) for cp in range(copies)]
    x = inputs.make_activations_device(m, k, "bench-c1", "x")
    h = inputs.make_activations_device(m, k, "bench-c1", "h")
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    am = torch.empty((m,), dtype=torch.int32, device="cuda")
    ws_l = binding.alloc_workspace(binding.qgemm_workspace_bytes(n, k, m))
    ws_h = binding.alloc_workspace(binding.lmhead_workspace_bytes(v, m))
    calls = []
    for cp in range(copies):
        binding.lmhead_argmax(heads[cp], h, m, am, None, ws_h, stream)
        d = inputs.drafts_first_equal(am.cpu().numpy(), 3, v, "bench-c1", cp)
        dd = torch.from_numpy(np.ascontiguousarray(d, dtype=np.int32)).cuda()
        res = torch.empty((1 + m,), dtype=torch.int32, pin_memory=True)
        calls.append((binding.prepare_qgemm(lins[cp], x, m, y, ws_l, stream),
                      binding.prepare_lmhead_accept_greedy(heads[cp], h, 1, m, am, None, dd, res[:1],
                                                           res[1:].view(1, m), ws_h, stream), dd, res))
    times, committed = [], []
    for it in range(warmup + steps):
        lin, head, _, res = calls[it % copies]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        lin()
        head()
        e1.record(stream)
        e1.synchronize()
        if it >= warmup:
            times.append(e0.elapsed_time(e1) * 1e3)
            committed.append(int(res[0]))
    wb = inputs.weight_bytes(n, k, 8) + inputs.weight_bytes(v, k, 8)
    med = float(np.median(times))
    return {"workload": "one 2048x2048 8-bit g64 linear at 6 rows + lm_head 8192x2048 8-bit with greedy accept of 5 "
                        f"drafts (first 3 = the head's tokens), {copies} rotating copies",
            "weight_bytes_per_round": wb, "round_us": round(med, 2),
            "round_us_p10_p90": [round(float(np.percentile(times, 10)), 2),
                                 round(float(np.percentile(times, 90)), 2)],
            "weight_GBps": round(wb / (med * 1e-6) / 1e9, 1), "committed_tokens_per_round": float(np.mean(committed))}


def variant_curves(args):
    """t(M) of each Qwen3-4B 8-bit projection launch under each forced
    decomposition -- stream-K and slab on the matrix cores, and the slab with
    the K reduction on the vector ALUs (dot2, at most 4 rows) -- from HIP
    events around single launches on the launch stream, rotating six weight
    copies per shape so no launch is served from the MALL.  Prints one JSON
    line; under rocprofv3 --kernel-trace the same launches give the kernel
    durations (kernel names carry the decomposition and the row class)."""
    import torch
    from speculative_decoding_verify_dspk_amd import binding, inputs
    binding.lib()
    s = inputs.LAYER_SHAPES["qwen3-4b"]
    H, Q, KV, F = s["hidden"], s["q"], s["kv"], s["inter"]
    shapes = {"qkv": ([Q, KV, KV], H), "o": ([H], Q), "gate_up": ([F, F], H), "down": ([H], F)}
    widths = list(range(1, 17))
    copies = 6
    stream = torch.cuda.current_stream()
    out = {"metric": "per-launch device time t(M) by projection decomposition", "unit": "us",
           "workload": "qwen3-4b layer projections, 8-bit g64, one launch per call (grouped q/k/v and gate/up), "
                       f"{copies} rotating weight copies", "curves": {}, "launch_plan": []}
    names = {binding.VARIANT_STREAMK: "mfma_streamk", binding.VARIANT_SLAB: "mfma_slab",
             binding.VARIANT_DOT: "dot_slab"}
    prev = binding.set_projection_variant(binding.VARIANT_AUTO)
    try:
        for pname, (ns, k) in shapes.items():
            ws = [[binding.DeviceQWeight(n, k, 8, *inputs.make_qweight_device(n, k, 8, "curves", pname, i, c))
                   for i, n in enumerate(ns)] for c in range(copies)]
            x = inputs.make_activations_device(16, k, "curves", pname)
            ys = [torch.empty((16, n), dtype=torch.float32, device="cuda") for n in ns]
            wsp = binding.alloc_workspace(sum(binding.qgemm_workspace_bytes(n, k, 16) for n in ns))
            for var, vname in names.items():
                binding.set_projection_variant(var)
                curve = {}
                for m in widths:
                    if var == binding.VARIANT_DOT and m > 4:
                        continue
                    calls = [binding.prepare_qgemm_grouped(ws[c], x, m, ys, wsp, stream) for c in range(copies)]
                    for c in range(args.warmup):
                        calls[c % copies]()
                    # back-to-back batches of `copies` launches, as in a round:
                    # per-launch time = batch time / copies
                    ts = []
                    for r in range(args.steps):
                        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        e0.record(stream)
                        for c in range(copies):
                            calls[c]()
                        e1.record(stream)
                        e1.synchronize()
                        ts.append(e0.elapsed_time(e1) * 1e3 / copies)
                    curve[m] = round(float(np.median(ts)), 2)
                    out["launch_plan"].append([pname, vname, m, args.warmup + args.steps * copies])
                out["curves"].setdefault(pname, {})[vname] = curve
            del ws
    finally:
        binding.set_projection_variant(prev)
    print(json.dumps(out))


def main():
    args = parse()
    if args.variant_curves:
        variant_curves(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the verify pass runs on one GPU here (it is not sharded); "
              "use --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.prefill > 0:
        prefill_bench(args)
        return
    out = run_workload(args)
    if not args.no_extras and args.config == "qwen3-4b" and args.layers == 1 and args.batch == 1:
        out["other_configs"] = other_configs(args)
    print(json.dumps(out))


# The scope's other workloads, run after the headline one through the same
# round machinery (fewer steps, no extras): their wall-clock weight-GB/s and
# per-width device curve.
OTHER_CONFIGS = [
    ("ornith-9b 4-bit knee", ["--config", "ornith-9b", "--bits", "4", "--sweep", "1,2,4,8,12,16", "--copies", "2"]),
    ("ornith-9b 8-bit knee", ["--config", "ornith-9b", "--bits", "8", "--sweep", "1,2,4,8,12,16", "--copies", "2"]),
    ("ornith-9b bf16 knee", ["--config", "ornith-9b", "--bits", "16", "--sweep", "1,2,4,8,12,16", "--copies", "2"]),
    ("dense-27b 64 layers, 17 rows, speculative sampling T=1",
     ["--config", "dense-27b", "--layers", "64", "--sweep", "17", "--copies", "1", "--accept", "sample"]),
    ("qwen3-8b, 4 requests x 6 rows, greedy per request",
     ["--config", "qwen3-8b", "--batch", "4", "--sweep", "6", "--alpha", "0.3,0.5,0.7,0.9", "--copies", "2"]),
]


def other_configs(args):
    import torch
    res = {"single linear + 8192-vocab head, 6 rows": single_linear_section(max(30, args.steps), 5)}
    torch.cuda.empty_cache()
    for name, extra in OTHER_CONFIGS:
        sub = parse(extra + ["--steps", str(max(3, args.steps // 2)), "--warmup", "1", "--no-extras",
                             "--no-cpu-baseline", "--draft-sets", "2"])
        o = run_workload(sub)
        torch.cuda.empty_cache()
        res[name] = {"workload": o["config"]["workload"], "weight_bytes_per_round": o["config"]["weight_bytes_per_round"],
                     "value_weight_GBps": o["value"], "hbm_frac": o["hbm_frac"],
                     "round_wall_us_p50": o["round_wall_us"]["p50"],
                     "committed_tokens_per_round": o["committed_tokens_per_round"],
                     "committed_by_width": o["committed_by_width"],
                     "curve": {k: {kk: v[kk] for kk in ("round_us", "layer_us", "head_us", "accept_us",
                                                          "hbm_frac", "t_over_t1")}
                               for k, v in o["curve"].items()},
                     "head_avg_launch_us": o["roofline"]["avg_launch_us"]}
    return res


def run_workload(args) -> dict:
    """The verify rounds of one workload: the timed serving loop, then the
    event-instrumented pass; returns the result line as a dict."""
    import torch
    from speculative_decoding_verify_dspk_amd import binding, inputs
    from speculative_decoding_verify_dspk_amd.verify_round import VerifyStack

    binding.lib()   # fail loudly if the HIP library is missing
    sweep = [int(s) for s in args.sweep.split(",")]
    B = args.batch
    alpha = np.array([float(a) for a in args.alpha.split(",")])
    alpha = np.broadcast_to(alpha, (B,)).copy() if alpha.size in (1, B) else None
    if alpha is None or B * max(sweep) > binding.MAX_ROWS or (args.accept == "sample" and B != 1):
        print("bench.py: --alpha needs 1 or --batch values, batch * rows <= 32, sampling one request",
              file=sys.stderr)
        sys.exit(2)
    sample = args.accept == "sample"
    filtered = sample and (args.top_k > 0 or args.top_p < 1.0 or args.presence != 0.0 or args.frequency != 0.0)
    max_m = B * max(sweep)
    stack = VerifyStack(args.config, args.layers, args.bits, max_m, copies=args.copies)
    stream = torch.cuda.current_stream()
    V = stack.vocab

    # untimed pre-pass per (width, weight copy): that copy's target tokens
    # (and logits), then the drafter's side for S draft sets -- draft ids with
    # the match rates, or (sampling) draft distributions q from noisy target
    # logits, draft ids drawn from q, and the round's uniforms.  Each copy is
    # a different synthetic target, so each gets drafts of its own; rounds
    # cycle through the sets, so the committed counts average S x copies
    # independent draws per width.
    S = args.draft_sets
    sample_ws = binding.alloc_workspace(binding.sample_workspace_bytes(V, max_m)) if sample else None
    counts_t = torch.from_numpy(inputs.history_counts(V, args.history, "bench", args.config)).cuda() \
        if filtered else None
    rounds_in = {}
    for m in sweep:
        M = B * m
        for cp in range(args.copies):
            stack.launch_head(M, cp, want_logits=sample, stream=stream)
            t = stack.argmax[:M].cpu().numpy().reshape(B, m)
            z = stack.logits[:m].cpu().numpy() if sample else None
            for si in range(S):
                # [accept_len | committed] in pinned host memory: the acceptance
                # writes the round's result straight to the host (no copy launch)
                res = torch.empty((B + B * m,), dtype=torch.int32, pin_memory=True)
                r = dict(res=res, res_np=res.numpy(), alen=res[:B], com=res[B:].view(B, m))
                r["res_np"][:] = PENDING
                if sample:
                    q, d = inputs.draft_distribution(z, args.temperature, args.noise, "bench", args.config, m, cp,
                                                     si)
                    r["q"] = torch.from_numpy(np.ascontiguousarray(q)).cuda()
                    r["d"] = torch.from_numpy(d).cuda()
                    r["u"] = torch.from_numpy(inputs.make_uniforms(m, "bench", args.config, m, cp, si)).cuda()
                    r["ws"] = sample_ws
                    if filtered:
                        r["params"] = binding.sample_params(args.temperature, args.top_k, args.top_p,
                                                            args.presence, args.frequency)
                        r["counts"] = counts_t
                else:
                    d = inputs.drafts_match_rate(t, alpha, V, "bench", args.config, m, cp, si) if m > 1 else None
                    r["d"] = torch.from_numpy(np.ascontiguousarray(d, dtype=np.int32)).cuda() if m > 1 else None
                rounds_in[(m, cp, si)] = r

    def accept_call(m, r, prepare=True):
        if filtered:
            args_ = (stack.logits, r["q"], r["d"], r["u"], m, V, r["params"], r["counts"], r["alen"], r["com"],
                     r["ws"])
            return binding.prepare_accept_sample_ex(*args_, stream) if prepare else \
                (lambda: binding.accept_sample_ex(*args_))
        if sample:
            args_ = (stack.logits, r["q"], r["d"], r["u"], m, V, args.temperature, r["alen"], r["com"], r["ws"])
            return binding.prepare_accept_sample(*args_, stream) if prepare else \
                (lambda: binding.accept_sample(*args_))
        args_ = (stack.argmax, r["d"], B, m, r["alen"], r["com"])
        return binding.prepare_accept_greedy(*args_, stream) if prepare else (lambda: binding.accept_greedy(*args_))

    ev = lambda: torch.cuda.Event(enable_timing=True)   # noqa: E731

    # each round's calls, marshalled once per (width, weight copy); with
    # --graph, captured once as HIP graphs (layers, head, accept) instead
    prepared, graphs = {}, {}
    for m in sweep:
        for cp in range(args.copies):
            layers = None if args.graph else stack.prepare_round(B * m, cp, want_logits=sample, stream=stream)[0]
            for si in range(S):
                r = rounds_in[(m, cp, si)]
                if args.graph:
                    graphs[(m, cp, si)] = stack.capture_calls(B * m, cp, accept_call(m, r, prepare=False),
                                                              want_logits=sample)
                elif sample:
                    head = binding.prepare_lmhead(stack.heads[cp], stack.h, B * m, stack.argmax, stack.logits,
                                                  stack.ws_head, stream)
                    prepared[(m, cp, si)] = (layers, head, accept_call(m, r))
                else:
                    # greedy: the head's last workgroup runs the acceptance
                    # (dspk_lmhead_argmax_accept_greedy), no accept launch
                    fused = binding.prepare_lmhead_accept_greedy(stack.heads[cp], stack.h, B, m, stack.argmax, None,
                                                                 r["d"], r["alen"], r["com"], stack.ws_head, stream)
                    prepared[(m, cp, si)] = (layers, fused, lambda: None)

    def run_round(m: int, k: int, record: list | None):
        """Round number k at width m: weight copy k % copies, draft set (k // copies) % S."""
        copy, si = k % args.copies, (k // args.copies) % S
        r = rounds_in[(m, copy, si)]
        r["res_np"][:] = PENDING
        e = [ev() for _ in range(4)] if record is not None else None
        if e: e[0].record(stream)
        if args.graph:
            gl, gh, ga = graphs[(m, copy, si)]
            gl.replay()
            if e: e[1].record(stream)
            gh.replay()
            if e: e[2].record(stream)
            ga.replay()
        else:
            calls, head, accept = prepared[(m, copy, si)]
            for f in calls:
                f()
            if e: e[1].record(stream)
            head()
            if e: e[2].record(stream)
            accept()
        if e: e[3].record(stream)
        if e is None:
            wait_result(r["res_np"], stream)
        else:
            stream.synchronize()   # the event-instrumented pass
        if record is not None:
            record.append((m, e))
        return r["res_np"]         # the round's result, in host memory

    step_copy = 0
    for _ in range(args.warmup):
        for m in sweep:
            run_round(m, step_copy, None)
            step_copy += 1

    # A serving loop's long-lived objects (weights, prepared calls, the torch
    # module) move to the permanent generation, so that a full collection
    # scans only what the loop itself allocates (one scan of everything takes
    # tens of milliseconds with torch loaded).
    import gc
    gc.collect()
    gc.freeze()
    # Timed region: K steps of rounds as a serving loop runs them -- launch,
    # wait for the result words in pinned host memory, read the accept
    # lengths -- with no timing events.
    committed = 0
    committed_by_width = {m: 0 for m in sweep}
    faults = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    walls = []
    for _ in range(args.steps):
        for m in sweep:
            tr = time.perf_counter()
            res_np = run_round(m, step_copy, None)
            for a in res_np[:B]:
                if a < 0:
                    faults += 1
                else:
                    committed += int(a)
                    committed_by_width[m] += int(a)
            walls.append(time.perf_counter() - tr)
            step_copy += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Second pass, not part of the timed region: the same K steps with HIP
    # events on the launch stream around the layers, the head and the accept
    # step, for the per-width curve and the head kernel's launch time.
    records = []
    for _ in range(args.steps):
        for m in sweep:
            run_round(m, step_copy, records)
            step_copy += 1
    torch.cuda.synchronize()

    layer_b = stack.layer_weight_bytes() * args.layers
    head_b = stack.head_weight_bytes()
    round_b = layer_b + head_b
    n_rounds = args.steps * len(sweep)
    value = round_b * n_rounds / wall / 1e9

    # per-width device times from the events (median over steps)
    curve = {}
    head_ms_all, head_bytes_all = [], []
    for m in sweep:
        M = B * m
        rs = [e for (mm, e) in records if mm == m]
        t_rounds = [e[0].elapsed_time(e[3]) for e in rs]
        t_round = np.median(t_rounds)
        t_layer = np.median([e[0].elapsed_time(e[1]) for e in rs])
        t_head = [e[1].elapsed_time(e[2]) for e in rs]
        t_acc = np.median([e[2].elapsed_time(e[3]) for e in rs])
        head_ms_all += t_head
        head_bytes_all += [head_b + M * stack.hidden * 2 + (M * V * 4 if sample else M * 4)] * len(t_head)
        curve[M] = {"round_us": round(float(t_round) * 1e3, 2),
                    "round_us_p10_p90": [round(float(np.percentile(t_rounds, 10)) * 1e3, 2),
                                         round(float(np.percentile(t_rounds, 90)) * 1e3, 2)],
                    "layer_us": round(float(t_layer) * 1e3, 2),
                    "head_us": round(float(np.median(t_head)) * 1e3, 2),
                    "accept_us": round(float(t_acc) * 1e3, 2),
                    "weight_GBps": round(round_b / (t_round * 1e-3) / 1e9, 1),
                    "hbm_frac": round(round_b / (t_round * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    first = curve[B * sweep[0]]["round_us"]
    for M in curve:
        curve[M]["t_over_t1"] = round(curve[M]["round_us"] / first, 4)

    # the cap policy on the measured curve (verify round at widths 1..max,
    # interpolated between the measured widths; drafter time not included)
    cap_policy = None
    if B == 1 and len(sweep) > 1 and sweep[0] == 1:
        widths = np.arange(1, max(sweep) + 1)
        t_us = np.interp(widths, sweep, [curve[m]["round_us"] for m in sweep])
        cap_policy = {}
        for a in (0.3, 0.5, 0.7, 0.9):
            cap, rate = binding.choose_cap(t_us, None, a)
            cap_policy[str(a)] = {"cap": cap, "speedup_vs_plain": round(rate * t_us[0], 3)}

    head_avg_s = float(np.mean(head_ms_all)) * 1e-3
    head_bytes = float(np.mean(head_bytes_all))
    achieved = head_bytes / head_avg_s / 1e9
    profiled = args.config == "qwen3-4b" and args.bits == 8 and not sample and B == 1
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic() if profiled else None,
                "kernel": f"qgemm_kernel<{args.bits},MT,true> (vocabulary head + argmax)",
                "avg_launch_us": round(head_avg_s * 1e6, 2), "bytes_per_launch": int(head_bytes)}

    if args.calibrate:
        src = torch.empty(1 << 26, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    achievable = None if args.no_extras else achievable_bandwidth(head_b)
    if achievable is not None:
        roofline["achievable"] = achievable
        roofline["frac_of_achievable"] = round(achieved / achievable["GBps"], 4)
    dense = None
    if not args.no_extras and args.config == "qwen3-4b":
        dense = dense27b_section(max(args.steps, 5), max(args.warmup, 2))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.config, args.bits, min(B * max(sweep), 8), args.cpu_sample_s)

    workload = (f"{args.config} layer x{args.layers} + lm_head {V}x{stack.hidden}, "
                f"{'bf16' if args.bits == 16 else str(args.bits) + '-bit g64'}, "
                + (f"speculative sampling T={args.temperature}" if sample
                   else f"greedy alpha={','.join(f'{a:g}' for a in alpha)}")
                + (f" top_k={args.top_k} top_p={args.top_p:g} presence={args.presence:g} "
                   f"frequency={args.frequency:g} over a {args.history}-token history" if filtered else "")
                + (f", {B} requests x rows" if B > 1 else "") + f", one round per rows in {sweep}")
    out = {
        "metric": "verify weight-GB/s & % HBM peak vs width M=1..16; t(M)/t(1) cost curve",
        "value": round(value, 1), "unit": "weight-GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "widths": [B * m for m in sweep], "weight_bytes_per_round": round_b,
                   "rotating_copies": args.copies,
                   "launch": "hip-graph replays" if args.graph else "host launches, arguments marshalled once"},
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "t16_over_t1": curve[max(curve)]["t_over_t1"],
        "curve": curve,
        "rounds_per_s": round(n_rounds / wall, 1),
        "round_wall_us": {"p50": round(float(np.median(walls)) * 1e6, 1), "max": round(max(walls) * 1e6, 1)},
        "rows_per_s": round(B * sum(sweep) * args.steps / wall, 1),
        "committed_tokens_per_round": round(committed / n_rounds, 3),
        "committed_tokens_per_s": round(committed / wall, 1),
        # per request and round at each width: measured, and the closed form
        # 1 + sum_{i=1..m-1} alpha^i of independent per-position matches
        "committed_by_width": None if sample else {
            str(B * m): {"measured": round(committed_by_width[m] / (args.steps * B), 3),
                         "expected": [round(float(sum(a ** i for i in range(m))), 3) for a in alpha]}
            for m in sweep},
        "accept_faults": faults,
        "cap_policy": cap_policy,
        "roofline": roofline,
        "dense27b": dense,
        "cpu_baseline": cpu,
        "device": torch.cuda.get_device_name(0), "device_info": device_info(), "host": platform.node(),
    }
    del stack
    return out


if __name__ == "__main__":
    main()
