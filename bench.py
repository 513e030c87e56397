"""Benchmark of the Q4_0 decode hot path on one MI355X.

Default workload: the Q4_0 matvec at the 31B FFN projection shape,
K=5376 -> N=21504 (65,028,096 weight bytes), B=1.  One step = one matvec
dispatch over one activation batch; dispatches rotate over 16 independently
drawn weight copies (1.04 GB, larger than the 256 MB last-level cache) so every
step streams its weights from HBM.  Inputs are resident in HBM before timing.

Prints one JSON line (rank 0, N=1 only):
  value      = algorithmic bytes per dispatch / mean dispatch time (GB/s)
  roofline   = the matvec kernel against the 8 TB/s HBM3E peak
  cpu_baseline = the fp64 oracle timed on a bounded sample on the host cores
Extra keys report B=8 at the same shape and the decode workloads.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def matvec_bytes(n, k, b):
    return n * (k // 32) * 18 + 4 * b * k + 4 * b * n


def time_dispatches(torch, launch, steps, warmup):
    """Mean time per dispatch (ms) over `steps` back-to-back launches after
    `warmup` untimed ones, HIP events on the stream the kernels are launched
    on.  (Host submission takes about half a dispatch, so the GPU stays busy;
    the same dispatches replayed as one HIP graph take the same time per
    dispatch, see time_matvec_graph.)
    The part's clocks take about 15 ms of sustained memory traffic to settle
    (a 65 MB matvec runs ~15 % slower before that), hence the long default
    warm-up."""
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        launch(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def time_matvec(q, torch, Ws, x, y, steps, warmup):
    """B = 1 and vector-path B > 1: the C entry point called with prepared
    arguments, so host submission stays far below a dispatch (also under a
    tracing profiler, whose per-launch hooks would otherwise leave gaps)."""
    fn = q.lib().q4_0_matvec
    B, K = x.shape
    N = y.shape[1]
    stream = torch.cuda.current_stream().cuda_stream
    args = [(W.data_ptr(), N, K, x.data_ptr(), B, y.data_ptr(), None, stream) for W in Ws]
    for a in args[:1]:
        assert fn(*a) == 0, q.lib().q4dec_last_error()
    return time_dispatches(torch, lambda i: fn(*args[i % len(args)]), steps, warmup)


def matvec_repeats(q, torch, Ws, x, y, steps, windows=5):
    """Spread of the B = 1 timing: `windows` more timed windows of `steps`
    dispatches each (the clocks are settled by then), median and coefficient
    of variation of the per-dispatch time."""
    import statistics
    t = [time_matvec(q, torch, Ws, x, y, steps, 50) for _ in range(windows)]
    med = statistics.median(t)
    return {"windows": windows, "dispatches_per_window": steps, "median_ms": round(med, 6),
            "cv": round(statistics.pstdev(t) / statistics.mean(t), 4)}


def time_matvec_graph(q, torch, Ws, x, y, nodes, replays=5):
    """The same B = 1 dispatches captured as one HIP graph of `nodes` kernel
    nodes (rotating over the weight copies) and replayed: mean time per node
    over `replays` timed replays after three untimed ones."""
    fn = q.lib().q4_0_matvec
    B, K = x.shape
    N = y.shape[1]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        stream = torch.cuda.current_stream().cuda_stream
        for i in range(nodes):
            W = Ws[i % len(Ws)]
            assert fn(W.data_ptr(), N, K, x.data_ptr(), B, y.data_ptr(), None, stream) == 0, \
                q.lib().q4dec_last_error()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(replays):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (replays * nodes)


def time_matvec_batched(q, torch, Ws, x, y, K, B, steps, warmup):
    """As time_matvec for the matrix-core path."""
    N = y.shape[1]
    ws = torch.zeros(q.matvec_batched_workspace(N, K, B), dtype=torch.uint8, device=x.device)
    return time_dispatches(
        torch, lambda i: q.q4_0_matvec_batched(Ws[i % len(Ws)], x, K, B, K, y=y, ws=ws), steps,
        warmup)


def settle(torch, fn, ms=40.0):
    """Runs fn until `ms` of wall time has passed (untimed): the clocks take
    about 15 ms of sustained memory traffic to reach their steady state."""
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        fn()
        torch.cuda.synchronize()


def bench_attention_stack(q, torch, batch, reps=20, kv16=False):
    """The 28-layer Qwen3-1.7B-shaped attention stack at n_cache = 4096: per
    layer one fused call (QK-norm + RoPE + KV append at position 4096, then
    split-K attention over the 4097 keys) reading raw q | k | v rows.  Every
    layer has its own cache, so a pass streams 28 * B * 2 * 8 * 4097 * 128 * e
    bytes of K/V (e = 4, or 2 with binary16 caches)."""
    import numpy as np

    from q4_quantized_matvec_amd._lib import kv_layout_of
    from synth import workloads as wl
    w = wl.ATTN_QWEN3_1P7B
    dev = torch.device("cuda:0")
    hq, hkv, hd, pos = w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_cache
    pos_d = torch.tensor([pos, pos + 1], dtype=torch.int64, device=dev)
    layers = []
    for l in range(w.n_layers):
        qh, kh, vh, qn, kn, kc, vc = wl.attn_layer_inputs(w, batch, l)
        if kv16:
            kc, vc = kc.astype(np.float16), vc.astype(np.float16)
        kcd = torch.from_numpy(kc).to(dev)
        qkv = np.concatenate([qh.reshape(batch, -1), kh.reshape(batch, -1), vh.reshape(batch, -1)],
                             axis=1)
        layers.append(dict(qkv=torch.from_numpy(np.ascontiguousarray(qkv)).to(dev),
                           qn=torch.from_numpy(qn).to(dev), kn=torch.from_numpy(kn).to(dev),
                           kc=kcd, vc=torch.from_numpy(vc).to(dev), kv=kv_layout_of(kcd)))
        del kc, vc
    ws = torch.empty(q.gqa_decode_attn_workspace(layers[0]["kv"], hq, 0), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((batch, hq * hd), dtype=torch.float32, device=dev)
    scale = 1.0 / np.sqrt(hd)

    ld = hq * hd + 2 * hkv * hd

    def one_pass():
        for L in layers:
            q.gqa_decode_attn_rope(L["qkv"], ld, hq, L["qn"], L["kn"], L["kv"], pos_d[0:1],
                                   w.rope_theta, w.eps, False, L["kc"], L["vc"], 0, scale, out,
                                   hq * hd, ws)

    settle(torch, one_pass)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        one_pass()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    n = pos + 1
    e = 2 if kv16 else 4
    nbytes = w.n_layers * batch * (2 * hkv * hd * n * e + 2 * hq * hd * 4 + 2 * hkv * hd * 4 +
                                   2 * hkv * hd * e)
    del layers
    torch.cuda.empty_cache()
    return {"ms_per_pass": round(ms, 4), "batch": batch, "layers": w.n_layers, "n_keys": n,
            "kv": "f16" if kv16 else "f32",
            "algorithmic_GB_per_pass": round(nbytes / 1e9, 4),
            "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def decode_algorithmic_bytes(m, step, kv_bytes=4):
    """Bytes one decode step must move: every weight byte (Q4_0 matrices, the
    Q8_0 logit table, the gathered embedding rows, norm gains), every visible
    KV-cache byte, the appended KV rows and the logits."""
    from synth import workloads as wl
    d, F, V, B = m.d_model, m.ffn, m.vocab, m.batch
    q4 = lambda n, k: n * (k // 32) * 18
    total = V * (d // 32) * 34 + B * (d // 32) * 34 + 4 * d + 4 * B * V
    n = m.start_pos + step + 1
    for ly in m.layers:
        nq, nk, nv = wl.layer_rows(m, ly)
        total += q4(nq + nk + nv, d) + q4(d, nq) + q4(2 * F, d) + q4(d, F)
        total += 4 * (2 * d + 2 * ly.head_dim) + (8 * d if m.sandwich else 0)
        vis = min(n, ly.window) if ly.window else n
        total += B * ly.n_kv_heads * ly.head_dim * kv_bytes * (2 * vis + 2)
    return total


def device_prefilled_caches(torch, m, dev, kv16=False):
    """Per layer a (k, v) pair of device caches laid out as the host recipe's
    (positions below start_pos in slot p % cap, N(0,1); other slots 0), drawn
    by torch's seeded device generator: long contexts hold tens of GB of cache,
    too much to draw on the host in a benchmark."""
    gen = torch.Generator(device=dev)
    caches = []
    for l, ly in enumerate(m.layers):
        pair = []
        for which in (0, 1):
            gen.manual_seed(m.seed * 1000 + 2 * l + which)
            c = torch.zeros((m.batch, ly.n_kv_heads, ly.cap, ly.head_dim),
                            dtype=torch.float16 if kv16 else torch.float32, device=dev)
            filled = min(m.start_pos, ly.cap)
            c[:, :, :filled].normal_(generator=gen)
            pair.append(c)
        caches.append(tuple(pair))
    return caches


def bench_decode(q, torch, m, reps=3, warmup=2, device_caches=False, kv16=False):
    """Times 16-step greedy decode runs from the prefilled position (HIP graph
    replay, two graphs ping-ponging the token buffers)."""
    from synth import workloads as wl
    from synth.device import model_kwargs, prefilled_caches, upload_model
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    weights = wl.model_weights(m)
    if device_caches:
        caches = device_prefilled_caches(torch, m, dev, kv16=kv16)
    else:
        caches = prefilled_caches(m, kv16=kv16)
    dmod = upload_model(m, weights, dev, caches=caches)
    del caches
    del weights
    log(f"{m.name}: generated and uploaded in {time.perf_counter() - t0:.1f} s")
    dm = q.DecodeModel(**model_kwargs(m, dmod))
    a = torch.from_numpy(wl.start_tokens(m)).to(dev)
    b = torch.empty_like(a)
    stream = torch.cuda.current_stream()

    def run(steps):
        dm.set_position(m.start_pos)
        for s_ in range(steps):
            src, dst = (a, b) if s_ % 2 == 0 else (b, a)
            dm.step(src, dst)

    for _ in range(warmup):
        run(m.steps)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run(m.steps)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / m.steps)
    ms = sorted(times)[len(times) // 2]
    nbytes = sum(decode_algorithmic_bytes(m, s_, 2 if kv16 else 4) for s_ in range(m.steps)) / m.steps
    dm.close()
    del dmod
    torch.cuda.empty_cache()
    return {"tok/s": round(m.batch * 1e3 / ms, 2), "ms_per_step": round(ms, 4), "batch": m.batch,
            "steps": m.steps, "start_pos": m.start_pos,
            "kv_fill": "device generator" if device_caches else "host recipe",
            "kv": "f16" if kv16 else "f32",
            "algorithmic_GB_per_step": round(nbytes / 1e9, 4),
            "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def copy_calibration(torch, nbytes=1 << 30, reps=4):
    """A plain device-to-device copy of a known size, launched after the timed
    matvecs so that an HBM byte counter (FETCH_SIZE, WRITE_SIZE) can be scaled
    to bytes: each launch reads and writes exactly `nbytes`."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} launches of {nbytes} bytes")


def pmc_traffic(fetch_csv, write_csv, kernel="mv_b1_kernel", copy_bytes=1 << 30):
    """HBM traffic per matvec launch from two rocprofv3 --pmc passes (FETCH_SIZE,
    then WRITE_SIZE; both in KiB per dispatch), each scaled by the ratio of the
    known copy size to what the same counter read for the calibration copy."""
    import csv

    def per_kernel(path, counter):
        vals = {"mv": [], "copy": []}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            if kernel in name:
                vals["mv"].append(float(r["Counter_Value"]))
            elif "copy" in name.lower() or "elementwise" in name.lower():
                vals["copy"].append(float(r["Counter_Value"]))
        assert vals["mv"] and vals["copy"], f"{path}: no {counter} rows for both kernels"
        mv = sorted(vals["mv"])[len(vals["mv"]) // 2]
        cp = sorted(vals["copy"])[len(vals["copy"]) // 2]
        return mv, cp

    mv_f, cp_f = per_kernel(fetch_csv, "FETCH_SIZE")
    mv_w, cp_w = per_kernel(write_csv, "WRITE_SIZE")
    f_scale = copy_bytes / (cp_f * 1024.0)
    w_scale = copy_bytes / (cp_w * 1024.0)
    return {"fetch_kib_raw": mv_f, "write_kib_raw": mv_w,
            "copy_fetch_kib_raw": cp_f, "copy_write_kib_raw": cp_w,
            "fetch_scale": f_scale, "write_scale": w_scale,
            "bytes_per_launch": round(mv_f * 1024.0 * f_scale + mv_w * 1024.0 * w_scale)}


def kernel_source_hash():
    """Digest of the matvec kernel's sources: stored counter readings are used
    only while it is unchanged."""
    import hashlib
    h = hashlib.sha256()
    for f in ("matvec.hip", "common.hpp"):
        with open(os.path.join(ROOT, "q4_quantized_matvec_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(key):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f).get(key)
    if not t or t.get("kernel_source") != kernel_source_hash():
        return None
    return t["bytes_per_launch"]


def cpu_baseline_matvec(w, budget_s=12.0):
    import numpy as np

    import oracle
    from synth import workloads as wl
    W, x = wl.matvec_inputs(w, 1)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.q4_0_matvec(W, w.n, w.k, x)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 20000:
            break
    per = el / reps
    return {"value": round(matvec_bytes(w.n, w.k, 1) / per / 1e9, 3), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{reps} full {w.k}x{w.n} B=1 fp64 matvecs ({el:.1f} s), "
                      f"{per * 1e3:.1f} ms each"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--copies", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-matvec", action="store_true")
    ap.add_argument("--decode",
                    default="qwen3_4b,gemma4_31b,gemma4_31b_128k,qwen3_4b_f16kv,gemma4_31b_128k_f16kv,"
                            "gemma4_31b_exact",
                    help="decode workloads to time (comma list, empty for none)")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the B=1 HBM-streaming matvec (for profiler runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run a 1 GiB device copy to scale byte counters")
    ap.add_argument("--no-attention", action="store_true",
                    help="skip the 28-layer attention-stack timing")
    ap.add_argument("--only-decode", action="store_true",
                    help="time only the decode workloads (for profiler runs)")
    ap.add_argument("--pmc-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc passes and exit")
    args = ap.parse_args()
    if args.pmc_traffic:
        t = pmc_traffic(*args.pmc_traffic)
        t["source"] = ("rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE over "
                       "'bench.py --headline-only --copy-calibration --no-cpu-baseline'")
        path = os.path.join(ROOT, "profiles", "traffic.json")
        data = json.load(open(path)) if os.path.exists(path) else {}
        t["kernel_source"] = kernel_source_hash()
        data["q4_0_matvec_5376x21504_B1"] = t
        with open(path, "w") as f:
            json.dump(data, f, indent=1)
        print(json.dumps(t))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import torch

    import q4_quantized_matvec_amd as q
    from synth import workloads as wl

    dev = torch.device("cuda:0")
    # decode legs: key -> (workload, caches drawn on the device, binary16 caches)
    legs = {"qwen3_4b": (wl.QWEN3_4B, False, False), "gemma4_31b": (wl.GEMMA4_31B, False, False),
            "gemma4_31b_128k": (wl.GEMMA4_31B_128K, True, False),
            "qwen3_4b_f16kv": (wl.QWEN3_4B, False, True),
            "gemma4_31b_128k_f16kv": (wl.GEMMA4_31B_128K, True, True),
            "gemma4_31b_exact": (wl.GEMMA4_31B_EXACT, False, False)}
    decode_keys = [k for k in args.decode.split(",") if k] if not args.only_matvec else []

    def run_leg(key):
        m, on_dev, kv16 = legs[key]
        name = m.name + ("_f16kv" if kv16 else "")
        return name, bench_decode(q, torch, m, device_caches=on_dev, kv16=kv16)

    if args.only_decode:
        print(json.dumps({"decode": dict(run_leg(k) for k in decode_keys)}), flush=True)
        return

    w = wl.MATVEC_5376x21504
    log(f"generating {args.copies} weight copies of {w.k}x{w.n}")
    Ws = []
    for c in range(args.copies):
        W, _ = wl.matvec_inputs(w, 1, copy=c)
        Ws.append(torch.from_numpy(W).to(dev))
    _, x1 = wl.matvec_inputs(w, 1)
    x1 = torch.from_numpy(x1).to(dev)
    y1 = torch.empty((1, w.n), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    log("timing B=1")
    ms1 = time_matvec(q, torch, Ws, x1, y1, args.steps, args.warmup)
    bytes1 = matvec_bytes(w.n, w.k, 1)
    gbs1 = bytes1 / (ms1 * 1e-3) / 1e9
    traffic = stored_traffic("q4_0_matvec_5376x21504_B1")
    out = {
        "metric": "Q4_0 matvec GB/s (% of HBM peak) at 5376x21504; decode tok/s at B=1 and B=8",
        "value": round(gbs1, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms1, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded Philox; Q4_0 codes uniform, binary16 scales U[0.005,0.02], x N(0,1))",
        "config": {"workload": w.name, "N": w.n, "K": w.k, "B": 1, "weight_copies": args.copies,
                   "weight_bytes": w.n * (w.k // 32) * 18,
                   "algorithmic_bytes_per_launch": bytes1},
        "roofline": {"bound": "hbm", "achieved": round(gbs1, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs1 / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
    }
    if args.copy_calibration:
        copy_calibration(torch)
    if not args.headline_only:
        _, x8 = wl.matvec_inputs(w, 8)
        x8 = torch.from_numpy(x8).to(dev)
        y8 = torch.empty((8, w.n), dtype=torch.float32, device=dev)
        log("timing B=8 (matrix cores)")
        ms8 = time_matvec_batched(q, torch, Ws, x8, y8, w.k, 8, args.steps, args.warmup)
        log("timing B=1 cache-resident (one copy)")
        ms1r = time_matvec(q, torch, Ws[:1], x1, y1, args.steps, args.warmup)
        gbs8 = matvec_bytes(w.n, w.k, 8) / (ms8 * 1e-3) / 1e9
        out["matvec_B8"] = {"GB/s": round(gbs8, 2), "ms": round(ms8, 6),
                            "frac_hbm": round(gbs8 / HBM_PEAK_GBS, 4), "path": "mfma"}
        for bb in (16, 32):
            _, xb = wl.matvec_inputs(w, bb)
            xb = torch.from_numpy(xb).to(dev)
            yb = torch.empty((bb, w.n), dtype=torch.float32, device=dev)
            log(f"timing B={bb} (matrix cores, batch groups of 8)")
            msb = time_matvec_batched(q, torch, Ws, xb, yb, w.k, bb, args.steps, args.warmup)
            gbsb = matvec_bytes(w.n, w.k, bb) / (msb * 1e-3) / 1e9
            out[f"matvec_B{bb}"] = {"GB/s": round(gbsb, 2), "ms": round(msb, 6),
                                    "frac_hbm": round(gbsb / HBM_PEAK_GBS, 4), "path": "mfma"}
            del xb, yb
        out["matvec_B1_cache_resident"] = {"GB/s": round(bytes1 / (ms1r * 1e-3) / 1e9, 2),
                                           "ms": round(ms1r, 6)}
        log("timing B=1: repeat windows, then as one HIP graph")
        out["matvec_B1_repeats"] = matvec_repeats(q, torch, Ws, x1, y1, args.steps)
        msg = time_matvec_graph(q, torch, Ws, x1, y1, args.steps)
        out["matvec_B1_graph"] = {"nodes": args.steps, "GB/s": round(bytes1 / (msg * 1e-3) / 1e9, 2),
                                  "ms_per_node": round(msg, 6)}
        del Ws
        torch.cuda.empty_cache()
        if not args.no_attention:
            for kv16 in (False, True):
                key = "attn_qwen3_1p7b" + ("_f16kv" if kv16 else "")
                out[key] = {}
                for bb in (1, 8):
                    log(f"timing the 28-layer attention stack, B={bb}, {'f16' if kv16 else 'f32'} KV")
                    out[key][f"B{bb}"] = bench_attention_stack(q, torch, bb, kv16=kv16)
        if decode_keys:
            out["decode"] = {}
            for key in decode_keys:
                log(f"timing decode {key}")
                name, res = run_leg(key)
                out["decode"][name] = res
    if not args.no_cpu_baseline and not args.headline_only:
        log("timing the oracle on the host")
        out["cpu_baseline"] = cpu_baseline_matvec(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
