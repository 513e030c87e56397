"""Benchmark of the Q4_0 decode hot path on one MI355X.

Headline workload: the Q4_0 matvec at the 31B FFN projection shape,
K=5376 -> N=21504 (65,028,096 weight bytes), B=1.  One step = one matvec
dispatch over one activation batch; dispatches rotate over 16 independently
drawn weight copies (1.04 GB, larger than the 256 MB last-level cache) so every
step streams its weights from HBM.  Inputs are resident in HBM before timing.

Timing method (every GPU line): untimed dispatches until both `--warmup`
dispatches and at least 50 ms of GPU work have run (the part's clocks take
about 15 ms of sustained memory traffic to settle), then `--windows` timed
windows of exactly `--steps` back-to-back dispatches each, timing-only HIP
events (no system-scope cache release at a window boundary) on the stream the
kernels run on; a line reports the median window (per dispatch) and the
coefficient of variation over the windows.

Prints one JSON line (rank 0, N=1 only):
  value        = algorithmic bytes per dispatch / median dispatch time (GB/s)
  roofline     = the matvec kernel against the 8 TB/s HBM3E peak, with the
                 counter-measured HBM bytes per launch when they were taken
                 from the current kernel sources
  cpu_baseline = the fp64 oracle on the host cores: the headline workload on
                 a bounded sample, plus per-workload lines (single thread and
                 all threads)
Extra keys report the small matvec, B = 2..32 at the headline shape (vector
and matrix-core paths), the attention stack and the decode workloads.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
SETTLE_MS = 50.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def matvec_bytes(n, k, b, block_bytes=18):
    return n * (k // 32) * block_bytes + 4 * b * k + 4 * b * n


def summarize(per_dispatch_ms):
    med = statistics.median(per_dispatch_ms)
    return {"median_ms": round(med, 6), "min_ms": round(min(per_dispatch_ms), 6),
            "max_ms": round(max(per_dispatch_ms), 6),
            "cv": round(statistics.pstdev(per_dispatch_ms) / statistics.mean(per_dispatch_ms), 4),
            "windows": len(per_dispatch_ms)}


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence


class TimingEvents:
    """Timing-only HIP events on the launch stream.  A default event record
    ends with a system-scope release (the caches are written back and
    invalidated), which costs the work after it about a microsecond per
    dispatch when windows are as short as 20 dispatches; these events are
    created with hipEventDisableSystemFence, so a window boundary adds only
    the timestamp.  They are read after a full device synchronisation.  The
    HIP runtime is the one torch has loaded (the library links the same one)."""

    _rt = None

    @classmethod
    def runtime(cls):
        import ctypes
        if cls._rt is None:
            path = None
            with open("/proc/self/maps") as f:
                for line in f:
                    p = line.split()[-1]
                    if "libamdhip64" in p and p.startswith("/"):
                        path = p
                        break
            rt = ctypes.CDLL(path or "libamdhip64.so.7")
            rt.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._rt = rt
        return cls._rt

    def __init__(self, torch, n):
        import ctypes
        self._c = ctypes
        rt = self.runtime()
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = rt.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE)
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            self.ev.append(e)
        self.stream = torch.cuda.current_stream().cuda_stream

    def record(self, i):
        rc = self.runtime().hipEventRecord(self.ev[i], self.stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def ms(self, i, j):
        t = self._c.c_float()
        rc = self.runtime().hipEventElapsedTime(self._c.byref(t), self.ev[i], self.ev[j])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(t.value)

    def __del__(self):
        try:
            for e in self.ev:
                self.runtime().hipEventDestroy(e)
        except Exception:
            pass


def settle(torch, launch, warmup, ms=SETTLE_MS):
    """Untimed dispatches until `warmup` of them and `ms` of wall time with
    the GPU kept busy have passed (the host waits for each batch, so wall time
    is GPU time)."""
    i = 0
    t0 = time.perf_counter()
    while i < warmup or (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(32):
            launch(i)
            i += 1
        torch.cuda.synchronize()
    return i


def time_windows(torch, launch, steps, warmup, windows):
    """Median per-dispatch time over `windows` windows of exactly `steps`
    back-to-back dispatches (events recorded between the windows on the launch
    stream, so the GPU never idles between them; a few untimed dispatches
    before the first event keep the queue ahead of the GPU)."""
    i = settle(torch, launch, warmup)
    for _ in range(8):
        launch(i)
        i += 1
    ev = TimingEvents(torch, windows + 1)
    ev.record(0)
    for w in range(windows):
        for _ in range(steps):
            launch(i)
            i += 1
        ev.record(w + 1)
    torch.cuda.synchronize()
    return summarize([ev.ms(w, w + 1) / steps for w in range(windows)])


def matvec_launcher(q, torch, Ws, x, y, check=True):
    """The C entry point q4_0_matvec called with prepared arguments on the
    current stream, so host submission stays far below a dispatch (also under
    a tracing profiler, whose per-launch hooks would otherwise leave gaps)."""
    fn = q.lib().q4_0_matvec
    B, K = x.shape
    N = y.shape[1]
    stream = torch.cuda.current_stream().cuda_stream
    args = [(W.data_ptr(), N, K, x.data_ptr(), B, y.data_ptr(), None, stream) for W in Ws]
    if check:
        assert fn(*args[0]) == 0, q.lib().q4dec_last_error()
    return lambda i: fn(*args[i % len(args)])


def batched_launcher(q, torch, Ws, x, y, K, B):
    N = y.shape[1]
    ws = torch.zeros(q.matvec_batched_workspace(N, K, B), dtype=torch.uint8, device=x.device)
    return lambda i: q.q4_0_matvec_batched(Ws[i % len(Ws)], x, K, B, K, y=y, ws=ws)


def time_graph(torch, make_launch, nodes, replays=5):
    """`nodes` dispatches (of the launcher `make_launch()` builds on the
    capture stream) captured as one HIP graph and replayed: median time per
    node over `replays` timed replays after a settle of at least 50 ms."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch = make_launch()
        for i in range(nodes):
            launch(i)
    settle(torch, lambda i: g.replay(), 3)
    ev = TimingEvents(torch, replays + 1)
    ev.record(0)
    for r in range(replays):
        g.replay()
        ev.record(r + 1)
    torch.cuda.synchronize()
    return summarize([ev.ms(r, r + 1) / nodes for r in range(replays)])


def gbs(nbytes, ms):
    return nbytes / (ms * 1e-3) / 1e9


def line(nbytes, t, **extra):
    v = gbs(nbytes, t["median_ms"])
    return dict({"GB/s": round(v, 2), "frac_hbm": round(v / HBM_PEAK_GBS, 4),
                 "ms": t["median_ms"], "cv": t["cv"]}, **extra)


def weight_copies(torch, w, copies, dev):
    from synth import workloads as wl
    Ws = []
    for c in range(copies):
        W, _ = wl.matvec_inputs(w, 1, copy=c)
        Ws.append(torch.from_numpy(W).to(dev))
    return Ws


def activations(torch, w, b, dev):
    from synth import workloads as wl
    _, x = wl.matvec_inputs(w, b)
    return torch.from_numpy(x).to(dev), torch.empty((b, w.n), dtype=torch.float32, device=dev)


def bench_small_matvec(q, torch, args, dev):
    """K=2048 -> N=6144 at B=1: 128 rotating copies (906 MB, every dispatch
    from HBM) and one copy (cache-resident).  A dispatch takes about as long as
    its host submission here, so the figures are graph replays (node times);
    the eager rate is reported beside them."""
    from synth import workloads as wl
    w = wl.MATVEC_2048x6144
    log(f"generating 128 weight copies of {w.k}x{w.n}")
    Ws = weight_copies(torch, w, 128, dev)
    x, y = activations(torch, w, 1, dev)
    nb = matvec_bytes(w.n, w.k, 1)
    out = {"workload": w.name, "N": w.n, "K": w.k, "B": 1, "algorithmic_bytes": nb}
    log("timing the small matvec (128 copies, then one)")
    launch = matvec_launcher(q, torch, Ws, x, y)
    out["rotating_128"] = line(
        nb, time_graph(torch, lambda: matvec_launcher(q, torch, Ws, x, y, check=False), args.steps),
        timing="graph")
    out["rotating_128_eager"] = line(nb, time_windows(torch, launch, args.steps, args.warmup,
                                                      args.windows), timing="eager")
    out["cache_resident"] = line(
        nb, time_graph(torch, lambda: matvec_launcher(q, torch, Ws[:1], x, y, check=False),
                       args.steps), timing="graph")
    del Ws
    torch.cuda.empty_cache()
    return out


def bench_attention_stack(q, torch, batch, windows, reps=4, kv16=False):
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
    ws = torch.zeros(q.gqa_decode_attn_workspace(layers[0]["kv"], hq, 0), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((batch, hq * hd), dtype=torch.float32, device=dev)
    scale = 1.0 / np.sqrt(hd)
    ld = hq * hd + 2 * hkv * hd

    def one_pass(_i=0):
        for L in layers:
            q.gqa_decode_attn_rope(L["qkv"], ld, hq, L["qn"], L["kn"], L["kv"], pos_d[0:1],
                                   w.rope_theta, w.eps, False, L["kc"], L["vc"], 0, scale, out,
                                   hq * hd, ws)

    t = time_windows(torch, one_pass, reps, 1, windows)
    ms = t["median_ms"]
    n = pos + 1
    e = 2 if kv16 else 4
    nbytes = w.n_layers * batch * (2 * hkv * hd * n * e + 2 * hq * hd * 4 + 2 * hkv * hd * 4 +
                                   2 * hkv * hd * e)
    del layers
    torch.cuda.empty_cache()
    return {"ms_per_pass": round(ms, 4), "cv": t["cv"], "batch": batch, "layers": w.n_layers,
            "n_keys": n, "kv": "f16" if kv16 else "f32",
            "algorithmic_GB_per_pass": round(nbytes / 1e9, 4),
            "GB/s": round(gbs(nbytes, ms), 1), "frac_hbm": round(gbs(nbytes, ms) / HBM_PEAK_GBS, 4)}


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


def oracle_decode_baseline(m, weights, caches):
    """The oracle's decode step on the host cores: one step of the whole model
    with all threads, and one step of a one-layer slice of it (layer 0 plus the
    embedding and logit tables) on one thread."""
    import oracle
    from synth import workloads as wl
    full_threads = oracle.num_threads()
    om = oracle.Model(wl.oracle_spec(m, weights, caches))
    tok = wl.start_tokens(m)
    t0 = time.perf_counter()
    om.step(m.start_pos, tok)
    t_all = time.perf_counter() - t0
    del om
    sub = wl.submodel(m, [0])
    sw = dict(weights, layers=weights["layers"][:1])
    oracle.set_num_threads(1)
    try:
        om = oracle.Model(wl.oracle_spec(sub, sw, caches[:1]))
        t0 = time.perf_counter()
        om.step(m.start_pos + 1, tok)
        t_one = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(full_threads)
    return {"all_threads": {"s_per_step": round(t_all, 3), "tok/s": round(m.batch / t_all, 4),
                            "threads": full_threads,
                            "sample": f"one step of the whole {m.n_layers}-layer model at B={m.batch}"},
            "one_thread": {"s_per_step": round(t_one, 3), "threads": 1,
                           "sample": "one step of layer 0 with the embedding and logit tables"}}


def bench_decode(q, torch, m, reps=5, warmup=2, device_caches=False, kv16=False, oracle_cpu=False,
                 counter_steps=0):
    """Times 16-step greedy decode runs from the prefilled position (HIP graph
    replay, two graphs ping-ponging the token buffers); median step time over
    `reps` runs.  With `counter_steps`, instead runs that many eager steps
    between two marker copies (for byte counters) and returns."""
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
    log(f"{m.name}: generated and uploaded in {time.perf_counter() - t0:.1f} s")
    cpu = None
    if oracle_cpu and not device_caches and not kv16:
        log(f"{m.name}: oracle decode step on the host")
        cpu = oracle_decode_baseline(m, weights, caches)
    del caches
    del weights
    dm = q.DecodeModel(**model_kwargs(m, dmod))
    a = torch.from_numpy(wl.start_tokens(m)).to(dev)
    b = torch.empty_like(a)

    def run(steps, eager=False):
        dm.set_position(m.start_pos)
        for s_ in range(steps):
            src, dst = (a, b) if s_ % 2 == 0 else (b, a)
            dm.step(src, dst, eager=eager)

    if counter_steps:
        run(1, eager=True)
        torch.cuda.synchronize()
        marker_copy(torch)
        run(counter_steps, eager=True)
        torch.cuda.synchronize()
        marker_copy(torch)
        dm.close()
        return {"counter_steps": counter_steps}
    for _ in range(warmup):
        run(m.steps)
    torch.cuda.synchronize()
    times = []
    ev = TimingEvents(torch, 2)
    for _ in range(reps):
        ev.record(0)
        run(m.steps)
        ev.record(1)
        torch.cuda.synchronize()
        times.append(ev.ms(0, 1) / m.steps)
    t = summarize(times)
    ms = t["median_ms"]
    nbytes = sum(decode_algorithmic_bytes(m, s_, 2 if kv16 else 4) for s_ in range(m.steps)) / m.steps
    dm.close()
    del dmod
    torch.cuda.empty_cache()
    res = {"tok/s": round(m.batch * 1e3 / ms, 2), "ms_per_step": round(ms, 4), "cv": t["cv"],
           "batch": m.batch, "steps": m.steps, "start_pos": m.start_pos,
           "kv_fill": "device generator" if device_caches else "host recipe",
           "kv": "f16" if kv16 else "f32",
           "algorithmic_GB_per_step": round(nbytes / 1e9, 4),
           "GB/s": round(gbs(nbytes, ms), 1), "frac_hbm": round(gbs(nbytes, ms) / HBM_PEAK_GBS, 4)}
    return res, cpu


COPY_BYTES = 1 << 30


_MARKER = {}


def marker_copy(torch, nbytes=COPY_BYTES, reps=1):
    """A plain device-to-device copy of a known size: it scales an HBM byte
    counter (FETCH_SIZE, WRITE_SIZE) to bytes (each launch reads and writes
    exactly `nbytes`) and marks the start and end of the dispatches that a
    counter run sums.  The buffers are made (and filled) on the first call
    only, so no fill lands between two markers."""
    if nbytes not in _MARKER:
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        _MARKER[nbytes] = (src, torch.empty_like(src))
        torch.cuda.synchronize()
    src, dst = _MARKER[nbytes]
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"marker copy: {reps} launch(es) of {nbytes} bytes")


def _pmc_rows(path, counter):
    import csv
    rows = []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    return rows


def _is_copy(name):
    """The runtime's device-to-device copy kernel (what the marker copy runs)."""
    return "copyBuffer" in name


def pmc_traffic(fetch_csv, write_csv, kernel="mv_b1_kernel"):
    """HBM traffic per matvec launch from two rocprofv3 --pmc passes (FETCH_SIZE,
    then WRITE_SIZE; both in KiB per dispatch), each scaled by the ratio of the
    known copy size to what the same counter read for the calibration copy."""
    def per_kernel(path, counter):
        vals = {"mv": [], "copy": []}
        for _, name, v in _pmc_rows(path, counter):
            if kernel in name:
                vals["mv"].append(v)
            elif _is_copy(name) and v * 1024.0 > COPY_BYTES / 4:
                vals["copy"].append(v)
        assert vals["mv"] and vals["copy"], f"{path}: no {counter} rows for both kernels"
        return statistics.median(vals["mv"]), statistics.median(vals["copy"])

    mv_f, cp_f = per_kernel(fetch_csv, "FETCH_SIZE")
    mv_w, cp_w = per_kernel(write_csv, "WRITE_SIZE")
    f_scale = COPY_BYTES / (cp_f * 1024.0)
    w_scale = COPY_BYTES / (cp_w * 1024.0)
    return {"fetch_kib_raw": mv_f, "write_kib_raw": mv_w,
            "copy_fetch_kib_raw": cp_f, "copy_write_kib_raw": cp_w,
            "fetch_scale": f_scale, "write_scale": w_scale,
            "bytes_per_launch": round(mv_f * 1024.0 * f_scale + mv_w * 1024.0 * w_scale)}


def pmc_traffic_span(fetch_csv, write_csv, units):
    """HBM traffic per unit (decode step, attention pass) of the dispatches
    between the two large marker copies, scaled as in pmc_traffic."""
    def span(path, counter):
        rows = _pmc_rows(path, counter)
        marks = [i for i, (_, name, v) in enumerate(rows)
                 if _is_copy(name) and v * 1024.0 > COPY_BYTES / 4]
        assert len(marks) >= 2, f"{path}: expected two marker copies"
        a, b = marks[-2], marks[-1]
        total = sum(v for _, _, v in rows[a + 1:b])
        scale = COPY_BYTES / (statistics.median([rows[a][2], rows[b][2]]) * 1024.0)
        return total, scale, b - a - 1

    f, fs, nd = span(fetch_csv, "FETCH_SIZE")
    w_, ws, _ = span(write_csv, "WRITE_SIZE")
    return {"units": units, "dispatches_per_unit": nd / units, "fetch_scale": fs, "write_scale": ws,
            "bytes_per_unit": round((f * 1024.0 * fs + w_ * 1024.0 * ws) / units),
            "fetch_bytes_per_unit": round(f * 1024.0 * fs / units),
            "write_bytes_per_unit": round(w_ * 1024.0 * ws / units)}


def kernel_source_hash(files=("matvec.hip", "common.hpp")):
    """Digest of kernel sources: stored counter readings are used only while
    the kernels they were taken from are unchanged."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "q4_quantized_matvec_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def all_sources():
    d = os.path.join(ROOT, "q4_quantized_matvec_amd", "csrc")
    return tuple(sorted(f for f in os.listdir(d) if f.endswith((".hip", ".hpp"))))


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


def stored_traffic(key, files=("matvec.hip", "common.hpp")):
    if not os.path.exists(TRAFFIC_JSON):
        return None
    with open(TRAFFIC_JSON) as f:
        t = json.load(f).get(key)
    if not t or t.get("kernel_source") != kernel_source_hash(files):
        return None
    return t


def store_traffic(key, t, files):
    data = json.load(open(TRAFFIC_JSON)) if os.path.exists(TRAFFIC_JSON) else {}
    t["kernel_source"] = kernel_source_hash(files)
    data[key] = t
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(data, f, indent=1)
    print(json.dumps(t))


def host_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity": affinity}


def timed_calls(fn, budget_s, max_reps=20000):
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= max_reps:
            return reps, el


def cpu_matvec(w, batch, budget_s, threads=None):
    """The oracle's matvec on a bounded sample of the workload: as many full
    calls as fit in `budget_s` (at least one)."""
    import oracle
    from synth import workloads as wl
    full = oracle.num_threads()
    W, _ = wl.matvec_inputs(w, 1)
    _, x = wl.matvec_inputs(w, batch)
    if threads:
        oracle.set_num_threads(threads)
    try:
        used = oracle.num_threads()
        reps, el = timed_calls(lambda: oracle.q4_0_matvec(W, w.n, w.k, x), budget_s)
    finally:
        oracle.set_num_threads(full)
    per = el / reps
    return {"value": round(matvec_bytes(w.n, w.k, batch) / per / 1e9, 3), "unit": "GB/s",
            "cores": used, "kind": "oracle", "ms_per_call": round(per * 1e3, 2),
            "sample": f"{reps} full {w.k}x{w.n} B={batch} fp64 matvecs ({el:.1f} s)"}


def cpu_attention(batch, layers, threads=None):
    """The oracle's attention-stack step (QK-norm, RoPE, attention over the
    4096 cached keys and the new one) on a sample of the 28 layers; the pass
    time is the per-layer mean times 28."""
    import numpy as np

    import oracle
    from synth import workloads as wl
    w = wl.ATTN_QWEN3_1P7B
    full = oracle.num_threads()
    hd, pos = w.head_dim, w.n_cache
    if threads:
        oracle.set_num_threads(threads)
    try:
        used = oracle.num_threads()
        el = 0.0
        for l in layers:
            qh, kh, vh, qn, kn, kc, vc = wl.attn_layer_inputs(w, batch, l)
            # position-indexed fp64 copies of the caches, one slot for the new row
            kk = np.empty((batch, pos + 1, w.n_kv_heads, hd))
            vv = np.empty_like(kk)
            kk[:, :pos] = kc[:, :, :pos].transpose(0, 2, 1, 3)
            vv[:, :pos] = vc[:, :, :pos].transpose(0, 2, 1, 3)
            del kc, vc
            t0 = time.perf_counter()
            for b in range(batch):
                qr = oracle.rope_neox(oracle.rmsnorm(qh[b], qn, w.eps), pos, w.rope_theta)
                kk[b, pos] = oracle.rope_neox(oracle.rmsnorm(kh[b], kn, w.eps), pos, w.rope_theta)
                vv[b, pos] = vh[b]
                oracle.gqa_attention(qr, kk[b], vv[b], 0, 1.0 / np.sqrt(hd))
            el += time.perf_counter() - t0
    finally:
        oracle.set_num_threads(full)
    per_pass = el / len(layers) * w.n_layers
    n = pos + 1
    nbytes = w.n_layers * batch * (2 * w.n_kv_heads * hd * n * 4)
    return {"value": round(nbytes / per_pass / 1e9, 3), "unit": "GB/s", "cores": used,
            "kind": "oracle", "ms_per_pass": round(per_pass * 1e3, 1),
            "sample": f"layers {list(layers)} of 28 at B={batch} ({el:.1f} s), pass = mean x 28"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200,
                    help="dispatches per timed window (exactly this many)")
    ap.add_argument("--warmup", type=int, default=2000,
                    help="minimum untimed dispatches (at least 50 ms of GPU work runs regardless)")
    ap.add_argument("--windows", type=int, default=7, help="timed windows per line (median, cv)")
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
    ap.add_argument("--counter-run", metavar="LEG",
                    help="for a --pmc pass: run one leg (a decode workload, or attn_B1 / attn_B8, "
                         "between two marker copies; or matvec_B1_B8) and exit")
    ap.add_argument("--pmc-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="store the headline matvec's counter bytes in profiles/traffic.json")
    ap.add_argument("--pmc-traffic-leg", nargs=3, metavar=("LEG", "FETCH_CSV", "WRITE_CSV"),
                    help="store a --counter-run leg's counter bytes per unit in profiles/traffic.json")
    args = ap.parse_args()
    if args.pmc_traffic:
        t = pmc_traffic(*args.pmc_traffic)
        t["source"] = ("rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE over "
                       "'bench.py --headline-only --copy-calibration --no-cpu-baseline'")
        store_traffic("q4_0_matvec_5376x21504_B1", t, ("matvec.hip", "common.hpp"))
        return
    if args.pmc_traffic_leg:
        leg, fc, wc = args.pmc_traffic_leg
        units = COUNTER_UNITS
        t = pmc_traffic_span(fc, wc, units)
        t["source"] = f"rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE over 'bench.py --counter-run {leg}'"
        store_traffic(f"counter_run_{leg}", t, all_sources())
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
    want_cpu = not args.no_cpu_baseline

    if args.counter_run:
        leg = args.counter_run
        if leg == "matvec_B1_B8":
            res = counter_run_matvec(q, torch)
        elif leg.startswith("attn_B"):
            batch = int(leg[len("attn_B"):])
            res = counter_run_attention(q, torch, batch)
        else:
            m, on_dev, kv16 = legs[leg]
            res = bench_decode(q, torch, m, device_caches=on_dev, kv16=kv16,
                               counter_steps=COUNTER_UNITS)
        print(json.dumps({"counter_run": leg, **res}), flush=True)
        return

    def run_leg(key, oracle_cpu=False):
        m, on_dev, kv16 = legs[key]
        name = m.name + ("_f16kv" if kv16 else "")
        res, cpu = bench_decode(q, torch, m, device_caches=on_dev, kv16=kv16, oracle_cpu=oracle_cpu)
        t = stored_traffic(f"counter_run_{key}", all_sources())
        if t:
            res["counter_GB_per_step"] = round(t["bytes_per_unit"] / 1e9, 4)
            res["counter_over_algorithmic"] = round(
                t["bytes_per_unit"] / (res["algorithmic_GB_per_step"] * 1e9), 3)
        return name, res, cpu

    if args.only_decode:
        print(json.dumps({"decode": {n: r for n, r, _ in (run_leg(k) for k in decode_keys)}}),
              flush=True)
        return

    w = wl.MATVEC_5376x21504
    log(f"generating {args.copies} weight copies of {w.k}x{w.n}")
    Ws = weight_copies(torch, w, args.copies, dev)
    x1, y1 = activations(torch, w, 1, dev)
    torch.cuda.synchronize()

    log("timing B=1")
    t1 = time_windows(torch, matvec_launcher(q, torch, Ws, x1, y1), args.steps, args.warmup,
                      args.windows)
    ms1 = t1["median_ms"]
    bytes1 = matvec_bytes(w.n, w.k, 1)
    gbs1 = gbs(bytes1, ms1)
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
        "timing": dict(t1, dispatches_per_window=args.steps, settle_ms=SETTLE_MS,
                       statistic="median window"),
        "roofline": {"bound": "hbm", "achieved": round(gbs1, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs1 / HBM_PEAK_GBS, 4),
                     "traffic": traffic["bytes_per_launch"] if traffic else None},
        "env": {"device": torch.cuda.get_device_name(0), "hip": torch.version.hip,
                "torch": torch.__version__, "library": q.version(),
                "kernel_source": kernel_source_hash(all_sources())},
    }
    if args.copy_calibration:
        marker_copy(torch, reps=4)
    if not args.headline_only:
        # B = 2..8 through the workspace-free entry point (at B = 2 the vector
        # kernel once per row, W re-read from the caches; from B = 3 on this
        # shape the matrix-core tile kernel without a K split) and through the
        # matrix-core entry point with a workspace
        for bb in (2, 4, 8, 16, 32):
            xb, yb = activations(torch, w, bb, dev)
            nb = matvec_bytes(w.n, w.k, bb)
            if bb <= 8:
                kern = "vector kernel per row" if bb < 3 else "matrix-core tiles, whole K"
                log(f"timing B={bb} (q4_0_matvec, {kern})")
                out[f"matvec_B{bb}_plain_entry"] = line(
                    nb, time_windows(torch, matvec_launcher(q, torch, Ws, xb, yb), args.steps,
                                     args.warmup, args.windows), path=f"q4_0_matvec ({kern})")
            log(f"timing B={bb} (q4_0_matvec_batched, matrix cores)")
            out[f"matvec_B{bb}"] = line(
                nb, time_windows(torch, batched_launcher(q, torch, Ws, xb, yb, w.k, bb), args.steps,
                                 args.warmup, args.windows), path="q4_0_matvec_batched (mfma)")
            del xb, yb
        log("timing B=1 cache-resident (one copy), then as one HIP graph")
        out["matvec_B1_cache_resident"] = line(
            bytes1, time_windows(torch, matvec_launcher(q, torch, Ws[:1], x1, y1), args.steps,
                                 args.warmup, args.windows))
        out["matvec_B1_graph"] = line(
            bytes1, time_graph(torch, lambda: matvec_launcher(q, torch, Ws, x1, y1, check=False),
                               args.steps),
            nodes=args.steps)
        del Ws
        torch.cuda.empty_cache()
        out["matvec_2048x6144"] = bench_small_matvec(q, torch, args, dev)
        if not args.no_attention:
            for kv16 in (False, True):
                key = "attn_qwen3_1p7b" + ("_f16kv" if kv16 else "")
                out[key] = {}
                for bb in (1, 8):
                    log(f"timing the 28-layer attention stack, B={bb}, {'f16' if kv16 else 'f32'} KV")
                    r = bench_attention_stack(q, torch, bb, args.windows, kv16=kv16)
                    t = stored_traffic(f"counter_run_attn_B{bb}", all_sources()) if not kv16 else None
                    if t:
                        r["counter_GB_per_pass"] = round(t["bytes_per_unit"] / 1e9, 4)
                        r["counter_over_algorithmic"] = round(
                            t["bytes_per_unit"] / (r["algorithmic_GB_per_pass"] * 1e9), 3)
                    out[key][f"B{bb}"] = r
        cpu_decode = {}
        if decode_keys:
            out["decode"] = {}
            for key in decode_keys:
                log(f"timing decode {key}")
                name, res, cpu = run_leg(key, oracle_cpu=want_cpu and key in ("qwen3_4b",
                                                                              "gemma4_31b"))
                out["decode"][name] = res
                if cpu:
                    cpu_decode[name] = cpu
    if want_cpu and not args.headline_only:
        log("timing the oracle on the host")
        base = cpu_matvec(w, 1, 10.0)
        base["host"] = host_info()
        per = {"matvec_5376x21504_B1_one_thread": cpu_matvec(w, 1, 4.0, threads=1),
               "matvec_5376x21504_B8": cpu_matvec(w, 8, 4.0),
               "matvec_5376x21504_B8_one_thread": cpu_matvec(w, 8, 4.0, threads=1),
               "matvec_2048x6144": cpu_matvec(wl.MATVEC_2048x6144, 1, 2.0),
               "matvec_2048x6144_one_thread": cpu_matvec(wl.MATVEC_2048x6144, 1, 2.0, threads=1)}
        if not args.no_attention:
            per["attn_qwen3_1p7b_B1"] = cpu_attention(1, (0, 9, 18, 27))
            per["attn_qwen3_1p7b_B1_one_thread"] = cpu_attention(1, (0, 27), threads=1)
        for name, cpu in cpu_decode.items():
            per[name] = cpu
        base["per_workload"] = per
        out["cpu_baseline"] = base
    print(json.dumps(out), flush=True)


COUNTER_UNITS = 4


def counter_run_matvec(q, torch, launches=60, copies=12):
    """The headline shape at B = 1 (q4_0_matvec, vector kernel) then at B = 8
    (q4_0_matvec_batched, matrix cores), `launches` calls each over `copies`
    weight copies, for per-kernel counter passes."""
    from synth import workloads as wl
    w = wl.MATVEC_5376x21504
    dev = torch.device("cuda:0")
    Ws = weight_copies(torch, w, copies, dev)
    x1, y1 = activations(torch, w, 1, dev)
    launch = matvec_launcher(q, torch, Ws, x1, y1)
    for i in range(launches):
        launch(i)
    torch.cuda.synchronize()
    x8, y8 = activations(torch, w, 8, dev)
    launch = batched_launcher(q, torch, Ws, x8, y8, w.k, 8)
    for i in range(launches):
        launch(i)
    torch.cuda.synchronize()
    return {"launches": launches, "copies": copies}


def counter_run_attention(q, torch, batch):
    """COUNTER_UNITS passes of the attention stack between two marker copies."""
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
        kcd = torch.from_numpy(kc).to(dev)
        qkv = np.concatenate([qh.reshape(batch, -1), kh.reshape(batch, -1), vh.reshape(batch, -1)],
                             axis=1)
        layers.append(dict(qkv=torch.from_numpy(np.ascontiguousarray(qkv)).to(dev),
                           qn=torch.from_numpy(qn).to(dev), kn=torch.from_numpy(kn).to(dev),
                           kc=kcd, vc=torch.from_numpy(vc).to(dev), kv=kv_layout_of(kcd)))
    ws = torch.zeros(q.gqa_decode_attn_workspace(layers[0]["kv"], hq, 0), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((batch, hq * hd), dtype=torch.float32, device=dev)
    ld = hq * hd + 2 * hkv * hd

    def one_pass():
        for L in layers:
            q.gqa_decode_attn_rope(L["qkv"], ld, hq, L["qn"], L["kn"], L["kv"], pos_d[0:1],
                                   w.rope_theta, w.eps, False, L["kc"], L["vc"], 0,
                                   1.0 / np.sqrt(hd), out, hq * hd, ws)

    one_pass()
    torch.cuda.synchronize()
    marker_copy(torch)
    for _ in range(COUNTER_UNITS):
        one_pass()
    torch.cuda.synchronize()
    marker_copy(torch)
    return {"counter_passes": COUNTER_UNITS}


if __name__ == "__main__":
    main()
