"""Benchmark of the lossless BF16 coding hot path on one MI355X.

Default (``--workload layerset``): the 96-tensor layer set, 10.87e9 weights
(20.25 GiB of BF16), every container resident in HBM.  One step encodes the
96 tensors (per-tensor dictionary pass, which reads 48 bytes back and waits
for its stream, then encode) and decodes them back to back, in each layout
(byte-split and K15).  ``value`` is the decode kernel's rate: BF16 bytes
rebuilt exactly per second over the timed decode passes of both layouts.
``roofline`` holds that kernel's algorithmic HBM traffic (container read +
BF16 written) per launch over its average launch time, measured with HIP
events on the launch stream around the timed passes, against the 8 TB/s
peak; ``copy_reference`` is a plain device copy that moves the same bytes
per launch, timed the same way (the practical ceiling).  ``gemv_banded``
times the fused decode-GEMV on the banded 6144 x 24576 tensor (5% escapes in
64-row bands) at batches 1, 4 and 16 against the plain BF16 GEMV (own
kernel) and torch's F.linear (hipBLASLt) on the same weights.
``cpu_baseline`` is the CPU oracle, as it stands, decoding a sample of the
same layer set: one tensor slice per host thread on all cores the process
may use, and on one core.

Other workloads (``--workload small|square|mlp|banded``): one step = the
whole path on one tensor per layout (dictionary, encode, decode, fused
GEMV, the two BF16 comparators), with per-call HIP event pairs.

``--bursts`` prints, instead of the bench line, burst timings of decode,
fused GEMV, plain GEMV and F.linear for the chosen workload and batch, in
both escape forms (full and compact): the tables of the design notes come
from it.

Printed: one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("decoded BF16 GB/s (% HBM peak); fused decode-GEMV µs vs BF16 GEMV; "
          "bits/weight")
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
LAYOUT_NAMES = {0: "byte-split", 1: "K15"}
WORKSET_BYTES = 512 << 20  # rotate copies until the inputs span 2x the 256 MB cache
ENC_THREADS = 2  # layer set: host threads (one stream each) that encode tensors side by side
CPU_THREADS_MAX = 16  # the host-core share of one GPU
BURST = 20  # back-to-back launches per timed burst
GEMV_BATCHES = (1, 4, 16)

WORKLOADS = {
    "small": "1024x1024 N(0,0.02), 0.05% entries x1000; batch 1",
    "square": "4096x4096 N(0,0.02), 1% zeros, 0.1% outliers N(0,2); batch 1",
    "mlp": "14336x4096 + 4096x14336, row std 10^U(-4,-1); batch 1",
    "banded": "6144x24576 N(0,0.02) + 5% escapes in 64-row bands; batch 1/4/16",
    "layer": "6144x24576 N(0,0.015), the layer set's first tensor (host draw); batch 1..256",
    "layerset": "96 tensors, 20.25 GiB: 48 x (6144x24576), 24 x (24576x6144) N(0,0.015), "
                "24 x [6144] N(1,0.05); streamed encode + decode, per-tensor dictionaries",
}


def parse(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", choices=sorted(WORKLOADS), default="layerset")
    p.add_argument("--batch", type=int, default=1)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-gemv", action="store_true",
                   help="layer set: skip the banded fused-GEMV section")
    p.add_argument("--cpu-seconds", type=float, default=8.0,
                   help="minimum wall time of each oracle baseline sample")
    p.add_argument("--parity-tensors", type=int, default=8,
                   help="layer set: tensors whose containers the oracle re-encodes and compares")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run one 256 MiB device copy first (a known-size kernel for HBM counters)")
    p.add_argument("--bursts", action="store_true",
                   help="print burst timings (decode, fused/plain GEMV, both escape forms)")
    p.add_argument("--once", action="store_true",
                   help="with --bursts: launch each kernel once instead (for counter runs)")
    return p.parse_args(argv)


def load_workload(name: str, batch: int):
    import synth
    if name == "small":
        d = synth.small()
        return [d["W"]], synth.vectors(synth.SEEDS["small"], batch, 1024)
    if name == "square":
        d = synth.square()
        return [d["W"]], synth.vectors(synth.SEEDS["square"], batch, 4096)
    if name == "mlp":
        m = synth.mlp()
        return [m["W1"], m["W2"]], None
    if name == "banded":
        d = synth.banded()
        # the same draw as the workload's own x, extended to `batch` rows
        return [d["W"]], synth.vectors(synth.SEEDS["banded"], batch, d["W"].shape[1])
    if name == "layer":
        _, W = synth.layerset_tensor(0)
        return [W], synth.vectors(synth.SEEDS["layerset"], batch, W.shape[1])
    raise ValueError(name)


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


DECODE_SOURCES = ["decode_gemv_sign_amd/csrc/wc_decode.hip", "decode_gemv_sign_amd/csrc/wc_tile.h",
                  "decode_gemv_sign_amd/csrc/wc_common.h"]
COUNTERS_JSON = os.path.join(ROOT, "profiles", "decode_counters.json")


def counter_traffic(workload: str, layout_name: str):
    """HBM bytes per decode launch from committed rocprofv3 counter runs, or None
    when absent or taken on a different version of the kernel."""
    if not os.path.exists(COUNTERS_JSON):
        return None
    data = json.load(open(COUNTERS_JSON))
    if data.get("source_hash") != source_hash(DECODE_SOURCES):
        return None
    e = data.get("workloads", {}).get(workload, {}).get(layout_name)
    return None if e is None else float(e["traffic_bytes_per_launch"])


def cpu_threads() -> int:
    """Host threads the oracle baseline uses: the cores this process may run
    on, at most the host-core share of one GPU."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return max(1, min(avail, CPU_THREADS_MAX))


def run_threads(fn, items, nthreads):
    """fn(item) for every item on nthreads host threads (the oracle's ctypes
    calls release the interpreter lock).  Returns results in item order."""
    out = [None] * len(items)
    errors = []
    lock = threading.Lock()
    nxt = [0]

    def worker():
        while True:
            with lock:
                i = nxt[0]
                nxt[0] += 1
            if i >= len(items):
                return
            try:
                out[i] = fn(items[i])
            except Exception as e:  # reported after the join
                errors.append(e)
                return

    ths = [threading.Thread(target=worker) for _ in range(max(1, nthreads))]
    for t in ths:
        t.start()
    for t in ths:
        t.join()
    if errors:
        raise errors[0]
    return out


def median(v):
    v = sorted(v)
    return v[len(v) // 2]


# ---------------------------------------------------------------- the layer set

def oracle_decode_baseline(samples, min_seconds: float):
    """The oracle decoding host copies of layer-set slices: per layout, one
    slice per thread on all cores, then one slice on one core; each repeated
    until min_seconds have passed.  The containers are the oracle's own
    encodes (not timed).  Returns the cpu_baseline object."""
    import oracle
    oracle.build(force=False)
    nt = len(samples)
    res = {}
    tot_bytes = 0.0
    tot_time = 0.0
    one_bytes = 0.0
    one_time = 0.0
    for lay in (0, 1):
        conts = run_threads(lambda w: oracle.encode(lay, w), samples, nt)
        n_each = [w.size for w in samples]
        # all cores: one slice per thread, rounds until min_seconds
        rounds = 0
        t0 = time.perf_counter()
        while True:
            run_threads(oracle.decode, conts, nt)
            rounds += 1
            el = time.perf_counter() - t0
            if el >= min_seconds:
                break
        b = 2.0 * sum(n_each) * rounds
        tot_bytes += b
        tot_time += el
        # one core: the first slice
        r1 = 0
        t0 = time.perf_counter()
        while True:
            oracle.decode(conts[0])
            r1 += 1
            el1 = time.perf_counter() - t0
            if el1 >= min_seconds / 2:
                break
        one_bytes += 2.0 * n_each[0] * r1
        one_time += el1
        res[LAYOUT_NAMES[lay]] = {"all_cores_gbps": round(b / el / 1e9, 4),
                                  "one_core_gbps": round(2.0 * n_each[0] * r1 / el1 / 1e9, 4)}
    rows = samples[0].shape[0]
    return {
        "value": round(tot_bytes / tot_time / 1e9, 4), "unit": "GB/s", "cores": nt,
        "kind": "oracle",
        "sample": (f"oracle decode (plain single-threaded C, one call per thread) of {nt} layer-set "
                   f"slices ({rows} leading rows of {nt} different matrices, "
                   f"{sum(w.size for w in samples) / 1e6:.1f}M weights), both layouts, "
                   f"repeated for >= {min_seconds:.0f} s each; containers from the oracle's "
                   "own encode (not timed)"),
        "one_core": {"value": round(one_bytes / one_time / 1e9, 4), "unit": "GB/s", "cores": 1},
        "host_cpu_count": os.cpu_count(),
        "layouts": res,
    }


def layerset_section(args, wc, torch, dev):
    """Encode + decode of the 96 tensors in both layouts; returns the pieces
    of the bench line."""
    import numpy as np

    import synth
    stream = torch.cuda.current_stream()
    lib = wc._lib
    layouts = [wc.BYTESPLIT, wc.K15]
    tensors, shapes = [], []
    for t in range(synth.LAYERSET_TENSORS):
        _, shape, w = synth.layerset_tensor_device(t, dev)
        tensors.append(w)
        shapes.append(shape)
    n_total = sum(w.numel() for w in tensors)
    nmax = max(w.numel() for w in tensors)
    work = torch.empty(wc.workspace_bytes(nmax), dtype=torch.uint8, device=dev)
    conts = {li: [] for li in layouts}
    hdrs = {li: [] for li in layouts}
    for li in layouts:  # containers allocated once, by a first (untimed) encode
        for w in tensors:
            h = wc.build_dict(w, li, work)
            hdrs[li].append(h)
            conts[li].append(wc.encode_into(h, w, torch.empty(h.total_bytes, dtype=torch.uint8,
                                                               device=dev), work))
    out_buf = torch.empty(nmax, dtype=torch.int16, device=dev)

    # Encode runs from ENC_THREADS host threads, each with its own stream and
    # workspace, so one tensor's dictionary pass (which waits for its stream)
    # overlaps the other threads' GPU work.
    enc_streams = [torch.cuda.Stream(device=dev) for _ in range(ENC_THREADS)]
    enc_work = [torch.empty_like(work) for _ in range(ENC_THREADS)]

    def encode_all(li):
        errors = []

        def worker(i):
            try:
                s = enc_streams[i]
                with torch.cuda.stream(s):
                    for k in range(i, len(tensors), ENC_THREADS):
                        h = wc.build_dict(tensors[k], li, enc_work[i], stream=s)
                        wc.encode_into(h, tensors[k], conts[li][k], enc_work[i], stream=s)
            except Exception as e:  # reported after the join
                errors.append(e)

        for s in enc_streams:  # after the work already queued (sources, earlier decodes)
            s.wait_stream(stream)
        ths = [threading.Thread(target=worker, args=(i,)) for i in range(ENC_THREADS)]
        for th in ths:
            th.start()
        for th in ths:
            th.join()
        for s in enc_streams:
            stream.wait_stream(s)
        if errors:
            raise errors[0]

    # decode calls pre-marshalled, so the host stays ahead of the GPU through
    # the 24 short norm-vector launches
    P = ctypes.c_void_p
    sp = P(stream.cuda_stream)
    dec_calls = {li: [(ctypes.byref(hdrs[li][k]), P(conts[li][k].data_ptr()), conts[li][k].numel(),
                       P(out_buf.data_ptr())) for k in range(len(tensors))] for li in layouts}

    def decode_all(li, check=False):
        ok = True
        for k, w in enumerate(tensors):
            rc = lib.wc_decode(*dec_calls[li][k], sp)
            if rc != 0:
                raise wc.WCError(rc, "wc_decode")
            if check:
                ok = ok and bool(torch.equal(out_buf[:w.numel()], w))
        return ok

    res = {}
    exact = True
    dec_time = {}
    for li in layouts:
        encode_all(li)
        exact = decode_all(li, check=True) and exact
        torch.cuda.synchronize()
        enc, dec = [], []
        for _ in range(args.warmup + args.steps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            encode_all(li)
            torch.cuda.synchronize()
            enc.append(time.perf_counter() - t0)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            decode_all(li)
            b.record(stream)
            b.synchronize()
            dec.append(a.elapsed_time(b) * 1e-3)
        enc_t = median(enc[args.warmup:])
        dec_t = median(dec[args.warmup:])
        dec_time[li] = (dec_t, sum(dec[args.warmup:]), len(dec) - args.warmup)
        cbytes = sum(h.total_bytes for h in hdrs[li])
        res[LAYOUT_NAMES[li]] = {
            "encode_ms": round(1e3 * enc_t, 3),
            "encode_decoded_gbps": round(2 * n_total / enc_t / 1e9, 1),
            "encode_hbm_frac": round((4 * n_total + cbytes) / enc_t / 1e9 / HBM_PEAK_GBPS, 4),
            "decode_ms": round(1e3 * dec_t, 3),
            "decode_decoded_gbps": round(2 * n_total / dec_t / 1e9, 1),
            "decode_hbm_gbps": round((cbytes + 2 * n_total) / dec_t / 1e9, 1),
            "decode_hbm_frac": round((cbytes + 2 * n_total) / dec_t / 1e9 / HBM_PEAK_GBPS, 4),
            "bpw": round(8 * cbytes / n_total, 4),
            "container_bytes": int(cbytes),
            "n_esc": int(sum(h.n_esc for h in hdrs[li])),
        }
    exact = decode_all(layouts[0], check=True) and decode_all(layouts[1], check=True) and exact
    torch.cuda.synchronize()

    # the decode kernel's roofline: algorithmic bytes per launch over the
    # average launch time of the timed passes (96 launches per pass); the
    # slower layout is reported
    launches = len(tensors)
    roof = {}
    for li in layouts:
        alg = (sum(h.total_bytes for h in hdrs[li]) + 2 * n_total) / launches
        t_launch = dec_time[li][1] / dec_time[li][2] / launches
        roof[LAYOUT_NAMES[li]] = {
            "kernel": f"k_decode ({LAYOUT_NAMES[li]})", "bound": "hbm",
            "achieved": round(alg / t_launch / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(alg / t_launch / 1e9 / HBM_PEAK_GBPS, 4),
            "traffic": counter_traffic("layerset", LAYOUT_NAMES[li]),
            "algorithmic_bytes_per_launch": int(alg), "launch_us": round(1e6 * t_launch, 2),
            "launches_per_pass": launches,
            "timing": (f"HIP events on the launch stream around each timed decode pass of the "
                       f"{launches} tensors ({dec_time[li][2]} passes); launch time = pass time / "
                       f"{launches}"),
        }
    worst = min(layouts, key=lambda li: roof[LAYOUT_NAMES[li]]["frac"])
    roofline = dict(roof[LAYOUT_NAMES[worst]])
    roofline["traffic_gbps"] = (round(roofline["traffic"] / (roofline["launch_us"] * 1e-6) / 1e9, 1)
                                if roofline["traffic"] else None)
    roofline["by_layout"] = {k: {"frac": v["frac"], "achieved": v["achieved"],
                                 "launch_us": v["launch_us"], "traffic": v["traffic"]}
                             for k, v in roof.items()}

    # the practical ceiling: a plain device copy moving the same bytes per
    # launch (read + write), rotating over buffers beyond the last-level cache
    per_launch = roofline["algorithmic_bytes_per_launch"]
    half = (per_launch // 2 + 4095) // 4096 * 4096
    nbuf = max(2, -(-WORKSET_BYTES // half))
    bufs = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(nbuf + 1)]
    for i in range(nbuf):
        bufs[i + 1].copy_(bufs[i])
    torch.cuda.synchronize()
    times = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(BURST):
            j = i % nbuf
            bufs[j + 1].copy_(bufs[j])
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3 / BURST)
    tc = median(times)
    copy_ref = {"bytes_read_plus_written": 2 * half, "us": round(1e6 * tc, 2),
                "gbps": round(2 * half / tc / 1e9, 1),
                "frac": round(2 * half / tc / 1e9 / HBM_PEAK_GBPS, 4),
                "decode_vs_copy": round(roofline["achieved"] / (2 * half / tc / 1e9), 4),
                "timing": f"torch copy_ of {half} bytes, median of 5 bursts of {BURST}"}
    del bufs

    # oracle parity of the containers on a spread of the set's tensors, and
    # host copies for the CPU baseline
    parity = exact
    host = {}
    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        k = max(0, min(args.parity_tensors, len(tensors)))
        picks = sorted({int(round(i * (len(tensors) - 1) / max(1, k - 1))) for i in range(k)}) if k else []
        items = []
        for t in picks:
            src = tensors[t].cpu().numpy().view(np.uint16)
            for li in layouts:
                items.append((t, li, src, conts[li][t].cpu().numpy()))

        def cmp(it):
            t, li, src, got = it
            return bool(np.array_equal(got, oracle.encode(li, src)))
        oks = run_threads(cmp, items, cpu_threads())
        parity = parity and all(oks)
        host["parity_tensors"] = picks
    return {"layouts": res, "roofline": roofline, "copy_reference": copy_ref, "exact": exact,
            "parity": parity, "n_total": n_total, "tensors": tensors, "shapes": shapes,
            "host": host}


def gemv_section(args, wc, torch, dev):
    """Fused decode-GEMV on the banded 6144 x 24576 tensor at batches 1, 4, 16
    against the plain BF16 GEMV and F.linear, in bursts over rotating copies;
    outputs checked against the oracle on sampled rows."""
    import numpy as np

    import synth
    d = synth.banded()
    W = d["W"]
    rows, cols = W.shape
    X = d["X"]  # 16 rows; batches 1 and 4 take its leading rows
    stream = torch.cuda.current_stream()
    lib = wc._lib
    P = ctypes.c_void_p
    sp = P(stream.cuda_stream)
    copies = 2  # 2 x (302 MB + 2 containers) > 512 MiB
    Wd = [torch.from_numpy(W.reshape(-1).view(np.int16)).to(dev) for _ in range(copies)]
    Wbf = [w.view(torch.bfloat16).view(rows, cols) for w in Wd]
    work = torch.empty(wc.workspace_bytes(W.size), dtype=torch.uint8, device=dev)
    layouts = [wc.BYTESPLIT, wc.K15]
    hc = {}
    for li in layouts:
        h = wc.build_dict(Wd[0], li, work)
        cs = [wc.encode_into(h, w, torch.empty(h.total_bytes, dtype=torch.uint8, device=dev), work)
              for w in Wd]
        hc[li] = (h, cs)
    Xd = torch.from_numpy(X.view(np.int16)).to(dev)
    Xbf = Xd.view(torch.bfloat16)
    out = {"workload": f"banded: {WORKLOADS['banded']}", "rows": rows, "cols": cols,
           "timing": f"HIP events on the launch stream around {BURST} back-to-back launches over "
                     f"{copies} rotating copies; median of 5 bursts; µs per launch",
           "batches": {}}
    ys = {}

    def burst(fn):
        for i in range(3):
            fn(i % copies)
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(BURST):
                fn(i % copies)
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / BURST)
        return median(ts)

    for B in GEMV_BATCHES:
        y = torch.empty((B, rows), dtype=torch.float32, device=dev)
        yb = torch.empty((B, rows), dtype=torch.float32, device=dev)
        xb = Xd[:B].contiguous()
        xbf = Xbf[:B].contiguous()

        def plain(k):
            rc = lib.wc_gemv_bf16(P(Wd[k].data_ptr()), rows, cols, P(xb.data_ptr()), B,
                                  P(yb.data_ptr()), sp)
            if rc != 0:
                raise wc.WCError(rc, "wc_gemv_bf16")

        t_plain = burst(plain)
        t_lin = burst(lambda k: torch.nn.functional.linear(xbf, Wbf[k]))
        entry = {"plain_bf16_us": round(t_plain, 2), "torch_linear_us": round(t_lin, 2)}
        for li in layouts:
            h, cs = hc[li]

            def fused(k, h=h, cs=cs):
                rc = lib.wc_decode_gemv(ctypes.byref(h), P(cs[k].data_ptr()), cs[k].numel(), rows,
                                        cols, P(xb.data_ptr()), B, P(y.data_ptr()), sp)
                if rc != 0:
                    raise wc.WCError(rc, "wc_decode_gemv")

            t_f = burst(fused)
            fused(0)
            torch.cuda.synchronize()
            ys[(li, B)] = y.cpu().numpy()
            entry[LAYOUT_NAMES[li]] = {
                "fused_us": round(t_f, 2),
                "fused_vs_best_bf16": round(t_f / min(t_plain, t_lin), 4),
                "fused_hbm_gbps": round((h.total_bytes + 2 * cols * B + 4 * rows * B) / t_f / 1e3, 1),
                "bpw": round(8 * h.total_bytes / W.size, 4),
            }
        out["batches"][str(B)] = entry
    parity = True
    if not args.no_cpu_baseline:
        import oracle
        from tests.tolerance import gemv_excess
        oracle.build(force=False)
        bands = [int(b) for b in d["bands"]]
        rs = sorted(set(list(range(0, 64)) + list(range(bands[0] * 64, bands[0] * 64 + 64)) +
                        list(np.random.default_rng(7).choice(rows, 64, replace=False))))
        y64, a = oracle.gemv_f64(np.ascontiguousarray(W[rs]), X)
        for (li, B), yv in ys.items():
            if not np.all(gemv_excess(yv[:, rs], y64[:B], a[:B]) <= 1.0):
                parity = False
        out["parity_rows_checked"] = len(rs)
    out["parity_vs_oracle"] = "ok" if parity else "FAILED"
    return out, parity


def calibration_copy(torch, dev):
    """One device-to-device copy of a known size (256 MiB read and written):
    the counter runs scale FETCH_SIZE / WRITE_SIZE by what they read for it.
    Then a timed burst of the same copy, the practical rate of a plain
    read+write stream."""
    a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e3 / 10
    return {"bytes_read_plus_written": 2 * a.numel(), "us": round(t, 2),
            "gbps": round(2 * a.numel() / t / 1e3, 1),
            "frac": round(2 * a.numel() / t / 1e3 / HBM_PEAK_GBPS, 4)}


def run_layerset(args):
    import numpy as np
    import torch

    import decode_gemv_sign_amd as wc

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_start = time.perf_counter()
    calib = calibration_copy(torch, dev) if args.calibrate_copy else None
    ls = layerset_section(args, wc, torch, dev)
    n_total = ls["n_total"]
    dec_ms = sum(r["decode_ms"] for r in ls["layouts"].values())
    value = 2.0 * n_total * len(ls["layouts"]) / (dec_ms * 1e-3) / 1e9
    hbm = sum(r["container_bytes"] + 2 * n_total for r in ls["layouts"].values()) / (dec_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(sum(r["encode_ms"] + r["decode_ms"] for r in ls["layouts"].values()), 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u16",
        "data": "synthetic",
        "config": {"workload": f"layerset: {WORKLOADS['layerset']}", "weights": int(n_total),
                   "layouts": list(ls["layouts"]),
                   "value_definition": "BF16 bytes rebuilt exactly (2 x weights per layout) / "
                                       "time of the decode passes over all 96 containers, both "
                                       "layouts (medians over the timed steps); a step encodes "
                                       "and decodes all 96 tensors per layout",
                   "value_hbm_frac": round(hbm / HBM_PEAK_GBPS, 4)},
        "roofline": ls["roofline"],
        "copy_reference": ls["copy_reference"],
        "layouts": ls["layouts"],
        "decode_exact": ls["exact"],
    }
    if calib is not None:
        out["calibration_copy"] = calib
    parity = ls["parity"]
    if not args.no_gemv:
        g, gp = gemv_section(args, wc, torch, dev)
        out["gemv_banded"] = g
        parity = parity and gp
    if not args.no_cpu_baseline:
        # host slices of the set's matrices for the oracle: the leading rows
        # of one matrix per thread, about 12.6M weights each
        nt = cpu_threads()
        mats = [t for t in range(len(ls["tensors"])) if len(ls["shapes"][t]) == 2]
        picks = [mats[int(i * len(mats) / nt)] for i in range(nt)]
        samples = []
        for t in picks:
            r, c = ls["shapes"][t]
            keep = max(1, (12_582_912 // c))
            samples.append(ls["tensors"][t][:keep * c].cpu().numpy().view(np.uint16).reshape(keep, c))
        del ls["tensors"]
        torch.cuda.empty_cache()
        out["cpu_baseline"] = oracle_decode_baseline(samples, args.cpu_seconds)
        out["parity_tensors_oracle"] = ls["host"].get("parity_tensors")
    else:
        out["cpu_baseline"] = None
    out["parity_vs_oracle"] = "ok" if parity else "FAILED"
    out["wall_s"] = round(time.perf_counter() - t_start, 1)
    print(json.dumps(out), flush=True)
    if not parity:
        sys.exit(1)


# ---------------------------------------------------------------- one tensor

def cpu_baseline_single(mats, xs, layouts, min_seconds: float, gpu_results):
    """The oracle, as it stands, on the same tensors: encode, decode and GEMV per
    layout, repeated until min_seconds have passed.  Also cross-checks the GPU
    step's outputs against it (containers byte-identical, GEMV within bound)."""
    import numpy as np

    import oracle
    from tests.tolerance import gemv_excess
    oracle.build(force=False)
    parity = True
    for (li, mi), res in gpu_results.items():
        W = mats[mi]
        ref = oracle.encode(layouts[li], W)
        if not np.array_equal(res["container"], ref):
            parity = False
        y64, a = oracle.gemv_f64(W, xs[mi])
        if not np.all(gemv_excess(res["y"], y64, a) <= 1.0):
            parity = False
    steps = 0
    t0 = time.perf_counter()
    while True:
        for mi, W in enumerate(mats):
            for lay in layouts:
                c = oracle.encode(lay, W)
                oracle.decode(c)
                oracle.gemv_f32(W, xs[mi])
        steps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    n_total = sum(W.size for W in mats)
    value = 2.0 * n_total * len(layouts) * steps / el / 1e9
    return {"value": round(value, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} full steps of the same workload ({el:.1f} s): per layout, "
                      f"oracle encode + decode + fp32 GEMV; single-threaded C",
            "host_cpu_count": os.cpu_count(),
            "ms_per_step": round(1e3 * el / steps, 3)}, parity


def prepare_single(args, wc, torch, dev):
    import numpy as np

    import synth
    mats, x = load_workload(args.workload, args.batch)
    if x is None:
        xs = [synth.vectors(synth.SEEDS[args.workload] * 10 + i, args.batch, W.shape[1])
              for i, W in enumerate(mats)]
    else:
        xs = [x]
    # the library is called with args.batch: every x must hold exactly that
    # many rows of its matrix's columns
    for W, xx in zip(mats, xs):
        if xx.shape != (args.batch, W.shape[1]):
            raise SystemExit(f"x has shape {xx.shape}, expected ({args.batch}, {W.shape[1]})")
    in_bytes = sum(W.nbytes for W in mats)
    copies = max(1, -(-WORKSET_BYTES // in_bytes))

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    Wd = [[to_dev(W.reshape(-1)) for W in mats] for _ in range(copies)]
    Xd = [to_dev(xx) for xx in xs]
    return mats, xs, copies, Wd, Xd


def run_single(args):
    import numpy as np
    import torch

    import decode_gemv_sign_amd as wc

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mats, xs, copies, Wd, Xd = prepare_single(args, wc, torch, dev)
    layouts = [wc.BYTESPLIT, wc.K15]
    Xbf = [xd.view(torch.bfloat16) for xd in Xd]
    Wbf = [[w.view(torch.bfloat16).view(W.shape) for w, W in zip(row, mats)] for row in Wd]
    work = [torch.empty(wc.workspace_bytes(max(W.size for W in mats)), dtype=torch.uint8,
                        device=dev) for _ in range(copies)]
    # container sizes are fixed by the data: size them with one dictionary pass
    hdr0 = {(li, mi): wc.build_dict(Wd[0][mi], lay, work[0]) for li, lay in enumerate(layouts)
            for mi in range(len(mats))}
    cont = [{k: torch.empty(h.total_bytes, dtype=torch.uint8, device=dev) for k, h in hdr0.items()}
            for _ in range(copies)]
    dec = [[torch.empty(W.size, dtype=torch.int16, device=dev) for W in mats] for _ in range(copies)]
    yf = {k: torch.empty((args.batch, mats[k[1]].shape[0]), dtype=torch.float32, device=dev)
          for k in hdr0}
    yb = [torch.empty((args.batch, W.shape[0]), dtype=torch.float32, device=dev) for W in mats]
    # Per-call argument tuples are built once, so that after the dictionary
    # pass (which waits for the GPU) the remaining calls of a step reach the
    # stream a few microseconds apart: the GPU keeps a backlog and each event
    # pair brackets only its own kernel.
    lib = wc._lib
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = ctypes.c_void_p

    def ptr(t):
        return P(t.data_ptr())

    def check(rc, what):
        if rc != 0:
            raise wc.WCError(rc, what)

    def step(s, events):
        k = s % copies
        out = {}

        def ev():
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            return e

        for mi in range(len(mats)):
            rows, cols = mats[mi].shape
            hs = {}
            for li, lay in enumerate(layouts):
                # the dictionary pass waits for its own work only: earlier
                # queued work is finished first, outside its timer
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                hs[li] = wc.build_dict(Wd[k][mi], lay, work[k])
                if events is not None:
                    events.setdefault(("build_dict", (li, mi)), []).append(time.perf_counter() - t0)
            marks = []
            for li in range(len(layouts)):
                h = hs[li]
                c = cont[k][(li, mi)]
                marks.append(("encode", (li, mi), ev()))
                check(lib.wc_encode(ctypes.byref(h), ptr(Wd[k][mi]), ptr(c), c.numel(), ptr(work[k]),
                                    work[k].numel(), stream), "wc_encode")
            for li in range(len(layouts)):
                h = hs[li]
                c = cont[k][(li, mi)]
                marks.append(("decode", (li, mi), ev()))
                check(lib.wc_decode(ctypes.byref(h), ptr(c), c.numel(), ptr(dec[k][mi]), stream),
                      "wc_decode")
            for li in range(len(layouts)):
                h = hs[li]
                c = cont[k][(li, mi)]
                marks.append(("decode_gemv", (li, mi), ev()))
                check(lib.wc_decode_gemv(ctypes.byref(h), ptr(c), c.numel(), rows, cols, ptr(Xd[mi]),
                                         args.batch, ptr(yf[(li, mi)]), stream), "wc_decode_gemv")
            marks.append(("gemv_bf16", (None, mi), ev()))
            check(lib.wc_gemv_bf16(ptr(Wd[k][mi]), rows, cols, ptr(Xd[mi]), args.batch, ptr(yb[mi]),
                                   stream), "wc_gemv_bf16")
            marks.append(("torch_linear", (None, mi), ev()))
            torch.nn.functional.linear(Xbf[mi], Wbf[k][mi])
            end = ev()
            if events is not None:
                for i, (name, key, e0) in enumerate(marks):
                    e1 = marks[i + 1][2] if i + 1 < len(marks) else end
                    events.setdefault((name, key), []).append((e0, e1))
            for li in range(len(layouts)):
                out[(li, mi)] = hs[li]
        return out

    copy_ref = calibration_copy(torch, dev) if args.calibrate_copy else None

    for s in range(args.warmup):
        step(s, None)
    events = {}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hdrs = None
    for s in range(args.steps):
        hdrs = step(args.warmup + s, events)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # every copy the steps decoded must equal its input bit for bit
    for k in range(min(copies, args.warmup + args.steps)):
        for mi in range(len(mats)):
            if not torch.equal(dec[k][mi], Wd[k][mi]):
                raise SystemExit(f"decode is not exact (copy {k}, tensor {mi})")

    # Launch durations of the decode kernel for the roofline: a burst of
    # back-to-back calls over the rotating copies between one event pair (in a
    # step, the event pair around one call also spans the queue's dispatch gap
    # before that kernel, which is large next to a 10-20 us kernel).
    burst = {}
    for mi in range(len(mats)):
        for li in range(len(layouts)):
            h = hdrs[(li, mi)]
            calls = [(ctypes.byref(h), ptr(cont[k][(li, mi)]), cont[k][(li, mi)].numel(),
                      ptr(dec[k][mi])) for k in range(copies)]
            for i in range(3):
                check(lib.wc_decode(*calls[i % copies], stream), "wc_decode")
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(BURST):
                check(lib.wc_decode(*calls[i % copies], stream), "wc_decode")
            e1.record()
            torch.cuda.synchronize()
            burst[(li, mi)] = e0.elapsed_time(e1) * 1e3 / BURST

    n_total = sum(W.size for W in mats)
    ms_step = 1e3 * wall / args.steps

    def avg_us(name, key):
        ev = events[(name, key)]
        if name == "build_dict":  # host wall time, including its wait for the GPU
            return 1e6 * sum(ev) / len(ev)
        return 1e3 * sum(e0.elapsed_time(e1) for e0, e1 in ev) / len(ev)

    kernels = {}
    roofline = None
    bpw = {}
    dec_total_us = 0.0
    for (li, mi), h in sorted(hdrs.items()):
        lname = LAYOUT_NAMES[layouts[li]]
        tag = lname if len(mats) == 1 else f"{lname}/W{mi + 1}"
        rows, cols = mats[mi].shape
        n = mats[mi].size
        b, p = wc.bits_per_weight(h)
        bpw[tag] = {"bpw": round(b, 4), "payload_bpw": round(p, 4),
                    "saving": round(1 - b / 16, 5), "n_esc": int(h.n_esc),
                    "escape_frac": round(h.n_esc / n, 6)}
        # the same tensor in the compact escape form (symbols only): header only
        hc = wc.build_dict(Wd[0][mi], layouts[li] | wc.COMPACT, work[0])
        bc, pc = wc.bits_per_weight(hc)
        bpw[tag]["compact_bpw"] = round(bc, 4)
        bpw[tag]["compact_payload_bpw"] = round(pc, 4)
        t_dec = avg_us("decode", (li, mi))
        t_burst = burst[(li, mi)]
        dec_total_us += t_burst
        dec_bytes = h.total_bytes + 2 * n
        t_gemv = avg_us("decode_gemv", (li, mi))
        gemv_bytes = h.total_bytes + 2 * cols * args.batch + 4 * rows * args.batch
        t_bf = avg_us("gemv_bf16", (None, mi))
        t_lin = avg_us("torch_linear", (None, mi))
        kernels[tag] = {
            "build_dict_host_us": round(avg_us("build_dict", (li, mi)), 2),
            "encode_us": round(avg_us("encode", (li, mi)), 2),
            "decode_us": round(t_dec, 2),
            "decode_burst_us": round(t_burst, 2),
            "decode_decoded_gbps": round(2 * n / t_burst / 1e3, 1),
            "decode_hbm_gbps": round(dec_bytes / t_burst / 1e3, 1),
            "decode_hbm_frac": round(dec_bytes / t_burst / 1e3 / HBM_PEAK_GBPS, 4),
            "decode_gemv_us": round(t_gemv, 2),
            "decode_gemv_hbm_gbps": round(gemv_bytes / t_gemv / 1e3, 1),
            "gemv_bf16_us": round(t_bf, 2),
            "torch_linear_us": round(t_lin, 2),
            "fused_vs_best_bf16": round(t_gemv / min(t_bf, t_lin), 4),
        }
        if roofline is None or t_burst > roofline["_t"]:
            roofline = {"_t": t_burst, "kernel": f"k_decode ({tag})", "bound": "hbm",
                        "achieved": round(dec_bytes / t_burst / 1e3, 1), "peak": HBM_PEAK_GBPS,
                        "unit": "GB/s", "frac": round(dec_bytes / t_burst / 1e3 / HBM_PEAK_GBPS, 4),
                        "traffic": counter_traffic(args.workload, tag),
                        "algorithmic_bytes_per_launch": int(dec_bytes),
                        "launch_us": round(t_burst, 2),
                        "timing": f"HIP events around {BURST} back-to-back launches"}
    roofline.pop("_t")
    roofline["traffic_gbps"] = (round(roofline["traffic"] / roofline["launch_us"] / 1e3, 1)
                                if roofline["traffic"] else None)
    # value: the decode kernel's rate over both layouts (burst launch times)
    value = 2.0 * n_total * len(layouts) / dec_total_us / 1e3

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {WORKLOADS[args.workload]}",
                   "layouts": [LAYOUT_NAMES[l] for l in layouts], "batch": args.batch,
                   "weights": int(n_total), "rotating_copies": copies,
                   "value_definition": "BF16 bytes rebuilt exactly by the decode kernel (2 x "
                                       "weights per layout) / its launch time (bursts of "
                                       f"{BURST}), both layouts; a step = dictionary + encode + "
                                       "decode + fused GEMV per layout, plus both BF16 GEMV "
                                       "comparators"},
        "roofline": roofline,
        "copy_reference": copy_ref,
        "kernels": kernels,
        "bits_per_weight": bpw,
    }
    if not args.no_cpu_baseline:
        gpu_results = {}
        for (li, mi) in hdrs:
            c = cont[(args.warmup + args.steps - 1) % copies][(li, mi)].cpu().numpy()
            y = yf[(li, mi)].cpu().numpy()
            gpu_results[(li, mi)] = {"container": c, "y": y}
        cb, parity = cpu_baseline_single([np.ascontiguousarray(W) for W in mats], xs, layouts,
                                         args.cpu_seconds, gpu_results)
        out["cpu_baseline"] = cb
        out["parity_vs_oracle"] = "ok" if parity else "FAILED"
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    if out.get("parity_vs_oracle") == "FAILED":
        sys.exit(1)


# ---------------------------------------------------------------- bursts

def run_bursts(args):
    """Burst timings for one workload and batch, both layouts, full and
    compact escape forms: decode, fused GEMV, plain GEMV, F.linear (µs per
    launch, median of 5 bursts over rotating copies).  Outputs are checked:
    decode bit-exact, fused GEMV equal (bitwise) between the two forms."""
    import numpy as np
    import torch

    import decode_gemv_sign_amd as wc

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mats, xs, copies, Wd, Xd = prepare_single(args, wc, torch, dev)
    stream = torch.cuda.current_stream()
    lib = wc._lib
    P = ctypes.c_void_p
    sp = P(stream.cuda_stream)
    work = torch.empty(wc.workspace_bytes(max(W.size for W in mats)), dtype=torch.uint8, device=dev)

    def burst(fn):
        if args.once:  # one launch of each kernel, for counter runs
            fn(0)
            torch.cuda.synchronize()
            return float("nan")
        for i in range(3):
            fn(i % copies)
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(BURST):
                fn(i % copies)
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / BURST)
        return median(ts)

    rows_out = []
    for mi, W in enumerate(mats):
        rows, cols = W.shape
        B = args.batch
        yb = torch.empty((B, rows), dtype=torch.float32, device=dev)
        Wbf = [Wd[k][mi].view(torch.bfloat16).view(rows, cols) for k in range(copies)]
        xbf = Xd[mi].view(torch.bfloat16)
        t_plain = burst(lambda k: lib.wc_gemv_bf16(P(Wd[k][mi].data_ptr()), rows, cols,
                                                   P(Xd[mi].data_ptr()), B, P(yb.data_ptr()), sp))
        t_lin = burst(lambda k: torch.nn.functional.linear(xbf, Wbf[k]))
        for li in (wc.BYTESPLIT, wc.K15):
            yref = None
            for form in (0, wc.COMPACT):
                h = wc.build_dict(Wd[0][mi], li | form, work)
                cs = [wc.encode_into(h, Wd[k][mi], torch.empty(h.total_bytes, dtype=torch.uint8,
                                                                device=dev), work)
                      for k in range(copies)]
                outb = torch.empty(W.size, dtype=torch.int16, device=dev)
                y = torch.empty((B, rows), dtype=torch.float32, device=dev)
                t_enc = burst(lambda k: lib.wc_encode(ctypes.byref(h), P(Wd[k][mi].data_ptr()),
                                                      P(cs[k].data_ptr()), cs[k].numel(),
                                                      P(work.data_ptr()), work.numel(), sp))
                t_dec = burst(lambda k: lib.wc_decode(ctypes.byref(h), P(cs[k].data_ptr()),
                                                      cs[k].numel(), P(outb.data_ptr()), sp))
                t_f = burst(lambda k: lib.wc_decode_gemv(ctypes.byref(h), P(cs[k].data_ptr()),
                                                         cs[k].numel(), rows, cols,
                                                         P(Xd[mi].data_ptr()), B, P(y.data_ptr()),
                                                         sp))
                torch.cuda.synchronize()
                exact = bool(torch.equal(outb, Wd[0][mi])) if copies else True
                # the containers the encode bursts rewrote must still decode exactly
                for k in range(copies):
                    wc.decode(h, cs[k], out=outb)
                    exact = exact and bool(torch.equal(outb, Wd[k][mi]))
                # the last launch ran on copy (BURST - 1) % copies; all copies are equal
                if yref is None:
                    yref = y.clone()
                neq = y.view(torch.int32) != yref.view(torch.int32)
                same = not bool(neq.any())
                diff = []
                if not same:
                    for b_, r_ in torch.nonzero(neq)[:4].cpu().tolist():
                        diff.append([b_, r_, float(y[b_, r_]), float(yref[b_, r_])])
                rows_out.append({
                    "tensor": mi, "layout": LAYOUT_NAMES[li], "form": "compact" if form else "full",
                    "bpw": round(8 * h.total_bytes / W.size, 4),
                    "encode_us": round(t_enc, 2),
                    "encode_hbm_frac": round((2 * W.size + h.total_bytes) / t_enc / 1e3 / HBM_PEAK_GBPS, 4),
                    "decode_us": round(t_dec, 2),
                    "decode_hbm_frac": round((h.total_bytes + 2 * W.size) / t_dec / 1e3 / HBM_PEAK_GBPS, 4),
                    "fused_us": round(t_f, 2), "plain_bf16_us": round(t_plain, 2),
                    "torch_linear_us": round(t_lin, 2),
                    "fused_vs_best_bf16": round(t_f / min(t_plain, t_lin), 4),
                    "decode_exact": exact, "gemv_same_as_full": same, "gemv_first_diffs": diff})
    print(json.dumps({"workload": f"{args.workload}: {WORKLOADS[args.workload]}", "batch": args.batch,
                      "timing": f"median of 5 bursts of {BURST} launches over {copies} rotating copies",
                      "rows": rows_out}), flush=True)
    if not all(r["decode_exact"] and r["gemv_same_as_full"] for r in rows_out):
        sys.exit(1)


# ---------------------------------------------------------------- counters

def _read_counters(path):
    """rocprofv3 counter CSV -> list of (kernel name, grid size, value) per
    dispatch, in dispatch order."""
    import csv
    files = [os.path.join(path, f) for f in sorted(os.listdir(path))
             if f.endswith("counter_collection.csv")]
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {path}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Grid_Size"]),
                             float(r["Counter_Value"])))
    rows.sort()
    return [(k, g, v) for _, k, g, v in rows]


def summarize_counters(fetch_dir, write_dir, workload, md_out=None, command=""):
    """HBM bytes per launch of the decode kernel from a FETCH_SIZE run and a
    WRITE_SIZE run (KiB per dispatch), each scaled by what the counter reads
    for the 256 MiB calibration copy at the start of the run; written into
    profiles/decode_counters.json for `workload` with the decode sources'
    hash.  With md_out, also a per-kernel table (medians per dispatch)."""
    F = _read_counters(fetch_dir)
    W = _read_counters(write_dir)

    def calib(rows):
        cps = [(g, v) for k, g, v in rows if k.startswith("__amd_rocclr_copyBuffer")]
        gmax = max(g for g, _ in cps)
        return next(v for g, v in cps if g == gmax)
    kib = 256 * 1024
    fs, ws = kib / calib(F), kib / calib(W)

    def per_kernel(rows):
        d = {}
        for k, g, v in rows:
            d.setdefault(k, []).append(v)
        return d
    pf, pw = per_kernel(F), per_kernel(W)
    entry = {}
    for lay, tag in ((0, "byte-split"), (1, "K15")):
        names = [k for k in pf if k.startswith(f"void wc::k_decode<{lay},")]
        fv = [v for k in names for v in pf[k]]
        wv = [v for k in names for v in pw.get(k, [])]
        if not fv or not wv:
            continue
        rb = 1024 * fs * sum(fv) / len(fv)
        wb = 1024 * ws * sum(wv) / len(wv)
        entry[tag] = {"traffic_bytes_per_launch": round(rb + wb), "read_bytes": round(rb),
                      "write_bytes": round(wb), "launches": len(fv), "kernels": names}
    data = {}
    if os.path.exists(COUNTERS_JSON):
        data = json.load(open(COUNTERS_JSON))
    h = source_hash(DECODE_SOURCES)
    if data.get("source_hash") != h:
        data = {"source_hash": h, "workloads": {}}
    data["fetch_scale"] = round(fs, 4)
    data["write_scale"] = round(ws, 4)
    data.setdefault("workloads", {})[workload] = entry
    with open(COUNTERS_JSON, "w") as fh:
        json.dump(data, fh, indent=1)
    if md_out:
        lines = [f"Commands: {command}", "",
                 f"Calibration: FETCH_SIZE x {fs:.4f}, WRITE_SIZE x {ws:.4f} (a 256 MiB copy reads "
                 "and writes 262144 KiB).  Medians per dispatch.", "",
                 "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB (scaled) | "
                 "write MB (scaled) |", "|---|---|---|---|---|---|"]
        for k in sorted(pf, key=lambda k: -sum(pf[k])):
            f_med = median(pf[k])
            w_med = median(pw.get(k, [0.0]))
            lines.append(f"| `{k[:70]}` | {len(pf[k])} | {f_med:.1f} | {w_med:.1f} | "
                         f"{1024 * fs * f_med / 1e6:.2f} | {1024 * ws * w_med / 1e6:.2f} |")
        lines += ["", "Decode per launch (means over the run's decode dispatches):", ""]
        for tag, e in entry.items():
            lines.append(f"* {tag}: read {e['read_bytes'] / 1e6:.2f} MB, write "
                         f"{e['write_bytes'] / 1e6:.2f} MB, total {e['traffic_bytes_per_launch'] / 1e6:.2f} MB "
                         f"per launch ({e['launches']} launches)")
        with open(md_out, "w") as fh:
            fh.write("\n".join(lines) + "\n")
    print(json.dumps({"workload": workload, "fetch_scale": fs, "write_scale": ws, "decode": entry}))


def summarize_trace(stats_csv, md_out, command, bench_json=None):
    """Markdown table of a `rocprofv3 --kernel-trace --stats` run's per-kernel
    statistics; with the profiled run's bench line, the decode kernel's mean
    launch time over the trace beside the one the bench line reports."""
    import csv
    with open(stats_csv, newline="") as fh:
        rows = list(csv.DictReader(fh))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    line = json.loads(open(bench_json).read().strip().splitlines()[-1]) if bench_json else None
    lines = [f"Command: {command}", ""]
    if line:
        lines += [f"Workload: {line['config']['workload']}", ""]
    lines += ["| kernel | calls | avg µs | min µs | max µs | % GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{r['Name'][:80]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} |")
    if line:
        roof = line.get("roofline") or {}
        by = roof.get("by_layout") or {}
        if not by and roof.get("kernel"):  # one tensor: the slower layout only
            by = {roof["kernel"].split("(")[1].rstrip(")"): {"launch_us": roof["launch_us"]}}
        lines += ["", "Decode launch time, the trace against the bench line of the same run "
                  "(the trace's mean covers every decode launch of the run):", ""]
        for lay, tag in ((0, "byte-split"), (1, "K15")):
            ks = [r for r in rows if r["Name"].startswith(f"void wc::k_decode<{lay},")]
            calls = sum(int(r["Calls"]) for r in ks)
            if not calls or tag not in by:
                continue
            avg = sum(float(r["TotalDurationNs"]) for r in ks) / calls / 1e3
            lines.append(f"* {tag}: trace mean {avg:.2f} µs over {calls} launches "
                         f"({', '.join(r['Name'].split('(')[0] for r in ks)}); bench "
                         f"launch_us {by[tag]['launch_us']} (ratio {by[tag]['launch_us'] / avg:.3f})")
    with open(md_out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def summarize_instructions(pmc_dir, md_out, tiles, command):
    """Per-kernel instruction counts of a `rocprofv3 --pmc SQ_...` run of
    `bench.py --bursts --once` (one launch of each kernel per layout and
    form, in that order): counts per 2048-weight tile of the tensor."""
    import csv
    files = [os.path.join(pmc_dir, f) for f in sorted(os.listdir(pmc_dir))
             if f.endswith("counter_collection.csv")]
    disp = {}
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                d = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"]})
                d[r["Counter_Name"]] = float(r["Counter_Value"])
    names = sorted({c for d in disp.values() for c in d if c != "name"})
    lines = [f"Command: {command}", "",
             f"Counts per dispatch divided by the tensor's {tiles} tiles of 2048 weights "
             "(dispatches in launch order: per layout, full then compact form: encode kernels, "
             "decode, fused GEMV; the plain kernels once per layout).", "",
             "| dispatch | kernel | " + " | ".join(n + " / tile" for n in names) + " |",
             "|---|---|" + "---|" * len(names)]
    for k in sorted(disp):
        d = disp[k]
        if not d["name"].startswith(("void wc::k_decode", "wc::k_decode", "void wc::k_gemv",
                                     "void wc::k_gemm")):
            continue
        lines.append(f"| {k} | `{d['name'].split('(')[0]}` | " +
                     " | ".join(f"{d.get(n, float('nan')) / tiles:.1f}" for n in names) + " |")
    with open(md_out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-instructions":
        # bench.py --summarize-instructions PMC_DIR MD_OUT TILES COMMAND
        a = sys.argv[2:]
        summarize_instructions(a[0], a[1], int(a[2]), a[3])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-trace":
        # bench.py --summarize-trace STATS_CSV MD_OUT COMMAND [BENCH_JSON]
        a = sys.argv[2:]
        summarize_trace(a[0], a[1], a[2], a[3] if len(a) > 3 else None)
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-counters":
        # bench.py --summarize-counters FETCH_DIR WRITE_DIR WORKLOAD [MD_OUT] [COMMAND]
        a = sys.argv[2:]
        summarize_counters(a[0], a[1], a[2], a[3] if len(a) > 3 else None,
                           a[4] if len(a) > 4 else "")
        return
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the codec shards per tensor with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)
    if args.bursts:
        if args.workload == "layerset":
            raise SystemExit("--bursts takes a single-tensor workload")
        run_bursts(args)
    elif args.workload == "layerset":
        run_layerset(args)
    else:
        run_single(args)


if __name__ == "__main__":
    main()
