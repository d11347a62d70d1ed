"""Benchmark of the lossless BF16 coding hot path on one MI355X.

One step = the whole path over one synthetic weight tensor, for each layout
(byte-split and K15): per-tensor dictionary (wc_build_dict, which reads 64
bytes back to the host), container encode (wc_encode), exact decode
(wc_decode) and decode fused into GEMV (wc_decode_gemv); then the two BF16
GEMV comparators the fused kernel is judged against (wc_gemv_bf16 and
torch.nn.functional.linear).  Inputs are resident in HBM before timing.
Several copies of the input rotate from step to step so the working set
exceeds the 256 MB last-level cache and every step streams from HBM.

Printed: one JSON line.  `value` = BF16 bytes decoded exactly per second of
whole-step wall time (2 n bytes per layout per step).  Per-call GPU times
(HIP event pairs on the launch stream around each call, averaged over the
timed steps; the dictionary pass is host wall time since it waits for the
GPU) are in `kernels`; `roofline` describes the decode kernel (the metric's
decoded-BF16 rate), timed over a burst of back-to-back launches after the
steps; `copy_reference` (with --calibrate-copy) is a plain 256 MiB device
copy timed the same way; `cpu_baseline` times the CPU oracle on the same
workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("decoded BF16 GB/s (% HBM peak); fused decode-GEMV µs vs BF16 GEMV; "
          "bits/weight")
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
LAYOUT_NAMES = {0: "byte-split", 1: "K15"}
WORKSET_BYTES = 512 << 20  # rotate copies until the inputs span 2x the 256 MB cache
ENC_THREADS = 4  # layer set: host threads (one stream each) that encode tensors side by side

WORKLOADS = {
    "small": "1024x1024 N(0,0.02), 0.05% entries x1000; batch 1",
    "square": "4096x4096 N(0,0.02), 1% zeros, 0.1% outliers N(0,2); batch 1",
    "mlp": "14336x4096 + 4096x14336, row std 10^U(-4,-1); batch 1",
    "banded": "6144x24576 N(0,0.02) + 5% escapes in 64-row bands; batch 1/4/16",
    "layerset": "96 tensors, 20.25 GiB: 48 x (6144x24576), 24 x (24576x6144) N(0,0.015), "
                "24 x [6144] N(1,0.05); streamed encode + decode, per-tensor dictionaries",
}


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", choices=sorted(WORKLOADS), default="square")
    p.add_argument("--batch", type=int, default=1)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="minimum CPU time for the oracle baseline sample")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run one 256 MiB device copy first (a known-size kernel for HBM counters)")
    return p.parse_args()


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
    raise ValueError(name)


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


DECODE_SOURCES = ["decode_gemv_sign_amd/csrc/wc_decode.hip", "decode_gemv_sign_amd/csrc/wc_tile.h",
                  "decode_gemv_sign_amd/csrc/wc_common.h"]


def counter_traffic(workload: str, layout_name: str):
    """HBM bytes per decode launch from committed rocprofv3 counter runs, or None
    when absent or taken on a different version of the kernel."""
    path = os.path.join(ROOT, "profiles", "decode_counters.json")
    if not os.path.exists(path):
        return None
    data = json.load(open(path))
    if data.get("source_hash") != source_hash(DECODE_SOURCES):
        return None
    e = data.get("workloads", {}).get(workload, {}).get(layout_name)
    return None if e is None else float(e["traffic_bytes_per_launch"])


def cpu_baseline(mats, xs, layouts, min_seconds: float, gpu_results):
    """The oracle, as it stands, on the same tensors: encode, decode and GEMV per
    layout, repeated until min_seconds have passed.  Also cross-checks the GPU
    step's outputs against it (containers byte-identical, GEMV within bound)."""
    import numpy as np

    import oracle
    from tests.tolerance import gemv_excess
    oracle.build(force=False)
    # parity of the timed GPU outputs
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
            "ms_per_step": round(1e3 * el / steps, 3)}, parity


def run_layerset(args):
    """The 96-tensor layer set, every container resident: one step encodes all
    96 tensors (dictionary pass, which waits for the GPU, then encode, per
    tensor; 4 host threads on 4 streams take turns, so the waits overlap) and
    then decodes them one after another on one stream, per layout.  The tensors
    are drawn on the device from a seeded generator with the set's shapes and
    distributions (20 GiB drawn on the host would take minutes); the GPU tests
    check six of the set's tensors as drawn by `synth`.  Every decode is
    checked bit for bit against its source; the oracle encodes a norm vector
    and a 6144 x 24576 matrix of the set, byte-compared with the GPU's."""
    import numpy as np
    import torch

    import decode_gemv_sign_amd as wc
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    layouts = [wc.BYTESPLIT, wc.K15]
    tensors = []
    for t in range(96):
        name, shape, mean, sigma = synth.layerset_spec(t)
        n = int(np.prod(shape))
        g = torch.Generator(device=dev)
        g.manual_seed(4000 + t)
        z = torch.randn(n, generator=g, device=dev, dtype=torch.float32) * sigma + mean
        tensors.append(z.to(torch.bfloat16).view(torch.int16))
        del z
    n_total = sum(w.numel() for w in tensors)
    work = torch.empty(wc.workspace_bytes(max(w.numel() for w in tensors)), dtype=torch.uint8,
                       device=dev)
    conts = {li: [] for li in layouts}
    hdrs = {li: [] for li in layouts}
    for li in layouts:  # containers allocated once, by a first (untimed) encode
        for w in tensors:
            h = wc.build_dict(w, li, work)
            hdrs[li].append(h)
            conts[li].append(wc.encode_into(h, w, torch.empty(h.total_bytes, dtype=torch.uint8,
                                                               device=dev), work))
    out_buf = torch.empty(max(w.numel() for w in tensors), dtype=torch.int16, device=dev)

    # Encode runs from ENC_THREADS host threads, each with its own stream and
    # workspace, so one tensor's dictionary pass (which waits for its stream)
    # overlaps the other threads' GPU work.
    import threading
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
        threads = [threading.Thread(target=worker, args=(i,)) for i in range(ENC_THREADS)]
        for th in threads:
            th.start()
        for th in threads:
            th.join()
        for s in enc_streams:
            stream.wait_stream(s)
        if errors:
            raise errors[0]

    def decode_all(li, check=False):
        ok = True
        for k, w in enumerate(tensors):
            o = out_buf[:w.numel()]
            wc.decode(hdrs[li][k], conts[li][k], out=o)
            if check:
                ok = ok and bool(torch.equal(o, w))
        return ok

    res = {}
    exact = True
    for li in layouts:
        encode_all(li)
        exact = decode_all(li, check=True) and exact
        torch.cuda.synchronize()
        enc, dec = [], []
        for _ in range(args.warmup + args.steps):
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
        enc = sorted(enc[args.warmup:])[len(enc[args.warmup:]) // 2]
        dec = sorted(dec[args.warmup:])[len(dec[args.warmup:]) // 2]
        cbytes = sum(h.total_bytes for h in hdrs[li])
        res[LAYOUT_NAMES[li]] = {
            "encode_ms": round(1e3 * enc, 3), "encode_decoded_gbps": round(2 * n_total / enc / 1e9, 1),
            "decode_ms": round(1e3 * dec, 3), "decode_decoded_gbps": round(2 * n_total / dec / 1e9, 1),
            "decode_hbm_gbps": round((cbytes + 2 * n_total) / dec / 1e9, 1),
            "decode_hbm_frac": round((cbytes + 2 * n_total) / dec / 1e9 / HBM_PEAK_GBPS, 4),
            "bpw": round(8 * cbytes / n_total, 4),
            "n_esc": int(sum(h.n_esc for h in hdrs[li])),
        }
    parity = exact
    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        for t in (0, 72):
            host = tensors[t].cpu().numpy().view(np.uint16)
            for li in layouts:
                if not np.array_equal(conts[li][t].cpu().numpy(), oracle.encode(li, host)):
                    parity = False
    best = max(layouts, key=lambda li: res[LAYOUT_NAMES[li]]["decode_decoded_gbps"])
    out = {
        "metric": METRIC,
        "value": res[LAYOUT_NAMES[best]]["decode_decoded_gbps"],
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(sum(r["encode_ms"] + r["decode_ms"] for r in res.values()), 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u16",
        "data": "synthetic",
        "config": {"workload": f"layerset: {WORKLOADS['layerset']}", "weights": int(n_total),
                   "value_definition": "2 bytes x weights / time to decode all 96 containers "
                                       f"back to back ({LAYOUT_NAMES[best]}, the faster layout); "
                                       "medians over the timed steps"},
        "layouts": res,
        "decode_exact": exact,
        "parity_vs_oracle": "ok" if parity else "FAILED",
    }
    print(json.dumps(out), flush=True)
    if not parity:
        sys.exit(1)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the codec shards per tensor with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)
    if args.workload == "layerset":
        run_layerset(args)
        return
    import numpy as np
    import torch

    import decode_gemv_sign_amd as wc
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
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
    layouts = [wc.BYTESPLIT, wc.K15]
    in_bytes = sum(W.nbytes for W in mats)
    copies = max(1, -(-WORKSET_BYTES // in_bytes))

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    Wd = [[to_dev(W.reshape(-1)) for W in mats] for _ in range(copies)]
    Xd = [to_dev(xx) for xx in xs]
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
    import ctypes
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

    copy_ref = None
    if args.calibrate_copy:
        # One device-to-device copy of a known size (the counter runs scale
        # FETCH_SIZE / WRITE_SIZE by what they read for it), then a timed burst
        # of the same copy: the practical rate of a plain read+write stream.
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
        copy_ref = {"bytes_read_plus_written": 2 * a.numel(), "us": round(t, 2),
                    "gbps": round(2 * a.numel() / t / 1e3, 1),
                    "frac": round(2 * a.numel() / t / 1e3 / HBM_PEAK_GBPS, 4)}
        del a, b

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
    burst_n = 20
    for mi in range(len(mats)):
        for li in range(len(layouts)):
            h = hdrs[(li, mi)]
            calls = [(ctypes.byref(h), ptr(cont[k][(li, mi)]), cont[k][(li, mi)].numel(),
                      ptr(dec[k][mi])) for k in range(copies)]
            for i in range(3):
                check(lib.wc_decode(*calls[i % copies], stream), "wc_decode")
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(burst_n):
                check(lib.wc_decode(*calls[i % copies], stream), "wc_decode")
            e1.record()
            torch.cuda.synchronize()
            burst[(li, mi)] = e0.elapsed_time(e1) * 1e3 / burst_n

    n_total = sum(W.size for W in mats)
    ms_step = 1e3 * wall / args.steps
    value = 2.0 * n_total * len(layouts) / (wall / args.steps) / 1e9

    def avg_us(name, key):
        ev = events[(name, key)]
        if name == "build_dict":  # host wall time, including its wait for the GPU
            return 1e6 * sum(ev) / len(ev)
        return 1e3 * sum(e0.elapsed_time(e1) for e0, e1 in ev) / len(ev)

    kernels = {}
    roofline = None
    bpw = {}
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
            "decode_decoded_gbps": round(2 * n / t_dec / 1e3, 1),
            "decode_hbm_gbps": round(dec_bytes / t_dec / 1e3, 1),
            "decode_hbm_frac": round(dec_bytes / t_dec / 1e3 / HBM_PEAK_GBPS, 4),
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
                        "timing": f"HIP events around {burst_n} back-to-back launches"}
    roofline.pop("_t")
    # the counter rate: the rocprofv3 HBM bytes of one launch over the same launch time
    roofline["traffic_gbps"] = (round(roofline["traffic"] / roofline["launch_us"] / 1e3, 1)
                                if roofline["traffic"] else None)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {WORKLOADS[args.workload]}",
                   "layouts": [LAYOUT_NAMES[l] for l in layouts], "batch": args.batch,
                   "weights": int(n_total), "rotating_copies": copies,
                   "value_definition": "2 bytes x weights x layouts per step / step wall time; "
                                       "step = dictionary + encode + decode + fused GEMV per "
                                       "layout, plus both BF16 GEMV comparators"},
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
        cb, parity = cpu_baseline([np.ascontiguousarray(W) for W in mats], xs, layouts,
                                  args.cpu_seconds, gpu_results)
        out["cpu_baseline"] = cb
        out["parity_vs_oracle"] = "ok" if parity else "FAILED"
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    if out.get("parity_vs_oracle") == "FAILED":
        sys.exit(1)


if __name__ == "__main__":
    main()
