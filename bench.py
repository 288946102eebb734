"""Benchmark of the fused attention forward on one MI355X.

One step = one fa_fwd call over the whole workload (default: B=4, H=32,
S=4096, D=128, fp16, causal, scale 1/sqrt(128)), inputs resident in HBM.
Prints one JSON line: TFLOP/s (4*D*B*H*visible pairs per call / average
kernel time), the roofline of the kernel against the dense fp16 MFMA peak,
and the fp64 CPU oracle timed on a bounded sample of the same workload.

With ``--workload decode_*`` one step is one fa_decode call (new query rows
against a key/value cache, HBM-bound): the line reports GB/s of algorithmic
bytes against the 8 TB/s HBM peak instead. With ``--workload varlen_*`` one
step is one fa_fwd_varlen call over a packed batch of ragged sequences
(TFLOP/s over the visible pairs of every sequence). With ``--workload
bwd_<forward workload>`` one step is one fa_bwd call (10 * D FLOPs per
visible pair).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--cpu-seconds T]
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X dense fp16/bf16 MFMA peak: 256 CUs x 4096 FLOP/clk/CU x 2.4 GHz.
PEAK_FP16_TFLOPS = 2516.6
# MI355X HBM3E peak bandwidth.
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ["tiled_attention_11_amd/csrc/fa_kernel.hip",
                  "tiled_attention_11_amd/csrc/fa_internal.h",
                  "tiled_attention_11_amd/csrc/fa_device.h"]
ROPE_SOURCES = KERNEL_SOURCES + ["tiled_attention_11_amd/csrc/fa_rope.hip"]
BWD_SOURCES = ["tiled_attention_11_amd/csrc/fa_bwd.hip",
               "tiled_attention_11_amd/csrc/fa_internal.h",
               "tiled_attention_11_amd/csrc/fa_device.h"]
DECODE_SOURCES = ["tiled_attention_11_amd/csrc/fa_decode.hip",
                  "tiled_attention_11_amd/csrc/fa_internal.h",
                  "tiled_attention_11_amd/csrc/fa_device.h"]


class ClockSampler:
    """Samples the GPU shader clock (the active level of the DPM table in
    sysfs) from a background thread while launches run; the median of the
    samples above idle is the clock the kernels ran at. None where the file
    is not readable."""

    def __init__(self, period_s=0.003):
        import glob
        import threading
        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))[:1]
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self._stop.is_set():
            for p in self.paths:
                try:
                    for line in open(p).read().splitlines():
                        m = re.search(r"(\d+)\s*Mhz\s*\*", line)
                        if m:
                            self.samples.append(int(m.group(1)))
                except OSError:
                    return
            time.sleep(self.period)

    def __enter__(self):
        if self.paths:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join()

    def mhz(self):
        busy = sorted(x for x in self.samples if x >= 1000)
        return busy[len(busy) // 2] if busy else None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def kernel_sha256(sources=None):
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counted_traffic(workload, prefix="fa_fwd", sources=None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{prefix}_{workload}.pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not sha or not val or sha.group(1) != kernel_sha256(sources):
        return None
    return int(val.group(1))


def c_abi_step(fn, *args):
    """One timed step: a direct call of a C ABI entry point (the binding of the
    same name) with its arguments bound once (raw device addresses and the
    stream handle), so that the host loop costs one ctypes call per launch
    rather than the argument checks of the torch wrappers, which the first,
    untimed call of each benchmark still goes through. On short kernels those
    checks (and the device context they set up) can outlast the kernel and
    starve the GPU between launches."""
    import tiled_attention_11_amd as fa

    def step():
        status = fn(*args)
        if status != 0:
            raise fa.FaError(status, fn.__name__)
    return step


def visible_per_row(S, mask, window, rows_i):
    """Visible keys of each query position (for FLOP accounting)."""
    import numpy as np
    i = np.asarray(rows_i, dtype=np.int64)
    if mask == "full":
        lo, hi = np.zeros_like(i), np.full_like(i, S - 1)
    elif mask == "causal":
        lo, hi = np.zeros_like(i), i
    else:
        wl, wr = window
        lo = np.maximum(0, i - wl) if wl >= 0 else np.zeros_like(i)
        hi = np.minimum(S - 1, i + wr) if wr >= 0 else np.full_like(i, S - 1)
    return np.maximum(0, hi - lo + 1)


def cpu_baseline(w, q, k, v, o_gpu, lse_gpu, seconds):
    """Time the fp64 oracle on a bounded random sample of the workload's rows;
    also report how those rows compare with the GPU output."""
    import numpy as np

    import oracle
    from tests.parity import compare

    orc = oracle.load()
    B, H, S, D = w["B"], w["H"], w["S"], w["D"]
    total = B * H * S
    rng = np.random.default_rng(1234)
    args = (q, k, v, w["dtype"], w["scale"], w["mask"], w["window"])
    if w.get("rope"):
        import synth
        cos, sin = synth.rope_tables(S, D, w["rope_base"])

        def rows_of(rows):
            return orc.attention_rope_rows(*args, cos, sin, w["rope"], rows=rows)
    else:
        def rows_of(rows):
            return orc.attention_rows(*args, rows=rows)
    probe = rng.choice(total, size=min(64, total), replace=False)
    t0 = time.perf_counter()
    rows_of(probe)
    dt = max(time.perf_counter() - t0, 1e-4)
    n = int(min(total, max(64, len(probe) * seconds / dt)))
    rows = np.sort(rng.choice(total, size=n, replace=False))
    t0 = time.perf_counter()
    o_ref, lse_ref = rows_of(rows)
    dt = time.perf_counter() - t0
    pairs = int(visible_per_row(S, w["mask"], w["window"], rows % S).sum())
    flops = 4 * D * pairs
    st = compare(o_gpu.reshape(-1, D)[rows], lse_gpu.reshape(-1)[rows], o_ref, lse_ref,
                 w["dtype"])
    base = {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": orc.max_threads(),
        "kind": "oracle", "cpu_model": cpu_model(),
        "sample": (f"{n} query rows drawn uniformly (seed 1234) from the same workload, "
                   f"{pairs} visible pairs, {dt:.2f} s wall, fp64"),
    }
    parity = {"rows": n, "pass": st["pass"], "max_abs": st["max_abs"],
              "mean_abs": st["mean_abs"], "lse_max_abs": st.get("lse_max_abs")}
    return base, parity


def decode_bytes(w):
    """Algorithmic HBM bytes of one fa_decode call: q read, the visible part of
    the cache (k and v) read once, o and lse written."""
    B, H, Sq, Sk, D = w["B"], w["H"], w["Sq"], w["Sk"], w["D"]
    lo_hi = []
    for i in (Sk - Sq, Sk - 1):  # positions of the first and the last new row
        lo = 0 if w["mask"] != "window" or w["window"][0] < 0 else max(0, i - w["window"][0])
        hi = Sk - 1 if w["mask"] == "full" or (w["mask"] == "window" and w["window"][1] < 0) else \
            min(Sk - 1, i + (0 if w["mask"] == "causal" else w["window"][1]))
        lo_hi.append((lo, hi))
    keys = lo_hi[1][1] - lo_hi[0][0] + 1
    return B * H * (2 * Sq * D * 2 + 2 * keys * D * 2 + Sq * 4)


def bench_decode(args, name):
    import numpy as np
    import torch

    import synth
    import tiled_attention_11_amd as fa

    w = synth.DECODE_WORKLOADS[name]
    B, H, Sq, Sk, D, dtype = w["B"], w["H"], w["Sq"], w["Sk"], w["D"], w["dtype"]
    wl, wr = w["window"]
    m = fa._mask_code(w["mask"])
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.perf_counter()
    q, k, v = synth.decode_inputs(name)
    tq, tk, tv = (torch.from_numpy(x.view(np.int16)).view(tdt).to(dev) for x in (q, k, v))
    out = torch.empty_like(tq)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
    ps = w.get("page_size")
    if ps:
        kp, vp, table = synth.paged_cache(k, v, ps, w["seed"])
        tkp, tvp = (torch.from_numpy(x.view(np.int16)).view(tdt).to(dev) for x in (kp, vp))
        ttab = torch.from_numpy(table).to(dev)
        tlen = torch.full((B,), Sk, dtype=torch.int32, device=dev)
        del tk, tv
        need = fa.fa_decode_paged_workspace_bytes(B, H, Sq, Sk, D, m, wl, wr)
    else:
        need = fa.fa_decode_workspace_bytes(B, H, Sq, Sk, D, m, wl, wr)
    ws = torch.empty(max(int(need), 16), dtype=torch.uint8, device=dev)
    print(f"[bench] {name}: inputs ready in {time.perf_counter() - t0:.1f}s, workspace "
          f"{need} B", file=sys.stderr, flush=True)

    code = fa.FA_DTYPE_FP16 if dtype == "f16" else fa.FA_DTYPE_BF16
    sh = torch.cuda.current_stream().cuda_stream
    if ps:
        fa.decode_paged(tq, tkp, tvp, ttab, tlen, Sk, scale=w["scale"], mask=w["mask"],
                        window=(wl, wr), out=out, lse=lse, workspace=ws)
        step = c_abi_step(fa.fa_decode_paged, tq.data_ptr(), tkp.data_ptr(), tvp.data_ptr(),
                          out.data_ptr(), lse.data_ptr(), ttab.data_ptr(), tlen.data_ptr(), B, H,
                          Sq, Sk, D, tkp.shape[0], tkp.shape[1], ttab.shape[1],
                          float(w["scale"]), m, wl, wr, code, ws.data_ptr(), ws.numel(), sh)
    else:
        fa.decode(tq, tk, tv, scale=w["scale"], mask=w["mask"], window=(wl, wr), out=out,
                  lse=lse, workspace=ws)
        step = c_abi_step(fa.fa_decode, tq.data_ptr(), tk.data_ptr(), tv.data_ptr(),
                          out.data_ptr(), lse.data_ptr(), B, H, Sq, Sk, D, float(w["scale"]), m,
                          wl, wr, code, ws.data_ptr(), ws.numel(), sh)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]) * 1e-3
    avg_s = evs[0].elapsed_time(evs[-1]) * 1e-3 / args.steps
    print(f"[bench] timed {args.steps} steps: avg {avg_s * 1e6:.1f} us, median "
          f"{np.median(per) * 1e6:.1f} us", file=sys.stderr, flush=True)
    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()

    nbytes = decode_bytes(w)
    gbs = nbytes / avg_s / 1e9
    flops = fa.fa_decode_flops(B, H, Sq, Sk, D, m, wl, wr)
    result = {
        "metric": "cache attention (new rows against a key/value cache) HBM GB/s",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(avg_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {
            "workload": (f"{name}: B={B} H={H} Sq={Sq} Sk={Sk} D={D} {dtype} {w['mask']}"
                         + (f" paged {ps}-key pages, shuffled" if ps else "")
                         + f" scale={w['scale']:.6g}"),
            "B": B, "H": H, "Sq": Sq, "Sk": Sk, "D": D, "mask": w["mask"], "window": [wl, wr],
            "bytes_per_step": nbytes, "flops_per_step": flops, "workspace_bytes": int(need),
        },
        "tflops": round(flops / avg_s / 1e12, 3),
        "median_launch_us": round(float(np.median(per)) * 1e6, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": counted_traffic(name, "fa", DECODE_SOURCES),
        },
        "cpu_baseline": None,
    }
    if args.cpu_seconds > 0:
        import oracle
        from tests.parity import compare
        orc = oracle.load()
        o_bits = out.cpu().view(torch.int16).numpy().view(np.uint16)
        lse_h = lse.cpu().numpy()
        # whole heads, in order, until the time budget is spent
        heads, t_used, pairs = 0, 0.0, 0
        stats = []
        per_head = flops // (4 * D * B * H)
        while heads < B * H and t_used < args.cpu_seconds:
            b, h = divmod(heads, H)
            sl = (slice(b, b + 1), slice(h, h + 1))
            t0 = time.perf_counter()
            o_ref, lse_ref = orc.attention_kv(q[sl], k[sl], v[sl], dtype, w["scale"], w["mask"],
                                              (wl, wr))
            t_used += time.perf_counter() - t0
            stats.append(compare(o_bits[sl], lse_h[sl], o_ref, lse_ref, dtype))
            heads += 1
            pairs += per_head
        head_bytes = nbytes // (B * H)
        result["cpu_baseline"] = {
            "value": round(heads * head_bytes / t_used / 1e9, 4), "unit": "GB/s",
            "cores": orc.max_threads(), "kind": "oracle",
            "sample": f"{heads} whole heads of the same workload ({heads * head_bytes} bytes, "
                      f"{pairs} visible pairs), {t_used:.2f} s wall, fp64",
        }
        result["parity_sample"] = {"heads": heads, "pass": all(s["pass"] for s in stats),
                                   "max_abs": max(s["max_abs"] for s in stats),
                                   "lse_max_abs": max(s.get("lse_max_abs", 0.0) for s in stats)}
    print(json.dumps(result), flush=True)


def bench_varlen(args, name):
    import numpy as np
    import torch

    import synth
    import tiled_attention_11_amd as fa

    w = synth.VARLEN_WORKLOADS[name]
    T, H, D, dtype = w["T"], w["H"], w["D"], w["dtype"]
    wl, wr = w["window"]
    m = fa._mask_code(w["mask"])
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.perf_counter()
    q, k, v, cu = synth.varlen_inputs(name)
    lengths = np.diff(cu)
    max_seqlen = int(lengths.max())
    tq, tk, tv = (torch.from_numpy(x.view(np.int16)).view(tdt).to(dev) for x in (q, k, v))
    tcu = torch.from_numpy(cu).to(dev)
    out = torch.empty_like(tq)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    print(f"[bench] {name}: inputs ready in {time.perf_counter() - t0:.1f}s, lengths "
          f"{lengths.tolist()}", file=sys.stderr, flush=True)

    fa.forward_varlen(tq, tk, tv, tcu, max_seqlen, scale=w["scale"], mask=w["mask"],
                      window=(wl, wr), out=out, lse=lse)
    step = c_abi_step(fa.fa_fwd_varlen, tq.data_ptr(), tk.data_ptr(), tv.data_ptr(),
                      out.data_ptr(), lse.data_ptr(), tcu.data_ptr(), len(lengths), max_seqlen,
                      T, H, D, float(w["scale"]), m, wl, wr,
                      fa.FA_DTYPE_FP16 if dtype == "f16" else fa.FA_DTYPE_BF16,
                      torch.cuda.current_stream().cuda_stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]) * 1e-3
    avg_s = evs[0].elapsed_time(evs[-1]) * 1e-3 / args.steps
    print(f"[bench] timed {args.steps} steps: avg {avg_s * 1e6:.1f} us, median "
          f"{np.median(per) * 1e6:.1f} us", file=sys.stderr, flush=True)
    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()

    flops = fa.fa_fwd_varlen_flops(cu.tolist(), H, D, m, wl, wr)
    tflops = flops / avg_s / 1e12
    result = {
        "metric": "packed variable-length attention fwd TFLOP/s and % of fp16 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(avg_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {
            "workload": (f"{name}: {len(lengths)} sequences packed into T={T} tokens, "
                         f"lengths uniform in [{w['len_lo']}, {w['len_hi']}] (seed {w['seed']}), "
                         f"H={H} D={D} {dtype} {w['mask']} scale={w['scale']:.6g}"),
            "T": T, "H": H, "D": D, "lengths": lengths.tolist(), "mask": w["mask"],
            "window": [wl, wr], "flops_per_step": flops,
        },
        "pct_of_peak": round(100.0 * tflops / PEAK_FP16_TFLOPS, 2),
        "median_launch_us": round(float(np.median(per)) * 1e6, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_FP16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_FP16_TFLOPS, 4),
            "traffic": counted_traffic(name),
        },
        "cpu_baseline": None,
    }
    if args.cpu_seconds > 0:
        import oracle
        from tests.parity import compare
        orc = oracle.load()
        o_bits = out.cpu().view(torch.int16).numpy().view(np.uint16)
        lse_h = lse.cpu().numpy()
        # query rows drawn uniformly from each sequence in turn, until the
        # time budget is spent
        rng = np.random.default_rng(1234)
        t_used, pairs, nrows, stats, rounds = 0.0, 0, 0, [], 0
        while t_used < args.cpu_seconds and rounds < 64:
            rounds += 1
            for a, b in zip(cu[:-1], cu[1:]):
                L = int(b - a)
                rows_i = rng.integers(0, L, 4)
                heads = rng.integers(0, H, 4)

                def head_major(x):
                    return np.ascontiguousarray(x[a:b].transpose(1, 0, 2))[None]

                hq, hk, hv = head_major(q), head_major(k), head_major(v)
                t1 = time.perf_counter()
                o_ref, lse_ref = orc.attention_rows(hq, hk, hv, dtype, w["scale"], w["mask"],
                                                    (wl, wr), rows=heads * L + rows_i)
                t_used += time.perf_counter() - t1
                stats.append(compare(o_bits[a + rows_i, heads], lse_h[a + rows_i, heads],
                                     o_ref, lse_ref, dtype))
                pairs += int(visible_per_row(L, w["mask"], (wl, wr), rows_i).sum())
                nrows += rows_i.size
        result["cpu_baseline"] = {
            "value": round(4 * D * pairs / t_used / 1e12, 6), "unit": "TFLOP/s",
            "cores": orc.max_threads(), "kind": "oracle",
            "sample": (f"{nrows} query rows, 4 per sequence per round over {rounds} rounds "
                       f"(seed 1234), {pairs} visible pairs, {t_used:.2f} s wall, fp64"),
        }
        result["parity_sample"] = {"rows": nrows, "pass": all(s["pass"] for s in stats),
                                   "max_abs": max(s["max_abs"] for s in stats),
                                   "lse_max_abs": max(s.get("lse_max_abs", 0.0) for s in stats)}
    print(json.dumps(result), flush=True)


def bench_bwd(args, name):
    """One step = one fa_bwd call (the forward's O and LSE computed beforehand)."""
    import numpy as np
    import torch

    import synth
    import tiled_attention_11_amd as fa

    fwd_name = name[len("bwd_"):]
    w = synth.WORKLOADS[fwd_name]
    B, H, S, D, dtype = w["B"], w["H"], w["S"], w["D"], w["dtype"]
    wl, wr = w["window"]
    m = fa._mask_code(w["mask"])
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.perf_counter()
    q, k, v = synth.workload_inputs(fwd_name)
    do, _, _ = synth.make_qkv(B, H, S, D, dtype, w["seed"] + 1000)
    tq, tk, tv, tdo = (torch.from_numpy(x.view(np.int16)).view(tdt).to(dev)
                       for x in (q, k, v, do))
    o, lse = fa.forward(tq, tk, tv, scale=w["scale"], mask=w["mask"], window=(wl, wr))
    dq, dk, dv = (torch.empty_like(tq) for _ in range(3))
    ws = torch.empty(int(fa.fa_bwd_workspace_bytes(B, H, S)), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    print(f"[bench] {name}: inputs and forward ready in {time.perf_counter() - t0:.1f}s",
          file=sys.stderr, flush=True)

    fa.backward(tq, tk, tv, o, lse, tdo, scale=w["scale"], mask=w["mask"], window=(wl, wr),
                dq=dq, dk=dk, dv=dv, workspace=ws)
    step = c_abi_step(fa.fa_bwd, tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(),
                      lse.data_ptr(), tdo.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                      dv.data_ptr(), B, H, S, D, float(w["scale"]), m, wl, wr,
                      fa.FA_DTYPE_FP16 if dtype == "f16" else fa.FA_DTYPE_BF16, ws.data_ptr(),
                      ws.numel(), torch.cuda.current_stream().cuda_stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]) * 1e-3
    avg_s = evs[0].elapsed_time(evs[-1]) * 1e-3 / args.steps
    print(f"[bench] timed {args.steps} steps: avg {avg_s * 1e6:.1f} us, median "
          f"{np.median(per) * 1e6:.1f} us", file=sys.stderr, flush=True)
    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
    flops = fa.fa_bwd_flops(B, H, S, D, m, wl, wr)
    tflops = flops / avg_s / 1e12
    result = {
        "metric": f"attention backward TFLOP/s and % of fp16 MFMA peak, {fwd_name}",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(avg_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {
            "workload": (f"{name}: fa_bwd (dQ kernel with the row dots + dK/dV kernel) at B={B} H={H} "
                         f"S={S} D={D} {dtype} {w['mask']} scale={w['scale']:.6g}, dO standard "
                         "normal; O and LSE from fa_fwd outside the timed region"),
            "B": B, "H": H, "S": S, "D": D, "mask": w["mask"], "window": [wl, wr],
            "flops_per_step": flops,
        },
        "pct_of_peak": round(100.0 * tflops / PEAK_FP16_TFLOPS, 2),
        "median_launch_us": round(float(np.median(per)) * 1e6, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_FP16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_FP16_TFLOPS, 4),
            "traffic": counted_traffic(name, prefix="fa", sources=BWD_SOURCES),
        },
        "cpu_baseline": None,
    }
    if args.cpu_seconds > 0:
        import oracle
        orc = oracle.load()
        got = [g.cpu().view(torch.int16).numpy().view(np.uint16) for g in (dq, dk, dv)]
        from tests.parity import decode as dec
        heads, t_used, worst = 0, 0.0, 0.0
        u = 2.0 ** -11 if dtype == "f16" else 2.0 ** -8
        while heads < B * H and t_used < args.cpu_seconds:
            b, h = divmod(heads * 37 % (B * H), H)  # spread over the batch
            sl = (slice(b, b + 1), slice(h, h + 1))
            t1 = time.perf_counter()
            refs, mags = orc.attention_bwd(q[sl], k[sl], v[sl], do[sl], dtype, w["scale"],
                                           w["mask"], (wl, wr))
            t_used += time.perf_counter() - t1
            for g, r, mg in zip(got, refs, mags):
                err = np.abs(dec(g[sl], dtype).reshape(r.shape) - r)
                worst = max(worst, float((err / (2 * u * mg + 2.0 ** -10 * np.abs(r) + 2.0 ** -24)).max()))
            heads += 1
        per_head = flops // (B * H)
        result["cpu_baseline"] = {
            "value": round(heads * per_head / t_used / 1e12, 6), "unit": "TFLOP/s",
            "cores": orc.max_threads(), "kind": "oracle",
            "sample": f"{heads} whole heads of the same workload, {t_used:.2f} s wall, fp64",
        }
        result["parity_sample"] = {"heads": heads, "worst_error_over_bound": round(worst, 4),
                                   "pass": worst <= 1.0}
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--cpu-seconds", type=float, default=25.0,
                    help="target wall time of the CPU oracle sample (0 = skip)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB "
                         "(reference kernel for rocprofv3 byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(attention heads shard across GPUs with no communication; run one "
              "process per GPU on its own heads).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import tiled_attention_11_amd as fa

    name = args.workload or synth.HEADLINE
    if name in synth.DECODE_WORKLOADS:
        return bench_decode(args, name)
    if name in synth.VARLEN_WORKLOADS:
        return bench_varlen(args, name)
    if name.startswith("bwd_") and name[len("bwd_"):] in synth.WORKLOADS:
        return bench_bwd(args, name)
    w = synth.WORKLOADS[name]
    B, H, S, D, dtype = w["B"], w["H"], w["S"], w["D"], w["dtype"]
    wl, wr = w["window"]
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t0 = time.perf_counter()
    q, k, v = synth.workload_inputs(name)
    tq, tk, tv = (torch.from_numpy(x.view(np.int16)).view(tdt).to(dev) for x in (q, k, v))
    out = torch.empty_like(tq)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    rope = w.get("rope")
    if rope:
        cos, sin = synth.rope_tables(S, D, w["rope_base"])
        tcos, tsin = torch.from_numpy(cos).to(dev), torch.from_numpy(sin).to(dev)
        k_rot = torch.empty_like(tk)
    print(f"[bench] {name}: inputs ready in {time.perf_counter() - t0:.1f}s", file=sys.stderr,
          flush=True)

    code = fa.FA_DTYPE_FP16 if dtype == "f16" else fa.FA_DTYPE_BF16
    mcode = fa._mask_code(w["mask"])
    sh = torch.cuda.current_stream().cuda_stream
    if rope:
        fa.forward_rope(tq, tk, tv, tcos, tsin, mode=rope, k_rot=k_rot, scale=w["scale"],
                        mask=w["mask"], window=(wl, wr), out=out, lse=lse)
        step = c_abi_step(fa.fa_fwd_rope, tq.data_ptr(), tk.data_ptr(), tv.data_ptr(),
                          out.data_ptr(), lse.data_ptr(), k_rot.data_ptr(), tcos.data_ptr(),
                          tsin.data_ptr(), tcos.shape[0], fa._rope_code(rope), B, H, S, D,
                          float(w["scale"]), mcode, wl, wr, code, sh)
    else:
        fa.forward(tq, tk, tv, scale=w["scale"], mask=w["mask"], window=(wl, wr), out=out,
                   lse=lse)
        step = c_abi_step(fa.fa_fwd, tq.data_ptr(), tk.data_ptr(), tv.data_ptr(),
                          out.data_ptr(), lse.data_ptr(), B, H, S, D, float(w["scale"]), mcode,
                          wl, wr, code, sh)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t_wall = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]) * 1e-3
    total_s = evs[0].elapsed_time(evs[-1]) * 1e-3
    avg_s = total_s / args.steps
    # the shader clock under this load: sampled over half a second of the
    # same launches, after (and outside) the timed region
    with ClockSampler() as clk:
        for _ in range(max(50, int(0.5 / avg_s))):
            step()
        torch.cuda.synchronize()
    print(f"[bench] timed {args.steps} steps: avg {avg_s * 1e6:.1f} us, median "
          f"{np.median(per) * 1e6:.1f} us, wall {t_wall:.3f} s", file=sys.stderr, flush=True)

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    flops = fa.fa_fwd_flops(B, H, S, D, fa._mask_code(w["mask"]), wl, wr)
    tflops = flops / avg_s / 1e12
    traffic = counted_traffic(name, sources=ROPE_SOURCES if w.get("rope") else None)

    result = {
        "metric": ("attention fwd TFLOP/s and % of fp16 MFMA peak, B4 H32 S4096 D128 causal"
                   if name == synth.HEADLINE else
                   "attention fwd" + (" with RoPE of q and k" if rope else "")
                   + f" TFLOP/s and % of fp16 MFMA peak, {name}"),
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(avg_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if dtype == "f16" else "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"{name}: B={B} H={H} S={S} D={D} {dtype} {w['mask']}"
                         + (f" window=({wl},{wr})" if w["mask"] == "window" else "")
                         + f" scale={w['scale']:.6g}"
                         + (f", RoPE of q and k ({rope}, base {w['rope_base']:g}): one fa_rope "
                            "launch over k + the forward with q rotated in registers"
                            if rope else "")),
            "B": B, "H": H, "S": S, "D": D, "mask": w["mask"], "window": [wl, wr],
            "flops_per_step": flops,
        },
        "pct_of_peak": round(100.0 * tflops / PEAK_FP16_TFLOPS, 2),
        "median_launch_us": round(float(np.median(per)) * 1e6, 2),
        "min_launch_us": round(float(np.min(per)) * 1e6, 2),
        "tflops_at_median": round(flops / float(np.median(per)) / 1e12, 2),
        # the shader clock under this load (sysfs DPM level, sampled over the
        # same launches run again right after the timed region) and the dense
        # fp16 MFMA peak at that clock
        "sclk_mhz": clk.mhz(),
        "pct_of_clock_adjusted_peak": (round(100.0 * tflops / (256 * 4096 * clk.mhz() * 1e-6), 2)
                                       if clk.mhz() else None),
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_FP16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_FP16_TFLOPS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": None,
    }
    if args.cpu_seconds > 0:
        torch.cuda.synchronize()
        o_bits = out.cpu().view(torch.int16).numpy().view(np.uint16)
        base, parity = cpu_baseline(w, q, k, v, o_bits, lse.cpu().numpy(), args.cpu_seconds)
        result["cpu_baseline"] = base
        result["parity_sample"] = parity
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
