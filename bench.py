"""Throughput of the rotated, quantized projections on one MI355X.

One step = one pass of the whole per-step hot path over the projections of one
diffusion-transformer block at 1024x1024 (M = 4096 latent rows):

  W8A8  qkv 3072->9216, out 3072->3072, gate+up 3072->24576, down 12288->3072:
        rotate + per-token int8 quantize (tp_quantize_rows_int8), then the i8
        product with its fused scale epilogue (tp_qgemm_w8a8_prequantized);
  W8    FFN up 3072->12288: rotate to bf16 (tp_hadamard_rotate_rows), then the
        weight-only int8 product (tp_qgemm_w8);
  W4    FFN down 12288->3072 at M = 4032: rotate, then the weight-only int4
        product (tp_qgemm_w4).

Weights are rotated and quantized once before timing (offline by definition);
that step is timed separately and reported as weight_prep. All inputs are
seeded synthetic tensors with the value distributions described in
workloads/__init__.py (Gaussian activations with outlier channels, Gaussian
weights with outlier input columns); no checkpoint or dataset is involved.

Printed: one JSON line with the step throughput (TOPS over all products of the
step), the dominant kernel's roofline fraction (HIP events around each launch
inside the timed region), a per-launch breakdown and the CPU oracle timed on a
bounded sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TOPS_I8 = 5000.0       # MI355X dense int8 MFMA, TOP/s
PEAK_TFLOPS_BF16 = 2500.0   # MI355X dense bf16 MFMA, TFLOP/s
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, GB/s
METRIC = "rotated int8/int4 QGEMM TOPS & % MFMA/HBM roofline at M=4096,K=3072 (1 GPU)"


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=0,
                   help="activation rows of the CPU oracle sample (0: all rows of every product)")
    p.add_argument("--cpu-only", action="store_true", help="time only the CPU oracle sample (no GPU)")
    p.add_argument("--small-m", action="store_true",
                   help="instead of the step: the M <= 64 HBM-bound sweep (one JSON line per case)")
    p.add_argument("--library-reference", action="store_true",
                   help="instead of the step: time the platform's own int8 / bf16 GEMMs (hipBLASLt through torch) on "
                        "the step's shapes, as context for the roofline fractions (one JSON line per shape)")
    p.add_argument("--only", default=None,
                   help="run only the launches whose name contains this text (for counter profiling)")
    p.add_argument("--no-next", action="store_true", help="skip the rows measured beside the step (\"next\")")
    p.add_argument("--no-small-m", action="store_true", help="skip the M <= 64 rows of the default run")
    p.add_argument("--next-only", action="store_true",
                   help="measure only the rows beside the step and print their JSON (for profiling)")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MB",
                   help="before the step, run a plain device copy of MB MiB (a kernel of known traffic)")
    return p.parse_args()


def step_plan():
    import workloads as W
    return [("w8a8", W.DIT_QKV), ("w8a8", W.DIT_OUT), ("w8a8", W.DIT_GATEUP), ("w8a8", W.DIT_DOWN),
            ("w8", W.FFN_UP), ("w4", W.FFN_DOWN)]


# The sources of the product kernels (the translation unit gemm.hip and what
# it includes): the counter profile of a product applies only while they are
# unchanged.
GEMM_SOURCES = ("gemm.hip", "gemm_pp.hpp", "gemm_skinny.hpp", "device_common.hpp", "kernels.hpp")


def _src_hash():
    """Hash of the product kernels' sources: a committed counter profile
    applies only to the kernels it was taken on."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "int4_quantized_gemm_amd", "csrc")
    for f in GEMM_SOURCES:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic_for(kernel_key):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != _src_hash():
        return None
    v = rec.get("kernels", {}).get(kernel_key)
    return None if v is None else v.get("bytes_per_launch")


# --------------------------------------------------------------- CPU baseline
def _cpu_model():
    """The host CPU's model name (the first "model name" of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_inputs(rows):
    """Activations (the first `rows` rows; 0: all) and the oracle's own
    quantized weights for every product of the step (untimed)."""
    import oracle
    import workloads as W
    out = []
    for kind, wl in step_plan():
        x, w = W.generate(wl, rows=rows or None)
        wn = w.numpy()
        if kind == "w4":
            q, s = oracle.quantize_weights_int4(wn)
            wd = oracle.dequantize_int4(q, s)
        else:
            q, s = oracle.quantize_weights_int8(wn)
            wd = oracle.dequantize_int8(q, s) if kind == "w8" else None
        out.append((kind, wl, x.double().numpy(), q, s, wd))
    return out


def _oracle_pass(inputs, rows, repeats):
    """The oracle as it stands over the first `rows` activation rows of every
    product of the step, each step of the path timed on its own: activation
    rotation (the dense H product per 256-group), activation quantization
    (W8A8) or the bf16 rounding of the rotated operand (W8, W4), the product
    (fp64 matrix product: exact on the integer codes of W8A8, against the
    dequantized weights for W8 and W4) and the W8A8 scale epilogue. Returns
    (ops, {step: seconds, each the median over repeats}, {product: seconds})."""
    import oracle
    steps = {"rotation": 0.0, "quantization": 0.0, "product": 0.0, "epilogue": 0.0}
    per = {}
    total_ops = 0.0
    for kind, wl, xall, q, s, wd in inputs:
        x64 = xall[:rows] if rows else xall
        times = {k: [] for k in steps}
        for _ in range(repeats):
            t0 = time.perf_counter()
            xr = oracle.rotate_groups(x64)
            t1 = time.perf_counter()
            if kind == "w8a8":
                qa, sa = oracle.quantize_activations_int8(xr, rotate=False)
                t2 = time.perf_counter()
                acc = oracle.int_accumulate(qa, q)
                t3 = time.perf_counter()
                _ = acc.astype(np.float64) * sa.astype(np.float64)[:, None] * s.astype(np.float64)[None, :]
                t4 = time.perf_counter()
            else:
                xb = oracle.bf16_round(xr)
                t2 = time.perf_counter()
                _ = np.matmul(xb, wd.T)
                t3 = t4 = time.perf_counter()
            for k, dt in zip(steps, (t1 - t0, t2 - t1, t3 - t2, t4 - t3)):
                times[k].append(dt)
        med = {k: float(np.median(v)) for k, v in times.items()}
        for k in steps:
            steps[k] += med[k]
        per[wl.name] = sum(med.values())
        total_ops += 2.0 * x64.shape[0] * wl.n * wl.k
    return total_ops, steps, per


def cpu_baseline(rows):
    """The oracle timed on the host: all threads on `rows` rows of every
    product (0: all rows), then one thread on a 64-row sample."""
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count() or 1])
    inputs = _oracle_inputs(rows)
    ops, steps, per = _oracle_pass(inputs, 0, repeats=5)
    total = sum(steps.values())
    one_rows = 64
    with threadpool_limits(limits=1):
        ops1, steps1, _ = _oracle_pass(inputs, one_rows, repeats=3)
    total1 = sum(steps1.values())
    return {
        "value": ops / total / 1e12,
        "unit": "TOPS",
        "cores": int(cores),
        "kind": "oracle",
        "cpu_model": _cpu_model(),
        "host_cpus": os.cpu_count(),
        "sample": f"{'first %d' % rows if rows else 'all'} activation rows of each of the 6 products of the step "
                  f"(all N, all K), fp64 numpy oracle: rotation, quantization or bf16 rounding, product, epilogue; "
                  f"median of 5 runs per step, {total:.1f} s per pass "
                  f"({', '.join(f'{k}:{v:.2f}s' for k, v in per.items())})",
        "steps_s": {k: round(v, 4) for k, v in steps.items()},
        "one_thread": {"value": ops1 / total1 / 1e12, "unit": "TOPS", "cores": 1,
                       "sample": f"first {one_rows} activation rows of each product, median of 3 runs per step, "
                                 f"{total1:.1f} s per pass",
                       "steps_s": {k: round(v, 4) for k, v in steps1.items()}},
    }


# ------------------------------------------------------- M <= 64 sweep (HBM)
def _graph_times(torch, fn, copies):
    """Median and min seconds per call of fn(i) over i = 0 .. copies-1, the
    calls captured in one HIP graph and replayed (5 repeats of at least 64
    calls), so the time is the GPU's, not the Python launch rate's."""
    for i in range(copies):
        fn(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(copies):
            fn(i)
    graph.replay()
    torch.cuda.synchronize()
    reps = max(2, -(-64 // copies))
    med = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        med.append(e0.elapsed_time(e1) / (reps * copies) * 1e-3)
    del graph
    return float(np.median(med)), float(np.min(med))


def small_m_sweep(args, emit=False):
    """Products with 1, 16 and 64 activation rows against the full-size
    weights of the step. They are bound by reading the weights, so each case
    cycles through enough distinct copies of the packed weight (at least
    2 x 256 MB) that no launch finds its weight in the 256 MB last-level cache.
    Bytes per launch = weight codes + scales + activation operand + output.
    Returns one dict per case (and prints each as a JSON line if emit)."""
    import torch
    import int4_quantized_gemm_amd as tp
    import workloads as W

    d = torch.device("cuda:0")
    torch.cuda.set_device(d)
    cases = [("w8", W.FFN_UP), ("w4", W.FFN_DOWN), ("w8a8", W.DIT_QKV), ("w8a8", W.DIT_GATEUP)]
    out_rows = []
    for kind, wl in cases:
        _, w = W.generate(wl, rows=1)
        bits = 4 if kind == "w4" else 8
        q, s = tp.tp_rotate_quantize_weights(w.to(d), bits=bits)
        del w
        wbytes = q.numel() + s.numel() * 4
        copies = max(2, -(-2 * 256 * 2 ** 20 // wbytes))
        qs = [(q.clone(), s.clone()) for _ in range(copies)]
        del q, s
        for m in (1, 16, 64):
            x, _ = W.generate(wl.with_(m=m), rows=m)
            xd = x.to(d)
            if kind == "w8a8":
                qa, sa = tp.tp_quantize_rows_int8(xd)
                out = torch.empty((m, wl.n), dtype=torch.float32, device=d)
                ws = torch.empty((max(1, tp.tp_workspace_size(4, m, wl.n, wl.k, 0)),), dtype=torch.uint8, device=d)
                fn = lambda i: tp.tp_qgemm_w8a8_prequantized(qa, sa, qs[i][0], qs[i][1], out=out, workspace=ws)
                abytes = m * wl.k + m * 4
            else:
                xr = tp.tp_hadamard_rotate_rows(xd, out_dtype=torch.bfloat16)
                out = torch.empty((m, wl.n), dtype=torch.bfloat16, device=d)
                op = 1 if kind == "w8" else 2
                ws = torch.empty((max(1, tp.tp_workspace_size(op, m, wl.n, wl.k, 0)),), dtype=torch.uint8, device=d)
                g = tp.tp_qgemm_w8 if kind == "w8" else tp.tp_qgemm_w4
                fn = lambda i, g=g: g(xr, qs[i][0], qs[i][1], rotate=False, out=out, workspace=ws)
                abytes = m * wl.k * 2
            nbytes = wbytes + abytes + out.numel() * out.element_size()
            t_med, t_min = _graph_times(torch, fn, copies)
            gbs = nbytes / t_med / 1e9
            row = {"case": f"{kind}[{wl.name}]", "m": m, "n": wl.n, "k": wl.k, "bytes": nbytes,
                   "us_median": round(t_med * 1e6, 2), "us_min": round(t_min * 1e6, 2), "gbs": round(gbs, 1),
                   "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "weight_copies": copies,
                   "tflops": round(2.0 * m * wl.n * wl.k / t_med / 1e12, 2)}
            out_rows.append(row)
            if emit:
                print(json.dumps({"metric": "small-M product HBM bandwidth", **row}), flush=True)
        del qs
        torch.cuda.empty_cache()
    return out_rows


# ------------------------------------------ rows measured beside the step
def _time_us(torch, fn, reps=5, inner=10):
    """Median over `reps` of the mean time of `inner` back-to-back calls (HIP
    events on the current stream, where the library launches)."""
    fn()
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(inner):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / inner * 1e3)
    return float(np.median(out))


def next_rows(args, cpu):
    """The fused FFN middle (SwiGLU -> rotation -> int8 codes or rotated bf16),
    at the two full-size workloads: its HBM roofline fraction (algorithmic
    bytes: gate and up read, output written), the unfused two-pass path for
    context (an ideal SwiGLU pass writing bf16 h at peak HBM bandwidth, plus
    this library's own rotation pass over h, measured), and the oracle on a
    bounded row sample."""
    import torch
    import int4_quantized_gemm_amd as tp
    import workloads as W
    d = torch.device("cuda:0")
    res = []
    for w in (W.FFN_MID_W8A8, W.FFN_MID_W4):
        gu = W.gate_up(w, fused=True).to(d)
        g, u = gu[:, :w.k], gu[:, w.k:]
        es = 4 if w.in_dtype == "f32" else 2
        # h for the unfused second pass: the same values the fused kernel forms
        # (computed here with plain torch ops, outside the timed region)
        h = (torch.nn.functional.silu(g.float()) * u.float()).to(torch.bfloat16)
        if w.out == "i8":
            y = torch.empty((w.m, w.k), dtype=torch.int8, device=d)
            sc = torch.empty((w.m,), dtype=torch.float32, device=d)
            fused = lambda: tp.tp_swiglu_rotate(g, u, out_kind="i8", out=y, scales=sc)
            second = lambda: tp.tp_quantize_rows_int8(h, qa=y, sa=sc)
            out_bytes, second_bytes = w.m * w.k + w.m * 4, w.m * w.k * 3 + w.m * 4
        else:
            y = torch.empty((w.m, w.k), dtype=torch.bfloat16, device=d)
            fused = lambda: tp.tp_swiglu_rotate(g, u, out_kind="bf16", out=y)
            second = lambda: tp.tp_hadamard_rotate_rows(h, out=y)
            out_bytes, second_bytes = w.m * w.k * 2, w.m * w.k * 4
        alg = 2 * w.m * w.k * es + out_bytes
        us = _time_us(torch, fused)
        us2 = _time_us(torch, second)
        # The unfused path as it would run: torch's SwiGLU (silu, multiply,
        # rounding to bf16: three elementwise kernels) then the second pass.
        tmp = torch.empty((w.m, w.k), dtype=g.dtype, device=d)
        hb = torch.empty((w.m, w.k), dtype=torch.bfloat16, device=d)

        def unfused(second_on=(lambda hh: tp.tp_quantize_rows_int8(hh, qa=y, sa=sc)) if w.out == "i8" else
                    (lambda hh: tp.tp_hadamard_rotate_rows(hh, out=y))):
            torch.mul(torch.nn.functional.silu(g), u, out=tmp)
            hb.copy_(tmp)
            second_on(hb)

        us3 = _time_us(torch, unfused)
        silu_pass_us = (2 * w.m * w.k * es + w.m * w.k * 2) / (PEAK_HBM_GBS * 1e3)
        row = {"row": "ffn_middle", "workload": f"{w.name}: M={w.m}, K={w.k}, {w.in_dtype} gate/up -> {w.out}",
               "us": round(us, 2), "roofline": {"bound": "hbm", "achieved": round(alg / us / 1e3, 1),
                                                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                                "frac": round(alg / us / 1e3 / PEAK_HBM_GBS, 4),
                                                "algorithmic_bytes": alg},
               "unfused_us": round(silu_pass_us + us2, 2),
               "unfused_note": f"ideal SwiGLU pass at peak HBM ({silu_pass_us:.1f} us) + measured rotation pass over "
                               f"bf16 h ({us2:.1f} us, {second_bytes / us2 / 1e3:.0f} GB/s)",
               "unfused_measured_us": round(us3, 2),
               "unfused_measured_note": "torch SwiGLU (silu, multiply, bf16 rounding) then the same second pass, "
                                        "timed the same way"}
        del gu, g, u, h, y, tmp, hb
        if cpu:
            rows = 256
            g64, u64 = (t.double().numpy() for t in W.gate_up(w, rows=rows))
            import oracle
            fn = (lambda: oracle.ffn_middle_int8(g64, u64)) if w.out == "i8" else \
                (lambda: oracle.bf16_round(oracle.ffn_middle_rotated(g64, u64)))
            times = []
            for _ in range(3):
                t0 = time.perf_counter()
                fn()
                times.append(time.perf_counter() - t0)
            dt = float(np.median(times))
            row["cpu_baseline"] = {"value": round(alg * rows / w.m / dt / 1e9, 3), "unit": "GB/s",
                                   "kind": "oracle", "sample": f"first {rows} rows, median of 3 ({dt:.2f} s)"}
        res.append(row)

    # NEXT-2: W4A8 on the two K = 12288 down projections (int4 weights with
    # group scales, per-token int8 activations already quantized).
    for wl in (W.DIT_DOWN, W.FFN_DOWN):
        x, w = W.generate(wl)
        xd = x.to(d)
        q4, s4 = tp.tp_rotate_quantize_weights(w.to(d), bits=4)
        qa, sa = tp.tp_quantize_rows_int8(xd)
        out = torch.empty((wl.m, wl.n), dtype=torch.float32, device=d)
        ws = torch.empty((max(1, tp.tp_workspace_size(_lib_op_w4a8_pre(), wl.m, wl.n, wl.k, 0)),), dtype=torch.uint8,
                         device=d)
        us = _time_us(torch, lambda: tp.tp_qgemm_w4a8_prequantized(qa, sa, q4, s4, out=out, workspace=ws))
        ops = 2.0 * wl.m * wl.n * wl.k
        row = {"row": "w4a8", "workload": f"{wl.name}: M={wl.m}, K={wl.k}, N={wl.n}, int8 codes -> fp32",
               "us": round(us, 2), "roofline": {"bound": "mfma", "achieved": round(ops / us / 1e6, 1),
                                                "peak": PEAK_TOPS_I8, "unit": "TOP/s",
                                                "frac": round(ops / us / 1e6 / PEAK_TOPS_I8, 4)}}
        if cpu:
            import oracle
            rows = 64
            x64 = x[:rows].double().numpy()
            qh, sh = q4.cpu().numpy(), s4.cpu().numpy()
            times = []
            for _ in range(3):
                t0 = time.perf_counter()
                oracle.qgemm_w4a8(x64, qh, sh)
                times.append(time.perf_counter() - t0)
            dt = float(np.median(times))
            row["cpu_baseline"] = {"value": round(2.0 * rows * wl.n * wl.k / dt / 1e12, 5), "unit": "TOP/s",
                                   "kind": "oracle", "sample": f"first {rows} rows incl. rotation and quantization, "
                                                               f"median of 3 ({dt:.2f} s)"}
        res.append(row)
        del x, w, xd, q4, s4, qa, sa, out, ws

    # NEXT-3: the loader path on the largest weight of the block (gate+up,
    # 24576 x 3072): undo the int8 codes to fp32, and requantize them to int4.
    wl = W.DIT_GATEUP
    _, w = W.generate(wl, rows=1)
    q8, s8 = tp.tp_rotate_quantize_weights(w.to(d), bits=8)
    wh = torch.empty((wl.n, wl.k), dtype=torch.float32, device=d)
    q4 = torch.empty((wl.n, wl.k // 2), dtype=torch.uint8, device=d)
    s4 = torch.empty((wl.n, wl.k // 256), dtype=torch.float32, device=d)
    nk = wl.n * wl.k
    for name, fn, alg in (
            ("dequantize_unrotate int8 -> fp32", lambda: tp.tp_dequantize_unrotate(q8, s8, 8, out=wh),
             nk * (1 + 4) + wl.n * 4),
            ("requantize int8 -> int4", lambda: tp.tp_requantize_weights(q8, s8, 8, 4, q_out=q4, scales_out=s4),
             nk * (1 + 0.5) + wl.n * 4 + wl.n * (wl.k // 256) * 4)):
        us = _time_us(torch, fn)
        row = {"row": "loader", "workload": f"{name}: {wl.name} weight N={wl.n}, K={wl.k}", "us": round(us, 2),
               "roofline": {"bound": "hbm", "achieved": round(alg / us / 1e3, 1), "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "frac": round(alg / us / 1e3 / PEAK_HBM_GBS, 4),
                            "algorithmic_bytes": int(alg)}}
        if cpu:
            import oracle
            rows = 512
            qh, sh = q8[:rows].cpu().numpy(), s8[:rows].cpu().numpy()
            f = (lambda: oracle.dequantize_unrotate(qh, sh, 8)) if "unrotate" in name else \
                (lambda: oracle.requantize(qh, sh, 8, 4))
            times = []
            for _ in range(3):
                t0 = time.perf_counter()
                f()
                times.append(time.perf_counter() - t0)
            dt = float(np.median(times))
            row["cpu_baseline"] = {"value": round(alg * rows / wl.n / dt / 1e9, 3), "unit": "GB/s", "kind": "oracle",
                                   "sample": f"first {rows} weight rows, median of 3 ({dt:.2f} s)"}
        res.append(row)
    del q8, s8, wh, q4, s4

    # NEXT-4: a LoRA side path (rank 32 and 64) added into the W8A8 qkv
    # projection's fp32 output, against the product's own time: as a second
    # pass over C (tp_lora_add), and in the product's store (tp_lora_down, then
    # tp_qgemm_w8a8_prequantized_lora against tp_qgemm_w8a8_prequantized).
    wl = W.DIT_QKV
    x, w = W.generate(wl)
    xd = x.to(d)
    q8, s8 = tp.tp_rotate_quantize_weights(w.to(d), bits=8)
    y = tp.tp_qgemm_w8a8(xd, q8, s8)
    prod_us = _time_us(torch, lambda: tp.tp_qgemm_w8a8(xd, q8, s8, out=y))
    qa, sa = tp.tp_quantize_rows_int8(xd)
    y2 = torch.empty_like(y)
    pre_us = _time_us(torch, lambda: tp.tp_qgemm_w8a8_prequantized(qa, sa, q8, s8, out=y2))
    tbuf = torch.empty((wl.m, 64), dtype=torch.float32, device=d)
    for r in (32, 64):
        a = (torch.randn((r, wl.k), device=d) * 0.02).to(torch.bfloat16)
        b = (torch.randn((wl.n, r), device=d) * 0.02).to(torch.bfloat16)
        wsl = torch.empty((tp.tp_lora_workspace_size(wl.m, r),), dtype=torch.uint8, device=d)
        us = _time_us(torch, lambda: tp.tp_lora_add(y, xd, a, b, 0.8, workspace=wsl))
        alg = wl.m * wl.k * 2 + r * wl.k * 2 + wl.n * r * 2 + 2 * wl.m * wl.n * 4 + 2 * wl.m * r * 4
        row = {"row": "lora", "workload": f"rank {r} beside dit_qkv: M={wl.m}, K={wl.k}, N={wl.n}, bf16 x/A/B, fp32 C",
               "us": round(us, 2), "roofline": {"bound": "hbm", "achieved": round(alg / us / 1e3, 1),
                                                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                                "frac": round(alg / us / 1e3 / PEAK_HBM_GBS, 4),
                                                "algorithmic_bytes": int(alg)},
               "vs_product": f"{us / prod_us * 100:.1f}% of the W8A8 qkv product ({prod_us:.1f} us incl. its "
                             f"activation quantization)"}
        fus_us = _time_us(torch, lambda: (tp.tp_lora_down(xd, a, t=tbuf),
                                          tp.tp_qgemm_w8a8_prequantized_lora(qa, sa, q8, s8, tbuf, b, 0.8, out=y2)))
        row["in_store"] = {"us": round(fus_us, 2), "product_alone_us": round(pre_us, 2),
                           "extra_us": round(fus_us - pre_us, 2),
                           "note": f"tp_lora_down + tp_qgemm_w8a8_prequantized_lora: the side path costs "
                                   f"{(fus_us - pre_us) / pre_us * 100:.1f}% of the prequantized product"}
        if cpu:
            import oracle
            rows = 64
            x64 = x[:rows].double().numpy()
            a64, b64 = a.double().cpu().numpy(), b.double().cpu().numpy()
            c64 = np.zeros((rows, wl.n))
            times = []
            for _ in range(3):
                t0 = time.perf_counter()
                oracle.lora_add(c64, x64, a64, b64, 0.8)
                times.append(time.perf_counter() - t0)
            dt = float(np.median(times))
            row["cpu_baseline"] = {"value": round(alg * rows / wl.m / dt / 1e9, 3), "unit": "GB/s", "kind": "oracle",
                                   "sample": f"first {rows} rows, median of 3 ({dt:.3f} s)"}
        res.append(row)
    return res


def _lib_op_w4a8_pre():
    from int4_quantized_gemm_amd import _lib
    return _lib.TP_OP_QGEMM_W4A8_PREQUANTIZED


# ------------------------------------------- platform library, for context only
def library_reference(args):
    """The platform's own GEMMs on the step's shapes: torch._int_mm (int8 x
    int8 -> int32) for the W8A8 products and a bf16 matmul for the
    weight-only ones. Plain products without rotation, quantization or scale
    epilogue; a measure of what the vendor library reaches on this GPU, not a
    part of the product path."""
    import statistics
    import torch
    d = torch.device("cuda:0")

    def timed(f, reps=20):
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        res = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                f()
            e1.record()
            torch.cuda.synchronize()
            res.append(e0.elapsed_time(e1) / reps * 1e-3)
        return statistics.median(res)

    for kind, wl in step_plan():
        m, k, n = wl.m, wl.k, wl.n
        if kind == "w8a8":
            a = torch.randint(-127, 128, (m, k), dtype=torch.int8, device=d)
            b = torch.randint(-127, 128, (n, k), dtype=torch.int8, device=d).t()
            f, what, peak = (lambda: torch._int_mm(a, b)), "torch._int_mm int8->int32", PEAK_TOPS_I8
        else:
            a = torch.randn((m, k), device=d).to(torch.bfloat16)
            b = torch.randn((n, k), device=d).to(torch.bfloat16).t()
            f, what, peak = (lambda: a @ b), "torch.matmul bf16", PEAK_TFLOPS_BF16
        sec = timed(f)
        rate = 2.0 * m * n * k / sec / 1e12
        print(json.dumps({"metric": "platform library GEMM (context)", "shape": wl.name, "m": m, "k": k, "n": n,
                          "op": what, "us": round(sec * 1e6, 1), "rate": round(rate, 1),
                          "frac_of_peak": round(rate / peak, 4)}), flush=True)


# ------------------------------------------------------------------ GPU path
def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    if args.cpu_only:
        print(json.dumps(cpu_baseline(args.cpu_rows)))
        return
    if args.small_m:
        small_m_sweep(args, emit=True)
        return
    if args.library_reference:
        library_reference(args)
        return
    if args.next_only:
        print(json.dumps({"next": next_rows(args, cpu=not args.no_cpu_baseline)}), flush=True)
        return

    import torch
    import int4_quantized_gemm_amd as tp
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    d = torch.device("cuda:0")
    torch.cuda.set_device(d)

    # ---- inputs and offline weight preparation (untimed)
    plan = []
    prep_s = 0.0
    prep_bytes = 0
    for kind, wl in step_plan():
        x, w = W.generate(wl)
        xd = x.to(d)
        wd = w.to(d)
        del x, w
        bits = 4 if kind == "w4" else 8
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        q, s = tp.tp_rotate_quantize_weights(wd, bits=bits)
        torch.cuda.synchronize()
        prep_s += time.perf_counter() - t0
        prep_bytes += wd.numel() * 4
        del wd
        e = {"kind": kind, "wl": wl, "x": xd, "q": q, "s": s}
        if kind == "w8a8":
            e["qa"] = torch.empty((wl.m, wl.k), dtype=torch.int8, device=d)
            e["sa"] = torch.empty((wl.m,), dtype=torch.float32, device=d)
            e["out"] = torch.empty((wl.m, wl.n), dtype=torch.float32, device=d)
        else:
            e["xr"] = torch.empty((wl.m, wl.k), dtype=torch.bfloat16, device=d)
            e["out"] = torch.empty((wl.m, wl.n), dtype=torch.bfloat16, device=d)
        plan.append(e)
    ws = torch.empty((256,), dtype=torch.uint8, device=d)

    # one launch list per step: (name, roofline kind, algorithmic units, callable)
    launches = []
    for e in plan:
        wl = e["wl"]
        if e["kind"] == "w8a8":
            launches.append((f"rotate_quantize_i8[{wl.name}]", "hbm", wl.m * wl.k * (2 + 1) + wl.m * 4,
                             lambda e=e: tp.tp_quantize_rows_int8(e["x"], qa=e["qa"], sa=e["sa"])))
            launches.append((f"gemm_w8a8[{wl.name}]", "i8", 2.0 * wl.m * wl.n * wl.k,
                             lambda e=e: tp.tp_qgemm_w8a8_prequantized(e["qa"], e["sa"], e["q"], e["s"],
                                                                       out=e["out"], workspace=ws)))
        else:
            launches.append((f"rotate_bf16[{wl.name}]", "hbm", wl.m * wl.k * (2 + 2),
                             lambda e=e: tp.tp_hadamard_rotate_rows(e["x"], out=e["xr"])))
            fn = tp.tp_qgemm_w8 if e["kind"] == "w8" else tp.tp_qgemm_w4
            launches.append((f"gemm_{e['kind']}[{wl.name}]", "bf16", 2.0 * wl.m * wl.n * wl.k,
                             lambda e=e, fn=fn: fn(e["xr"], e["q"], e["s"], rotate=False, out=e["out"],
                                                   workspace=ws)))
    step_ops = sum(u for _, k, u, _ in launches if k != "hbm")
    if args.calibrate_copy:
        n = args.calibrate_copy * 2 ** 20 // 4
        src = torch.ones((n,), dtype=torch.float32, device=d)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)  # one elementwise kernel: n*4 B read, n*4 B written
        torch.cuda.synchronize()
        del src, dst
    if args.only:
        launches = [l for l in launches if args.only in l[0]]
        assert launches, f"no launch matches {args.only!r}"

    def run_step(events=None, only=None):
        for i, (_, _, _, fn) in enumerate(launches):
            rec = events is not None and (only is None or i == only)
            if rec:
                events[i][0].record()
            fn()
            if rec:
                events[i][1].record()

    def rate(kind, units, ms):
        sec = ms * 1e-3
        if kind == "hbm":
            return units / sec / 1e9, PEAK_HBM_GBS, "GB/s"
        if kind == "i8":
            return units / sec / 1e12, PEAK_TOPS_I8, "TOP/s"
        return units / sec / 1e12, PEAK_TFLOPS_BF16, "TFLOP/s"

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    # Per-launch breakdown in a pass of its own, before the timed region: an
    # event pair around every launch serializes them (about 90 us per step).
    evb = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in launches]
           for _ in range(args.steps)]
    for s_i in range(args.steps):
        run_step(evb[s_i])
    torch.cuda.synchronize()
    per = []
    for i, (name, kind, units, _) in enumerate(launches):
        ts = [evb[s][i][0].elapsed_time(evb[s][i][1]) for s in range(args.steps)]
        ms = float(np.median(ts))
        ach, peak, unit = rate(kind, units, ms)
        per.append({"launch": name, "us": round(ms * 1e3, 2), "us_min": round(float(np.min(ts)) * 1e3, 2),
                    "achieved": round(ach, 1), "unit": unit, "peak": peak, "frac": round(ach / peak, 4),
                    "bound": "hbm" if kind == "hbm" else "mfma", "units": units, "kind": kind})
    dom_i = max(range(len(per)), key=lambda i: per[i]["us"])

    # Timed region: K steps, an event pair around each step and one around
    # the dominant launch (its roofline figure comes from these).
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in launches]
          for _ in range(args.steps)]
    evs = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_i in range(args.steps):
        evs[s_i][0].record()
        run_step(ev[s_i], only=dom_i)
        evs[s_i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom_ts = [ev[s][dom_i][0].elapsed_time(ev[s][dom_i][1]) for s in range(args.steps)]
    dom_ms = float(np.median(dom_ts))
    step_ts = [evs[s][0].elapsed_time(evs[s][1]) for s in range(args.steps)]
    name, kind, units, _ = launches[dom_i]
    ach, peak, unit = rate(kind, units, dom_ms)
    ms_per_step = wall / args.steps * 1e3
    value = step_ops / (wall / args.steps) / 1e12

    # The shader clock the GPU runs this step at: amd-smi polled while the
    # step repeats for about a second, outside the timed region.
    clock = sample_clock(run_step, torch, seconds=1.5)
    clk = clock.get("sclk_mhz_median")
    dom = {"launch": name, "us": round(dom_ms * 1e3, 2), "us_min": round(float(np.min(dom_ts)) * 1e3, 2),
           "achieved": round(ach, 1), "unit": unit, "peak": peak, "frac": round(ach / peak, 4),
           "bound": "hbm" if kind == "hbm" else "mfma"}

    # The int8 path at M = 4096, K = 3072 (qkv, out, gate+up): quantizer and
    # product per projection, and together.
    k3072 = {}
    tot_us = tot_q_us = tot_ops = 0.0
    for e in plan:
        wl = e["wl"]
        if e["kind"] != "w8a8" or wl.k != 3072:
            continue
        qn, gn = f"rotate_quantize_i8[{wl.name}]", f"gemm_w8a8[{wl.name}]"
        byname = {r["launch"]: r for r in per}
        if qn not in byname or gn not in byname:  # --only
            continue
        qr, gr = byname[qn], byname[gn]
        ops = 2.0 * wl.m * wl.n * wl.k
        k3072[wl.name] = {"n": wl.n, "gemm_us": gr["us"], "gemm_tops": round(ops / gr["us"] / 1e6, 1),
                          "gemm_frac": round(ops / gr["us"] / 1e6 / PEAK_TOPS_I8, 4), "quantize_us": qr["us"],
                          "with_quantize_tops": round(ops / (gr["us"] + qr["us"]) / 1e6, 1)}
        tot_us += gr["us"]
        tot_q_us += qr["us"]
        tot_ops += ops
    k3072_summary = None if not k3072 else {"projections": k3072, "gemm_tops": round(tot_ops / tot_us / 1e6, 1),
                     "gemm_frac": round(tot_ops / tot_us / 1e6 / PEAK_TOPS_I8, 4),
                     "with_quantize_tops": round(tot_ops / (tot_us + tot_q_us) / 1e6, 1),
                     "with_quantize_frac": round(tot_ops / (tot_us + tot_q_us) / 1e6 / PEAK_TOPS_I8, 4),
                     "note": "M=4096, K=3072 W8A8 projections of the block (qkv, out, gate+up): the i8 products "
                             "alone and with their activation rotation + quantization; medians of the breakdown "
                             "pass"}
    # The step against its own roofline: every launch at its peak (i8 or
    # bf16 MFMA, or HBM) against the measured step.
    ideal_us = 0.0
    for r in per:
        if r["kind"] == "hbm":
            ideal_us += r["units"] / (PEAK_HBM_GBS * 1e3)
        elif r["kind"] == "i8":
            ideal_us += r["units"] / (PEAK_TOPS_I8 * 1e6)
        else:
            ideal_us += r["units"] / (PEAK_TFLOPS_BF16 * 1e6)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+bf16",
        "data": "synthetic (seeded Gaussian activations with outlier channels, Gaussian weights with outlier "
                "input columns; no checkpoint)",
        "config": {
            "workload": "dit_block_1024: W8A8 qkv/out/gate+up/down (M=4096) + W8 FFN up (M=4096, K=3072, "
                        "N=12288) + W4 FFN down (M=4032, K=12288, N=3072), activation rotation included",
            "m": 4096,
            "step_ops": step_ops,
        },
        "roofline": {
            "kernel": dom["launch"],
            "bound": dom["bound"],
            "achieved": dom["achieved"],
            "peak": dom["peak"],
            "unit": dom["unit"],
            "frac": dom["frac"],
            "traffic": _traffic_for(dom["launch"]),
            "us": dom["us"],
            "us_min": dom["us_min"],
            "frac_at_measured_clock": round(dom["frac"] * 2400.0 / clk, 4) if clk else None,
        },
        "step_ms": {"median": round(float(np.median(step_ts)), 4), "min": round(float(np.min(step_ts)), 4),
                    "median_over_min": round(float(np.median(step_ts) / np.min(step_ts)), 4),
                    "note": "HIP events around each step of the timed region"},
        "step_roofline": {"ideal_us": round(ideal_us, 1), "measured_us": round(ms_per_step * 1e3, 1),
                          "frac": round(ideal_us / (ms_per_step * 1e3), 4),
                          "note": "every launch of the step at its own peak (i8 MFMA 5.0 POP/s, bf16 MFMA "
                                  "2.5 PFLOP/s, HBM 8 TB/s) against the measured step"},
        "k3072_int8_path": k3072_summary,
        "clock": clock,
        "breakdown": [{k: r[k] for k in ("launch", "us", "us_min", "achieved", "unit", "frac")} for r in per],
        "breakdown_note": "per-launch HIP events in a pass of their own before the timed region (events around "
                          "every launch cost about 90 us per step); median and min over the steps; the timed "
                          "region has events around each step and around the dominant launch only",
        "weight_prep": {"gbs_fp32_read": round(prep_bytes / prep_s / 1e9, 1), "seconds": round(prep_s, 4),
                        "note": "tp_rotate_quantize_weights over every weight of the step, once, untimed in value"},
        "cpu_baseline": None,
    }
    if not args.only and not args.no_small_m:
        rows = small_m_sweep(args)
        by_m = {}
        for r in rows:
            by_m.setdefault(r["m"], []).append(r["frac_hbm"])
        result["small_m"] = {"rows": rows, "min_frac_hbm_by_m": {str(m): min(v) for m, v in by_m.items()},
                             "note": "M <= 64 products against the full-size step weights, cycled through >= 512 "
                                     "MB of weight copies (no last-level-cache hits); bytes = weight codes + "
                                     "scales + activations + output; median of 5 graph replays"}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_rows)
    if not args.no_next and not args.only:
        result["next"] = next_rows(args, cpu=not args.no_cpu_baseline)
    print(json.dumps(result), flush=True)


def sample_clock(run_step, torch, seconds=1.5):
    """Median shader clock (MHz, over samples and XCDs) reported by amd-smi
    while the step repeats; {} where amd-smi is not usable."""
    import shutil
    import subprocess
    import threading
    if "rocprof" in os.environ.get("LD_PRELOAD", "") or any(k.startswith("ROCPROF") for k in os.environ):
        # under the profiler every launch is serialized (the clock means
        # nothing) and a child program would inherit the profiler's library
        return {"sclk_mhz_median": None, "samples": 0, "source": "not sampled under a profiler"}
    smi = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    samples = []
    stop = threading.Event()

    def poll():
        while not stop.is_set():
            try:
                r = subprocess.run([smi, "metric", "-c", "--json"], capture_output=True, text=True, timeout=5)
                j = json.loads(r.stdout[r.stdout.index("{"):] if "{" in r.stdout else r.stdout)
                gd = j["gpu_data"][0] if isinstance(j, dict) else j[0]
                clks = [v["clk"]["value"] for k, v in gd["clock"].items()
                        if k.startswith("gfx") and isinstance(v, dict) and isinstance(v.get("clk"), dict)
                        and isinstance(v["clk"].get("value"), (int, float))]
                if clks:
                    samples.append(float(np.mean(clks)))
            except Exception:
                return

    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        run_step()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=10)
    if not samples:
        return {"sclk_mhz_median": None, "samples": 0, "source": "amd-smi metric -c (not available)"}
    return {"sclk_mhz_median": round(float(np.median(samples)), 1), "sclk_mhz_min": round(float(np.min(samples)), 1),
            "sclk_mhz_max": round(float(np.max(samples)), 1), "samples": len(samples),
            "source": "amd-smi metric -c, mean over XCDs, polled while the step repeats for about 1.5 s "
                      "(outside the timed region)",
            "note": "peak figures are the published 2.4 GHz ones; frac_at_measured_clock rescales the dominant "
                    "launch's fraction to this clock"}


if __name__ == "__main__":
    main()
