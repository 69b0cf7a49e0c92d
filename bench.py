"""Decode throughput of the packed low-bit MLA cache on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload serve] [--no-cpu]

The default workload is the largest one-GPU configuration, the serving step:
B64 H128, lengths uniform in [1024, 131072], one token written per sequence
and then decoded (mla_lowbit_write_decode). The other workloads (tiny, v2lite,
v3, c2r4) are selected with --workload. A step is one mla_lowbit_decode over
one batch of the workload (for the serving workload: one
mla_lowbit_write_decode). The W warmup steps and the K timed
steps are each captured as one HIP graph; the timed region is one replay of
the K-step graph (--eager launches every step from Python instead). Inputs are
resident in HBM when timing starts. Step k uses cache copy k mod R, with R
copies covering more than twice the 256 MB Infinity Cache, so every step
streams its cache from HBM rather than from the previous step's cache lines.

Prints one JSON line: value = cache tokens attended per second (sum of sequence
lengths / step time), plus the roofline of the decode call (HIP events on the
launch stream) and the CPU oracle's throughput on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_MFMA_TFLOPS = 2500.0      # dense fp16/bf16 MFMA
MALL_BYTES = 256 << 20


def algorithmic_bytes(lens, H, c_bits, n_sink=4, n_local=128, max_pages=None):
    """Bytes the method must move per decode: per quantized token its packed copy
    (C4R4 360 B, C2R4 232 B), per protected token 1152 B of BF16, per (b, h) the
    query (1152 B), output (1024 B) and lse (4 B), and 4 B per page-table entry."""
    per_q = 360 if c_bits == 4 else 232
    total = 0
    for L in lens:
        prot = min(L, n_sink) + max(0, min(n_local, L - n_sink))
        total += (L - prot) * per_q + prot * 1152
        total += 4 * ((L + 63) // 64)
    total += len(lens) * H * (1152 + 1024 + 4)
    return total


def algorithmic_flops(lens, H):
    """2 * (576 + 512) flops per cached token per head (QK over 576 channels, PV over 512)."""
    return 2 * (576 + 512) * H * sum(lens)


DECODE_SOURCES = ("bit_mla_kv_lowbit_amd/csrc/decode.hip", "bit_mla_kv_lowbit_amd/csrc/decode_wide.hip",
                  "bit_mla_kv_lowbit_amd/csrc/decode_ops.h", "bit_mla_kv_lowbit_amd/csrc/mla_common.h",
                  "bit_mla_kv_lowbit_amd/csrc/mla_kernels.h")


def decode_source_hash() -> str:
    """Hash of the decode kernels' sources: HBM traffic counters taken on other
    sources no longer describe the kernel and are not reported."""
    import hashlib
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, prefix: str = "decode"):
    """HBM bytes per decode call from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary of this workload (prefix "decode": mla_lowbit_decode,
    "bf16_decode": mla_bf16_decode), or None when it is missing or was taken on
    other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{prefix}_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != decode_source_hash():
        return None
    try:
        return {"bytes_per_call": int(float(kv["traffic_bytes_per_call"])),
                "fetch_bytes": int(float(kv["fetch_bytes_per_call"])),
                "write_bytes": int(float(kv["write_bytes_per_call"])),
                "copy_calibration": float(kv["fetch_scale"]),
                "write_calibration": float(kv.get("write_scale", "1.0"))}
    except (KeyError, ValueError):
        return None


def time_steps(launch, R, steps, warmup, eager, outs):
    """Time `steps` calls of launch(k mod R, stream) after `warmup` untimed ones.
    Graph mode: the warmup and the timed steps are each captured as one HIP
    graph; the timed region is one replay bracketed by HIP events on the stream
    it runs on. Eager mode: every step is launched from Python between its own
    events. The outputs `outs` of the first eager call must be reproduced by the
    warmup replay and by the timed steps. Returns (wall ms per step, event ms
    per step list)."""
    import torch

    cur = torch.cuda.current_stream()
    launch(0, cur)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    def same():
        return all(torch.equal(a, b) for a, b in zip(outs, ref))

    def clear():
        for t in outs:
            t.zero_()

    if eager:
        for k in range(warmup):
            launch(k % R, cur)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            evs[k][0].record(cur)
            launch((warmup + k) % R, cur)
            evs[k][1].record(cur)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ev_ms = [a.elapsed_time(b) for a, b in evs]
    else:
        cap = torch.cuda.Stream()
        cap.wait_stream(cur)

        def capture(first, n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for k in range(first, first + n):
                    launch(k % R, torch.cuda.current_stream())
            return g

        g_warm = capture(0, max(1, warmup))
        g_timed = capture(warmup, steps)
        cur.wait_stream(cap)
        torch.cuda.synchronize()
        clear()
        g_warm.replay()
        torch.cuda.synchronize()
        if not same():
            raise RuntimeError("warmup graph replay differs from the eager call")
        clear()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(cur)
        g_timed.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ev_ms = [e0.elapsed_time(e1) / steps]
    if not same():
        raise RuntimeError("timed steps changed the result")
    return (t1 - t0) * 1e3 / steps, ev_ms


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="serve")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--eager", action="store_true",
                    help="launch every step from Python instead of replaying HIP graphs")
    ap.add_argument("--no-bf16", action="store_true",
                    help="skip the paired BF16-cache decode of the same batch")
    ap.add_argument("--sweep", default="",
                    help="context sweep instead of the workload: comma-separated lengths "
                         "(e.g. 1024,16384,131072,1048576), C4R4 and BF16 at --sweep-batch")
    ap.add_argument("--sweep-batch", type=int, default=8)
    ap.add_argument("--runs", type=int, default=1,
                    help="sweep: independent timing runs per length; with --eager each gives "
                         "--steps samples (the pages' Table 9 protocol is 2 runs x 60 samples)")
    ap.add_argument("--sq", type=int, default=1,
                    help="query tokens per sequence (multi-token prediction verification: "
                         "mla_lowbit_decode_mq; the BF16 pairing is skipped)")
    ap.add_argument("--qdq", action="store_true",
                    help="simulated quantize-dequantize throughput over the workload's tokens")
    ap.add_argument("--prefill", action="store_true",
                    help="bulk writer throughput: the workload's whole cache in one write call")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run one elementwise copy of this many MiB (fp32 negation), the "
                         "known-size kernel that scales the HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; multi-GPU sharding is "
                                   "not implemented, so --gpus must be 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    import bit_mla_kv_lowbit_amd as mla
    import synth

    dev = torch.device("cuda:0")
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 18  # fp32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        print(f"[bench] calibration copy: {args.calib_copy_mib} MiB read + "
              f"{args.calib_copy_mib} MiB written", file=sys.stderr, flush=True)

    if args.sweep:
        return run_sweep(args, [int(x) for x in args.sweep.split(",") if x])
    wl = synth.WORKLOADS[args.workload]
    cfg = mla.Config(c_bits=wl.c_bits)
    if args.prefill:
        return run_prefill(args, wl, cfg)
    if args.qdq:
        return run_qdq(args, wl, cfg)
    print(f"[bench] generating {wl.desc} on the GPU", file=sys.stderr, flush=True)
    inp, step = synth.workload_inputs(wl, device=dev)
    lens = (step.seq_lens if step is not None else inp.seq_lens).cpu().tolist()
    pages, sink, local = mla.allocate_cache(cfg, wl.B, inp.num_pages, dev)
    mla.write(cfg, inp.c_kv, inp.k_rope, inp.seq_idx, inp.pos, inp.seq_lens, inp.page_table,
              pages, sink, local)
    torch.cuda.synchronize()
    cache_bytes = pages.numel() + sink.numel() * 2 + local.numel() * 2
    R = max(1, math.ceil(2 * MALL_BYTES / cache_bytes) + 1) if cache_bytes < 2 * MALL_BYTES else 1
    reps = [(pages, sink, local)]
    for _ in range(R - 1):
        reps.append((pages.clone(), sink.clone(), local.clone()))
    max_pages = inp.page_table.shape[1]
    ws = torch.empty(max(16, mla.decode_workspace_bytes(cfg, wl.B, wl.H, max_pages)),
                     dtype=torch.uint8, device=dev)
    out = torch.empty(wl.B, wl.H, 512, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(wl.B, wl.H, dtype=torch.float32, device=dev)
    seq_lens_dev = step.seq_lens if step is not None else inp.seq_lens
    if args.sq > 1:
        if step is not None:
            raise SystemExit("--sq applies to the decode workloads, not the serving step")
        q_lat, q_rope = synth.queries(wl.B, args.sq * wl.H, wl.seed + 99, dev)
        q_lat = q_lat.view(wl.B, args.sq, wl.H, -1)
        q_rope = q_rope.view(wl.B, args.sq, wl.H, -1)
        ws = torch.empty(max(16, mla.decode_workspace_bytes(cfg, wl.B, args.sq * wl.H,
                                                            max_pages)),
                         dtype=torch.uint8, device=dev)
        out = torch.empty(wl.B, args.sq, wl.H, 512, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(wl.B, args.sq, wl.H, dtype=torch.float32, device=dev)

    def launch(r, stream):
        p, s, l = reps[r]
        if args.sq > 1:
            mla.decode_mq(cfg, q_lat, q_rope, p, inp.page_table, seq_lens_dev, s, l,
                          synth.SOFTMAX_SCALE, out=out, lse=lse, workspace=ws, stream=stream)
        elif step is None:
            mla.decode(cfg, inp.q_lat, inp.q_rope, p, inp.page_table, seq_lens_dev, s, l,
                       synth.SOFTMAX_SCALE, out=out, lse=lse, workspace=ws, stream=stream)
        else:
            mla.write_decode(cfg, step.c_kv, step.k_rope, step.pos, inp.q_lat, inp.q_rope, p,
                             inp.page_table, seq_lens_dev, s, l, synth.SOFTMAX_SCALE, out=out,
                             lse=lse, workspace=ws, stream=stream)

    print(f"[bench] cache {cache_bytes / 1e6:.1f} MB x {R} copies; warmup {args.warmup}",
          file=sys.stderr, flush=True)
    ms_per_step, ev_ms = time_steps(launch, R, args.steps, args.warmup, args.eager, (out, lse))
    ev_mean = float(np.mean(ev_ms))
    print(f"[bench] {args.steps} steps ({'eager' if args.eager else 'one graph'}): "
          f"{ms_per_step * 1e3:.1f} us/step wall, {ev_mean * 1e3:.1f} us/step events",
          file=sys.stderr, flush=True)

    tokens = float(sum(lens))
    value = tokens / (ms_per_step / 1e3)
    # s_q query tokens: s_q * H query rows (query i sees s_q - 1 - i fewer tokens)
    abytes = algorithmic_bytes(lens, args.sq * wl.H, wl.c_bits)
    aflops = sum(algorithmic_flops([max(0, L - (args.sq - 1 - i)) for L in lens], wl.H)
                 for i in range(args.sq))
    bw = abytes / (ev_mean / 1e3) / 1e9
    tf = aflops / (ev_mean / 1e3) / 1e12
    hbm_bound = aflops / abytes < PEAK_MFMA_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    roof = ({"bound": "hbm", "achieved": round(bw, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(bw / PEAK_HBM_GBS, 4)} if hbm_bound else
            {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_MFMA_TFLOPS,
             "unit": "TFLOP/s", "frac": round(tf / PEAK_MFMA_TFLOPS, 4)})
    tr = measured_traffic(args.workload) if args.sq == 1 else None
    roof["traffic"] = tr["bytes_per_call"] if tr else None
    roof["traffic_source"] = (
        f"profiles/decode_traffic_{args.workload}.txt: rocprofv3 FETCH_SIZE and WRITE_SIZE "
        f"passes over the same call on the same kernel sources (hash-checked), fetch scaled "
        f"x{tr['copy_calibration']:.4f} and write x{tr['write_calibration']:.4f} by what the "
        f"counters read for a 512 MiB copy kernel; not measured in this run"
        if tr else "null: no counter summary taken on these kernel sources")
    kernels = ("decode_wide_kernel + combine_wide_kernel" if wl.H == 128
               else "decode_kernel + combine_kernel")
    roof["kernel"] = (f"mla_lowbit_decode: {kernels}" if step is None else
                      f"mla_lowbit_write_decode: write_kernel + {kernels}")
    roof["algorithmic_bytes_per_launch"] = abytes
    roof["algorithmic_flops_per_launch"] = aflops
    roof["hbm_frac"] = round(bw / PEAK_HBM_GBS, 4)
    roof["mfma_frac"] = round(tf / PEAK_MFMA_TFLOPS, 4)
    roof["event_us_mean"] = round(ev_mean * 1e3, 2)
    if args.eager:
        roof["event_us_p10_p50_p90"] = [round(float(np.percentile(ev_ms, q)) * 1e3, 2)
                                       for q in (10, 50, 90)]
    if tr:
        roof["traffic_fetch_write"] = [tr["fetch_bytes"], tr["write_bytes"]]
        roof["traffic_copy_calibration"] = tr["copy_calibration"]

    roof["copy_GBps"] = copy_bandwidth()

    paired = None
    if not args.no_bf16 and args.sq == 1:
        paired = paired_bf16(args, wl, inp, ev_mean * 1e3, cache_bytes, step)

    cpu = None
    parity = None
    if not args.no_cpu and args.sq == 1:
        cpu, parity = cpu_baseline(cfg, wl, inp, step, out, lse, lens, args.cpu_seconds)

    line = {
        "metric": "decode cache tokens/sec and % of HBM/MFMA roofline, C4R4 MLA at 1 GPU",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("u4 codes (C4R4)" if wl.c_bits == 4 else "u2 content / u4 RoPE codes (C2R4)")
                 + ", f16 MFMA, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": wl.desc + (f", s_q={args.sq}" if args.sq > 1 else ""),
                   "B": wl.B, "H": wl.H, "s_q": args.sq,
                   "format": "C4R4" if wl.c_bits == 4 else "C2R4",
                   "tokens_per_step": int(tokens), "cache_copies_rotated": R,
                   "launch": "eager" if args.eager else "one_hip_graph_of_K_steps"},
        "roofline": roof,
        "paired_bf16": paired,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(cfg, wl, inp, step, out, lse, lens, budget_s):
    """Time the CPU oracle's decode on a bounded sample of the same workload:
    whole sequences (all heads), shortest first, repeated in passes until about
    budget_s seconds of oracle time; then check the GPU output on those rows."""
    import numpy as np
    import torch

    import oracle
    import synth

    oc = oracle.Cfg(c_bits=wl.c_bits)
    # one OpenMP thread per core this process may run on, capped by the
    # thread count the environment grants (OMP_NUM_THREADS), if it sets one
    n_affinity = len(os.sched_getaffinity(0))
    n_threads = n_affinity
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        n_threads = max(1, min(n_threads, int(os.environ["OMP_NUM_THREADS"])))
    oracle.set_num_threads(n_threads)
    u16 = lambda t: t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    pt = inp.page_table.cpu().numpy()
    pre = inp.seq_lens.cpu().numpy()
    final = np.array(lens, np.int32)
    D = 576
    seq_idx = inp.seq_idx
    # one oracle cache for the sampled sequences (their page-table rows are disjoint)
    op = np.zeros((inp.num_pages, oracle.page_bytes(oc)), np.uint8)
    osink = np.zeros((wl.B, oc.n_sink, D), np.uint16)
    olocal = np.zeros((wl.B, oc.n_local, D), np.uint16)

    def oracle_write(b):
        mask = seq_idx == b
        oracle.write(oc, u16(inp.c_kv[mask]), u16(inp.k_rope[mask]), seq_idx[mask].cpu().numpy(),
                     inp.pos[mask].cpu().numpy(), pre, pt, op, osink, olocal)
        if step is not None:
            sb = np.array([b], np.int32)
            oracle.write(oc, u16(step.c_kv[[b]]), u16(step.k_rope[[b]]), sb,
                         step.pos.cpu().numpy()[sb], final, pt, op, osink, olocal)

    ql, qr = u16(inp.q_lat), u16(inp.q_rope)
    order = [int(b) for b in np.argsort(final, kind="stable")]
    done, refs, ref_lse = [], {}, {}
    spent, n_tok, passes = 0.0, 0, 0
    while spent < budget_s:
        todo = order if passes == 0 else done
        for b in todo:
            if passes == 0:
                # stop before a sequence that would overrun the budget by much
                if done and spent + spent / n_tok * final[b] > 2 * budget_s:
                    break
                oracle_write(b)
            sel = [(b, h) for h in range(wl.H)]
            t0 = time.perf_counter()
            ref, rl = oracle.decode(oc, synth.SOFTMAX_SCALE, ql, qr, op, pt, final, osink, olocal,
                                    sel=sel)
            spent += time.perf_counter() - t0
            n_tok += int(final[b])
            if passes == 0:
                done.append(b)
                refs[b], ref_lse[b] = ref, rl
            if spent >= budget_s:
                break
        passes += 1
    tok_seq = int(sum(final[d] for d in done))
    cpu = {"value": round(n_tok / spent, 1), "unit": "tokens/s", "cores": n_threads,
           "kind": "oracle",
           "sample": f"{len(done)} of {wl.B} sequences ({tok_seq} cache tokens) x all {wl.H} "
                     f"heads, fp64 plain-loop decode, {passes} pass(es), {n_tok} tokens attended "
                     f"in {spent:.1f} s on {n_threads} OpenMP threads (one per core, heads of a "
                     f"sequence in parallel)",
           "affinity_cores": n_affinity, "cpu_model": cpu_model()}
    # the same oracle on one core, over the shortest sampled sequence
    b1 = done[0]
    oracle.set_num_threads(1)
    t0 = time.perf_counter()
    reps = 0
    while time.perf_counter() - t0 < min(budget_s / 2, 5.0):
        oracle.decode(oc, synth.SOFTMAX_SCALE, ql, qr, op, pt, final, osink, olocal,
                      sel=[(b1, h) for h in range(wl.H)])
        reps += 1
    t1 = time.perf_counter()
    oracle.set_num_threads(n_threads)
    cpu["single_core_value"] = round(reps * int(final[b1]) / (t1 - t0), 1)
    cpu["single_core_sample"] = (f"sequence {b1} ({int(final[b1])} cache tokens) x all {wl.H} "
                                 f"heads, {reps} run(s) in {t1 - t0:.1f} s")
    rows = [(b, h) for b in done for h in range(wl.H)]
    ref = np.concatenate([refs[b] for b in done])
    rl = np.concatenate([ref_lse[b] for b in done])
    got = np.stack([out[b, h].float().cpu().numpy() for b, h in rows])
    gl = lse.cpu().numpy()[[b for b, _ in rows], [h for _, h in rows]]
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    mx = float(np.max(np.abs(got - ref) / np.maximum(1.0, np.abs(ref))))
    dl = float(np.max(np.abs(gl - rl)))
    parity = {"rows": len(rows), "rel_l2": rel, "max_abs_rel": mx, "lse_abs": dl,
              "pass": bool(rel <= 2e-3 and mx <= 1e-2 and dl <= 1e-3)}
    return cpu, parity


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or the platform's processor string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def copy_bandwidth(nbytes=1 << 30, reps=5):
    """Achievable read + write bandwidth of a device-to-device copy of nbytes
    (context for the HBM fraction, not its denominator)."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / reps
    del src, dst
    return round(2 * nbytes / t / 1e9, 1)


def bf16_algorithmic_bytes(lens, H):
    """Bytes a BF16-cache decode must move: 1152 B per cached token, per (b, h)
    the query, output and lse, 4 B per page-table entry."""
    return (sum(L * 1152 + 4 * ((L + 63) // 64) for L in lens)
            + len(lens) * H * (1152 + 1024 + 4))


def _copies(nbytes):
    """Cache copies to rotate so that consecutive steps miss the Infinity Cache."""
    return max(1, math.ceil(2 * MALL_BYTES / nbytes) + 1) if nbytes < 2 * MALL_BYTES else 1


def time_bf16_decode(args, inp, B, H, step=None):
    """The same batch decoded from a BF16 paged cache (mla_bf16_decode), timed
    like the low-bit decode; with a serving step, each step first writes the new
    tokens (mla_bf16_write) and then decodes. Returns (event us per step, cache
    bytes)."""
    import numpy as np
    import torch

    import bit_mla_kv_lowbit_amd as mla
    import synth

    dev = inp.q_lat.device
    pages = mla.allocate_bf16_cache(inp.num_pages, dev)
    mla.bf16_write(inp.c_kv, inp.k_rope, inp.seq_idx, inp.pos, inp.page_table, pages)
    torch.cuda.synchronize()
    nbytes = pages.numel() * 2
    R = _copies(nbytes)
    reps = [pages] + [pages.clone() for _ in range(R - 1)]
    max_pages = inp.page_table.shape[1]
    ws = torch.empty(max(16, mla.bf16_decode_workspace_bytes(B, H, max_pages)),
                     dtype=torch.uint8, device=dev)
    out = torch.empty(B, H, 512, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, H, dtype=torch.float32, device=dev)

    lens = inp.seq_lens if step is None else step.seq_lens
    if step is not None:
        seq_ids = torch.arange(B, dtype=torch.int32, device=dev)

    def launch(r, stream):
        if step is not None:
            mla.bf16_write(step.c_kv, step.k_rope, seq_ids, step.pos, inp.page_table, reps[r],
                           stream=stream)
        mla.bf16_decode(inp.q_lat, inp.q_rope, reps[r], inp.page_table, lens,
                        synth.SOFTMAX_SCALE, out=out, lse=lse, workspace=ws, stream=stream)

    ev_ms = []
    for _ in range(max(1, args.runs)):
        ev_ms += time_steps(launch, R, args.steps, args.warmup, args.eager, (out, lse))[1]
    del reps, pages
    time_bf16_decode.samples_us = [v * 1e3 for v in ev_ms]
    return float(np.mean(ev_ms)) * 1e3, nbytes


def paired_bf16(args, wl, inp, t_lowbit_us, lowbit_cache_bytes, step=None):
    """Figure 5(b) / Table 9 of the pages: the low-bit decode's latency against
    a paired BF16-cache decode of the same batch, delta = t_lowbit / t_bf16 - 1
    (for a serving step: write + decode on both sides)."""
    lens = (inp.seq_lens if step is None else step.seq_lens).cpu().tolist()
    t_bf16, nbytes = time_bf16_decode(args, inp, wl.B, wl.H, step)
    bw = bf16_algorithmic_bytes(lens, wl.H) / (t_bf16 / 1e6) / 1e9
    print(f"[bench] paired BF16 cache: {t_bf16:.1f} us/step events "
          f"({bw:.0f} GB/s algorithmic)", file=sys.stderr, flush=True)
    tr = measured_traffic(wl.name, "bf16_decode") if step is None else None
    dec = ("decode_wide_kernel<BF16 pages> + combine_wide_kernel" if wl.H == 128
           else "decode_kernel<BF16 pages> + combine_kernel")
    return {"kernel": (f"mla_bf16_decode: {dec}" if step is None else
                       f"mla_bf16_write + mla_bf16_decode: write_bf16_kernel + {dec}"),
            "event_us_mean": round(t_bf16, 2), "hbm_frac": round(bw / PEAK_HBM_GBS, 4),
            "traffic": tr["bytes_per_call"] if tr else None,
            "delta_pct": round((t_lowbit_us / t_bf16 - 1.0) * 100.0, 2),
            "cache_bytes": nbytes, "lowbit_cache_bytes": lowbit_cache_bytes,
            "cache_compression": round(nbytes / lowbit_cache_bytes, 3)}


def sweep_cpu_check(inp, out, lse, B, L, H):
    """CPU leg of one sweep length: the oracle writes the last sequence's L
    tokens into a compact page table of its own (physical page ids do not enter
    the result) and decodes all H heads of it, timed; the GPU rows of that
    sequence are checked against it at the decode tolerance."""
    import numpy as np
    import torch

    import oracle
    import synth

    oc = oracle.Cfg(c_bits=4)
    n_thr = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        n_thr = max(1, min(n_thr, int(os.environ["OMP_NUM_THREADS"])))
    oracle.set_num_threads(n_thr)
    u16 = lambda t: t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    b = B - 1
    n_pages = max(1, -(-L // 64))
    pt = np.arange(n_pages, dtype=np.int32)[None]
    lens = np.array([L], np.int32)
    op = np.zeros((n_pages, oracle.page_bytes(oc)), np.uint8)
    osink = np.zeros((1, oc.n_sink, 576), np.uint16)
    olocal = np.zeros((1, oc.n_local, 576), np.uint16)
    t0 = time.perf_counter()
    oracle.write(oc, u16(inp.c_kv[b * L:(b + 1) * L]), u16(inp.k_rope[b * L:(b + 1) * L]),
                 np.zeros(L, np.int32), np.arange(L, dtype=np.int32), lens, pt, op, osink, olocal)
    t1 = time.perf_counter()
    ref, rl = oracle.decode(oc, synth.SOFTMAX_SCALE, u16(inp.q_lat[b:b + 1]),
                            u16(inp.q_rope[b:b + 1]), op, pt, lens, osink, olocal,
                            sel=[(0, h) for h in range(H)])
    t2 = time.perf_counter()
    got = out[b].float().cpu().numpy()
    gl = lse[b].cpu().numpy()
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    mx = float(np.max(np.abs(got - ref) / np.maximum(1.0, np.abs(ref))))
    dl = float(np.max(np.abs(gl - rl)))
    cpu = {"value": round(L / (t2 - t1), 1), "unit": "tokens/s", "cores": n_thr, "kind": "oracle",
           "sample": f"sequence {b} ({L} cache tokens) x all {H} heads, fp64 plain-loop decode "
                     f"in {t2 - t1:.1f} s after a {t1 - t0:.1f} s oracle write"}
    parity = {"rows": H, "rel_l2": rel, "max_abs_rel": mx, "lse_abs": dl,
              "pass": bool(rel <= 2e-3 and mx <= 1e-2 and dl <= 1e-3)}
    print(f"[sweep] L{L} oracle check on sequence {b}: rel_l2 {rel:.2e} max {mx:.2e} "
          f"lse {dl:.2e}", file=sys.stderr, flush=True)
    return cpu, parity


def run_sweep(args, lengths):
    """Context sweep (Figure 5 and Table 9 of the pages): for each length, B
    sequences of H = 16 heads decoded from a C4R4 cache and from a BF16 cache;
    one JSON line per length with both latencies, delta, throughput and the
    persistent allocation of both layouts."""
    import torch

    import bit_mla_kv_lowbit_amd as mla
    import synth

    dev = torch.device("cuda:0")
    B, H = args.sweep_batch, 16
    cfg = mla.C4R4
    for i, L in enumerate(lengths):
        print(f"[sweep] B{B} H{H} L{L}: generating", file=sys.stderr, flush=True)
        inp = synth.bulk_cache_inputs(B, L, H, seed=2000 + i, device=dev)
        pages, sink, local = mla.allocate_cache(cfg, B, inp.num_pages, dev)
        mla.write(cfg, inp.c_kv, inp.k_rope, inp.seq_idx, inp.pos, inp.seq_lens,
                  inp.page_table, pages, sink, local)
        torch.cuda.synchronize()
        low_bytes = pages.numel() + 2 * (sink.numel() + local.numel())
        R = _copies(low_bytes)
        reps = [(pages, sink, local)] + [(pages.clone(), sink.clone(), local.clone())
                                         for _ in range(R - 1)]
        max_pages = inp.page_table.shape[1]
        ws = torch.empty(max(16, mla.decode_workspace_bytes(cfg, B, H, max_pages)),
                         dtype=torch.uint8, device=dev)
        out = torch.empty(B, H, 512, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(B, H, dtype=torch.float32, device=dev)

        def launch(r, stream):
            p, s, l = reps[r]
            mla.decode(cfg, inp.q_lat, inp.q_rope, p, inp.page_table, inp.seq_lens, s, l,
                       synth.SOFTMAX_SCALE, out=out, lse=lse, workspace=ws, stream=stream)

        ev = []
        for _ in range(max(1, args.runs)):
            ev += time_steps(launch, R, args.steps, args.warmup, args.eager, (out, lse))[1]
        t_low = sum(ev) / len(ev) * 1e3
        low_samples = [v * 1e3 for v in ev]
        del reps, pages, sink, local
        check = None if args.no_cpu else sweep_cpu_check(inp, out, lse, B, L, H)
        t_bf16, bf16_bytes = time_bf16_decode(args, inp, B, H)
        lens = [L] * B
        table_bytes = inp.page_table.numel() * 4
        line = {"mode": "sweep", "B": B, "H": H, "L": L,
                "c4r4_us": round(t_low, 2), "bf16_us": round(t_bf16, 2),
                "delta_pct": round((t_low / t_bf16 - 1.0) * 100.0, 2),
                "c4r4_tokens_per_s": round(B * L / (t_low / 1e6), 1),
                "c4r4_hbm_frac": round(algorithmic_bytes(lens, H, 4) / (t_low / 1e6) / 1e9
                                       / PEAK_HBM_GBS, 4),
                "bf16_hbm_frac": round(bf16_algorithmic_bytes(lens, H) / (t_bf16 / 1e6) / 1e9
                                       / PEAK_HBM_GBS, 4),
                "alloc_c4r4_bytes": low_bytes + table_bytes,
                "alloc_bf16_bytes": bf16_bytes + table_bytes,
                "compression": round((bf16_bytes + table_bytes) / (low_bytes + table_bytes), 3)}
        if check is not None:
            line["cpu_baseline"], line["parity"] = check
        if args.eager:
            import numpy as np

            def stats(v):
                return {"n": len(v), "mean": round(float(np.mean(v)), 2),
                        "median": round(float(np.median(v)), 2),
                        "p10": round(float(np.percentile(v, 10)), 2),
                        "p90": round(float(np.percentile(v, 90)), 2)}
            line["c4r4_us_samples"] = stats(low_samples)
            line["bf16_us_samples"] = stats(time_bf16_decode.samples_us)
        print(json.dumps(line), flush=True)
        del inp, ws, out, lse
        torch.cuda.empty_cache()


def run_prefill(args, wl, cfg):
    """Bulk writer throughput: every token of the workload's cache quantized,
    packed and (if protected) copied in one mla_lowbit_write call per step."""
    import numpy as np
    import torch

    import bit_mla_kv_lowbit_amd as mla
    import synth

    dev = torch.device("cuda:0")
    print(f"[prefill] generating {wl.desc} on the GPU", file=sys.stderr, flush=True)
    inp, _ = synth.workload_inputs(wl, device=dev)
    pages, sink, local = mla.allocate_cache(cfg, wl.B, inp.num_pages, dev)

    def launch(r, stream):
        mla.write(cfg, inp.c_kv, inp.k_rope, inp.seq_idx, inp.pos, inp.seq_lens,
                  inp.page_table, pages, sink, local, stream=stream)

    ms, ev = time_steps(launch, 1, args.steps, args.warmup, args.eager, (pages, sink, local))
    t = float(np.mean(ev)) * 1e3
    lens = inp.seq_lens.cpu().tolist()
    n = int(sum(lens))
    per_tok = 360 if wl.c_bits == 4 else 232
    prot = sum(min(L, 4) + max(0, min(128, L - 4)) for L in lens)
    abytes = n * (1152 + 8 + per_tok) + prot * 1152
    bw = abytes / (t / 1e6) / 1e9
    print(json.dumps({"mode": "prefill", "workload": wl.desc, "tokens": n,
                      "event_us_mean": round(t, 2), "tokens_per_s": round(n / (t / 1e6), 1),
                      "roofline": {"bound": "hbm", "achieved": round(bw, 1),
                                   "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                   "frac": round(bw / PEAK_HBM_GBS, 4),
                                   "algorithmic_bytes_per_launch": abytes}}), flush=True)


def run_qdq(args, wl, cfg):
    """QDQ throughput (Figure 3 of the pages: simulated quantize-dequantize):
    every token of the workload's cache through mla_lowbit_qdq in one call."""
    import numpy as np
    import torch

    import bit_mla_kv_lowbit_amd as mla
    import synth

    dev = torch.device("cuda:0")
    print(f"[qdq] generating {wl.desc} on the GPU", file=sys.stderr, flush=True)
    inp, _ = synth.workload_inputs(wl, device=dev)
    out_c, out_r = torch.empty_like(inp.c_kv), torch.empty_like(inp.k_rope)

    def launch(r, stream):
        mla.qdq(cfg, inp.c_kv, inp.k_rope, out_c=out_c, out_r=out_r, stream=stream)

    _, ev = time_steps(launch, 1, args.steps, args.warmup, args.eager, (out_c, out_r))
    t = float(np.mean(ev)) * 1e3
    n = int(inp.c_kv.shape[0])
    abytes = n * 2 * 1152
    bw = abytes / (t / 1e6) / 1e9
    print(json.dumps({"mode": "qdq", "workload": wl.desc, "tokens": n,
                      "event_us_mean": round(t, 2), "tokens_per_s": round(n / (t / 1e6), 1),
                      "roofline": {"bound": "hbm", "achieved": round(bw, 1),
                                   "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                   "frac": round(bw / PEAK_HBM_GBS, 4),
                                   "algorithmic_bytes_per_launch": abytes}}), flush=True)


if __name__ == "__main__":
    main()
