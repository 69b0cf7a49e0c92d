"""Decode throughput of the packed low-bit MLA cache on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload v2lite] [--no-cpu]

A step is one mla_lowbit_decode over one batch of the workload (for the serving
workload: one mla_lowbit_write_decode). The W warmup steps and the K timed
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


DECODE_SOURCES = ("bit_mla_kv_lowbit_amd/csrc/decode.hip", "bit_mla_kv_lowbit_amd/csrc/mla_common.h",
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


def measured_traffic(workload: str):
    """HBM bytes per decode call from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary of this workload, or None when it is missing or was taken
    on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"decode_traffic_{workload}.txt")
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
                "copy_calibration": float(kv["fetch_scale"])}
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="v2lite")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--eager", action="store_true",
                    help="launch every step from Python instead of replaying HIP graphs")
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

    wl = synth.WORKLOADS[args.workload]
    cfg = mla.Config(c_bits=wl.c_bits)
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

    def launch(r, stream):
        p, s, l = reps[r]
        if step is None:
            mla.decode(cfg, inp.q_lat, inp.q_rope, p, inp.page_table, seq_lens_dev, s, l,
                       synth.SOFTMAX_SCALE, out=out, lse=lse, workspace=ws, stream=stream)
        else:
            mla.write_decode(cfg, step.c_kv, step.k_rope, step.pos, inp.q_lat, inp.q_rope, p,
                             inp.page_table, seq_lens_dev, s, l, synth.SOFTMAX_SCALE, out=out,
                             lse=lse, workspace=ws, stream=stream)

    print(f"[bench] cache {cache_bytes / 1e6:.1f} MB x {R} copies; warmup {args.warmup}",
          file=sys.stderr, flush=True)
    cur = torch.cuda.current_stream()
    launch(0, cur)
    torch.cuda.synchronize()
    eager_out, eager_lse = out.clone(), lse.clone()

    if args.eager:
        for k in range(args.warmup):
            launch(k % R, cur)
        # timed region: exactly K steps, each bracketed by HIP events on the launch stream
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            evs[k][0].record(cur)
            launch((args.warmup + k) % R, cur)
            evs[k][1].record(cur)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ev_ms = [a.elapsed_time(b) for a, b in evs]
    else:
        # the W warmup steps and the K timed steps are each captured in one HIP
        # graph (step k decodes cache copy k mod R); the timed region is one
        # replay, bracketed by HIP events on the stream it runs on
        cap = torch.cuda.Stream()
        cap.wait_stream(cur)

        def capture(first, n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for k in range(first, first + n):
                    launch(k % R, torch.cuda.current_stream())
            return g

        g_warm = capture(0, max(1, args.warmup))
        g_timed = capture(args.warmup, args.steps)
        cur.wait_stream(cap)
        torch.cuda.synchronize()
        out.zero_()
        lse.zero_()
        g_warm.replay()
        torch.cuda.synchronize()
        if not (torch.equal(out, eager_out) and torch.equal(lse, eager_lse)):
            raise RuntimeError("warmup graph replay differs from the eager decode")
        out.zero_()
        lse.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(cur)
        g_timed.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ev_ms = [e0.elapsed_time(e1) / args.steps]
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    ev_mean = float(np.mean(ev_ms))
    print(f"[bench] {args.steps} steps ({'eager' if args.eager else 'one graph'}): "
          f"{ms_per_step * 1e3:.1f} us/step wall, {ev_mean * 1e3:.1f} us/step events",
          file=sys.stderr, flush=True)
    if not (torch.equal(out, eager_out) and torch.equal(lse, eager_lse)):
        raise RuntimeError("timed steps changed the decode result")

    tokens = float(sum(lens))
    value = tokens / (ms_per_step / 1e3)
    abytes = algorithmic_bytes(lens, wl.H, wl.c_bits)
    aflops = algorithmic_flops(lens, wl.H)
    bw = abytes / (ev_mean / 1e3) / 1e9
    tf = aflops / (ev_mean / 1e3) / 1e12
    hbm_bound = aflops / abytes < PEAK_MFMA_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    roof = ({"bound": "hbm", "achieved": round(bw, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(bw / PEAK_HBM_GBS, 4)} if hbm_bound else
            {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_MFMA_TFLOPS,
             "unit": "TFLOP/s", "frac": round(tf / PEAK_MFMA_TFLOPS, 4)})
    tr = measured_traffic(args.workload) if step is None else None
    roof["traffic"] = tr["bytes_per_call"] if tr else None
    roof["kernel"] = ("mla_lowbit_decode: decode_kernel + combine_kernel"
                      if step is None else
                      "mla_lowbit_write_decode: write_kernel + decode_kernel + combine_kernel")
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

    cpu = None
    parity = None
    if not args.no_cpu:
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
        "dtype": "u4/u2 codes, f16 MFMA, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": wl.desc, "B": wl.B, "H": wl.H,
                   "format": "C4R4" if wl.c_bits == 4 else "C2R4",
                   "tokens_per_step": int(tokens), "cache_copies_rotated": R,
                   "launch": "eager" if args.eager else "one_hip_graph_of_K_steps"},
        "roofline": roof,
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
    cpu = {"value": round(n_tok / spent, 1), "unit": "tokens/s", "cores": oracle.num_threads(),
           "kind": "oracle",
           "sample": f"{len(done)} of {wl.B} sequences ({tok_seq} cache tokens) x all {wl.H} "
                     f"heads, fp64 plain-loop decode, {passes} pass(es), {n_tok} tokens attended "
                     f"in {spent:.1f} s"}
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


if __name__ == "__main__":
    main()
