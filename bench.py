"""Decode throughput of the packed low-bit MLA cache on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload v2lite] [--no-cpu]

A step is one mla_lowbit_decode over one batch of the workload (for the serving
workload: one mla_lowbit_write_decode). Inputs are resident in HBM when timing
starts. The step rotates over R independent copies of the cache (R * cache
bytes > 256 MB Infinity Cache), so every step streams its cache from HBM
rather than from the last step's cache lines.

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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="v2lite")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    import bit_mla_kv_lowbit_amd as mla
    import synth

    dev = torch.device("cuda:0")
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
    stream = torch.cuda.current_stream()
    seq_lens_dev = step.seq_lens if step is not None else inp.seq_lens

    def one_step(k):
        p, s, l = reps[k % R]
        if step is None:
            mla.decode(cfg, inp.q_lat, inp.q_rope, p, inp.page_table, seq_lens_dev, s, l,
                       synth.SOFTMAX_SCALE, out=out, lse=lse, workspace=ws, stream=stream)
        else:
            mla.write_decode(cfg, step.c_kv, step.k_rope, step.pos, inp.q_lat, inp.q_rope, p,
                             inp.page_table, seq_lens_dev, s, l, synth.SOFTMAX_SCALE, out=out,
                             lse=lse, workspace=ws, stream=stream)

    print(f"[bench] cache {cache_bytes / 1e6:.1f} MB x {R} copies; warmup {args.warmup}",
          file=sys.stderr, flush=True)
    for k in range(args.warmup):
        one_step(k)
    torch.cuda.synchronize()

    # timed region: exactly K steps; HIP events on the launch stream bracket each call
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        evs[k][0].record(stream)
        one_step(args.warmup + k)
        evs[k][1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    ev_ms = [a.elapsed_time(b) for a, b in evs]
    ev_mean = float(np.mean(ev_ms))
    print(f"[bench] {args.steps} steps: {ms_per_step * 1e3:.1f} us/step wall, "
          f"{ev_mean * 1e3:.1f} us/call events (median {np.median(ev_ms) * 1e3:.1f})",
          file=sys.stderr, flush=True)

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
    roof["traffic"] = None
    roof["kernel"] = "mla_lowbit_decode call (decode_h16 + combine kernels)"
    roof["algorithmic_bytes_per_launch"] = abytes
    roof["algorithmic_flops_per_launch"] = aflops
    roof["event_us_mean"] = round(ev_mean * 1e3, 2)
    roof["event_us_p10_p50_p90"] = [round(float(np.percentile(ev_ms, q)) * 1e3, 2)
                                   for q in (10, 50, 90)]

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
        "dtype": "int4/int2 codes, fp16 MFMA, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": wl.desc, "B": wl.B, "H": wl.H,
                   "format": "C4R4" if wl.c_bits == 4 else "C2R4",
                   "tokens_per_step": int(tokens), "cache_copies_rotated": R},
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(cfg, wl, inp, step, out, lse, lens, budget_s):
    """Time the CPU oracle's decode on a bounded sample of the same workload (whole
    sequences, all heads), and check the GPU output on those rows."""
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

    def oracle_state(seqs):
        mask = torch.zeros(seq_idx.numel(), dtype=torch.bool, device=seq_idx.device)
        for b in seqs:
            mask |= seq_idx == b
        op = np.zeros((inp.num_pages, oracle.page_bytes(oc)), np.uint8)
        osink = np.zeros((wl.B, oc.n_sink, D), np.uint16)
        olocal = np.zeros((wl.B, oc.n_local, D), np.uint16)
        oracle.write(oc, u16(inp.c_kv[mask]), u16(inp.k_rope[mask]),
                     seq_idx[mask].cpu().numpy(), inp.pos[mask].cpu().numpy(), pre, pt, op,
                     osink, olocal)
        if step is not None:
            sb = np.array(seqs, np.int32)
            oracle.write(oc, u16(step.c_kv[seqs]), u16(step.k_rope[seqs]), sb,
                         step.pos.cpu().numpy()[sb], final, pt, op, osink, olocal)
        return op, osink, olocal

    ql, qr = u16(inp.q_lat), u16(inp.q_rope)
    order = list(np.argsort(final))  # shortest first, to fit the time budget
    done, rows, refs, ref_lse = [], [], [], []
    spent = 0.0
    for b in order:
        b = int(b)
        op, osink, olocal = oracle_state([b])
        sel = [(b, h) for h in range(wl.H)]
        t0 = time.perf_counter()
        ref, rl = oracle.decode(oc, synth.SOFTMAX_SCALE, ql, qr, op, pt, final, osink, olocal,
                                sel=sel)
        spent += time.perf_counter() - t0
        done.append(b)
        rows += sel
        refs.append(ref)
        ref_lse.append(rl)
        if spent >= budget_s:
            break
        # estimated time of the next sequence
        nxt = order[len(done)] if len(done) < len(order) else None
        if nxt is None or spent + spent / sum(final[d] for d in done) * final[int(nxt)] > 2 * budget_s:
            break
    tok = float(sum(final[d] for d in done))
    cpu = {"value": round(tok / spent, 1), "unit": "tokens/s", "cores": oracle.num_threads(),
           "kind": "oracle",
           "sample": f"{len(done)} of {wl.B} sequences ({int(tok)} tokens) x all {wl.H} heads, "
                     f"fp64 plain-loop decode, {spent:.1f} s"}
    ref = np.concatenate(refs)
    rl = np.concatenate(ref_lse)
    got = np.stack([out[b, h].float().cpu().numpy() for b, h in rows])
    gl = np.array([lse[b, h].item() for b, h in rows])
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    mx = float(np.max(np.abs(got - ref) / np.maximum(1.0, np.abs(ref))))
    dl = float(np.max(np.abs(gl - rl)))
    parity = {"rows": len(rows), "rel_l2": rel, "max_abs_rel": mx, "lse_abs": dl,
              "pass": bool(rel <= 2e-3 and mx <= 1e-2 and dl <= 1e-3)}
    return cpu, parity


if __name__ == "__main__":
    main()
