"""Benchmark of the attention share on one MI355X.

One step = one pass of the whole hot path over one batch: the Ulysses share of a
sequence-parallel attention layer (8 ranks, 32 query heads, 8 key/value heads,
head dim 128) at S = 131072 tokens in 16 packed documents, as rank 0 sees it,
with the re-layouts fused into the attention loads and stores:

  1. usp_ulysses_attn_fwd: reads rank 0's heads of x_q, x_k, x_v in place from
     the sequence-sharded [8][16384][H][128] tensors (causal over packed documents
     via position_ids) and writes its heads of O back in that layout;
  2. usp_ulysses_attn_bwd: reads x_q, x_k, x_v, O and dO the same way and writes
     rank 0's heads of dX_q, dX_k, dX_v.

The same step through explicit re-layout kernels (seq->head permutes of x_q,
x_k, x_v and dO, blockattn_fwd/bwd on the head-sharded share [131072][4 | 1][128],
head->seq permutes of O and of the gradients) is timed after it and reported
under "components" with each kernel's share of the time.

The share is exactly the packed long-context attention workload (4 query heads
sharing 1 key/value head, 16 documents with multinomial lengths).  `value` is
the whole step's throughput in causal-adjusted attention TFLOP/s (fwd 4*d*vis*Hq,
bwd 2.5x that, vis = visible (query, key) pairs).  The merge of ring partials is
not part of this step; it is timed on its own at the ring workload's shapes and
reported under "components".

Prints ONE JSON line.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "causal attn fwd+bwd TFLOP/s & % bf16 MFMA peak at S=128k; permute GB/s"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E

P, H_Q, H_KV, D = 8, 32, 8, 128
S = 131072
N_DOCS, DOC_SEED, SEED = 16, 1, 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (profiling runs)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the unfused step and the stand-alone permute, merge, ring and "
                         "all-gather measurements (profiling runs)")
    ap.add_argument("--bandwidth-only", action="store_true",
                    help="only the stand-alone permute, copy and merge measurements (HBM byte "
                         "counter runs); prints their JSON line")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain device copy of CALIB_BYTES (calibrates the HBM "
                         "byte counters of a profiling run)")
    return ap.parse_args()


CALIB_BYTES = 512 << 20        # bytes read (and written) by the calibration copy
TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "attn_packed128k_traffic.md")


def kernel_source_hash():
    """sha1 over the HIP sources; a traffic figure counts only for the sources it was
    measured on."""
    import hashlib
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sequence_parallelism_amd", "csrc")
    h = hashlib.sha1()
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(d, name), "rb") as fh:
                h.update(name.encode() + fh.read())
    return h.hexdigest()[:12]


def measured_traffic(call):
    """HBM bytes per call of `call` ('fwd' or 'bwd') from the committed counter summary,
    or None when it is missing or was taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if line.startswith("traffic_bytes_per_call:"):
                    kv = dict(t.split("=") for t in line.split(":", 1)[1].split())
                    if kv.get("src_hash") == kernel_source_hash() and call in kv:
                        return int(kv[call])
    except (OSError, ValueError):
        pass
    return None


def stats(xs):
    """median / min / mean of per-step times (ms)."""
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "min": round(float(a.min()), 4),
            "mean": round(float(a.mean()), 4)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "one GPU only: the attention share runs on a single device; --gpus must be 1"}))
        sys.exit(2)

    import torch
    import sequence_parallelism_amd as usp
    from sequence_parallelism_amd import inputs

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    usp.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.bandwidth_only:
        g = torch.Generator(device=dev)
        g.manual_seed(SEED + 100)
        print(json.dumps({"bandwidth": bandwidth_measurement(torch, usp, dev, g)}), flush=True)
        return

    # ---- inputs, resident in HBM before timing -----------------------------------
    xq, xk, xv, xdo, pos, lengths = inputs.bench_layer(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(SEED + 100)        # the extras' own draws
    hq, hkv = H_Q // P, H_KV // P
    q = torch.empty((S, hq, D), dtype=torch.bfloat16, device=dev)
    k = torch.empty((S, hkv, D), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    o = torch.empty_like(q)
    lse = torch.empty((hq, S), dtype=torch.float32, device=dev)
    do = torch.empty_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    o_seq, dxq = torch.zeros_like(xq), torch.zeros_like(xq)
    dxk, dxv = torch.zeros_like(xk), torch.zeros_like(xv)
    ws = torch.empty(usp.bwd_workspace_bytes(S, S, hq, hkv, D), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(usp.fwd_workspace_bytes(S, S, hq, hkv, D), dtype=torch.uint8, device=dev)

    vis = int(np.sum(lengths * (lengths + 1) // 2))
    fwd_flop = 4.0 * D * vis * hq
    bwd_flop = 2.5 * fwd_flop
    eb = 2
    perm_bytes = {  # algorithmic bytes: every element read once and written once
        "seq_to_head_qkv": 2 * eb * (q.numel() + k.numel() + v.numel()),
        "head_to_seq_o": 2 * eb * o.numel(),
        "seq_to_head_do": 2 * eb * do.numel(),
        "head_to_seq_grads": 2 * eb * (dq.numel() + dk.numel() + dv.numel()),
    }
    stream = torch.cuda.current_stream()
    names_u = ["seq_to_head_qkv", "fwd", "head_to_seq_o", "seq_to_head_do", "bwd", "head_to_seq_grads"]
    names = ["fwd", "bwd"]

    def step(ev=None):
        """The fused step: the timed hot path."""
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        usp.ulysses_attn_fwd(xq, xk, xv, 0, pos, o_seq=o_seq, lse=lse, workspace=ws_f)
        mark(1)
        usp.ulysses_attn_bwd(xq, xk, xv, o_seq, lse, xdo, 0, pos, dxq=dxq, dxk=dxk, dxv=dxv,
                             workspace=ws)
        mark(2)

    def step_unfused(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        usp.seq_to_head(xq, P, group=0, out=q)
        usp.seq_to_head(xk, P, group=0, out=k)
        usp.seq_to_head(xv, P, group=0, out=v)
        mark(1)
        usp.blockattn_fwd(q, k, v, pos, o=o, lse=lse, workspace=ws_f)
        mark(2)
        usp.head_to_seq(o, P, H_Q, out=o_seq, group=0)
        mark(3)
        usp.seq_to_head(xdo, P, group=0, out=do)
        mark(4)
        usp.blockattn_bwd(q, k, v, o, lse, do, pos, dq=dq, dk=dk, dv=dv, workspace=ws)
        mark(5)
        usp.head_to_seq(dq, P, H_Q, out=dxq, group=0)
        usp.head_to_seq(dk, P, H_KV, out=dxk, group=0)
        usp.head_to_seq(dv, P, H_KV, out=dxv, group=0)
        mark(6)

    def run(fn, n_marks, steps):
        """Times `steps` calls of fn bracketed by synchronisations; per-component HIP
        events on the launch stream (per-step lists)."""
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_marks)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            fn(evs[i])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return (t1 - t0) * 1e3 / steps, [[e[j].elapsed_time(e[j + 1]) for e in evs]
                                         for j in range(n_marks - 1)]

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms_step, per = run(step, 3, args.steps)
    comp_stats = dict(zip(names, (stats(x) for x in per)))
    comp_ms = {n: float(np.mean(x)) for n, x in zip(names, per)}
    # the fused step's outputs (identical in every step: the kernels are deterministic),
    # rank 0's heads in global token order, for the parity check against the oracle
    got = {name: inputs.share_of(t, P, 0).cpu() for name, t in
           (("o", o_seq), ("dq", dxq), ("dk", dxk), ("dv", dxv))}
    got["lse"] = lse.cpu()

    ms_unfused, comp_u = None, {}
    if not args.no_extras:
        for _ in range(args.warmup):
            step_unfused()
        ms_unfused, per_u = run(step_unfused, 7, args.steps)
        comp_u = {n: float(np.mean(x)) for n, x in zip(names_u, per_u)}

    step_s = ms_step / 1e3
    value = (fwd_flop + bwd_flop) / step_s / 1e12
    fwd_tf = fwd_flop / (comp_ms["fwd"] / 1e3) / 1e12
    bwd_tf = bwd_flop / (comp_ms["bwd"] / 1e3) / 1e12
    components = {
        "ms": {n: round(v_, 4) for n, v_ in comp_ms.items()},
        "ms_stats": comp_stats,
        "attn_fwd_TFLOPs": round(fwd_tf, 2),
        "attn_bwd_TFLOPs": round(bwd_tf, 2),
        "attn_fwd_frac_of_bf16_peak": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
        "attn_bwd_frac_of_bf16_peak": round(bwd_tf / PEAK_BF16_TFLOPS, 4),
        "attn_fwd_TFLOPs_at_median": round(fwd_flop / (comp_stats["fwd"]["median"] / 1e3) / 1e12, 2),
        "attn_bwd_TFLOPs_at_median": round(bwd_flop / (comp_stats["bwd"]["median"] / 1e3) / 1e12, 2),
        "visible_pairs_per_head": vis,
    }
    if comp_u:
        perm_gbps = sum(perm_bytes.values()) / (sum(comp_u[n] for n in perm_bytes) / 1e3) / 1e9
        components.update({
            "unfused_step_ms": round(ms_unfused, 4),
            "unfused_ms": {n: round(v_, 4) for n, v_ in comp_u.items()},
            "permute_GBps_in_unfused_step": round(perm_gbps, 1),
            "permute_frac_of_hbm_peak_in_unfused_step": round(perm_gbps / PEAK_HBM_GBPS, 4),
        })

    # dominant launch: the backward call, its kernels timed together by the events around
    # it on the launch stream
    dominant = "bwd" if comp_ms["bwd"] >= comp_ms["fwd"] else "fwd"
    dom_flop = bwd_flop if dominant == "bwd" else fwd_flop
    achieved = dom_flop / (comp_ms[dominant] / 1e3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(dominant),
                "kernel": "usp_ulysses_attn_bwd call: launch-order schedules, dQ kernel (also D and the "
                          "row scalars), dK/dV kernel" if dominant == "bwd"
                else "usp_ulysses_attn_fwd call: launch-order schedule, attention kernel"}

    if args.calib_copy:
        src = torch.empty(CALIB_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1.0)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if not args.no_extras:
        components.update(causal_4k_measurement(torch, usp, dev, args.steps))
        components.update(single_doc_measurement(torch, usp, q, k, v, do))
        components.update(extra_measurements(torch, usp, dev, g))

    cpu, parity = None, None
    if not args.no_cpu_baseline:
        # rank 0's share of the inputs by plain slicing (host copies)
        host = [inputs.share_of(t, P, 0).cpu() for t in (xq, xk, xv, xdo)]
        cpu, parity = cpu_baseline(*host, lengths, got)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Ulysses SP=8 share, packed long context: S=131072, 16 docs "
                               "(multinomial lengths, seed 1), 4 query heads sharing 1 kv head, "
                               "d=128, bf16; fwd + bwd with the re-layouts fused",
                   "S": S, "Hq": hq, "Hkv": hkv, "D": D, "sp": P, "layer_heads_q": H_Q,
                   "layer_heads_kv": H_KV, "docs": N_DOCS},
        "tokens_per_s": round(S / step_s, 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        "components": components,
    }
    print(json.dumps(out), flush=True)
    if parity is not None and not parity["pass"]:
        sys.exit(1)


def causal_4k_measurement(torch, usp, dev, steps):
    """Single-device causal attention, [4096][8][128] bf16, one document (the small
    configuration; launch-bound, reported only): fwd and bwd timed by events, median
    and min over the steps."""
    from sequence_parallelism_amd import inputs
    qc, kc, vc, doc_, posc = inputs.causal_4k()
    qd, kd, vd, dod = (t.to(dev) for t in (qc, kc, vc, doc_))
    posd = torch.from_numpy(posc).to(dev)
    o, lse = usp.blockattn_fwd(qd, kd, vd, posd)
    dq, dk, dv = usp.blockattn_bwd(qd, kd, vd, o, lse, dod, posd)
    wsf = torch.empty(usp.fwd_workspace_bytes(4096, 4096, 8, 8, D), dtype=torch.uint8, device=dev)
    wsb = torch.empty(usp.bwd_workspace_bytes(4096, 4096, 8, 8, D), dtype=torch.uint8, device=dev)
    n = max(steps, 20)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    for _ in range(5):
        usp.blockattn_fwd(qd, kd, vd, posd, o=o, lse=lse, workspace=wsf)
        usp.blockattn_bwd(qd, kd, vd, o, lse, dod, posd, dq=dq, dk=dk, dv=dv, workspace=wsb)
    torch.cuda.synchronize()
    for e in ev:
        e[0].record()
        usp.blockattn_fwd(qd, kd, vd, posd, o=o, lse=lse, workspace=wsf)
        e[1].record()
        usp.blockattn_bwd(qd, kd, vd, o, lse, dod, posd, dq=dq, dk=dk, dv=dv, workspace=wsb)
        e[2].record()
    torch.cuda.synchronize()
    f = stats([e[0].elapsed_time(e[1]) for e in ev])
    b = stats([e[1].elapsed_time(e[2]) for e in ev])
    flop = 4.0 * D * (4096 * 4097 // 2) * 8
    return {"causal4k_fwd_ms": f, "causal4k_bwd_ms": b,
            "causal4k_fwd_TFLOPs_at_median": round(flop / (f["median"] / 1e3) / 1e12, 1),
            "causal4k_bwd_TFLOPs_at_median": round(2.5 * flop / (b["median"] / 1e3) / 1e12, 1)}


def single_doc_measurement(torch, usp, q, k, v, do, steps=5):
    """The packed 128K share's head-sharded tensors (rank 0's q [131072][4][128], k, v
    [131072][1][128], dO) as ONE causal document, position_ids 0..131071: the literal
    "causal at 128k" reading, reported beside the packed workload (supplementary)."""
    dev = q.device
    S, hq, hkv = q.shape[0], q.shape[1], k.shape[1]
    pos = torch.arange(S, dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((hq, S), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    wsf = torch.empty(usp.fwd_workspace_bytes(S, S, hq, hkv, D), dtype=torch.uint8, device=dev)
    wsb = torch.empty(usp.bwd_workspace_bytes(S, S, hq, hkv, D), dtype=torch.uint8, device=dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for _ in range(2):
        usp.blockattn_fwd(q, k, v, pos, o=o, lse=lse, workspace=wsf)
        usp.blockattn_bwd(q, k, v, o, lse, do, pos, dq=dq, dk=dk, dv=dv, workspace=wsb)
    torch.cuda.synchronize()
    for e in ev:
        e[0].record()
        usp.blockattn_fwd(q, k, v, pos, o=o, lse=lse, workspace=wsf)
        e[1].record()
        usp.blockattn_bwd(q, k, v, o, lse, do, pos, dq=dq, dk=dk, dv=dv, workspace=wsb)
        e[2].record()
    torch.cuda.synchronize()
    f = stats([e[0].elapsed_time(e[1]) for e in ev])
    b = stats([e[1].elapsed_time(e[2]) for e in ev])
    flop = 4.0 * D * (S * (S + 1) // 2) * hq
    ftf = flop / (f["median"] / 1e3) / 1e12
    btf = 2.5 * flop / (b["median"] / 1e3) / 1e12
    del o, lse, dq, dk, dv, wsf, wsb
    return {"single_doc128k_fwd_ms": f, "single_doc128k_bwd_ms": b,
            "single_doc128k_fwd_TFLOPs_at_median": round(ftf, 1),
            "single_doc128k_bwd_TFLOPs_at_median": round(btf, 1),
            "single_doc128k_fwd_frac_of_bf16_peak": round(ftf / PEAK_BF16_TFLOPS, 4),
            "single_doc128k_bwd_frac_of_bf16_peak": round(btf / PEAK_BF16_TFLOPS, 4)}


def extra_measurements(torch, usp, dev, g):
    """Stand-alone permute, copy and merge bandwidth, the emulated rings and the
    all-gather comparison."""
    res = bandwidth_measurement(torch, usp, dev, g)
    res.update(ring_measurement(torch, usp, dev, g))
    res.update(striped_measurement(torch, usp, dev, g))
    res.update(allgather_measurement(torch, usp, dev, g))
    return res


def bandwidth_measurement(torch, usp, dev, g):
    """Stand-alone permute (full bijection of the Ulysses SP=8, 32-head layer) and
    lse_merge (ring blocks of 16384 rows, 2 heads) bandwidth, buffers rotated so
    that the working set exceeds the 256 MB last-level cache; two copy ceilings of
    the same bytes: the runtime's device-to-device copy, and the permute kernel
    itself with one rank (an identity map: a plain contiguous copy)."""
    res = {}
    sets = 3
    xs = [torch.randn((8, 4096, 32, 128), generator=g, device=dev).to(torch.bfloat16)
          for _ in range(sets)]
    ys = [torch.empty((8, 32768, 4, 128), dtype=torch.bfloat16, device=dev) for _ in range(sets)]
    for i in range(sets):
        usp.seq_to_head(xs[i], 8, out=ys[i])
    torch.cuda.synchronize()
    n = 12
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        usp.seq_to_head(xs[i % sets], 8, out=ys[i % sets])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    nbytes = 2 * xs[0].numel() * 2
    res["permute_full_sp8_GBps"] = round(nbytes / (ms / 1e3) / 1e9, 1)
    res["permute_full_sp8_frac_of_hbm_peak"] = round(nbytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 4)
    e0.record()
    for i in range(n):
        usp.head_to_seq(ys[i % sets], 8, 32, out=xs[i % sets])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    res["permute_inverse_full_sp8_GBps"] = round(nbytes / (ms / 1e3) / 1e9, 1)
    # measured copy ceiling: a plain contiguous device-to-device copy of the same bytes
    # over the same rotating buffers (cold in the last-level cache, like the permutes)
    zs = [torch.empty_like(xs[0]) for _ in range(sets)]
    for i in range(sets):
        zs[i].copy_(xs[i])
    torch.cuda.synchronize()
    e0.record()
    for i in range(n):
        zs[i % sets].copy_(xs[i % sets])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    copy_gbps = nbytes / (ms / 1e3) / 1e9
    res["hbm_copy_measured_GBps"] = round(copy_gbps, 1)
    res["permute_full_sp8_frac_of_measured_copy"] = round(res["permute_full_sp8_GBps"] / copy_gbps, 4)
    # the permute kernel with P = 1: [1][32768][32][128] -> the same layout, a contiguous copy
    flat = lambda t: t.view(1, -1, t.shape[2], t.shape[3])
    for i in range(sets):
        usp.seq_to_head(flat(xs[i]), 1, out=flat(zs[i]))
    torch.cuda.synchronize()
    e0.record()
    for i in range(n):
        usp.seq_to_head(flat(xs[i % sets]), 1, out=flat(zs[i % sets]))
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    kcopy = nbytes / (ms / 1e3) / 1e9
    res["permute_kernel_as_copy_GBps"] = round(kcopy, 1)
    res["permute_full_sp8_frac_of_kernel_copy"] = round(res["permute_full_sp8_GBps"] / kcopy, 4)
    del xs, ys, zs

    blk, H, nb = 16384, 2, 16
    acc = torch.zeros((nb * blk, H, 128), dtype=torch.float32, device=dev)
    acc_l = torch.full((H, nb * blk), -float("inf"), dtype=torch.float32, device=dev)
    parts = [torch.randn((blk, H, 128), generator=g, device=dev) for _ in range(2)]
    pl = [torch.randn((H, blk), generator=g, device=dev) for _ in range(2)]
    for i in range(nb):
        usp.lse_merge(acc[i * blk:(i + 1) * blk], acc_l[:, i * blk:(i + 1) * blk], parts[0], pl[0])
    torch.cuda.synchronize()
    n = 4 * nb
    e0.record()
    for i in range(n):
        b = i % nb
        usp.lse_merge(acc[b * blk:(b + 1) * blk], acc_l[:, b * blk:(b + 1) * blk], parts[i % 2],
                      pl[i % 2])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    nbytes = 3 * blk * H * 128 * 4 + 3 * H * blk * 4   # O_acc r/w + O_part r; LSE r/w + r
    res["lse_merge_GBps"] = round(nbytes / (ms / 1e3) / 1e9, 1)
    res["lse_merge_frac_of_hbm_peak"] = round(nbytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 4)
    res["lse_merge_us"] = round(ms * 1e3, 2)
    del acc, acc_l, parts, pl
    return res


def timed(torch, fn, reps=1):
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def ring_measurement(torch, usp, dev, g):
    """The 256K single-document ring emulated on one GPU: query block i (16384 rows,
    2 heads) against key blocks 0..i, fp32 partials merged by lse_merge (136 block
    pairs); then the backward over the same pairs with the merged O and LSE.  The
    summing of partial gradients across pairs (torch additions) is not timed."""
    S, H, nb = 262144, 2, 16
    blk = S // nb
    mk = lambda: torch.randn((S, H, D), generator=g, device=dev).to(torch.bfloat16)
    q, k, v, do = mk(), mk(), mk(), mk()
    pos = torch.arange(S, dtype=torch.int32, device=dev)
    acc = torch.zeros((S, H, D), dtype=torch.float32, device=dev)
    acc_l = torch.full((H, S), -float("inf"), dtype=torch.float32, device=dev)
    po = torch.empty((blk, H, D), dtype=torch.float32, device=dev)
    pl = torch.empty((H, blk), dtype=torch.float32, device=dev)
    wsf = torch.empty(usp.fwd_workspace_bytes(blk, blk, H, H, D), dtype=torch.uint8, device=dev)
    wsb = torch.empty(usp.bwd_workspace_bytes(blk, blk, H, H, D), dtype=torch.uint8, device=dev)
    pq = torch.empty((blk, H, D), dtype=torch.bfloat16, device=dev)
    pk, pv = torch.empty_like(pq), torch.empty_like(pq)
    o = torch.empty((S, H, D), dtype=torch.bfloat16, device=dev)

    def fwd():
        acc.zero_()
        acc_l.fill_(-float("inf"))
        for i in range(nb):
            qs = slice(i * blk, (i + 1) * blk)
            for j in range(i + 1):
                ks = slice(j * blk, (j + 1) * blk)
                usp.blockattn_fwd(q[qs], k[ks], v[ks], pos, q_start=i * blk, k_start=j * blk,
                                  o=po, lse=pl, workspace=wsf)
                usp.lse_merge(acc[qs], acc_l[:, qs], po, pl)

    def bwd():
        for i in range(nb):
            qs = slice(i * blk, (i + 1) * blk)
            for j in range(i + 1):
                ks = slice(j * blk, (j + 1) * blk)
                usp.blockattn_bwd(q[qs], k[ks], v[ks], o[qs], acc_l[:, qs], do[qs], pos,
                                  q_start=i * blk, k_start=j * blk, dq=pq, dk=pk, dv=pv,
                                  workspace=wsb)

    ms_f = timed(torch, fwd)
    o.copy_(acc)
    ms_b = timed(torch, bwd)
    flop_f = 4.0 * D * (S * (S + 1) // 2) * H
    return {"ring256k_fwd_ms": round(ms_f, 2), "ring256k_fwd_TFLOPs": round(flop_f / ms_f / 1e9, 1),
            "ring256k_bwd_ms": round(ms_b, 2),
            "ring256k_bwd_TFLOPs": round(2.5 * flop_f / ms_b / 1e9, 1)}


def striped_measurement(torch, usp, dev, g):
    """The 256K single-document ring over 16 ranks, contiguous blocks against stripes
    (rank r holding tokens r, r + 16, ...), emulated on one GPU.  Every (query rank,
    key rank) call of the forward and of the backward is timed on its own; a ring step
    lasts as long as its slowest rank, so the ring's time is the sum over steps of
    the per-step maximum (a contiguous pair above the diagonal has no visible key and
    is skipped).  The work is the same in both layouts; the stripes balance it."""
    S, H, P = 262144, 2, 16
    n = S // P
    mk = lambda: torch.randn((S, H, D), generator=g, device=dev).to(torch.bfloat16)
    q, k, v, do = mk(), mk(), mk(), mk()
    pos = torch.arange(S, dtype=torch.int32, device=dev)
    po = torch.empty((n, H, D), dtype=torch.float32, device=dev)
    pl = torch.empty((H, n), dtype=torch.float32, device=dev)
    wsf = torch.empty(usp.fwd_workspace_bytes(n, n, H, H, D), dtype=torch.uint8, device=dev)
    wsb = torch.empty(usp.bwd_workspace_bytes(n, n, H, H, D), dtype=torch.uint8, device=dev)
    pq = torch.empty((n, H, D), dtype=torch.bfloat16, device=dev)
    pk, pv = torch.empty_like(pq), torch.empty_like(pq)
    acc = torch.zeros((P, n, H, D), dtype=torch.float32, device=dev)
    acc_l = torch.full((P, H, n), -float("inf"), dtype=torch.float32, device=dev)

    def per_call(calls):
        """calls: {(i, j): fn}; returns {(i, j): ms}, after one untimed pass."""
        for fn in calls.values():
            fn()
        torch.cuda.synchronize()
        evs = {key: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for key in calls}
        for key, fn in calls.items():
            evs[key][0].record()
            fn()
            evs[key][1].record()
        torch.cuda.synchronize()
        return {key: e[0].elapsed_time(e[1]) for key, e in evs.items()}

    def ring_time(ms):
        return sum(max(ms.get((i, (i - t) % P), 0.0) for i in range(P)) for t in range(P))

    res = {}
    # contiguous blocks: pairs j <= i
    blk = lambda t, i: t[i * n:(i + 1) * n]
    for i in range(P):
        for j in range(i + 1):
            usp.blockattn_fwd(blk(q, i), blk(k, j), blk(v, j), pos, q_start=i * n, k_start=j * n,
                              o=po, lse=pl, workspace=wsf)
            usp.lse_merge(acc[i], acc_l[i], po, pl)
    o_c = acc.to(torch.bfloat16)
    fwd_c = {(i, j): (lambda i=i, j=j: usp.blockattn_fwd(
        blk(q, i), blk(k, j), blk(v, j), pos, q_start=i * n, k_start=j * n, o=po, lse=pl, workspace=wsf))
        for i in range(P) for j in range(i + 1)}
    bwd_c = {(i, j): (lambda i=i, j=j: usp.blockattn_bwd(
        blk(q, i), blk(k, j), blk(v, j), o_c[i], acc_l[i], blk(do, i), pos, q_start=i * n,
        k_start=j * n, dq=pq, dk=pk, dv=pv, workspace=wsb))
        for i in range(P) for j in range(i + 1)}
    # stripes: every pair
    qs, ks, vs, dos = (usp.seq_to_stripe(t, P) for t in (q, k, v, do))
    acc.zero_()
    acc_l.fill_(-float("inf"))
    for i in range(P):
        for j in range(P):
            usp.striped_attn_fwd(qs[i], ks[j], vs[j], P, i, j, pos, o=po, lse=pl, workspace=wsf)
            usp.lse_merge(acc[i], acc_l[i], po, pl)
    o_s = acc.to(torch.bfloat16)
    fwd_s = {(i, j): (lambda i=i, j=j: usp.striped_attn_fwd(
        qs[i], ks[j], vs[j], P, i, j, pos, o=po, lse=pl, workspace=wsf)) for i in range(P) for j in range(P)}
    bwd_s = {(i, j): (lambda i=i, j=j: usp.striped_attn_bwd(
        qs[i], ks[j], vs[j], o_s[i], acc_l[i], dos[i], P, i, j, pos, dq=pq, dk=pk, dv=pv, workspace=wsb))
        for i in range(P) for j in range(P)}
    t = {name: per_call(c) for name, c in (("fc", fwd_c), ("bc", bwd_c), ("fs", fwd_s), ("bs", bwd_s))}
    ring_c = ring_time(t["fc"]) + ring_time(t["bc"])
    ring_s = ring_time(t["fs"]) + ring_time(t["bs"])
    res["ring16_256k_contiguous_fwd_bwd_ms"] = round(ring_c, 2)
    res["ring16_256k_striped_fwd_bwd_ms"] = round(ring_s, 2)
    res["ring16_256k_striped_speedup"] = round(ring_c / ring_s, 3)
    res["ring16_256k_serial_contiguous_ms"] = round(sum(t["fc"].values()) + sum(t["bc"].values()), 2)
    res["ring16_256k_serial_striped_ms"] = round(sum(t["fs"].values()) + sum(t["bs"].values()), 2)
    return res


def allgather_measurement(torch, usp, dev, g):
    """The 32-head, S = 32768 layer (8 key/value heads, one causal document) under the
    two decompositions, each GPU's compute emulated on this one: Ulysses (rank 0's 4
    query heads over all 32768 tokens) and all-gather-KV (rank r's 4096 rows of all 32
    heads against the full K, V).  The slowest rank sets the layer's pace."""
    S, P, Hq, Hkv = 32768, 8, 32, 8
    n = S // P
    mk = lambda *shape: torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
    pos = torch.arange(S, dtype=torch.int32, device=dev)
    res = {}
    # Ulysses share: [S][4][128] q, [S][1][128] k, v
    q, k, v, do = mk(S, Hq // P, D), mk(S, Hkv // P, D), mk(S, Hkv // P, D), mk(S, Hq // P, D)
    o, lse = usp.blockattn_fwd(q, k, v, pos)

    def uly():
        usp.blockattn_fwd(q, k, v, pos, o=o, lse=lse)
        usp.blockattn_bwd(q, k, v, o, lse, do, pos)
    res["cmp32k_ulysses_share_fwd_bwd_ms"] = round(timed(torch, uly, 3), 3)
    # all-gather-KV: rank r's rows of all heads
    q, k, v, do = mk(S, Hq, D), mk(S, Hkv, D), mk(S, Hkv, D), mk(S, Hq, D)
    per_rank = []
    for r in (0, P - 1):
        rs = slice(r * n, (r + 1) * n)
        o, lse = usp.blockattn_fwd(q[rs], k, v, pos, q_start=r * n)

        def ag():
            usp.blockattn_fwd(q[rs], k, v, pos, q_start=r * n, o=o, lse=lse)
            usp.blockattn_bwd(q[rs], k, v, o, lse, do[rs], pos, q_start=r * n)
        per_rank.append(round(timed(torch, ag, 3), 3))
    res["cmp32k_allgather_rank0_fwd_bwd_ms"] = per_rank[0]
    res["cmp32k_allgather_rank7_fwd_bwd_ms"] = per_rank[1]
    return res


def host_info():
    """CPU model, numpy's BLAS, physical and logical cores of the host."""
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), "")
    except OSError:
        pass
    blas = ""
    try:
        b = np.show_config(mode="dicts").get("Build Dependencies", {}).get("blas", {})
        blas = f"{b.get('name', '')} {b.get('version', '')}".strip()
    except Exception:
        pass
    try:
        import psutil
        physical = psutil.cpu_count(logical=False)
    except Exception:
        physical = None
    return {"cpu_model": model, "blas": blas, "physical_cores": physical,
            "logical_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}


O_ATOL, O_RTOL, LSE_ATOL, GRAD_REL = 2e-2, 1e-2, 1e-3, 5e-2


def cpu_baseline(q, k, v, do, lengths, got):
    """The fp64 CPU oracle, untuned, on the whole workload: every packed document
    (fwd + bwd, all 4 query heads) of rank 0's share, on the host's cores.  Its
    outputs are then compared with what the timed fused step wrote (`got`: O, LSE,
    dQ, dK, dV of rank 0's heads) at the acceptance tolerances: O within 2e-2 + 1e-2
    |ref| elementwise, LSE within 1e-3, each gradient within 5e-2 of its max-norm
    (per document)."""
    import oracle

    threads = len(os.sched_getaffinity(0))
    f64 = lambda t: t.float().numpy().astype(np.float64)
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    done_flop, spent = 0.0, 0.0
    hq = q.shape[1]
    err = {"o_max_abs": 0.0, "o_max_excess": -np.inf, "lse_max_abs": 0.0,
           "dq_max_rel": 0.0, "dk_max_rel": 0.0, "dv_max_rel": 0.0}
    g = {n: f64(t) if n != "lse" else t.numpy().astype(np.float64) for n, t in got.items()}
    for a, L in zip(starts, lengths):
        a, L = int(a), int(L)
        sl = slice(a, a + L)
        args = (f64(q[sl]), f64(k[sl]), f64(v[sl]))
        dd = f64(do[sl])
        pos = np.arange(L, dtype=np.int32)
        t0 = time.perf_counter()
        ro, rl = oracle.attention_fwd(*args, pos=pos, causal=True, threads=threads)
        rq, rk, rv = oracle.attention_bwd(*args, dd, pos=pos, causal=True, threads=threads)
        spent += time.perf_counter() - t0
        done_flop += 3.5 * 4.0 * D * (L * (L + 1) // 2) * hq
        e = np.abs(g["o"][sl] - ro)
        err["o_max_abs"] = max(err["o_max_abs"], float(e.max()))
        err["o_max_excess"] = max(err["o_max_excess"], float((e - O_RTOL * np.abs(ro)).max()))
        err["lse_max_abs"] = max(err["lse_max_abs"], float(np.abs(g["lse"][:, sl] - rl).max()))
        for n, ref in (("dq", rq), ("dk", rk), ("dv", rv)):
            rel = np.abs(g[n][sl] - ref).max() / max(np.abs(ref).max(), 1e-3)
            err[n + "_max_rel"] = max(err[n + "_max_rel"], float(rel))
    ok = (err["o_max_excess"] <= O_ATOL and err["lse_max_abs"] <= LSE_ATOL and
          max(err["dq_max_rel"], err["dk_max_rel"], err["dv_max_rel"]) <= GRAD_REL)
    parity = {"checked": "every document of rank 0's share, O, LSE, dQ, dK, dV of the timed "
                         "fused step against the fp64 oracle",
              "tolerances": {"o": "abs <= 2e-2 + 1e-2 |ref|", "lse_abs": LSE_ATOL,
                             "grad_rel_to_max": GRAD_REL},
              "max_errors": {n: round(x, 7) for n, x in err.items()}, "pass": bool(ok)}
    cpu = {"value": round(done_flop / spent / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
           "kind": "oracle",
           "sample": f"all {len(lengths)} documents of the packed S=131072 input "
                     f"({int(sum(lengths))} tokens, 4 query heads), fwd+bwd in fp64 numpy, "
                     f"{spent:.1f} s",
           "host": host_info()}
    return cpu, parity


if __name__ == "__main__":
    main()
