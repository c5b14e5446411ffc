"""Benchmark of the shared-prompt (DualKV) attention hot path on one MI355X.

One step = the per-micro-batch path of one attention layer:
  1. repack GATHER of the micro-batch's per-token rows (token id, position,
     loss mask, advantage: 16 bytes per token) from N(P+R) to P+NR rows;
  2. forward  (dualkv_fwd)  -> O, LSE;
  3. backward (dualkv_bwd)  -> dQ, dK, dV (delta, dq, dkdv, slot reduction);
  4. repack SCATTER of per-token fp32 outputs back to N(P+R) rows.
Inputs are resident in HBM before the timed region.  `value` is useful
fwd+bwd TFLOP/s: visible (query, key) pairs of the packed layout times
14*D*Hq, divided by the measured step time.

A workload is one layer shape (one prompt group, the single-group entry
points) or a grouped micro-batch (several prompt groups laid one after the
other, the *_groups entry points); the step is the same.

Also reported: forward / backward alone, the same library on the replicated
N(P+R) layout (P'=0, R'=P+R, valid lengths P+L_n: N independent causal
sequences) and the speedup over it (both layouts timed as back-to-back
fwd+bwd calls over the same number of steps, one after the other), the
dominant kernel's roofline (HIP
events bracketing its launches inside the timed steps), and the fp64 CPU
oracle timed on a bounded sample on this host.
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

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_8b",
                    help="a layer shape (one prompt group) or a grouped micro-batch")
    ap.add_argument("--no-replicated", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target length of the CPU oracle sample")
    ap.add_argument("--layer", action="store_true",
                    help="time a whole packed decoder layer (projections, norms, RoPE, attention, MLP) "
                         "instead of the attention step")
    return ap.parse_args()


def timed(fn, steps, torch):
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(steps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def _cpu_description():
    """CPU model, affinity core count and BLAS library of this host."""
    import os
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    from threadpoolctl import threadpool_info
    info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    blas = ", ".join(f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)" for i in info)
    threads = max((i.get("num_threads", 1) for i in info), default=1)
    return model, len(os.sched_getaffinity(0)), blas or "unknown", int(threads)


def cpu_baseline(w, groups, x, seconds):
    """The fp64 oracle on a bounded sample: the replicated sequences of the
    groups in order (group 0's n = 0, 1, ..., then group 1's ...), KV head 0
    (all its query heads), forward + backward, until `seconds` have passed.
    The sample's time is scaled to the whole job (every sequence, every KV
    head; the work of a sequence and head is proportional to its visible
    replicated pairs) and `value` is the job's useful FLOPs of the packed
    layout (the GPU metric's count) over that extrapolated time."""
    import numpy as np

    from oracle import replicated
    from shared_prompt_exact_amd import workcount

    g = w.n_q_heads // w.n_kv_heads
    total = sum(N for N, _, _ in groups)
    done, t0, pairs_done, row0, vl0 = 0, time.perf_counter(), 0, 0, 0
    pairs_all = packed_all = 0
    for N, P, R in groups:
        L = [R] * N if x.valid_len is None else [int(a) for a in x.valid_len[vl0:vl0 + N]]
        pairs_all += workcount.replicated_pairs(N, P, R, w.window, L)
        packed_all += workcount.visible_pairs(N, P, R, w.window, L)
        vl0 += N
    vl0 = 0
    for N, P, R in groups:
        L = [R] * N if x.valid_len is None else [int(a) for a in x.valid_len[vl0:vl0 + N]]
        for n in range(N):
            idx = row0 + replicated.sequence_rows(n, N, P, R)
            replicated.causal_sequence(x.q[idx].astype(np.float64), x.k[idx].astype(np.float64),
                                       x.v[idx].astype(np.float64), x.do[idx].astype(np.float64),
                                       P + L[n], w.window, None, 1024, kv_heads=[0])
            pairs_done += workcount.replicated_pairs(1, P, L[n], w.window)
            done += 1
            if time.perf_counter() - t0 >= seconds:
                break
        if time.perf_counter() - t0 >= seconds:
            break
        row0 += P + N * R
        vl0 += N
    dt = time.perf_counter() - t0
    t_job = dt * (pairs_all / max(pairs_done, 1)) * w.n_kv_heads
    useful = 14 * packed_all * w.n_q_heads * w.head_dim
    model, affinity, blas, threads = _cpu_description()
    return {"value": useful / t_job / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": (f"fp64 oracle (replicated causal attention + analytic backward), KV head 0 "
                       f"of {w.n_kv_heads} with its {g} query heads, {done} of {total} sequences "
                       f"(prompt + response) in {dt:.1f} s; extrapolated to the whole job "
                       f"(all sequences and KV heads, by visible replicated pairs): {t_job:.0f} s; "
                       f"value = the job's useful packed-layout FLOPs / that time"),
            "extrapolated": True, "sample_s": round(dt, 2), "job_s_extrapolated": round(t_job, 1),
            "sample_rate_replicated_tflops": 14 * pairs_done * g * w.head_dim / dt / 1e12,
            "cpu_model": model, "affinity_cores": affinity, "blas": blas}


# Decoder-layer shapes of the attention workloads (hidden size, MLP width,
# RoPE base): Qwen3-8B and the 30B MoE's attention width with a dense MLP of
# the same width as Qwen3-8B's.
LAYER_SHAPES = {"qwen3_8b": (4096, 12288, 1e6), "dapo_long": (4096, 12288, 1e6), "moe_30b": (4096, 12288, 1e6),
                "qwen3_8b_groups": (4096, 12288, 1e6)}


def layer_bench(args, dk, workloads, workcount, torch, dev):
    """One step = forward + backward of one packed decoder layer (x and dy
    resident), against the same layer on the replicated rows."""
    import numpy as np
    if args.workload not in LAYER_SHAPES:
        print(f"no layer shape for {args.workload}", file=sys.stderr)
        sys.exit(2)
    grouped = args.workload in workloads.GROUPED
    w = workloads.GROUPED[args.workload] if grouped else workloads.WORKLOADS[args.workload]
    groups = w.groups if grouped else ((w.n_resp, w.prompt_len, w.resp_len),)
    Hm, F, base = LAYER_SHAPES[args.workload]
    Hq, Hkv, D, Wn = w.n_q_heads, w.n_kv_heads, w.head_dim, w.window
    T, T_rep = w.packed_len, w.replicated_len
    rng = np.random.default_rng(w.seed)
    L = []
    if grouped and w.len_ranges is not None:
        for (N, P, R), (lo, hi) in zip(groups, w.len_ranges):
            L += rng.integers(lo, hi, endpoint=True, size=N).tolist()
    elif not grouped and w.len_range is not None:
        L = rng.integers(w.len_range[0], w.len_range[1], endpoint=True, size=w.n_resp).tolist()
    else:
        L = [R for N, P, R in groups for _ in range(N)]
    g = torch.Generator(device=dev).manual_seed(w.seed)
    shapes = {"norm1": (Hm,), "wq": (Hm, Hq * D), "wk": (Hm, Hkv * D), "wv": (Hm, Hkv * D), "wo": (Hq * D, Hm),
              "norm2": (Hm,), "w1": (Hm, F), "w3": (Hm, F), "w2": (F, Hm)}
    W = {}
    for n, sh in shapes.items():
        if n.startswith("norm"):
            W[n] = (1 + 0.1 * torch.randn(sh, generator=g, device=dev)).to(torch.bfloat16)
        else:
            W[n] = (torch.randn(sh, generator=g, device=dev) / np.sqrt(sh[0])).to(torch.bfloat16)
    x = torch.randn((T, Hm), generator=g, device=dev).to(torch.bfloat16)
    dy = torch.randn((T, Hm), generator=g, device=dev).to(torch.bfloat16)
    valid = torch.tensor(L, dtype=torch.int32, device=dev)

    def setup(groups_, x_, dy_, valid_):
        p = dk.make_layer_params(Hm, Hq, Hkv, D, F, Wn, base, 1e-6, valid_)
        saved = torch.empty(dk.dualkv_layer_saved_bytes(p, groups_), dtype=torch.uint8, device=dev)
        ws = torch.empty(dk.dualkv_layer_workspace_bytes(p, groups_), dtype=torch.uint8, device=dev)
        y, dx = torch.empty_like(x_), torch.empty_like(x_)
        grads = {n: torch.empty_like(W[n]) for n in W}

        def step():
            dk.dualkv_layer_fwd(x_, W, groups_, p, saved=saved, out=y)
            dk.dualkv_layer_bwd(x_, saved, dy_, W, groups_, p, workspace=ws, dx=dx, grads=grads)
        return step

    print(f"[bench] layer {w.name}: packed {T} rows", file=sys.stderr, flush=True)
    step = setup(groups, x, dy, valid)
    for _ in range(args.warmup):
        step()
    ms = timed(step, args.steps, torch)
    dk.dualkv_profile_start()
    for _ in range(args.steps):
        step()
    prof = {k: round(v[1] / args.steps, 3) for k, v in dk.dualkv_profile_stop().items()}
    torch.cuda.empty_cache()
    rep = None
    if not args.no_replicated:
        print(f"[bench] layer {w.name}: replicated {T_rep} rows", file=sys.stderr, flush=True)
        rgroups = tuple((N, 0, P + R) for N, P, R in groups)
        xr = torch.empty((T_rep, Hm), dtype=torch.bfloat16, device=dev)
        dyr = torch.empty_like(xr)
        dk.dualkv_repack_groups(x, groups, dk.DUALKV_SCATTER, out=xr)
        dk.dualkv_repack_groups(dy, groups, dk.DUALKV_SCATTER, out=dyr)
        vr, i = [], 0
        for N, P, R in groups:
            vr += [P + l for l in L[i:i + N]]
            i += N
        rstep = setup(rgroups, xr, dyr, torch.tensor(vr, dtype=torch.int32, device=dev))
        rstep()
        rsteps = max(2, args.steps // 2)
        rms = timed(rstep, rsteps, torch)
        rep = {"ms_fwd_bwd": round(rms, 3), "speedup": round(rms / ms, 3)}
        del rstep, xr, dyr
        torch.cuda.empty_cache()
    lin = Hm * (Hq * D + 2 * Hkv * D) + Hq * D * Hm + 3 * Hm * F
    Li, pairs, rep_pairs = 0, 0, 0
    for N, P, R in groups:
        pairs += workcount.visible_pairs(N, P, R, Wn, L[Li:Li + N])
        rep_pairs += workcount.replicated_pairs(N, P, R, Wn, L[Li:Li + N])
        Li += N
    gemm_fl = 6 * T * lin
    att_fl = 14 * pairs * Hq * D
    line = {"metric": "packed decoder layer fwd+bwd TFLOP/s (projections, norms, RoPE, attention, MLP)",
            "value": round((gemm_fl + att_fl) / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (random weights and activations of the layer shape)",
            "config": {"workload": w.name, "groups": [list(x_) for x_ in groups], "hidden": Hm, "ffn": F,
                       "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": D, "window": Wn,
                       "packed_tokens": T, "replicated_tokens": T_rep},
            "flops": {"gemm": gemm_fl, "attention": att_fl},
            "rho": round(T_rep / T, 4),
            # useful-FLOP ratio of the two layouts: token-wise work scales with
            # the rows, attention with the visible pairs
            "rho_layer": round((6 * T_rep * lin + 14 * rep_pairs * Hq * D) / (gemm_fl + att_fl), 4),
            "replicated": rep, "kernels_ms_per_step": prof}
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the attention "
              "layer is sharded across GPUs by data parallelism over prompt groups, "
              "each GPU running this library on its own micro-batches", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import shared_prompt_exact_amd as dk
    import workloads
    from shared_prompt_exact_amd import profiling, workcount

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if args.layer:
        layer_bench(args, dk, workloads, workcount, torch, dev)
        return
    grouped = args.workload in workloads.GROUPED
    if grouped:
        w = workloads.GROUPED[args.workload]
        groups = w.groups
    else:
        w = workloads.WORKLOADS[args.workload]
        groups = ((w.n_resp, w.prompt_len, w.resp_len),)
    D, Hq, Hkv, Wn = w.head_dim, w.n_q_heads, w.n_kv_heads, w.window
    T, T_rep = w.packed_len, w.replicated_len
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    x = workloads.generate_groups(w) if grouped else workloads.generate(w)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    to = lambda a: torch.from_numpy(a).to(tdt).to(dev)
    q, k, v, do = to(x.q), to(x.k), to(x.v), to(x.do)
    valid = None if x.valid_len is None else torch.from_numpy(x.valid_len).to(dev)
    Ls, vl0 = [], 0          # valid lengths per group
    for N, P, R in groups:
        Ls.append([R] * N if x.valid_len is None else x.valid_len[vl0:vl0 + N].tolist())
        vl0 += N

    pairs = sum(workcount.visible_pairs(N, P, R, Wn, L) for (N, P, R), L in zip(groups, Ls))
    rep_pairs = sum(workcount.replicated_pairs(N, P, R, Wn, L) for (N, P, R), L in zip(groups, Ls))
    fl = workcount.flops(pairs, Hq, D)

    # The library calls of one step, on one group (the single-group entry
    # points) or on several (the grouped ones).
    if grouped:
        def repack(src, direction, out):
            return dk.dualkv_repack_groups(src, groups, direction, out=out)

        def lib_fwd(q_, k_, v_, gs, **kw_):
            return dk.dualkv_fwd_groups(q_, k_, v_, gs, **kw_)

        def lib_bwd(q_, k_, v_, o_, l_, do_, gs, **kw_):
            return dk.dualkv_bwd_groups(q_, k_, v_, o_, l_, do_, gs, **kw_)

        def lib_ws(q_, k_, gs, **kw_):
            return dk.dualkv_bwd_groups_workspace_bytes(q_, k_, gs, **kw_)
    else:
        def repack(src, direction, out):
            return dk.dualkv_repack(src, *groups[0], direction, out=out)

        def lib_fwd(q_, k_, v_, gs, **kw_):
            return dk.dualkv_fwd(q_, k_, v_, *gs[0], **kw_)

        def lib_bwd(q_, k_, v_, o_, l_, do_, gs, **kw_):
            return dk.dualkv_bwd(q_, k_, v_, o_, l_, do_, *gs[0], **kw_)

        def lib_ws(q_, k_, gs, **kw_):
            return dk.dualkv_bwd_workspace_bytes(q_, k_, *gs[0], **kw_)

    # per-micro-batch token rows (id, position, loss mask, advantage bits)
    g = torch.Generator().manual_seed(w.seed)
    tok_rep = torch.randint(0, 2 ** 31 - 1, (T_rep, 4), generator=g, dtype=torch.int32).to(dev)
    tok_packed = torch.empty((T, 4), dtype=torch.int32, device=dev)
    tok_out_packed = torch.zeros((T,), dtype=torch.float32, device=dev)
    tok_out_rep = torch.empty((T_rep,), dtype=torch.float32, device=dev)

    o = torch.empty_like(q)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    dq, dkk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    kw = dict(window=Wn, valid_len=valid)
    ws = torch.empty(max(256, lib_ws(q, k, groups, **kw)), dtype=torch.uint8, device=dev)

    def fwd():
        lib_fwd(q, k, v, groups, out=o, lse=lse, **kw)

    def bwd():
        lib_bwd(q, k, v, o, lse, do, groups, workspace=ws, dq=dq, dk=dkk, dv=dv, **kw)

    def step():
        repack(tok_rep, dk.DUALKV_GATHER, tok_packed)
        fwd()
        bwd()
        repack(tok_out_packed, dk.DUALKV_SCATTER, tok_out_rep)

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms_step = timed(step, args.steps, torch)
    ms_fwd = timed(fwd, args.steps, torch)
    ms_bwd = timed(bwd, args.steps, torch)
    print(f"[bench] step {ms_step:.3f} ms  fwd {ms_fwd:.3f}  bwd {ms_bwd:.3f}", file=sys.stderr, flush=True)

    # Kernel durations from HIP events bracketing each launch (timed steps).
    dk.dualkv_profile_start()
    for _ in range(args.steps):
        step()
    prof = dk.dualkv_profile_stop()
    kernel_flops = {"fwd": fl["kernel_fwd"], "bwd_dq": fl["kernel_bwd_dq"], "bwd_dkdv": fl["kernel_bwd_dkdv"]}
    kernels = {name: {"launches": n, "avg_ms": ms / n} for name, (n, ms) in prof.items()}
    for name, kf in kernel_flops.items():
        if name in kernels:
            kernels[name]["tflops"] = kf / (kernels[name]["avg_ms"] * 1e-3) / 1e12
    dom = max(kernel_flops, key=lambda n: kernels.get(n, {"avg_ms": 0})["avg_ms"] * kernels.get(n, {"launches": 0})["launches"])
    dom_ach = kernels[dom]["tflops"]
    # HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE counter
    # record of this kernel and workload; null once its sources have changed.
    trec = profiling.load_traffic(dom, w.name)
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(dom_ach, 2),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(dom_ach / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": None if trec is None else trec["bytes_per_launch"]}

    # The dense bf16 rate this device sustains (MFMA-only probe, no memory
    # traffic), reported beside the published peak.
    dk.dualkv_mfma_probe(1024, 50)
    torch.cuda.synchronize()
    s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s_ev.record()
    probe_fl = dk.dualkv_mfma_probe(1024, 2000)
    e_ev.record()
    torch.cuda.synchronize()
    achievable = probe_fl / (s_ev.elapsed_time(e_ev) * 1e-3) / 1e12
    roofline["achievable_peak"] = round(achievable, 1)
    roofline["frac_of_achievable"] = round(dom_ach / achievable, 4)

    # Repack of hidden-state-sized rows (Hq*D bf16 per token), HBM bound.
    rep_rows = torch.empty((T_rep,) + tuple(do.shape[1:]), dtype=do.dtype, device=dev)
    repack(do, dk.DUALKV_SCATTER, rep_rows)
    packed_rows = torch.empty_like(do)
    ms_gather = timed(lambda: repack(rep_rows, dk.DUALKV_GATHER, packed_rows), args.steps, torch)
    ms_scatter = timed(lambda: repack(do, dk.DUALKV_SCATTER, rep_rows), args.steps, torch)
    row_b = Hq * D * do.element_size()
    gather_gbs = 2 * T * row_b / (ms_gather * 1e-3) / 1e9
    scatter_gbs = (T + T_rep) * row_b / (ms_scatter * 1e-3) / 1e9
    del rep_rows, packed_rows

    # Same kernels on the replicated layout: every group's N sequences as
    # independent causal sequences (P' = 0, R' = P+R, valid lengths P+L_n).
    rep = None
    if not args.no_replicated:
        print("[bench] replicated layout", file=sys.stderr, flush=True)
        rgroups = tuple((N, 0, P + R) for N, P, R in groups)

        def scatter(t):
            out = torch.empty((T_rep,) + tuple(t.shape[1:]), dtype=t.dtype, device=dev)
            return repack(t, dk.DUALKV_SCATTER, out)

        qr, kr, vr, dor = (scatter(t) for t in (q, k, v, do))
        vr_len = torch.tensor([P + l for (N, P, R), L in zip(groups, Ls) for l in L], dtype=torch.int32,
                              device=dev)
        rkw = dict(window=Wn, valid_len=vr_len)
        orr = torch.empty_like(qr)
        lr = torch.empty((Hq, qr.shape[0]), dtype=torch.float32, device=dev)
        dqr, dkr, dvr = torch.empty_like(qr), torch.empty_like(kr), torch.empty_like(vr)
        wsr = torch.empty(max(256, lib_ws(qr, kr, rgroups, **rkw)), dtype=torch.uint8, device=dev)

        def rfwd():
            lib_fwd(qr, kr, vr, rgroups, out=orr, lse=lr, **rkw)

        def rstep():
            rfwd()
            lib_bwd(qr, kr, vr, orr, lr, dor, rgroups, workspace=wsr, dq=dqr, dk=dkr, dv=dvr, **rkw)

        def pstep():
            fwd()
            bwd()

        # both layouts timed the same way: back-to-back fwd+bwd calls over the
        # same number of steps, one right after the other
        rsteps = max(2, args.steps // 2)
        rstep()
        ms_pk = timed(pstep, rsteps, torch)
        ms_rep = timed(rstep, rsteps, torch)
        ms_pk_fwd = timed(fwd, rsteps, torch)
        ms_rep_fwd = timed(rfwd, rsteps, torch)
        dk.dualkv_profile_start()
        for _ in range(rsteps):
            rstep()
        rprof = dk.dualkv_profile_stop()
        rep = {"ms_fwd_bwd": round(ms_rep, 3), "ms_fwd": round(ms_rep_fwd, 3),
               "kernels_avg_ms": {name: round(ms / n, 4) for name, (n, ms) in rprof.items()},
               "tflops_fwd_bwd": round(14 * rep_pairs * Hq * D / (ms_rep * 1e-3) / 1e12, 2),
               "ms_fwd_bwd_packed": round(ms_pk, 3),
               "speedup_fwd_bwd": round(ms_rep / ms_pk, 3),
               "speedup_fwd": round(ms_rep_fwd / ms_pk_fwd, 3),
               "speedup_step": round(ms_rep / ms_step, 3)}
        del qr, kr, vr, dor, orr, lr, dqr, dkr, dvr, wsr
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu oracle sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, groups, x, args.cpu_seconds)

    value = fl["fwd_bwd"] / (ms_step * 1e-3) / 1e12
    config = {"workload": w.name}
    if grouped:
        config["groups"] = [list(gr) for gr in groups]
    else:
        config.update(N=groups[0][0], P=groups[0][1], R=groups[0][2])
    config.update(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, window=Wn, packed_tokens=T, replicated_tokens=T_rep)
    line = {
        "metric": "DualKV attn fwd+bwd TFLOP/s, % bf16 MFMA peak, speedup vs replicated layout",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded i.i.d. Gaussian activations of the layer shape)",
        "config": config,
        "pct_bf16_peak": round(100 * value / MFMA_BF16_PEAK_TFLOPS, 2),
        "fwd": {"ms": round(ms_fwd, 3), "tflops": round(fl["fwd"] / (ms_fwd * 1e-3) / 1e12, 2)},
        "bwd": {"ms": round(ms_bwd, 3), "tflops": round(fl["bwd"] / (ms_bwd * 1e-3) / 1e12, 2)},
        "rho": round(T_rep / T, 4),
        "rho_attn": round(rep_pairs / pairs, 4),
        "replicated": rep,
        "kernels": {k_: {kk: round(vv, 4) for kk, vv in d.items()} for k_, d in kernels.items()},
        "repack_hidden_rows": {"gather_GBs": round(gather_gbs, 1), "scatter_GBs": round(scatter_gbs, 1),
                               "row_bytes": row_b},
        # Delta / scaled-LSE kernel: reads O, dO (bf16) and LSE, writes Delta
        # and the scaled LSE (fp32): T*Hq*(4*D + 12) bytes
        "bwd_delta_GBs": round(T * Hq * (4 * D + 12) / (kernels["bwd_delta"]["avg_ms"] * 1e-3) / 1e9, 1)
        if "bwd_delta" in kernels else None,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
