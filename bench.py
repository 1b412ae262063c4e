"""Benchmark of the Sol-Attn hot path on one MI355X.

A step = one pass of the whole path over one batch: sol_attn_pool -> sol_attn_select
-> sol_attn_fwd, on seeded synthetic Q/K/V already resident in HBM.  Default workload:
the 1344x768 refinement stage (16 latent frames x 48 x 84 = 64,512 tokens, B=1,
H=40, d=128, bf16, 128-token blocks, top-76 of 504 key blocks).

Prints ONE JSON line.  `value` = effective TFLOP/s of the whole step, counting the
two contractions over the selected key blocks only (4*B*H*L*k*Bs*d flops per step).
`roofline` covers the dominant kernel (sol_attn_fwd): algorithmic flops per launch
divided by its average launch time, from HIP events recorded on its stream between
the kernels of every timed step.
`cpu_baseline` times the float64 CPU oracle on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 matrix peak: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0

# Memory-side traffic of one sol_attn_fwd launch on the headline workload (bytes):
# rocprofv3 FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0 (KiB per dispatch; the factors are what
# the same counters read for the pool kernel in the same command, which reads Q and K
# once and writes the pooled means: profiles/fwd_bf16_refine_1344x768.md).
# The figure belongs to the kernel code whose SHA-256 prefix is stored beside it (the code
# of csrc/fwd_bf16.hip with comments removed and whitespace collapsed): when the code
# differs, the traffic is reported as null until re-measured.
FWD_TRAFFIC_BYTES = 42330755243
FWD_TRAFFIC_SRC_SHA256 = "51a3cbd0bf2c5870"
FWD_SRC = os.path.join(ROOT, "block_sparse_attention_attn_amd", "csrc", "fwd_bf16.hip")
_C_COMMENT_OR_LITERAL = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\])*"|\'(?:\\.|[^\'\\])*\'', re.S)


def code_sha(text: str) -> str:
    """SHA-256 prefix of C/C++ source with comments removed and whitespace collapsed
    (string and character literals are kept as written)."""
    code = _C_COMMENT_OR_LITERAL.sub(lambda m: m.group(0) if m.group(0)[0] in "\"'" else " ", text)
    return hashlib.sha256(" ".join(code.split()).encode()).hexdigest()[:16]


def fwd_source_sha() -> str:
    with open(FWD_SRC, encoding="utf-8") as f:
        return code_sha(f.read())


def fwd_traffic_bytes():
    """The measured traffic if it was taken on the kernel source built here, else None."""
    return FWD_TRAFFIC_BYTES if fwd_source_sha() == FWD_TRAFFIC_SRC_SHA256 else None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="refine_1344x768")
    p.add_argument("--topk", type=int, default=None, help="override k (e.g. all blocks for a dense run)")
    p.add_argument("--pattern", choices=["selected", "window", "cube", "quant"], default="selected",
                   help="selected: pool -> select -> fwd (the method); window: fwd alone with the static "
                        "window pattern of sol_attn_window_blocks (same k); cube: the method with 3-D "
                        "cube blocks read in place from the frame-major tensors (pool_cube, select, fwd_cube); "
                        "quant: the method between the 8-bit exchange formats (Q/K/V INT8 in, output FP8 out), "
                        "with the error against the bf16 path")
    p.add_argument("--cube-reorder", action="store_true",
                   help="cube pattern through reordered copies instead: cube_permute Q/K/V to cube-major "
                        "order, pool -> select -> fwd, cube_permute O back")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-probe", action="store_true",
                   help="after timing, run one plain device copy of Q (size known) to calibrate traffic counters")
    p.add_argument("--cpu-workers", type=int, default=16,
                   help="single-threaded oracle worker processes for the CPU baseline, one head each "
                        "(at most the CPUs this process may use)")
    return p.parse_args()


def _oracle_head(job):
    """One (b, h) head of the oracle's whole path (runs in a single-threaded worker)."""
    import oracle
    wl, q, k, v, topk, pattern = job
    if pattern == "cube":
        oracle.run_cube(q, k, v, wl.dtype, wl.grid, wl.cube, topk)
    elif pattern == "window":
        sel = oracle.window_selection(wl.n_blocks, topk)[None]
        oracle.attend(oracle.widen(q, wl.dtype), oracle.widen(k, wl.dtype), oracle.widen(v, wl.dtype), sel,
                      wl.block)
    else:
        oracle.run(q, k, v, wl.dtype, wl.block, topk)
    return True


def _single_thread_worker():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def cpu_baseline(wl, q, k, v, topk, max_workers, pattern="selected"):
    """Time the float64 oracle as it stands -- pool, select and attend of every query
    block (for the static window pattern: attend alone) -- on the first `workers` (b, h)
    heads of the workload, one head per single-threaded worker process.  Runs before the
    GPU is initialised (the workers are forked from a process that has not touched it)."""
    import concurrent.futures as cf
    import multiprocessing as mp
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count() or 1
    workers = max(1, min(max_workers, avail, wl.B * wl.H))
    if pattern == "quant":
        pattern = "selected"
    qs, ks, vs = (x.reshape(-1, 1, wl.L, wl.d)[:workers] for x in (q, k, v))
    jobs = [(wl, qs[i], ks[i], vs[i], topk, pattern) for i in range(workers)]
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("fork"),
                                initializer=_single_thread_worker) as ex:
        list(ex.map(lambda_ok, range(workers)))            # workers up before the clock starts
        t0 = time.perf_counter()
        list(ex.map(_oracle_head, jobs))
        dt = time.perf_counter() - t0
    if pattern == "cube":
        what = (f"whole path with {'x'.join(map(str, wl.cube))} cube blocks (pool, scores, top-{topk}, float64 "
                f"attention of all {wl.n_blocks} query boxes)")
    elif pattern == "window":
        what = f"float64 attention of all {wl.n_blocks} query blocks over the static window of {topk} blocks"
    else:
        what = f"whole path (pool, scores, top-{topk}, float64 attention of all {wl.n_blocks} query blocks)"
    flops = 4.0 * workers * wl.L * (topk * wl.block) * wl.d
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(workers), "kind": "oracle",
            "seconds": round(dt, 3), "host_cpus_visible": int(avail),
            "sample": f"{workers} of {wl.B * wl.H} heads, one head per single-threaded worker process, {what}; "
                      f"TFLOP/s in the same effective-flop count"}


def lambda_ok(_):
    return True


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); the sparse-attention path has no "
              f"multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    from block_sparse_attention_attn_amd import workloads as W

    wl = W.get(args.workload)
    topk = args.topk or wl.topk
    t_gen = time.perf_counter()
    q, k, v = W.make_qkv(wl)
    t_gen = time.perf_counter() - t_gen
    # the CPU baseline runs first, in worker processes forked before anything touches the GPU
    cpu_rec = None if args.no_cpu_baseline else cpu_baseline(wl, q, k, v, topk, args.cpu_workers, args.pattern)

    import torch
    from block_sparse_attention_attn_amd import sol_attn as S
    S.load_library()

    def dev(x):
        x = np.ascontiguousarray(x)
        if wl.dtype == "bf16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    Q, K, V = dev(q), dev(k), dev(v)
    nb = wl.n_blocks
    qp = torch.empty((wl.B, wl.H, nb, wl.d), dtype=torch.float64, device="cuda")
    kp = torch.empty_like(qp)
    idx = torch.empty((wl.B, wl.H, nb, topk), dtype=torch.int32, device="cuda")
    out = torch.empty_like(Q)
    # schedule query blocks covering the same latent rows of all frames together (cache reuse)
    order = S.sol_attn_frame_order(wl.L, wl.block, wl.lat_h * wl.lat_w, wl.lat_w).cuda()
    stream = torch.cuda.current_stream()
    lib = S.load_library()
    dtc = 0 if wl.dtype == "bf16" else 1
    s_ptr = stream.cuda_stream

    window = args.pattern == "window"
    cube = args.pattern == "cube"
    quant = args.pattern == "quant"
    if window:
        idx.copy_(S.sol_attn_window_blocks(nb, topk).view(1, 1, nb, topk).expand(wl.B, wl.H, nb, topk))
        # a window's tiles are shared by consecutive query blocks: run them side by side
        order = torch.arange(nb, dtype=torch.int32, device="cuda")
    T, h, w = wl.grid
    bt, by, bx = wl.cube
    reorder = cube and args.cube_reorder
    if cube:
        # boxes of bt x by x bx latents, read in place (or, with --cube-reorder, tokens
        # reordered to cube-major order so that a block of consecutive tokens is one box)
        if bt * by * bx != wl.block:
            raise SystemExit(f"cube {wl.cube} does not hold one block of {wl.block} tokens")
        Qc, Kc, Vc, Oc = (torch.empty_like(Q) for _ in range(4)) if reorder else (Q, K, V, out)
        ny, nx = h // by, w // bx
        order = S.sol_attn_frame_order(wl.L, wl.block, wl.block * ny * nx, wl.block * nx).cuda()
    elif quant:
        # one GPU's share of the 8-bit exchange around the attention: Q/K/V as INT8 codes
        # (as received), decoded, the method, the output coded as FP8 (as sent back), decoded
        if wl.dtype != "bf16":
            raise SystemExit("the 8-bit exchange formats take bf16 tensors")
        Qc, Kc, Vc, Oc = (torch.empty_like(Q) for _ in range(4))
        codes = [torch.empty(Q.shape, dtype=torch.uint8, device="cuda") for _ in range(4)]
        scales = [torch.empty(Q.shape[:3], dtype=torch.float32, device="cuda") for _ in range(4)]
    else:
        Qc, Kc, Vc, Oc = Q, K, V, out
    row_bytes = wl.d * Q.element_size()

    def quantize(x, n, fmt):
        S._check("quantize", lib.sol_attn_quantize(x.data_ptr(), wl.B, wl.H, wl.L, wl.d, fmt, codes[n].data_ptr(),
                                                   scales[n].data_ptr(), s_ptr))

    def dequantize(n, fmt, dst):
        S._check("dequantize", lib.sol_attn_dequantize(codes[n].data_ptr(), scales[n].data_ptr(), wl.B, wl.H, wl.L,
                                                       wl.d, fmt, dst.data_ptr(), s_ptr))

    def permute(src, dst, inverse):
        S._check("cube_permute", lib.sol_attn_cube_permute(src.data_ptr(), dst.data_ptr(), wl.B, wl.H, T, h, w,
                                                           row_bytes, bt, by, bx, int(inverse), s_ptr))

    def run_pool():
        S._check("pool", lib.sol_attn_pool(Qc.data_ptr(), Kc.data_ptr(), dtc, wl.B, wl.H, wl.L, wl.d, wl.block,
                                           qp.data_ptr(), kp.data_ptr(), s_ptr))

    def run_select():
        S._check("select", lib.sol_attn_select(qp.data_ptr(), kp.data_ptr(), wl.B, wl.H, nb, wl.d, topk,
                                               idx.data_ptr(), None, s_ptr))

    def run_fwd():
        S._check("fwd", lib.sol_attn_fwd(Qc.data_ptr(), Kc.data_ptr(), Vc.data_ptr(), dtc, wl.B, wl.H, wl.L, wl.d,
                                         wl.block, topk, idx.data_ptr(), order.data_ptr(), 0.0, Oc.data_ptr(),
                                         None, s_ptr))

    def run_pool_cube():
        S._check("pool_cube", lib.sol_attn_pool_cube(Q.data_ptr(), K.data_ptr(), dtc, wl.B, wl.H, T, h, w, wl.d,
                                                     bt, by, bx, qp.data_ptr(), kp.data_ptr(), s_ptr))

    def run_fwd_cube():
        S._check("fwd_cube", lib.sol_attn_fwd_cube(Q.data_ptr(), K.data_ptr(), V.data_ptr(), wl.B, wl.H, T, h, w,
                                                   bt, by, bx, topk, idx.data_ptr(), order.data_ptr(), 0.0,
                                                   out.data_ptr(), None, s_ptr))

    def run_permute_in():
        for src, dst in ((Q, Qc), (K, Kc), (V, Vc)):
            permute(src, dst, False)

    # the phases of one step (HIP events between them give per-kernel durations)
    if window:      # static pattern: the step is the attention alone
        phases = [("fwd", run_fwd)]
    elif reorder:
        phases = [("permute_in", run_permute_in), ("pool", run_pool), ("select", run_select), ("fwd", run_fwd),
                  ("permute_out", lambda: permute(Oc, out, True))]
    elif cube:
        phases = [("pool", run_pool_cube), ("select", run_select), ("fwd", run_fwd_cube)]
    elif quant:
        phases = [("quant_qkv_int8", lambda: [quantize(x, n, S.INT8) for n, x in enumerate((Q, K, V))]),
                  ("dequant_qkv", lambda: [dequantize(n, S.INT8, x) for n, x in enumerate((Qc, Kc, Vc))]),
                  ("pool", run_pool), ("select", run_select), ("fwd", run_fwd),
                  ("quant_o_fp8", lambda: quantize(Oc, 3, S.FP8_E4M3)),
                  ("dequant_o", lambda: dequantize(3, S.FP8_E4M3, out))]
    else:
        phases = [("pool", run_pool), ("select", run_select), ("fwd", run_fwd)]

    def step(ev=None):
        for n, (_, fn) in enumerate(phases):
            if ev is not None:
                ev[n].record(stream)
            fn()
        if ev is not None:
            ev[len(phases)].record(stream)

    quant_err = None
    if quant:
        # error of the 8-bit exchange against the bf16 path (outside the timed region)
        Qc, Kc, Vc, Oc, keep = Q, K, V, out, (Qc, Kc, Vc, Oc)
        run_pool(), run_select(), run_fwd()
        ref_out, ref_idx = out.clone(), idx.clone()
        Qc, Kc, Vc, Oc = keep
        step()
        torch.cuda.synchronize()
        diff = (out.float() - ref_out.float()).abs()
        same = (idx.unsqueeze(-1) == ref_idx.unsqueeze(-2)).any(-1).float().mean().item()
        changed = ~(idx == ref_idx).all(-1)                       # query blocks whose key set moved
        row_changed = changed.repeat_interleave(wl.block, dim=-1)[..., :wl.L]
        kept = diff[~row_changed]
        # the FP8 round trip of the output alone (same selection, exact attention inputs)
        quantize(ref_out, 3, S.FP8_E4M3)
        dequantize(3, S.FP8_E4M3, Oc)
        torch.cuda.synchronize()
        fp8_diff = (Oc.float() - ref_out.float()).abs()
        # the same exchange with the selection made from the exact pooled means (a sender
        # can ship float64 block sums beside the codes): only the attention sees 8-bit data
        idx.copy_(ref_idx)
        for n, x in enumerate((Q, K, V)):
            quantize(x, n, S.INT8)
            dequantize(n, S.INT8, (Qc, Kc, Vc)[n])
        run_fwd()
        quantize(Oc, 3, S.FP8_E4M3)
        dequantize(3, S.FP8_E4M3, Oc)
        torch.cuda.synchronize()
        exact_sel_diff = (Oc.float() - ref_out.float()).abs()
        quant_err = {"o_max_abs_err": round(diff.max().item(), 5), "o_mean_abs_err": round(diff.mean().item(), 6),
                     "o_rms_ref": round(ref_out.float().pow(2).mean().sqrt().item(), 5),
                     "selected_blocks_kept": round(same, 5),
                     "query_blocks_changed": round(changed.float().mean().item(), 5),
                     "o_err_unchanged_blocks": {"max": round(kept.max().item(), 5),
                                                "mean": round(kept.mean().item(), 6)},
                     "o_err_changed_blocks": ({"max": round(diff[row_changed].max().item(), 5),
                                               "mean": round(diff[row_changed].mean().item(), 6)}
                                              if bool(changed.any()) else None),
                     "o_fp8_round_trip": {"max": round(fp8_diff.max().item(), 5),
                                          "mean": round(fp8_diff.mean().item(), 6)},
                     "o_err_selection_from_exact_means": {"max": round(exact_sel_diff.max().item(), 5),
                                                          "mean": round(exact_sel_diff.mean().item(), 6)},
                     "bytes_per_row": {"bf16": 2 * wl.d, "8-bit + scale": wl.d + 4}}
        del ref_out, ref_idx, diff, kept, fp8_diff, row_changed, exact_sel_diff

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps, bracketed by synchronisation; HIP events on the
    # launch stream between the kernels of every step give the per-kernel durations
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for e in evs:
        step(e)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(stop) / args.steps
    samples = {name: np.array([e[n].elapsed_time(e[n + 1]) for e in evs]) for n, (name, _) in enumerate(phases)}
    t_phase = {name: float(np.mean(x)) for name, x in samples.items()}
    t_pool, t_sel, t_fwd = t_phase.get("pool"), t_phase.get("select"), t_phase["fwd"]
    fwd_stats = {"mean": round(t_fwd, 4), "median": round(float(np.median(samples["fwd"])), 4),
                 "min": round(float(np.min(samples["fwd"])), 4),
                 "p90": round(float(np.percentile(samples["fwd"], 90)), 4)}

    # the matrix rate the chip sustains (diagnostic kernel, outside the timed region)
    mfma_tflops = S.sol_attn_probe_mfma()

    if args.copy_probe:
        out.copy_(Q)
        torch.cuda.synchronize()

    flops = wl.effective_flops(topk)
    value = flops / (ms_per_step * 1e-3) / 1e12
    fwd_tflops = flops / (t_fwd * 1e-3) / 1e12
    pool_bytes = 2 * wl.B * wl.H * wl.L * wl.d * (2 if wl.dtype == "bf16" else 4) + 2 * wl.B * wl.H * nb * wl.d * 8
    rec = {
        "metric": "sparse-attn fwd effective TFLOP/s @64.5k tokens; % bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded smooth field + noise, unit RMS)",
        "config": {"workload": wl.name + ("+" + args.pattern if args.pattern != "selected" else "")
                   + ("-reorder" if reorder else ""), "B": wl.B,
                   "H": wl.H, "L": wl.L, "d": wl.d, "block": wl.block, "topk": topk, "n_blocks": nb,
                   "latent": [wl.frames, wl.lat_h, wl.lat_w], "pattern": args.pattern,
                   **({"cube": list(wl.cube)} if cube else {})},
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "kernels_ms": {name: round(t, 4) for name, t in t_phase.items()},
        "fwd_tflops": round(fwd_tflops, 2),
        "fwd_ms_stats": fwd_stats,
        "mfma_measured_tflops": round(mfma_tflops, 1),
        "fwd_pct_measured_mfma": round(100.0 * fwd_tflops / mfma_tflops, 2),
        "pool_gbs": None if t_pool is None else round(pool_bytes / (t_pool * 1e-3) / 1e9, 1),
        # select: pooled float64 in + int32 indices out; 2*nB^2*d float64 flops per head
        "select_gbs": None if t_sel is None else round(
            (2 * wl.B * wl.H * nb * wl.d * 8 + wl.B * wl.H * nb * topk * 4) / (t_sel * 1e-3) / 1e9, 1),
        "select_fp64_gflops": None if t_sel is None else round(
            2.0 * wl.B * wl.H * nb * nb * wl.d / (t_sel * 1e-3) / 1e9, 1),
        "roofline": {"bound": "mfma", "achieved": round(fwd_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": fwd_traffic_bytes() if (wl.name == "refine_1344x768" and topk == wl.topk
                                                        and args.pattern == "selected") else None},
        **({"permute_gbs": round(4 * 2 * wl.B * wl.H * wl.L * row_bytes
                                 / ((t_phase["permute_in"] + t_phase["permute_out"]) * 1e-3) / 1e9, 1)}
           if reorder else {}),
        **({"exchange_8bit": quant_err} if quant else {}),
        "timed_wall_s": round(wall, 3),
        "input_gen_s": round(t_gen, 2),
    }
    if cpu_rec is not None:
        rec["cpu_baseline"] = cpu_rec
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
