"""Benchmark: GPTQ layer quantization of the 4096x11008 (LLaMA-7B down_proj) layer.

One step = the whole per-layer path on one GPU, inputs resident in HBM:
zero H, Hessian accumulation over 262144 bf16 tokens, act-order + damping +
Cholesky/inverse, the blocked column sweep with lazy updates (4-bit, group
128), and packing.  Prints one JSON line (see the keys below).

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--no-cpu-baseline]
    python bench.py --workload dequant [--steps 5] [--no-cpu-baseline]

The second form measures the product with the packed layer instead (decode:
one token against the same 4096x11008 layer packed at 4 bits, g128,
act-order in quantization order, activations gathered through perm); the
default line carries a short summary of it under "dequant_matmul".

The CPU baseline is the fp64 oracle on a bounded sample of the same layer
(token, row and column subsets, scaled to weights/s; the sample is stated in
the output).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GPTQ layer-quantize ms & weights/sec (4096×11008, 4-bit g128); % MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F64_TFLOPS = 78.6         # MI355X fp64 (matrix and vector)
PEAK_HBM_GBS = 8000.0


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hess_tile_kernel_4096x11008_traffic.json")
TRAFFIC_SOURCES = ("post_weight_quantization_accum_amd/csrc/hessian.hip",
                   "post_weight_quantization_accum_amd/csrc/common.hpp")
DQ_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "dequant_staged_kernel_4096x11008_traffic.json")
DQ_TRAFFIC_SOURCES = ("post_weight_quantization_accum_amd/csrc/dequant.hip",
                      "post_weight_quantization_accum_amd/csrc/common.hpp",
                      "post_weight_quantization_accum_amd/csrc/internal.hpp")


def source_digest(sources=TRAFFIC_SOURCES):
    import hashlib
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(path=TRAFFIC_FILE, sources=TRAFFIC_SOURCES):
    """HBM bytes per launch of a kernel, from the committed rocprofv3 counter
    runs (FETCH_SIZE and WRITE_SIZE, each scaled by the reading of a plain
    copy of known size); None if the kernel source has changed since they
    were taken."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_digest(sources):
        return None
    return t.get("bytes_per_launch")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dequant", action="store_true", help="skip the summary of the packed-layer product")
    ap.add_argument("--tokens", type=int, default=None, help="override the token count (testing only)")
    ap.add_argument("--workload", choices=("quantize", "dequant", "shapes", "stack"), default="quantize")
    ap.add_argument("--blocks", type=int, default=2, help="stack workload: decoder blocks")
    ap.add_argument("--stack-tokens", type=int, default=2048, help="stack workload: calibration tokens")
    ap.add_argument("--rounds", type=int, default=None, help="dequant workload: timed rounds per token count")
    ap.add_argument("--dq-tokens", type=str, default="1,4,16", help="dequant workload: token counts")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def cpu_baseline(layer_w, layer_x, d_out, d_in, n_tok, q):
    """Time the oracle on a bounded sample and scale to weights/s of the full layer."""
    import threadpoolctl

    import oracle as O

    cores = len(os.sched_getaffinity(0))
    with threadpoolctl.threadpool_limits(cores):
        info = threadpoolctl.threadpool_info()
        used = max([i.get("num_threads", 1) for i in info] or [1])
        tok_s = 4096
        rows_s = 256
        Xs = layer_x[:tok_s]
        t0 = time.perf_counter()
        Hs = O.hessian(Xs)
        t_h = (time.perf_counter() - t0) * (n_tok / tok_s)
        H = Hs * (n_tok / tok_s)  # stands in for the full-token Hessian (same shape)
        t0 = time.perf_counter()
        perm = O.act_order_permutation(H)
        U = O.inverse_hessian_upper(O.damp_hessian(H[np.ix_(perm, perm)], q.damp))
        t_c = time.perf_counter() - t0
        Ws = layer_w[:rows_s][:, perm]
        t0 = time.perf_counter()
        codes, *_ = O.sweep(Ws, U, q.bits, q.group_size, q.sym, q.block)
        t_s = (time.perf_counter() - t0) * (d_out / rows_s)
        t0 = time.perf_counter()
        O.pack(codes, q.bits)
        t_p = (time.perf_counter() - t0) * (d_out / rows_s)
    total = t_h + t_c + t_s + t_p
    return {
        "value": d_out * d_in / total, "unit": "weights/s", "cores": int(used), "kind": "oracle",
        "sample": (f"Hessian on {tok_s} of {n_tok} tokens (x{n_tok // tok_s}); order + Cholesky form on the full "
                   f"{d_in}x{d_in} matrix; sweep and packing on {rows_s} of {d_out} rows (x{d_out // rows_s}); "
                   f"est. full-layer seconds {total:.1f} (H {t_h:.1f}, chol {t_c:.1f}, sweep {t_s:.1f}, pack {t_p:.2f})"),
    }


def factored_prepare_flops(d, leaf=128):
    """Flops of the factored form's preparation: the recursion of the
    Cholesky factorisation with the inverse products only where a parent
    reads them (left children), plus the products R[K_k, K_l] U_ll (K = 128
    each, taken whole)."""
    def rec(n, need_m):
        if n <= leaf:
            return 2.0 / 3.0 * n ** 3
        nb = -(-n // leaf)
        n1 = leaf * ((nb + 1) // 2)
        n2 = n - n1
        f = rec(n1, True) + n2 * n1 * n1 + n2 * n2 * n1   # L21 (triangular operand), Schur update (half)
        if need_m:
            f += n2 * n1 * n1 + n2 * n2 * n1                # T, M21
        return f + rec(n2, need_m)
    nb = d // leaf
    return rec(float(d), False) + nb * (nb - 1) / 2 * 2.0 * leaf ** 3


def phase_rooflines(d_out, d_in, n_tok, bits, block, phases_ms, x_bytes=2, factored=False):
    """Each phase's algorithmic work over its measured time, against the peak
    that bounds it (the solver runs in float64: its phases are priced at the
    float64 peak)."""
    h_flops = float(n_tok) * d_in * (d_in + 1)
    # Cholesky + triangular inverse; the factored form skips the inverse
    # products that nothing reads
    chol_flops = factored_prepare_flops(d_in) if factored else 2.0 / 3.0 * float(d_in) ** 3
    lazy = 0.0
    for i1 in range(0, d_in, block):
        i2 = min(i1 + block, d_in)
        lazy += 2.0 * d_out * (i2 - i1) * (d_in - i2)
    sweep_flops = lazy + float(d_out) * d_in * (block - 1)
    pack_bytes = d_out * d_in * (1 + bits / 8)

    def fl(flops, ms, peak):
        a = flops / (ms * 1e-3) / 1e12
        return {"achieved": round(a, 2), "peak": peak, "unit": "TFLOP/s", "frac": round(a / peak, 4),
                "algorithmic_flops": flops}
    out = {"hessian": dict(fl(h_flops, phases_ms["hessian"], PEAK_BF16_TFLOPS if x_bytes == 2 else PEAK_F64_TFLOPS),
                           bound="mfma"),
           "prepare_hinv": dict(fl(chol_flops, phases_ms["prepare_hinv"], PEAK_F64_TFLOPS), bound="mfma (fp64)"),
           "quantize_layer": dict(fl(sweep_flops, phases_ms["quantize_layer"], PEAK_F64_TFLOPS), bound="mfma (fp64)")}
    gbs = pack_bytes / (phases_ms["pack"] * 1e-3) / 1e9
    out["pack"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                   "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": pack_bytes}
    # the column sweep's bytes: every weight's float64 running value read and
    # its code byte written once (9 B per weight), over the whole quantize
    # phase (the sweep kernels alone: the kernel statistics under profiles/)
    sweep_bytes = 9.0 * d_out * d_in
    gbs = sweep_bytes / (phases_ms["quantize_layer"] * 1e-3) / 1e9
    out["column_sweep"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": sweep_bytes,
                           "timed": "quantize_layer phase"}
    return out


DQ_COPIES = 16   # distinct packed layers cycled through (406 MB > the 256 MB last-level cache)


def dequant_bytes(d_out, d_in, bits, n_groups, n_tok):
    """Algorithmic HBM bytes of one product: packed words, scales and zeros,
    perm, activations (bf16) and outputs (float32), each once."""
    wpr = -(-(d_in * bits) // 32)
    return d_out * wpr * 4 + 2 * n_groups * d_out * 4 + d_in * 4 + n_tok * d_in * 2 + n_tok * d_out * 4


def dequant_measure(d_out, d_in, bits, gs, token_counts, rounds, cpu=False):
    """Time gptq_dequant_matmul on DQ_COPIES copies of one packed layer, cycled
    so that every launch reads its weights from HBM.  Each round of
    DQ_COPIES launches is captured once in a HIP graph and replayed; HIP
    events on the replay stream bracket `rounds` replays.  Three routes per
    token count:
      perm:    act-order layer packed in quantization order, the product
               gathering the activations itself (the per-token kernels);
      gather:  the same layer, gptq_gather_columns first, then the
               natural-order product (the matrix cores from 2 tokens on);
      natural: a layer packed in original order (no act-order, or static
               groups with act-order): no gather."""
    import torch

    import post_weight_quantization_accum_amd as P
    from post_weight_quantization_accum_amd import synth

    dev = torch.device("cuda:0")
    n_max = max(token_counts)
    L = synth.make_packed_layer(d_out, d_in, n_max, bits=bits, group_size=gs, dtype="bf16", seed=4242)
    codes = torch.from_numpy(L.codes).to(dev)
    perm = torch.from_numpy(L.perm).to(dev)
    packed0 = P.pack_permuted(codes, bits, perm)
    packed_nat = P.pack(codes, bits)
    del codes
    sc0 = torch.from_numpy(L.scales).to(dev)
    z0 = torch.from_numpy(L.zeros).to(dev)
    layers = [(packed0.clone(), sc0.clone(), z0.clone(), perm.clone(), packed_nat.clone()) for _ in range(DQ_COPIES)]
    del packed_nat
    X = torch.from_numpy(L.X.view(np.int16)).view(torch.bfloat16).to(dev)
    ng = sc0.shape[0]
    out = {}
    for n in token_counts:
        Xn = X[:n]
        Xg = torch.empty((n, d_in), dtype=torch.bfloat16, device=dev)
        Y = torch.empty((n, d_out), dtype=torch.float32, device=dev)

        def rounds_of(mode):
            def one_round():
                for pk, sc, z, pm, pkn in layers:
                    if mode == "perm":
                        P.dequant_matmul(Xn, pk, bits, sc, z, perm=pm, group_size=gs, out=Y)
                    elif mode == "gather":
                        P.gather_columns(Xn, pm, out=Xg)
                        P.dequant_matmul(Xg, pk, bits, sc, z, group_size=gs, out=Y)
                    else:
                        P.dequant_matmul(Xn, pkn, bits, sc, z, group_size=gs, out=Y)
            return one_round

        row = {}
        for mode in ("perm", "gather", "natural"):
            one_round = rounds_of(mode)
            one_round()
            torch.cuda.synchronize()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                one_round()
            torch.cuda.current_stream().wait_stream(s)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                one_round()
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            cur = torch.cuda.current_stream()
            e0.record(cur)
            for _ in range(rounds):
                g.replay()
            e1.record(cur)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (rounds * DQ_COPIES)
            del g
            nbytes = dequant_bytes(d_out, d_in, bits, ng, n)
            if mode == "natural":
                nbytes -= d_in * 4   # no perm
            row[mode] = {"us_per_launch": round(us, 3), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                         "bytes": nbytes}
        best = min(("perm", "gather"), key=lambda m: row[m]["us_per_launch"])
        out[n] = dict(row["perm"], routes=row, act_order_best=best)
    res = {"layer": f"{d_out}x{d_in}", "bits": bits, "group_size": gs, "copies": DQ_COPIES, "rounds": rounds,
           "by_tokens": out}
    if cpu:
        import oracle as O
        t0 = time.perf_counter()
        words = O.pack_permuted(L.codes, bits, L.perm)
        t_pack = time.perf_counter() - t0
        t0 = time.perf_counter()
        O.dequant_matmul(L.X_f64()[:1], words, bits, d_in, L.scales, L.zeros, perm=L.perm, group_size=gs)
        t_mm = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(1.0 / t_mm, 4), "unit": "products/s (1 token)",
                               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
                               "sample": f"one full 1-token product {d_out}x{d_in} ({t_mm:.2f} s; "
                                         f"packing in quantization order {t_pack:.2f} s, not counted)"}
    return res


def dequant_main(a):
    from post_weight_quantization_accum_amd.configs import HEADLINE, layer_spec

    cfg_id, lname = HEADLINE
    wl, li, d_out, d_in, xl = layer_spec(cfg_id, lname)
    q = wl.quants[0]
    rounds = a.rounds or max(10, 20 * a.steps)
    toks = tuple(int(t) for t in a.dq_tokens.split(","))
    if 1 not in toks:
        toks = (1,) + toks
    r = dequant_measure(d_out, d_in, q.bits, q.group_size, toks, rounds, cpu=not a.no_cpu_baseline)
    d1 = r["by_tokens"][1]
    ng = -(-d_in // q.group_size)
    res = {
        "metric": "W4A16 dequant-GEMM decode (4096x11008, 4-bit g128 act-order, 1 token): HBM GB/s",
        "value": d1["GBps"], "unit": "GB/s", "n_gpus": 1, "steps": rounds, "warmup": 1,
        "ms_per_step": round(d1["us_per_launch"] * 1e-3, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 x / 4-bit codes, f32 accumulate", "data": "synthetic",
        "config": {"workload": f"product with the packed {d_out}x{d_in} layer, {q.bits}-bit g{q.group_size} "
                               f"act-order (sorted packing, perm gather), bf16 activations, 1 token; "
                               f"{DQ_COPIES} layer copies cycled", "d_out": d_out, "d_in": d_in, "tokens": 1},
        "roofline": {"bound": "hbm", "achieved": d1["GBps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(d1["GBps"] / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(DQ_TRAFFIC_FILE, DQ_TRAFFIC_SOURCES),
                     "kernel": "dequant_staged_kernel<4,1,bf16>", "launch_us": d1["us_per_launch"],
                     "algorithmic_bytes_per_launch": dequant_bytes(d_out, d_in, q.bits, ng, 1)},
        "by_tokens": r["by_tokens"],
    }
    if "cpu_baseline" in r:
        res["cpu_baseline"] = r["cpu_baseline"]
    if a.calib_copy_mib:
        import torch
        src = torch.empty(a.calib_copy_mib << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        res["calib_copy_bytes"] = int(src.numel())
    print(json.dumps(res))


def shapes_main(a):
    """Every distinct layer shape of the five workloads at its full size
    (token count, dtype, quantizer), one layer-quantize step each after a
    warm-up; inputs drawn on the device (normal weights, normal activations:
    the times do not depend on the values)."""
    import torch

    import post_weight_quantization_accum_amd as P
    from post_weight_quantization_accum_amd.configs import WORKLOADS

    dev = torch.device("cuda:0")
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
    rows = []
    for cid, wl in WORKLOADS.items():
        seen = set()
        for (name, d_out, d_in, _xl) in wl.layers:
            if (d_out, d_in) in seen:
                continue
            seen.add((d_out, d_in))
            for q in wl.quants:
                log(f"workload {cid} {name} {d_out}x{d_in} {q.bits}-bit g{q.group_size}")
                g = torch.Generator(device=dev)
                g.manual_seed(1000 * cid + d_in)
                X = (torch.randn((wl.n_tok, d_in), generator=g, device=dev) * 0.5).to(tdt[wl.dtype])
                W = (torch.randn((d_out, d_in), generator=g, device=dev) * wl.sigma_w).to(tdt[wl.dtype])
                cfg = P.make_config(bits=q.bits, group_size=q.group_size, sym=q.sym, act_order=q.act_order,
                                    block=q.block, damp=q.damp)
                H = torch.empty((d_in, d_in), dtype=torch.float64, device=dev)
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
                times = []
                for it in range(1 + max(1, a.steps // 2)):
                    ev[0].record()
                    H.zero_()
                    P.hessian_accumulate(H, X)
                    ev[1].record()
                    fac = P.factored_supported(d_out, d_in, cfg)
                    if fac:
                        perm = P.prepare_hinv_factored(H, cfg)
                        ev[2].record()
                        out = P.quantize_layer_factored(W, H, perm, cfg, want_w_hat=False, want_row_loss=False)
                    else:
                        perm = P.prepare_hinv(H, cfg)
                        ev[2].record()
                        out = P.quantize_layer(W, H, perm, cfg, want_w_hat=False, want_row_loss=False)
                    ev[3].record()
                    P.pack(out["codes"], q.bits)
                    ev[4].record()
                    torch.cuda.synchronize()
                    if it > 0:
                        times.append([ev[i].elapsed_time(ev[i + 1]) for i in range(4)])
                t = np.mean(np.array(times), axis=0)
                ph = dict(zip(("hessian", "prepare_hinv", "quantize_layer", "pack"), (float(v) for v in t)))
                total = float(sum(t))
                rows.append({"workload": cid, "layer": name, "d_out": d_out, "d_in": d_in, "tokens": wl.n_tok,
                             "dtype": wl.dtype, "bits": q.bits, "group_size": q.group_size,
                             "act_order": bool(q.act_order), "ms": round(total, 3),
                             "solver_only_ms": round(total - ph["hessian"], 3),
                             "phases_ms": {k: round(v, 3) for k, v in ph.items()},
                             "weights_per_s": d_out * d_in / (total * 1e-3),
                             "hinv_form": "factored" if fac else "U",
                             "phase_roofline": phase_rooflines(d_out, d_in, wl.n_tok, q.bits, q.block, ph,
                                                               x_bytes=4 if wl.dtype == "f32" else 2,
                                                               factored=fac)})
                log(f"  {total:.2f} ms (H {ph['hessian']:.2f}, prepare {ph['prepare_hinv']:.2f}, "
                    f"quantize {ph['quantize_layer']:.2f}, pack {ph['pack']:.3f})")
                del X, W, H, out, perm
                torch.cuda.empty_cache()
    print(json.dumps({"metric": "GPTQ layer-quantize ms per distinct layer shape (workloads 1-5)",
                      "unit": "ms", "higher_is_better": False, "n_gpus": 1, "data": "synthetic (device normal)",
                      "shapes": rows}))


def stack_main(a):
    """Blocks of workload 5's shape (hidden 12288, ffn 49152, fp16, 3-bit
    g128) quantized in sequence by the sequential driver: every layer's
    Hessian from the already-quantized upstream outputs, products from the
    packed words.  Weights and X0 drawn on the device."""
    import torch

    import post_weight_quantization_accum_amd as P
    from post_weight_quantization_accum_amd import sequential as S
    from post_weight_quantization_accum_amd.configs import WORKLOADS

    wl = WORKLOADS[5]
    q = wl.quants[0]
    hidden, ffn = 12288, 49152
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(5005)
    cfg = P.make_config(bits=q.bits, group_size=q.group_size, sym=q.sym, act_order=q.act_order, block=q.block,
                        damp=q.damp)

    def block(hh, ff):
        def w(o, i):
            return (torch.randn((o, i), generator=g, device=dev) * wl.sigma_w).half()
        return S.Block(q=w(hh, hh), k=w(hh, hh), v=w(hh, hh), out=w(hh, hh), fc1=w(ff, hh), fc2=w(hh, ff))

    # warm-up on a small stack (first launches, allocator)
    S.quantize_stack([block(256, 1024)], torch.randn((2048, 256), generator=g, device=dev).half(), cfg,
                     want_w_hat=False)
    blocks = [block(hidden, ffn) for _ in range(a.blocks)]
    X0 = torch.randn((a.stack_tokens, hidden), generator=g, device=dev).half()
    torch.cuda.synchronize()
    stats = S.new_stats()
    t0 = time.perf_counter()
    _, Xout = S.quantize_stack(blocks, X0, cfg, stats, want_w_hat=False)
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    n_w = a.blocks * (4 * hidden * hidden + 2 * hidden * ffn)
    print(json.dumps({"metric": "sequential quantization of decoder blocks (workload 5 shapes)",
                      "value": n_w / total, "unit": "weights/s", "n_gpus": 1, "higher_is_better": True,
                      "s_total": round(total, 3), "s_per_block": round(total / a.blocks, 3),
                      "breakdown_s": {k.replace("_ms", ""): round(v / 1e3, 3) for k, v in stats.items()},
                      "config": {"workload": f"{a.blocks} blocks, hidden {hidden}, ffn {ffn}, fp16, {q.bits}-bit "
                                             f"g{q.group_size}, {a.stack_tokens} calibration tokens",
                                 "weights": n_w},
                      "data": "synthetic (device normal)", "output_finite": bool(torch.isfinite(Xout).all())}))


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; "
                                   "--gpus N > 1 is not supported (single-GPU solver)"}))
        sys.exit(2)
    if a.workload == "dequant":
        dequant_main(a)
        return
    if a.workload == "shapes":
        shapes_main(a)
        return
    if a.workload == "stack":
        stack_main(a)
        return

    import torch

    import post_weight_quantization_accum_amd as P
    from post_weight_quantization_accum_amd import synth
    from post_weight_quantization_accum_amd.configs import HEADLINE, layer_spec

    cfg_id, lname = HEADLINE
    wl, li, d_out, d_in, xl = layer_spec(cfg_id, lname)
    q = wl.quants[0]
    n_tok = a.tokens or wl.n_tok
    t0 = time.perf_counter()
    L = synth.make_layer(d_out, d_in, n_tok, dtype=wl.dtype, sigma_w=wl.sigma_w, dist=wl.dist,
                         outlier_frac=wl.outlier_frac, outlier_scale=wl.outlier_scale, config=cfg_id,
                         layer=li, x_layer=xl)
    gen_s = time.perf_counter() - t0
    log(f"inputs generated in {gen_s:.1f} s")
    dev = torch.device("cuda:0")
    W = torch.from_numpy(L.W.view(np.int16)).view(torch.bfloat16).to(dev)
    X = torch.from_numpy(L.X.view(np.int16)).view(torch.bfloat16).to(dev)
    torch.cuda.synchronize()

    cfg = P.make_config(bits=q.bits, group_size=q.group_size, sym=q.sym, act_order=q.act_order,
                        block=q.block, damp=q.damp)
    lib = P.load()
    import ctypes
    H = torch.empty((d_in, d_in), dtype=torch.float64, device=dev)
    perm = torch.empty(d_in, dtype=torch.int32, device=dev)
    # the factored form of the inverse's factor where the shape allows it
    # (the headline layer does), else U
    factored = P.factored_supported(d_out, d_in, cfg)
    prep, quant = ((P.prepare_hinv_factored, P.quantize_layer_factored) if factored
                   else (P.prepare_hinv, P.quantize_layer))
    ws_h = torch.empty((lib.gptq_prepare_hinv_factored_workspace if factored else lib.gptq_prepare_hinv_workspace)(d_in),
                       dtype=torch.uint8, device=dev)
    ws_q = torch.empty((lib.gptq_quantize_layer_factored_workspace if factored else lib.gptq_quantize_layer_workspace)(
        d_out, d_in, ctypes.byref(cfg)), dtype=torch.uint8, device=dev)
    ng = P.n_groups(d_in, q.group_size)
    out = dict(codes=torch.empty((d_out, d_in), dtype=torch.uint8, device=dev),
               scales=torch.empty((ng, d_out), dtype=torch.float32, device=dev),
               zeros=torch.empty((ng, d_out), dtype=torch.float32, device=dev),
               g_idx=torch.empty(d_in, dtype=torch.int32, device=dev))
    packed = torch.empty((d_out, P.packed_words_per_row(d_in, q.bits)), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    phase_ms = {"hessian": [], "prepare_hinv": [], "quantize_layer": [], "pack": []}

    def step(record):
        if record:
            ev[0].record(stream)
        H.zero_()
        P.hessian_accumulate(H, X)
        if record:
            ev[1].record(stream)
        prep(H, cfg, perm=perm, workspace=ws_h)
        if record:
            ev[2].record(stream)
        quant(W, H, perm, cfg, workspace=ws_q, out=out)
        if record:
            ev[3].record(stream)
        P.pack(out["codes"], q.bits, out=packed)
        if record:
            ev[4].record(stream)

    for _ in range(a.warmup):
        step(False)
    torch.cuda.synchronize()
    log("warmup done")
    t_start = time.perf_counter()
    for _ in range(a.steps):
        step(True)
        torch.cuda.synchronize()
        names = list(phase_ms)
        for i, n in enumerate(names):
            phase_ms[n].append(ev[i].elapsed_time(ev[i + 1]))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1000.0 / a.steps
    phases = {k: float(np.mean(v)) for k, v in phase_ms.items()}
    phases_median = {k: float(np.median(v)) for k, v in phase_ms.items()}

    # Dominant kernel: the Hessian product (hess_tile_kernel).  One launch
    # runs up to 1792 (256x128 tile, 32768-token window) work items; the
    # launches of one Hessian are timed with HIP events on the stream they
    # run on (same kernels and launch configuration as above).  Algorithmic
    # work: n_tok * d_in * (d_in + 1) flops for the whole Hessian (2 flops
    # per product over the upper triangle with the diagonal), divided evenly
    # over the launches for the per-launch figure.
    hk, nl = [], 0
    for _ in range(max(1, min(a.steps, 3))):
        H.zero_()
        ms, nl = P.hessian_accumulate_timed(H, X)
        hk.append(ms)
    h_ms = float(np.mean(hk))
    h_flops = float(n_tok) * d_in * (d_in + 1) / nl
    achieved = h_flops / (h_ms * 1e-3) / 1e12
    traffic = measured_traffic()
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "kernel": "hess_tile_kernel<bf16> (Hessian product, 256x128 tiles of the upper triangle)",
                "launch_ms": round(h_ms, 4), "launches_per_step": nl,
                "algorithmic_flops_per_launch": h_flops}

    res = {
        "metric": METRIC,
        "value": d_out * d_in / (ms_per_step * 1e-3),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 MFMA (Hessian) + f64 (solver)",
        "data": "synthetic (seeded Student-t(4) activations with outlier channels; N(0,0.02^2) weights)",
        "config": {"workload": f"llama-7b down_proj {d_out}x{d_in} bf16; X {n_tok}x{d_in} bf16 Student-t(4), "
                               f"{wl.outlier_frac * 100:g}% outlier channels x{wl.outlier_scale:g}; {q.bits}-bit "
                               f"asym g{q.group_size} act-order B{q.block} damp {q.damp}",
                   "d_out": d_out, "d_in": d_in, "tokens": n_tok, "bits": q.bits, "group_size": q.group_size,
                   "act_order": bool(q.act_order), "parallelism": "single GPU",
                   "hinv_form": "factored" if factored else "U"},
        "phases_ms": {k: round(v, 3) for k, v in phases.items()},
        "phases_ms_median": {k: round(v, 3) for k, v in phases_median.items()},
        "solver_only_ms": round(phases["prepare_hinv"] + phases["quantize_layer"] + phases["pack"], 3),
        "phase_roofline": phase_rooflines(d_out, d_in, n_tok, q.bits, q.block, phases, factored=factored),
        "roofline": roofline,
    }
    log(f"timed {a.steps} steps: {ms_per_step:.2f} ms/step; phases {res['phases_ms']}")
    if not a.no_dequant:
        log("product with the packed layer ...")
        dq = dequant_measure(d_out, d_in, q.bits, q.group_size, (1, 16), 20)
        res["dequant_matmul"] = {"workload": "1 and 16 tokens x packed 4096x11008 4-bit g128 act-order (sorted), "
                                             "bf16", "by_tokens": dq["by_tokens"], "peak_GBps": PEAK_HBM_GBS}
    if a.calib_copy_mib:
        src = torch.empty(a.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        res["calib_copy_bytes"] = int(src.numel())
        del src, dst
    if not a.no_cpu_baseline:
        log("oracle CPU baseline ...")
        res["cpu_baseline"] = cpu_baseline(L.W_f64(), L.X_f64() if n_tok <= 8192 else
                                           synth.to_f64(L.X[:4096], L.dtype), d_out, d_in, n_tok, q)
    res["input_generation_s"] = round(gen_s, 1)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
