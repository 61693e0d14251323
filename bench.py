#!/usr/bin/env python3
"""Benchmark of one MoE layer step on one MI355X: route -> permute -> grouped SwiGLU FFN -> combine.

A step is one `moe_layer` call (every step of the path, one batch of T tokens) with all inputs
resident in HBM. Prints ONE JSON line on stdout (progress goes to stderr):
  value        layer tokens/s = T / (time per step), whole job (one GPU)
  roofline     the dominant step (the grouped FFN) against its bound, from HIP-event timing of
               that call on the stream it runs on, with algorithmic bytes / flops from
               token_dispatch_expert_amd.traffic; traffic = counter-measured HBM bytes when a
               profiles/ counter summary exists for the current kernel source, else null
  cpu_baseline the fp64 oracle timed on the host cores (a bounded sample of the workload)
  breakdown    per-call time (mean, p10 / median / p90 over the timed passes, each pass starting
               with the L2s and MALL flushed) and roofline fraction of every step; calls this short
               include the host's launch gap, the kernel trace in profiles/ has the kernel times

Workloads (--config, default c4 = the DeepSeek-V3-shaped prefill layer, T=8192, the largest
workload that the metric is quoted on; c2/c3 are the decode shapes, c5 the fp8-weight prefill):
c1..c5 as in synth.CONFIGS. bf16 and fp8 weights are put into their blocked layout
(MOE_BF16_BLOCKED / MOE_FP8_E4M3FN_BLOCKED, by moe_block_weights) once before anything is timed,
as a caller would at load time; --row-major-weights keeps them row-major. Other modes: --calibrate-copy runs a plain device copy of
known size, the reference for scaling the FETCH_SIZE / WRITE_SIZE counters.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at 1 GPU; % MFMA peak (GEMM) and % HBM BW (permute/combine)"
HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}
COPY_CAL_BYTES = 1 << 30          # --calibrate-copy moves exactly this many bytes each way
FFN_SOURCE = os.path.join(ROOT, "token_dispatch_expert_amd", "csrc", "ffn.hip")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def counter_traffic(workload: str):
    """HBM bytes per FFN call from a committed counter summary, if it matches this source."""
    p = os.path.join(ROOT, "profiles", f"grouped_ffn_{workload}_counters.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        c = json.load(f)
    if c.get("ffn_source_sha") != source_sha(FFN_SOURCE):
        return None
    return c.get("hbm_bytes_per_call")


def calibrate_copy(steps: int) -> None:
    import torch
    n = COPY_CAL_BYTES // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copied {COPY_CAL_BYTES} bytes x {steps}")


def _gpu_busy(us: float = 150.0) -> None:
    """Keeps the GPU busy for about `us` microseconds (a spin kernel), so that the host can enqueue
    a timed call before the GPU reaches it: the events then bracket GPU execution only."""
    import torch
    torch.cuda._sleep(int(us * 2.5e3))  # cycles at most ~2.5 GHz


def _time_calls(fn, reps: int, warmup: int = 2) -> list:
    """Per-call times in microseconds of fn() on the current stream (HIP events), each call
    enqueued behind a spin kernel so that host launch latency is not timed."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        _gpu_busy()
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) * 1e3)
    return out


def fit_max_affine(P):
    """One max-affine model t = max(a + b*G, c + beta*N) over every point (G active experts, N
    rows in all, time t): the two branches are first fitted by least squares on the points each
    one wins, alternating until the assignment settles; the four parameters are then refined to
    minimise the largest relative misfit (Nelder-Mead). Returns (a, b, c, beta, max_rel_misfit,
    rms_rel_misfit)."""
    import numpy as np
    from scipy.optimize import minimize
    G, N, t = P[:, 0], P[:, 1], P[:, 2]
    small = P[:, 1] / P[:, 0] <= 8
    for _ in range(20):
        A1 = np.stack([np.ones(small.sum()), G[small]], 1)
        A2 = np.stack([np.ones((~small).sum()), N[~small]], 1)
        w1, w2 = 1.0 / t[small], 1.0 / t[~small]     # relative least squares
        a, b = np.linalg.lstsq(A1 * w1[:, None], t[small] * w1, rcond=None)[0]
        c, beta = np.linalg.lstsq(A2 * w2[:, None], t[~small] * w2, rcond=None)[0]
        new_small = (a + b * G) >= (c + beta * N)
        if np.array_equal(new_small, small) or new_small.all() or (~new_small).all():
            break
        small = new_small

    def misfit(th):
        m = np.maximum(th[0] + th[1] * G, th[2] + th[3] * N)
        return np.max(np.abs(m - t) / t)

    th = minimize(misfit, np.array([a, b, c, beta]), method="Nelder-Mead",
                  options={"maxiter": 20000, "xatol": 1e-9, "fatol": 1e-9}).x
    m = np.maximum(th[0] + th[1] * G, th[2] + th[3] * N)
    rel = (m - t) / t
    return (*[float(v) for v in th], float(np.max(np.abs(rel))), float(np.sqrt(np.mean(rel * rel))))


def expert_time_sweep(args) -> int:
    """Expert-time profile of moe_grouped_ffn (the makespan abstract's max-affine model on this
    GPU): G active experts with n rows each (n up to 4096), every other expert empty, at the
    decode (d=4096, d_ff=1536, E=128, bf16) and DeepSeek-V3 (d=7168, d_ff=2048, E=256) shapes,
    the latter with bf16 and with fp8 e4m3fn weights (128 x 128 block scales). One max-affine
    model t = max(a + b*G, c + beta*N) (N = G*n rows) is fitted over all points of a shape;
    n* = b / beta is the row count where an expert's time stops being its weight streaming
    (compared with the HBM/MFMA ridge of the weight format: ~312 rows bf16, ~156 fp8).
    Then the tutorial's exercise A on the routing side: active experts and load imbalance
    (max / mean assignments per expert) against batch size T in {1, 16, 128, 1024} under the
    decode and prefill workloads' Zipf logit biases, routed by moe_route on the GPU."""
    import numpy as np
    import torch
    import synth
    import token_dispatch_expert_amd as moe
    dev = torch.device("cuda:0")
    ns = [1, 2, 4, 8, 16, 32, 64, 96, 128, 160, 192, 256, 320, 384, 512, 768, 1024, 2048, 4096]
    Gs = [1, 4, 16, 64]
    shapes = [("decode Qwen3-like, bf16 weights", 4096, 1536, 128, "bf16"),
              ("DeepSeek-V3-like, bf16 weights", 7168, 2048, 256, "bf16"),
              ("DeepSeek-V3-like, fp8 e4m3fn weights", 7168, 2048, 256, "fp8")]
    result = {"metric": "grouped-FFN time vs rows per expert and active experts",
              "unit": "us", "data": "synthetic N(0,1) x, N(0,1/fan_in) weights (fp8: scaled codes)",
              "timing": "median of per-call GPU times (HIP events, each call enqueued behind a spin kernel)",
              "shapes": []}
    for name, d, d_ff, E, wfmt in shapes:
        g = torch.Generator(device=dev).manual_seed(0)
        skw = {}
        if wfmt == "bf16":
            W = [torch.randn((E, a, b), generator=g, device=dev, dtype=torch.float32).div_(b ** 0.5).to(torch.bfloat16)
                 for a, b in ((d_ff, d), (d_ff, d), (d, d_ff))]
            ridge = 2500e12 / 8e12
        else:
            W = [torch.randn((E, a, b), generator=g, device=dev, dtype=torch.float32).mul_(64.0)
                 .clamp_(-448, 448).to(torch.float8_e4m3fn) for a, b in ((d_ff, d), (d_ff, d), (d, d_ff))]
            skw = {"s_gate": torch.full((E, d_ff // 128, d // 128), 1.0 / (64 * d ** 0.5), device=dev),
                   "s_up": torch.full((E, d_ff // 128, d // 128), 1.0 / (64 * d ** 0.5), device=dev),
                   "s_down": torch.full((E, d // 128, d_ff // 128), 1.0 / (64 * d_ff ** 0.5), device=dev)}
            ridge = 2500e12 / 8e12 / 2
        # the weights in their blocked layout, as the layer benchmark uses them (row-major with
        # --row-major-weights)
        if not args.row_major_weights:
            for i in range(3):
                b = torch.empty_like(W[i])
                moe.moe_block_weights(W[i], b)
                W[i] = b
            skw["weights_blocked"] = True
        pts = []
        for G in Gs:
            for n in ns:
                rows = G * n
                if rows > 65536:
                    continue
                counts = np.zeros(E, np.int64)
                counts[np.linspace(0, E - 1, G).astype(int)] = n   # spread over the expert range
                offs = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).to(dev)
                xs = torch.randn((rows, d), generator=g, device=dev).to(torch.bfloat16)
                ys = torch.empty((rows, d), device=dev)
                ws = moe.Workspace(moe.moe_ffn_workspace_size(rows, E, d, d_ff, torch.bfloat16, W[0].dtype), device=dev)
                t = _time_calls(lambda: moe.moe_grouped_ffn(xs, offs, W[0], W[1], W[2], ys, ws, **skw),
                                max(args.steps // 2, 5))
                us = float(np.median(t))
                pts.append((G, n, rows, us))
                log(f"{name}: G={G} n={n}: {us:.1f} us")
                del xs, ys, ws
        P = np.array([(G, N, us) for G, _, N, us in pts], dtype=np.float64)
        a, b, c, beta, mx, rms = fit_max_affine(P)
        wbytes = 3 * d * d_ff * (2 if wfmt == "bf16" else 1)
        result["shapes"].append({
            "shape": name, "d": d, "d_ff": d_ff, "E": E, "weights": wfmt,
            "weight_layout": "row-major" if args.row_major_weights else "blocked (8 rows x 128 bytes)",
            "points": [{"G": int(G), "n": int(n), "us": round(us, 2)} for G, n, _, us in pts],
            "fit": {"a_us": round(a, 2), "b_us_per_expert": round(b, 3), "c_us": round(c, 2),
                    "beta_us_per_row": round(beta, 5), "max_rel_misfit": round(mx, 3),
                    "rms_rel_misfit": round(rms, 3)},
            "n_star_measured": round(b / beta, 1),
            "crossover_rows_per_expert_at_G": {str(G): round((a - c) / (beta * G) + b / beta, 1) for G in Gs},
            "per_expert_stream_GBps": round(wbytes / (b * 1e-6) / 1e9, 1),
            "row_rate_TFLOPs": round(6 * d * d_ff / (beta * 1e-6) / 1e12, 1),
            "n_star_roofline": round(ridge, 1)})
        log(f"{name}: fit max|misfit| {mx:.1%}, n* = {b / beta:.0f} rows (ridge {ridge:.0f})")
        del W, skw
        torch.cuda.empty_cache()
    # exercise A: imbalance vs batch size under the workloads' logit biases
    ex = []
    for wl in ("c2", "c3", "c4"):
        base = synth.CONFIGS[wl]
        for T in (1, 16, 128, 1024):
            cfg = base.with_(T=T, name=f"{wl}-T{T}")
            logits, _ = synth.make_routing_inputs(cfg)
            lg = torch.from_numpy(logits).to(dev)
            ids = torch.empty((T, cfg.k), dtype=torch.int32, device=dev)
            gates = torch.empty((T, cfg.k), dtype=torch.float32, device=dev)
            counts = torch.empty((cfg.E,), dtype=torch.int32, device=dev)
            moe.moe_route(lg, cfg.k, ids, gates, counts)
            c = counts.cpu().numpy().astype(np.int64)
            mean = T * cfg.k / cfg.E
            act = c[c > 0]
            ex.append({"bias": f"{wl} (E={cfg.E}, k={cfg.k}, Zipf s={cfg.zipf_s})", "T": T,
                       "active_experts": int(len(act)), "max_rows": int(c.max()),
                       "max_over_mean": round(float(c.max() / mean), 2),
                       "max_over_mean_active": round(float(c.max() / act.mean()), 2)})
            log(f"exercise A {wl} T={T}: {len(act)} active, max/mean {c.max() / mean:.2f}")
    result["exercise_A"] = ex
    print(json.dumps(result), flush=True)
    return 0


def _timed_steps(fn, steps: int, warmup: int) -> float:
    """ms per call of fn over `steps` calls after `warmup` untimed ones (synchronised)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps * 1e3


def router_bench(args) -> int:
    """moe_route_gemm (router scores + top-k in one launch, logits not written) at the c2 and c4
    router shapes: time per call with cold caches, against HBM (x once, router weights once, ids
    and gates) and against the bf16 MFMA peak."""
    import numpy as np
    import torch
    import token_dispatch_expert_amd as moe
    dev = torch.device("cuda:0")
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    res = []
    for name, T, d, E, k in (("c2", 128, 4096, 128, 8), ("c4", 8192, 7168, 256, 8)):
        g = torch.Generator(device=dev).manual_seed(1)
        x = torch.randn((T, d), generator=g, device=dev).to(torch.bfloat16)
        w = torch.randn((E, d), generator=g, device=dev).div_(d ** 0.5).to(torch.bfloat16)
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        gates = torch.empty((T, k), dtype=torch.float32, device=dev)
        samples = []
        for _ in range(max(args.steps, 5)):
            flush.sum()
            torch.cuda.synchronize()
            samples += _time_calls(lambda: moe.moe_route_gemm(x, w, k, ids, gates), 1, 0)
        us = float(np.median(samples))
        byts = T * d * 2 + E * d * 2 + T * k * 8
        flops = 2.0 * T * E * d
        res.append({"shape": name, "T": T, "d": d, "E": E, "k": k, "median_us": round(us, 2),
                    "GB_per_s": round(byts / (us * 1e-6) / 1e9, 1),
                    "hbm_frac": round(byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                    "TFLOP_per_s": round(flops / (us * 1e-6) / 1e12, 2)})
        log(f"router {name}: {us:.1f} us")
    print(json.dumps({"metric": "fused router GEMM + top-k time", "unit": "us", "results": res}), flush=True)
    return 0


def capacity_sweep(args, cfg, logits, x, W, out, ws, skw) -> int:
    """Capacity factor C = 1.0..2.0 (tutorial page, section 10, exercise D): layer tokens/s and
    the fraction of dropped assignments, next to the uncapped layer."""
    import torch
    import token_dispatch_expert_amd as moe
    T, E, k = cfg.T, cfg.E, cfg.k
    rows = []
    for pct in (None, 200, 175, 150, 125, 110, 100):
        cap = None if pct is None else moe.moe_expert_capacity(T, E, k, pct)
        ms = _timed_steps(lambda: moe.moe_layer(logits, x, W["gate"], W["up"], W["down"], k, out, ws,
                                                capacity=cap, **skw), args.steps, args.warmup)
        kept = int(out["offsets"][-1].item())
        rows.append({"C": None if pct is None else pct / 100, "capacity": cap, "ms_per_step": round(ms, 4),
                     "tokens_per_s": round(T / (ms / 1e3), 1), "dropped_frac": round(1 - kept / (T * k), 4),
                     "active_experts": int(torch.count_nonzero(out["counts"]).item())})
        log(f"C={rows[-1]['C']}: capacity {cap}, {ms * 1e3:.1f} us/step, dropped {rows[-1]['dropped_frac']:.2%}")
    print(json.dumps({"metric": "layer tokens/s and dropped fraction vs capacity factor",
                      "config": {"workload": f"{cfg.name}: {cfg.note}", "T": T, "E": E, "k": k,
                                 "d": cfg.d, "d_ff": cfg.d_ff, "weights": cfg.w},
                      "steps": args.steps, "warmup": args.warmup, "sweep": rows}), flush=True)
    return 0


def naive_baselines(args, cfg, logits, x, W, out, ws, skw) -> int:
    """The tutorial's exercise C (section 10; "sorting matters", section 8): (i) a per-token
    loop with no sort, every (token, expert) pair its own GEMV chain, and (ii) a per-expert
    launch loop after a sort, each expert's rows as separate library GEMMs, both in torch on the
    same GPU, against the grouped path (one moe_layer call). bf16 weights only."""
    import numpy as np
    import torch
    import token_dispatch_expert_amd as moe
    if cfg.w != "bf16":
        log("naive baselines are written for bf16 weights")
        return 2
    T, E, k = cfg.T, cfg.E, cfg.k
    Wg, Wu, Wd = W["gate"], W["up"], W["down"]

    def grouped():
        moe.moe_layer(logits, x, Wg, Wu, Wd, k, out, ws)

    ms_grouped = _timed_steps(grouped, args.steps, args.warmup)
    y_ref = out["y"].clone()
    ids = out["topk_ids"].long()
    gates = out["topk_gates"]
    ids_h = ids.cpu().numpy()

    def silu_mul(g, u):
        gf = g.float()
        return (gf * torch.sigmoid(gf) * u.float()).to(torch.bfloat16)

    def per_token():
        y = torch.zeros((T, cfg.d), dtype=torch.float32, device=x.device)
        for t in range(T):
            xt = x[t:t + 1]
            for j in range(k):
                e = int(ids_h[t, j])
                h = silu_mul(xt @ Wg[e].t(), xt @ Wu[e].t())
                y[t] += gates[t, j] * (h @ Wd[e].t()).float()[0]
        return y

    def per_expert():
        flat = ids.reshape(-1)
        order = torch.argsort(flat, stable=True)
        counts = torch.bincount(flat, minlength=E).cpu().tolist()
        xs = x[order // k]
        ys = torch.empty((T * k, cfg.d), dtype=torch.float32, device=x.device)
        r = 0
        for e, n in enumerate(counts):
            if n:
                xe = xs[r:r + n]
                h = silu_mul(xe @ Wg[e].t(), xe @ Wu[e].t())
                ys[r:r + n] = (h @ Wd[e].t()).float()
                r += n
        y = torch.zeros((T, cfg.d), dtype=torch.float32, device=x.device)
        y.index_add_(0, order // k, ys * gates.reshape(-1)[order, None])
        return y

    n_tok = 1 if T > 1024 else max(1, args.steps // 4)
    ms_tok = _timed_steps(per_token, n_tok, 1)
    ms_exp = _timed_steps(per_expert, args.steps, args.warmup)
    def rel(a):
        a, b = a.double(), y_ref.double()
        return float((a - b).abs().max() / b.pow(2).mean().sqrt())
    err_tok, err_exp = rel(per_token()), rel(per_expert())
    res = {"metric": "layer time: grouped path vs naive per-token and per-expert loops",
           "config": {"workload": f"{cfg.name}: {cfg.note}", "T": T, "E": E, "k": k, "d": cfg.d,
                      "d_ff": cfg.d_ff},
           "grouped_ms": round(ms_grouped, 4),
           "per_token_loop_ms": round(ms_tok, 2), "per_expert_loop_ms": round(ms_exp, 4),
           "speedup_vs_per_token": round(ms_tok / ms_grouped, 1),
           "speedup_vs_per_expert": round(ms_exp / ms_grouped, 2),
           "rel_err_vs_grouped": {"per_token": round(err_tok, 4), "per_expert": round(err_exp, 4)},
           "per_token_steps_timed": n_tok}
    log(json.dumps(res))
    print(json.dumps(res), flush=True)
    return 0


def cpu_baseline(cfg, logits_np, x_np, host_w) -> dict:
    """The fp64 oracle, as it stands, on the host cores: decode workloads whole, prefill
    workloads on their first 64 tokens (the same logits, x and weights), repeated until at least
    10 s have run. The time is split into the oracle's Python loops (route, permute, gather,
    combine) and its per-expert FFN (exact weight decode + fp64 BLAS)."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info
    threads = max([i["num_threads"] for i in threadpool_info()] or [1])
    T, k = cfg.T, cfg.k
    if T <= 256:
        Ts, sample = T, f"whole workload ({T} tokens), repeated until >= 10 s"
    else:
        Ts = 64
        sample = f"first {Ts} of {T} tokens (same logits, x and weights), repeated until >= 10 s"
    lg_s, x_s = logits_np[:Ts], np.ascontiguousarray(x_np[:Ts])
    log(f"cpu baseline: oracle on {Ts} tokens ...")
    n_done, t_loops, t_ffn = 0, 0.0, 0.0
    dec = oracle.make_weight_decoder(lambda e: host_w[e], cfg.w)
    while t_loops + t_ffn < 10.0 and n_done < 20:
        t0 = time.perf_counter()
        ids, gates = oracle.route(lg_s, k)
        p = oracle.permute(ids, cfg.E)
        xs = oracle.decode_activations(oracle.gather_rows(x_s, p["sorted_to_flat"], k), cfg.act)
        t1 = time.perf_counter()
        ys = oracle.ffn(xs, p["offsets"], dec)
        t2 = time.perf_counter()
        oracle.combine(ys, p["flat_to_sorted"], gates)
        t3 = time.perf_counter()
        t_loops += (t1 - t0) + (t3 - t2)
        t_ffn += t2 - t1
        n_done += 1
    t_cpu = t_loops + t_ffn
    return {"value": round(Ts * n_done / t_cpu, 2), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "sample": sample, "seconds": round(t_cpu, 2), "passes": n_done,
            "host_cpus": os.cpu_count(), "blas_threads": int(threads),
            "split_s": {"route_permute_gather_combine_loops": round(t_loops, 2),
                        "ffn_decode_and_blas": round(t_ffn, 2)}}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c4", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--zipf", type=float, default=None,
                    help="override the workload's Zipf logit-bias exponent (0 = no bias), for "
                         "robustness runs of the same shape")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--row-major-weights", action="store_true",
                    help="keep the weights row-major instead of the blocked layout")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--capacity-sweep", action="store_true",
                    help="layer tokens/s and drop rate for capacity factors 1.0..2.0")
    ap.add_argument("--expert-time-sweep", action="store_true",
                    help="grouped-FFN time over rows per expert and active experts (max-affine fit)")
    ap.add_argument("--naive-baselines", action="store_true",
                    help="per-token and per-expert torch loops against the grouped path")
    ap.add_argument("--router", action="store_true",
                    help="time the fused router GEMM + top-k at the decode and prefill shapes")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library is one GPU's share of the layer and "
              "has no multi-GPU path (the design notes describe how it would shard)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synth
    import token_dispatch_expert_amd as moe
    from token_dispatch_expert_amd import traffic as tr
    from token_dispatch_expert_amd.binding import layer_buffers

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.calibrate_copy:
        calibrate_copy(max(args.steps, 1))
        return 0
    if args.expert_time_sweep:
        return expert_time_sweep(args)
    if args.router:
        return router_bench(args)

    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[args.config]
    if args.zipf is not None:
        cfg = cfg.with_(zipf_s=args.zipf if args.zipf > 0 else None,
                        note=f"{cfg.note}, logit bias Zipf s={args.zipf}")
    T, E, k, d, d_ff = cfg.T, cfg.E, cfg.k, cfg.d, cfg.d_ff
    act_t = torch.float32 if cfg.act == "f32" else torch.bfloat16
    w_t = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3fn": torch.float8_e4m3fn}[cfg.w]

    # ---- inputs (seeded, synthetic; every expert's weights exist, active or not)
    t0 = time.time()
    logits_np, x_np = synth.make_routing_inputs(cfg)
    logits = torch.from_numpy(logits_np).to(dev)
    if cfg.act == "f32":
        x = torch.from_numpy(x_np).to(dev)
    else:
        x = torch.from_numpy(x_np.view(np.int16)).to(dev).view(torch.bfloat16)
    wshape = {"gate": (E, d_ff, d), "up": (E, d_ff, d), "down": (E, d, d_ff)}
    W = {n: torch.empty(s, dtype=w_t, device=dev) for n, s in wshape.items()}
    S = None
    if cfg.w == "fp8_e4m3fn":
        S = {"s_gate": torch.empty((E, d_ff // 128, d // 128), device=dev),
             "s_up": torch.empty((E, d_ff // 128, d // 128), device=dev),
             "s_down": torch.empty((E, d // 128, d_ff // 128), device=dev)}
    host_w = {}
    keep_host = not args.no_cpu_baseline
    for e, w in synth.iter_expert_weights(cfg, range(E)):
        for n in ("gate", "up", "down"):
            src = torch.from_numpy(w[n].view(np.int16) if cfg.w == "bf16" else w[n])
            W[n][e].copy_(src.to(dev).view(w_t))
            if S is not None:
                S["s_" + n][e].copy_(torch.from_numpy(w[n + "_scale"]).to(dev))
        if keep_host:
            host_w[e] = w
        if e % 32 == 31:
            log(f"weights: {e + 1}/{E} experts generated and uploaded")
    torch.cuda.synchronize()
    # bf16 and fp8 weights go into their blocked layout once, before anything is timed (weights
    # are prepared at load time); the naive baselines use the weights as plain torch matrices
    blockable = ((cfg.w == "bf16" and d % 64 == 0 and d_ff % 64 == 0) or
                 (cfg.w == "fp8_e4m3fn" and d <= 65536 and d_ff <= 65536))
    blocked = blockable and not args.row_major_weights and not args.naive_baselines
    if blocked:
        for n in ("gate", "up", "down"):
            b = torch.empty_like(W[n])
            moe.moe_block_weights(W[n], b)
            W[n] = b
        torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s ({cfg.name}: T={T} d={d} E={E} k={k} d_ff={d_ff}, "
        f"weights {'blocked' if blocked else 'row-major'})")

    out = layer_buffers(T, E, k, d, act_t, device=dev)
    ws = moe.Workspace(moe.moe_layer_workspace_size(T, E, k, d, d_ff, act_t, w_t), device=dev)
    skw = dict(S or {})
    if blocked:
        skw["weights_blocked"] = True

    def step():
        moe.moe_layer(logits, x, W["gate"], W["up"], W["down"], k, out, ws, **skw)

    if args.capacity_sweep:
        return capacity_sweep(args, cfg, logits, x, W, out, ws, skw)
    if args.naive_baselines:
        return naive_baselines(args, cfg, logits, x, W, out, ws, skw)

    # ---- warmup, then exactly K timed steps bracketed by synchronisation
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed / args.steps * 1e3
    tokens_per_s = T / (ms_per_step / 1e3)
    log(f"layer: {ms_per_step * 1e3:.1f} us/step, {tokens_per_s:,.0f} tokens/s")

    # ---- per-call timing with events on the stream the library launches on
    counts = out["counts"].cpu().numpy()
    active = int(np.count_nonzero(counts))
    R = T * k
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    perm_ws = moe.Workspace(moe.moe_permute_workspace_size(T, E, k), device=dev)
    ffn_ws = moe.Workspace(moe.moe_ffn_workspace_size(R, E, d, d_ff, act_t, w_t), device=dev)
    # every timed call starts with cold caches: reading 512 MiB evicts the L2s and the 256 MB MALL
    # (a read, so that no dirty lines are left to be written back inside the timed calls)
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    calls = [
        lambda: moe.moe_route(logits, k, out["topk_ids"], out["topk_gates"]),
        lambda: moe.moe_permute(x, out["topk_ids"], E, out["counts"], out["offsets"],
                                out["sorted_to_flat"], out["flat_to_sorted"], out["x_sorted"], perm_ws),
        lambda: moe.moe_grouped_ffn(out["x_sorted"], out["offsets"], W["gate"], W["up"], W["down"],
                                    out["y_sorted"], ffn_ws, **skw),
        lambda: moe.moe_combine(out["y_sorted"], out["flat_to_sorted"], out["topk_gates"], out["y"]),
    ]
    # Each call is timed on its own, on the inputs the layer steps above left in place (every call
    # recomputes the same outputs). Nothing synchronises between the flush and the call: the host
    # enqueues the call while the flush still runs (~140 us), so the events bracket the call's GPU
    # execution and not the host's launch latency.
    reps = max(args.steps, 1)
    samples = np.zeros((reps, len(calls)))
    for i, fn in enumerate(calls):
        for r in range(reps):
            flush.sum()
            ev[0].record(stream)
            fn()
            ev[1].record(stream)
            torch.cuda.synchronize()
            samples[r, i] = ev[0].elapsed_time(ev[1]) * 1e3
    t_us = samples.mean(axis=0)
    pct = np.percentile(samples, [10, 50, 90], axis=0)
    a = 4 if cfg.act == "f32" else 2
    wb = {"f32": 4, "bf16": 2, "fp8_e4m3fn": 1}[cfg.w]
    sb = tr.fp8_scale_bytes(d, d_ff) if cfg.w == "fp8_e4m3fn" else 0
    bytes_ = {
        "route": tr.route_bytes(T, E, k),
        "permute": tr.permute_bytes(T, E, k, d, a),
        "grouped_ffn": tr.ffn_bytes(active, R, d, d_ff, wb, a, sb),
        "combine": tr.combine_bytes(T, k, d),
    }
    flops = tr.ffn_flops(R, d, d_ff)
    breakdown = {}
    for i, name in enumerate(["route", "permute", "grouped_ffn", "combine"]):
        gbps = bytes_[name] / (t_us[i] * 1e-6) / 1e9
        breakdown[name] = {"us": round(float(t_us[i]), 2), "p10_us": round(float(pct[0, i]), 2),
                           "median_us": round(float(pct[1, i]), 2), "p90_us": round(float(pct[2, i]), 2),
                           "alg_bytes": int(bytes_[name]),
                           "GB_per_s": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}
    mfma_peak = MFMA_PEAK_TFLOPS["fp32" if cfg.act == "f32" else "bf16"]
    ffn_tflops = flops / (t_us[2] * 1e-6) / 1e12
    breakdown["grouped_ffn"]["TFLOP_per_s"] = round(ffn_tflops, 2)
    breakdown["grouped_ffn"]["mfma_frac"] = round(ffn_tflops / mfma_peak, 4)
    # the FFN is HBM-bound when its intensity is below the ridge, MFMA-bound above it
    intensity = flops / bytes_["grouped_ffn"]
    ridge = mfma_peak * 1e12 / (HBM_PEAK_GBPS * 1e9)
    if intensity < ridge:
        roof = {"bound": "hbm", "achieved": round(bytes_["grouped_ffn"] / (t_us[2] * 1e-6) / 1e9, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(ffn_tflops, 2), "peak": mfma_peak, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["kernel"] = "moe_grouped_ffn (gate/up launch + down launch)"
    roof["alg_bytes"] = int(bytes_["grouped_ffn"])
    roof["alg_flops"] = int(flops)
    roof["us"] = round(float(t_us[2]), 2)
    roof["traffic"] = counter_traffic(cfg.name)
    log(f"grouped_ffn: {t_us[2]:.1f} us, {roof['achieved']} {roof['unit']} = {roof['frac']:.1%} of peak")

    # ---- CPU baseline: the fp64 oracle on the host cores
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, logits_np, x_np, host_w)
        log(f"cpu baseline: {cpu['value']} tokens/s on {cpu['cores']} threads "
            f"({cpu['host_cpus']} host CPUs)")

    line = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8_e4m3fn": "bf16 (fp8 e4m3fn weights)"}[cfg.w],
        "data": "synthetic (seeded: Zipf-biased N(0,1) router logits, N(0,1) x, N(0,1/fan_in) weights)",
        "config": {"workload": f"{cfg.name}: {cfg.note}", "T": T, "d": d, "E": E, "k": k, "d_ff": d_ff,
                   "activations": cfg.act, "weights": cfg.w,
                   "weight_layout": "blocked (8 rows x 128 bytes)" if blocked else "row-major",
                   "zipf_s": cfg.zipf_s, "seed": cfg.seed,
                   "active_experts": active, "max_rows_per_expert": int(counts.max())},
        "roofline": roof,
        "cpu_baseline": cpu,
        "breakdown": breakdown,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
