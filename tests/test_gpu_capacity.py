"""GPU parity of the capacity factor ("Expert Parallelism" tutorial page, section 5,
mitigation 1; section 10, exercise D): moe_layer_capped / moe_permute_capped against the
oracle with the same capacity, on the single-workgroup (T*k <= 8192) and the tiled
(T*k > 8192) permutation paths. Routing, counts, offsets and both maps are compared bit for
bit; outputs within the format's tolerance."""
import numpy as np
import pytest
import torch

import gpu_harness as H
import oracle
import synth
import token_dispatch_expert_amd as moe
from token_dispatch_expert_amd.binding import layer_buffers

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return H.require_gpu()


def run_capped(cfg, logits, x, W, dev, cap):
    lg = torch.from_numpy(logits).to(dev)
    xd = H.to_dev(x, cfg.act, dev)
    out = layer_buffers(cfg.T, cfg.E, cfg.k, cfg.d, H.ACT_TORCH[cfg.act], device=dev)
    for t in out.values():  # poison: rows past the kept ones must not be needed
        if t.dtype in (torch.float32, torch.bfloat16):
            t.fill_(float("nan"))
        else:
            t.fill_(-7)
    ws = moe.Workspace(moe.moe_layer_workspace_size(cfg.T, cfg.E, cfg.k, cfg.d, cfg.d_ff,
                                                    H.ACT_TORCH[cfg.act], H.W_TORCH[cfg.w]), device=dev)
    moe.moe_layer(lg, xd, W.gate, W.up, W.down, cfg.k, out, ws, capacity=cap, **W.kwargs())
    torch.cuda.synchronize()
    return {n: H.to_host(t) for n, t in out.items()}


def check_capped(cfg, got, ref, cap):
    kept = int(ref["offsets"][-1])
    assert int(got["offsets"][-1]) == kept
    for n in ("topk_ids", "counts", "offsets", "flat_to_sorted"):
        assert np.array_equal(got[n], ref[n]), n
    H.check_gates(got["topk_gates"], ref["topk_gates"], cfg.k)
    assert np.array_equal(got["sorted_to_flat"][:kept], ref["sorted_to_flat"]), "sorted_to_flat"
    assert np.array_equal(got["x_sorted"][:kept], ref["x_sorted"]), "x_sorted"
    tol = H.TOL[cfg.w]
    assert np.all(np.isfinite(got["y"]))
    # a token whose every slot was dropped gets exactly 0; the others are compared with the
    # tolerance over those rows only (the rms over a mostly-zero y would not measure anything)
    live = (ref["flat_to_sorted"].reshape(cfg.T, cfg.k) >= 0).any(axis=1)
    assert np.all(got["y"][~live] == 0.0), "a token with every slot dropped is not zero"
    if kept:
        e_ys = oracle.rel_max_err(got["y_sorted"][:kept], ref["y_sorted"])
        e_y = oracle.rel_max_err(got["y"][live], ref["y"][live])
        print(f"capacity {cap}: kept {kept}/{cfg.T * cfg.k} ({live.sum()} tokens), "
              f"y_sorted err {e_ys:.3e}, y err {e_y:.3e}", flush=True)
        assert e_ys <= tol and e_y <= tol


@pytest.mark.parametrize("T,E,k,d,d_ff,act,w", [
    (100, 300, 6, 256, 256, "bf16", "bf16"),   # many experts (5 per lane in the route)
    (300, 16, 4, 256, 256, "bf16", "bf16"),    # single-workgroup permutation
    (3000, 64, 4, 128, 128, "f32", "f32"),     # T*k = 12000: tiled permutation
])
def test_layer_with_capacity(dev, T, E, k, d, d_ff, act, w):
    cfg = synth.tiny_config(T=T, d=d, E=E, k=k, d_ff=d_ff, act=act, w=w, zipf_s=1.2, seed=21)
    logits, x = synth.make_routing_inputs(cfg)
    W = H.DeviceWeights(cfg, dev)
    caps = [0, 1] + [oracle.expert_capacity(T, E, k, p) for p in (100, 125, 150, 200)] + [T]
    for cap in caps:
        assert moe.moe_expert_capacity(T, E, k, 125) == oracle.expert_capacity(T, E, k, 125)
        got = run_capped(cfg, logits, x, W, dev, cap)
        ref = oracle.layer(logits, x, act, W.raw, w, k, capacity=cap)
        check_capped(cfg, got, ref, cap)


def test_permute_capacity_prefill_size(dev):
    """Routing and maps only, at the 65,536-assignment prefill size."""
    cfg = synth.CONFIGS["c4"]
    logits, _ = synth.make_routing_inputs(cfg)
    T, E, k = cfg.T, cfg.E, cfg.k
    ids = torch.from_numpy(oracle.route(logits, k)[0]).to(dev)
    x = torch.zeros((T, 8), dtype=torch.bfloat16, device=dev)
    ws = moe.Workspace(moe.moe_permute_workspace_size(T, E, k), device=dev)
    for p in (100, 150):
        cap = moe.moe_expert_capacity(T, E, k, p)
        out = layer_buffers(T, E, k, 8, torch.bfloat16, device=dev)
        moe.moe_permute(x, ids, E, out["counts"], out["offsets"], out["sorted_to_flat"],
                        out["flat_to_sorted"], out["x_sorted"], ws, capacity=cap)
        torch.cuda.synchronize()
        ref = oracle.permute(ids.cpu().numpy(), E, cap)
        kept = int(ref["offsets"][-1])
        print(f"C = {p / 100}: capacity {cap}, dropped {T * k - kept} of {T * k}", flush=True)
        for n in ("counts", "offsets", "flat_to_sorted"):
            assert np.array_equal(out[n].cpu().numpy(), ref[n]), n
        assert np.array_equal(out["sorted_to_flat"][:kept].cpu().numpy(), ref["sorted_to_flat"])


@pytest.mark.parametrize("T,E,k,cap_pct,zipf", [
    (9000, 1, 1, None, 0),       # one expert
    (1000, 17, 9, None, 0),      # the last 16-expert scan workgroup holds one expert
    (600, 1024, 16, None, 0),    # the expert limit: every rank wavefront scans 16 counts per lane
    (40000, 33, 8, None, 0),     # 1,250 tiles: more than the scan keeps in registers
    (3000, 300, 4, 110, 0),      # capacity on a partial scan workgroup
    (8193, 256, 1, None, 0),     # one assignment past the one-workgroup kernel: count-and-rank launch
    (2731, 200, 3, None, 1.5),   # the same with 200 experts, skewed (a hot expert per wave)
    (16384, 256, 4, 125, 1.5),   # count-and-rank at its largest batch, capacity, skewed
    (8200, 256, 8, 125, 0),      # 65,600 assignments: histogram and rank launches, capacity
    (12000, 257, 2, None, 1.2),  # 257 experts: histogram and rank launches
])
def test_permute_large_batches(dev, T, E, k, cap_pct, zipf):
    """The multi-launch permutation (more than 8192 assignments) at expert counts and tile
    counts the prefill workloads do not reach, and on both sides of the count-and-rank
    kernel's limits: counts, offsets, both maps and the sorted rows bit for bit against the
    oracle's stable counting sort."""
    rng = np.random.default_rng(T * 31 + E)
    # k distinct experts per token: top k of Gumbel-perturbed log weights (Zipf weights when
    # zipf > 0, uniform otherwise)
    logw = -zipf * np.log(np.arange(1, E + 1, dtype=np.float64))
    ids = np.argsort(-(logw + rng.gumbel(size=(T, E))), axis=1)[:, :k].astype(np.int32)
    x = rng.integers(-32768, 32768, size=(T, 8), dtype=np.int16)          # bf16 bit patterns
    cap = None if cap_pct is None else moe.moe_expert_capacity(T, E, k, cap_pct)
    ref = oracle.permute(ids, E, cap)
    xd = torch.from_numpy(x).to(dev).view(torch.bfloat16)
    out = layer_buffers(T, E, k, 8, torch.bfloat16, device=dev)
    ws = moe.Workspace(moe.moe_permute_workspace_size(T, E, k), device=dev)
    kw = {} if cap is None else {"capacity": cap}
    moe.moe_permute(xd, torch.from_numpy(ids).to(dev), E, out["counts"], out["offsets"],
                    out["sorted_to_flat"], out["flat_to_sorted"], out["x_sorted"], ws, **kw)
    torch.cuda.synchronize()
    kept = int(ref["offsets"][-1])
    for n in ("counts", "offsets", "flat_to_sorted"):
        assert np.array_equal(out[n].cpu().numpy(), ref[n]), n
    assert np.array_equal(out["sorted_to_flat"][:kept].cpu().numpy(), ref["sorted_to_flat"])
    xs = out["x_sorted"][:kept].view(torch.int16).cpu().numpy()
    assert np.array_equal(xs, x[ref["sorted_to_flat"] // k])


def test_combine_skips_dropped_slots(dev):
    rng = np.random.default_rng(5)
    T, k, d = 37, 3, 64
    R = T * k
    ys = rng.standard_normal((R, d)).astype(np.float32)
    f2s = rng.permutation(R).astype(np.int32)
    f2s[rng.random(R) < 0.3] = -1
    gates = rng.random((T, k)).astype(np.float32)
    y = torch.empty((T, d), dtype=torch.float32, device=dev)
    moe.moe_combine(torch.from_numpy(ys).to(dev), torch.from_numpy(f2s).to(dev),
                    torch.from_numpy(gates).to(dev), y)
    torch.cuda.synchronize()
    ref = oracle.combine(ys.astype(np.float64), f2s, gates.astype(np.float64))
    assert oracle.rel_max_err(y.cpu().numpy(), ref) <= 1e-6
