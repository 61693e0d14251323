"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Bar: topk_ids, counts, offsets, both index maps and x_sorted bytes bit-exact; gates within
1e-5 (max|err|/rms) with sum-to-one within k*2^-23; y and y_sorted within 1e-5 (fp32),
2e-2 (bf16) or 5e-2 (fp8 weights). Workloads small enough for the whole oracle are compared
element by element; the full-size decode/prefill/fp8 workloads compare routing and the
permutation in full and the float outputs on a seeded sample of tokens (each token's output
depends only on its own row, ids and gates).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import token_dispatch_expert_amd as moe
from token_dispatch_expert_amd.binding import layer_buffers

import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return H.require_gpu()


def run_full(cfg, dev, logits=None, x=None, plain_bar=True):
    """Whole layer vs the whole oracle. plain_bar=False keeps the plain fp64 comparison as a
    printed figure only (see the narrow-width case) and asserts the rounding-point bar."""
    lg0, x0 = synth.make_routing_inputs(cfg)
    logits = lg0 if logits is None else logits
    x = x0 if x is None else x
    ids, _ = oracle.route(logits, cfg.k)
    W = H.DeviceWeights(cfg, dev, experts=H.active_experts(np.bincount(ids.ravel(), minlength=cfg.E)))
    got = H.run_layer(cfg, logits, x, W, dev)
    ref = oracle.layer(logits, x, cfg.act, W.raw, cfg.w, cfg.k)
    H.check_routing_exact(got, ref, cfg.E)
    H.check_gates(got["topk_gates"], ref["topk_gates"], cfg.k)
    assert np.array_equal(got["x_sorted"], ref["x_sorted"]), "x_sorted bytes differ"
    tol = H.TOL[cfg.w]
    e_ys = oracle.rel_max_err(got["y_sorted"], ref["y_sorted"])
    e_y = oracle.rel_max_err(got["y"], ref["y"])
    print(f"{cfg.name}: y_sorted err {e_ys:.3e}, y err {e_y:.3e} (tol {tol})", flush=True)
    if plain_bar:
        assert e_ys <= tol and e_y <= tol
    else:
        assert cfg.act == "bf16", "only the bf16 rounding point replaces the plain bar"
    if cfg.act == "bf16":
        refh = oracle.layer(logits, x, cfg.act, W.raw, cfg.w, cfg.k, h_round="bf16")
        e_ys2 = oracle.rel_max_err(got["y_sorted"], refh["y_sorted"])
        e_y2 = oracle.rel_max_err(got["y"], refh["y"])
        print(f"{cfg.name}: vs bf16-h oracle: y_sorted err {e_ys2:.3e}, y err {e_y2:.3e} "
              f"(tol {H.TOL_ROUNDING_POINT})", flush=True)
        assert e_ys2 <= H.TOL_ROUNDING_POINT and e_y2 <= H.TOL_ROUNDING_POINT
    return got, ref


def run_sampled(cfg, dev, n_tokens, seed=0, logits=None):
    """Full-size layer: routing/permutation in full, float outputs on a token sample that
    reaches every active expert, every row tile and every kernel role.

    Float bars on the sample: y and y_sorted within the workload's tolerance of the plain fp64
    oracle; the implementation's bf16 h (its rounding point between the GEMMs) element by
    element within one bf16 unit of the fp64 h; y_sorted within the fp32 bar (1e-5) of the
    fp64 down projection of the implementation's own h, and y within it of their combine. (A
    y-level comparison with a bf16-h oracle is statistical at this size: the rare h element
    whose fp32 and fp64 values round to different bf16 neighbours moves its row's outputs by one
    bf16 unit of h, and over thousands of rows the largest such move exceeds 5e-3 of rms.)"""
    lg0, x = synth.make_routing_inputs(cfg)
    logits = lg0 if logits is None else logits
    ref_ids, ref_gates = oracle.route(logits, cfg.k)
    perm = oracle.permute(ref_ids, cfg.E)
    W = H.DeviceWeights(cfg, dev, experts=H.active_experts(perm["counts"]))
    toks = H.covering_tokens(cfg, perm, n_tokens, seed)
    keys = [(t, j) for t in toks for j in range(cfg.k)]
    srows = [int(perm["flat_to_sorted"][t * cfg.k + j]) for t, j in keys]
    print(f"{cfg.name}: weights on the device, running the layer", flush=True)
    got = H.run_layer(cfg, logits, x, W, dev, h_rows=srows if cfg.act == "bf16" else None)
    H.check_routing_exact(got, dict(topk_ids=ref_ids, **perm), cfg.E)
    H.check_gates(got["topk_gates"], ref_gates, cfg.k)
    xs_ref = oracle.gather_rows(x, perm["sorted_to_flat"], cfg.k)
    assert np.array_equal(got["x_sorted"], xs_ref), "x_sorted bytes differ"
    assert np.all(np.isfinite(got["y"])), "non-finite output (an expert without rows was read?)"
    print(f"{cfg.name}: routing exact; oracle on {len(toks)} tokens", flush=True)
    h_gpu = {key: got["h"][n] for n, key in enumerate(keys)} if "h" in got else None
    ref = H.sampled_reference(toks, ref_ids, ref_gates, x, cfg, W, h_gpu=h_gpu)
    ys_got = got["y_sorted"][srows]
    tol = H.TOL[cfg.w]
    e_y = oracle.rel_max_err(got["y"][toks], ref["y"])
    e_ys = oracle.rel_max_err(ys_got, np.stack([ref["rows"][key] for key in keys]))
    covered = {int(np.searchsorted(perm["offsets"], r, side="right")) - 1 for r in srows}
    active = set(H.active_experts(perm["counts"]))
    print(f"{cfg.name}: {len(toks)} sampled tokens, {len(keys)} y_sorted rows of {len(covered)}/{len(active)} "
          f"active experts: y_sorted err {e_ys:.3e}, y err {e_y:.3e} (tol {tol})", flush=True)
    e_ys2 = oracle.rel_max_err(ys_got, np.stack([ref["rows_bf16h"][key] for key in keys]))
    e_y2 = oracle.rel_max_err(got["y"][toks], ref["y_bf16h"])
    print(f"{cfg.name}: vs bf16-h oracle (figure only): y_sorted err {e_ys2:.3e}, y err {e_y2:.3e}", flush=True)
    assert covered == active, "the sample misses an active expert"
    assert e_ys <= tol and e_y <= tol
    if h_gpu is not None:
        H.check_h_rounding_point(np.stack([h_gpu[key] for key in keys]),
                                 np.stack([ref["h64"][key] for key in keys]), cfg.name)
        e_ys3 = oracle.rel_max_err(ys_got, np.stack([ref["rows_gpu_h"][key] for key in keys]))
        e_y3 = oracle.rel_max_err(got["y"][toks], ref["y_gpu_h"])
        print(f"{cfg.name}: vs fp64 down projection + combine of the GPU's own h: y_sorted err {e_ys3:.3e}, "
              f"y err {e_y3:.3e} (tol {H.TOL['f32']})", flush=True)
        assert e_ys3 <= H.TOL["f32"] and e_y3 <= H.TOL["f32"]


# ----------------------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------------------
def test_c1_tiny_fp32_full(dev):
    run_full(synth.CONFIGS["c1"], dev)


def test_c2_decode_bf16_full(dev):
    run_full(synth.CONFIGS["c2"], dev)


@pytest.mark.timeout(900)
def test_c3_decode_mixed_bf16_sampled(dev):
    run_sampled(synth.CONFIGS["c3"], dev, n_tokens=16)


@pytest.mark.timeout(900)
def test_c4_prefill_bf16_sampled(dev):
    run_sampled(synth.CONFIGS["c4"], dev, n_tokens=8)


@pytest.mark.timeout(900)
def test_c5_prefill_fp8_sampled(dev):
    run_sampled(synth.CONFIGS["c5"], dev, n_tokens=8)


# ----------------------------------------------------------------------------------------
# edge cases
# ----------------------------------------------------------------------------------------
def _onehot_logits(owner_lists, E, seed=0):
    """Logits whose top-k for token t is exactly owner_lists[t] (in that order)."""
    T = len(owner_lists)
    lg = np.random.default_rng(seed).uniform(-1, 0, size=(T, E)).astype(np.float32)
    for t, owners in enumerate(owner_lists):
        for j, e in enumerate(owners):
            lg[t, e] = np.float32(4.0 - 0.5 * j)
    return lg


@pytest.mark.parametrize("act,w", [("f32", "f32"), ("bf16", "bf16")])
def test_single_token(dev, act, w):
    run_full(synth.tiny_config(T=1, d=128, E=8, k=2, d_ff=256, act=act, w=w, seed=3), dev)


@pytest.mark.parametrize("name", ["c2", "c3"])
def test_single_token_full_width(dev, name):
    # one decode token at the full layer widths: each GEMM has few enough tiles that its
    # contraction is split across workgroups and summed by a second launch
    run_full(synth.CONFIGS[name].with_(T=1, name=f"{name}-T1"), dev)


def test_k_equals_e(dev):
    run_full(synth.tiny_config(T=33, d=64, E=4, k=4, d_ff=96, act="bf16", w="bf16", seed=4), dev)


def test_all_tokens_on_two_experts(dev):
    cfg = synth.tiny_config(T=300, d=128, E=16, k=2, d_ff=192, act="bf16", w="bf16", seed=5)
    lg = _onehot_logits([[11, 3]] * cfg.T, cfg.E)
    got, _ = run_full(cfg, dev, logits=lg)
    assert got["counts"][11] == 300 and got["counts"][3] == 300 and got["counts"].sum() == 600


@pytest.mark.parametrize("act,w", [("bf16", "bf16"), ("f32", "f32")])
def test_row_counts_at_tile_boundaries(dev, act, w):
    counts = [1, 15, 16, 17, 31, 32, 33, 0, 63, 64, 65, 0, 127, 128, 129, 255, 256, 257]
    E = len(counts)
    owners = [[e] for e, c in enumerate(counts) for _ in range(c)]
    np.random.default_rng(6).shuffle(owners)
    cfg = synth.tiny_config(T=len(owners), d=128, E=E, k=1, d_ff=160, act=act, w=w, seed=6)
    got, _ = run_full(cfg, dev, logits=_onehot_logits(owners, E))
    assert got["counts"].tolist() == counts


@pytest.mark.parametrize("w,d,d_ff", [("bf16", 128, 192), ("fp8_e4m3fn", 256, 384)])
def test_prefill_fragment_counts(dev, w, d, d_ff):
    # the large prefill tiles deal an expert's rows to its row tiles in whole 16-row fragments
    # and each wave runs a body compiled for the fragments of its row half that hold rows: these
    # counts (21, 37, ..., 245 rows, and experts of 300-1000 rows over 2-4 tiles) reach every
    # count in both halves of the 256-row bf16 and 128-row fp8 tiles
    counts = [16 * j + 5 for j in range(1, 16)] + [300, 520, 777, 1000]
    E = len(counts)
    owners = [[e] for e, c in enumerate(counts) for _ in range(c)]
    np.random.default_rng(8).shuffle(owners)
    cfg = synth.tiny_config(T=len(owners), d=d, E=E, k=1, d_ff=d_ff, act="bf16", w=w, seed=8)
    assert cfg.T * cfg.k >= 32 * cfg.E  # the prefill launch
    got, _ = run_full(cfg, dev, logits=_onehot_logits(owners, E))
    assert got["counts"].tolist() == counts


@pytest.mark.parametrize("act,w,d,d_ff", [("bf16", "bf16", 136, 200), ("f32", "f32", 40, 24),
                                           ("bf16", "bf16", 8, 8)])
def test_dims_not_multiples_of_tiles(dev, act, w, d, d_ff):
    run_full(synth.tiny_config(T=70, d=d, E=6, k=3, d_ff=d_ff, act=act, w=w, zipf_s=1.0, seed=7), dev)


@pytest.mark.parametrize("w,E,zipf", [("bf16", 5, 1.0), ("bf16", 40, 1.5), ("fp8_e4m3fn", 40, 1.5)])
def test_prefill_tile_paths(dev, w, E, zipf):
    # T*k >= 32*E selects the prefill tiles (256-row tiles; direct-to-LDS ring for bf16);
    # skewed counts also leave some experts with <= 16 rows on the streaming kernel, and no
    # expert's row count is a multiple of the tile
    d, d_ff = (192, 320) if w == "bf16" else (256, 384)
    cfg = synth.tiny_config(T=700, d=d, E=E, k=2, d_ff=d_ff, act="bf16", w=w, zipf_s=zipf, seed=13)
    got, _ = run_full(cfg, dev)
    assert cfg.T * cfg.k >= 32 * cfg.E


def _small_beside_large(counts, d, d_ff):
    """Per GEMM (gate/up, down): whether the experts with 1..16 rows of a prefill-sized bf16
    launch go to the lean streaming kernel on the library's second stream. This restates the
    library's rule, which compares their weight bytes at 3.5 GB/s per CU with the other
    experts' 256-row-tile-padded flops at 4 TFLOP/s per CU (the CU count cancels)."""
    out = []
    for N, K, mats in ((d_ff, d, 2), (d, d_ff, 1)):
        small = sum(mats * N * K * 2 for n in counts if 0 < n <= 16)
        large = sum(2 * ((n + 255) // 256 * 256) * K * mats * N for n in counts if n > 16)
        out.append(small > 0 and large > 0 and small / 3.5e9 <= large / 4e12)
    return out


@pytest.mark.parametrize("zipf,lean", [(2.0, True), (0.9, False)])
def test_prefill_small_experts_beside_tiles(dev, zipf, lean):
    # A prefill-sized bf16 layer whose experts with <= 16 rows go to the lean kernel on the
    # second stream beside the large tiles (few of them beside much tile work), or stay in the
    # prefill kernel's streaming role (more of them): both checked element-wise.
    cfg = synth.tiny_config(T=4096, d=512, E=128, k=4, d_ff=384, act="bf16", w="bf16",
                            zipf_s=zipf, seed=17)
    assert cfg.T * cfg.k >= 32 * cfg.E
    lg, _ = synth.make_routing_inputs(cfg)
    ids, _ = oracle.route(lg, cfg.k)
    counts = np.bincount(ids.ravel(), minlength=cfg.E)
    regime = _small_beside_large(counts, cfg.d, cfg.d_ff)
    print(f"small experts {int(((counts > 0) & (counts <= 16)).sum())}, lean (gate/up, down) {regime}",
          flush=True)
    assert regime == [lean, lean]
    run_full(cfg, dev)


def test_lean_kernel_every_small_count(dev):
    # every count from 1 to 16 rows once, two empty experts, and four experts of 5,000 rows
    # (enough tile work beside them for the rule to send the small ones to the lean kernel),
    # interleaved so that the lean kernel's walker steps over large and empty experts
    small = list(range(1, 17))
    counts = []
    for j, c in enumerate(small):
        counts.append(c)
        if j % 4 == 3:
            counts.append(5000 if j < 15 else 0)
    counts = [0] + counts + [5000]
    E = len(counts)
    assert sorted(c for c in counts if 0 < c <= 16) == small and counts.count(5000) == 4
    owners = [[e] for e, c in enumerate(counts) for _ in range(c)]
    np.random.default_rng(12).shuffle(owners)
    cfg = synth.tiny_config(T=len(owners), d=256, E=E, k=1, d_ff=256, act="bf16", w="bf16", seed=12)
    assert cfg.T * cfg.k >= 32 * cfg.E
    assert _small_beside_large(np.array(counts), cfg.d, cfg.d_ff) == [True, True]
    # 20,136 rows: the sampled check (every row of the small experts; the implementation's own h
    # element by element, then its down projection at the fp32 bar), since a y-level comparison
    # with the bf16-h oracle is a tail statistic at thousands of rows
    run_sampled(cfg, dev, n_tokens=64, seed=12, logits=_onehot_logits(owners, E))


@pytest.mark.parametrize("T", [24, 90])
def test_fp8_small(dev, T):
    # T = 24: 8 rows per expert, the decode-sized fp8 tiles; T = 90: the prefill kernel
    run_full(synth.tiny_config(T=T, d=256, E=6, k=2, d_ff=384, act="bf16", w="fp8_e4m3fn",
                               zipf_s=1.0, seed=8), dev)


@pytest.mark.parametrize("T", [20, 80])
def test_fp8_long_contraction(dev, T):
    # fp8 weights with d > 65536: the direct-to-LDS kernels stage an item's scale rows in LDS up
    # to that length, so these launches take the register-staged tiles (64-row tiles at T = 20,
    # 128-row at T = 80) beside the streaming kernel for experts with <= 16 rows
    cfg = synth.tiny_config(T=T, d=65664, E=2, k=1, d_ff=128, act="bf16", w="fp8_e4m3fn",
                            zipf_s=1.5, seed=9)
    assert (cfg.T * cfg.k >= 32 * cfg.E) == (T == 80)
    run_full(cfg, dev)


def test_many_experts_and_topk_limits(dev):
    # E and k at their limits
    run_full(synth.tiny_config(T=20, d=128, E=1024, k=32, d_ff=256, act="bf16", w="bf16", seed=9), dev)


def test_narrow_expert_width(dev):
    # d_ff = 64: the down GEMM's whole contraction is one 64-wide step of the direct-to-LDS ring.
    # At this width the bf16 rounding of h alone moves y by 2.09e-2 of its rms for this seed (a
    # CPU emulation of that rounding point gives the GPU's figure), over the 2e-2 bound stated for
    # the workloads' widths, so the case is held to the bf16-h oracle's 5e-3 bar instead.
    cfg = synth.tiny_config(T=20, d=128, E=1024, k=32, d_ff=64, act="bf16", w="bf16", seed=9)
    assert cfg.T * cfg.k < 32 * cfg.E  # the decode-sized tiles
    run_full(cfg, dev, plain_bar=False)


def test_bf16_output_is_rounded_fp32_sum(dev):
    # MOE_BF16 output: the fp32 combine result rounded to nearest even, bit for bit (torch's
    # float32 -> bfloat16 conversion rounds to nearest even), through moe_combine and moe_layer
    rng = np.random.default_rng(21)
    T, k, d = 300, 6, 520
    ys = torch.from_numpy((rng.standard_normal((T * k, d)) * np.exp(rng.uniform(-20, 20, (T * k, 1))))
                          .astype(np.float32)).to(dev)
    f2s = torch.from_numpy(rng.permutation(T * k).astype(np.int32)).to(dev)
    g = torch.from_numpy(rng.dirichlet(np.ones(k), size=T).astype(np.float32)).to(dev)
    y32 = torch.full((T, d), float("nan"), dtype=torch.float32, device=dev)
    y16 = torch.full((T, d), float("nan"), dtype=torch.bfloat16, device=dev)
    moe.moe_combine(ys, f2s, g, y32)
    moe.moe_combine(ys, f2s, g, y16)
    torch.cuda.synchronize()
    assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
    cfg = synth.tiny_config(T=70, d=256, E=12, k=4, d_ff=384, act="bf16", w="bf16", zipf_s=1.0, seed=22)
    logits, x = synth.make_routing_inputs(cfg)
    W = H.DeviceWeights(cfg, dev)
    outs = {}
    for ydt in (torch.float32, torch.bfloat16):
        out = layer_buffers(cfg.T, cfg.E, cfg.k, cfg.d, torch.bfloat16, device=dev, y_dtype=ydt)
        ws = moe.Workspace(moe.moe_layer_workspace_size(cfg.T, cfg.E, cfg.k, cfg.d, cfg.d_ff,
                                                        torch.bfloat16, torch.bfloat16), device=dev)
        out["y"].fill_(float("nan"))
        moe.moe_layer(torch.from_numpy(logits).to(dev), H.to_dev(x, "bf16", dev), W.gate, W.up, W.down,
                      cfg.k, out, ws)
        torch.cuda.synchronize()
        outs[ydt] = out["y"]
    assert torch.equal(outs[torch.bfloat16].view(torch.int16), outs[torch.float32].to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("E,k", [(12, 3), (300, 7)])
def test_ties_and_signed_zero(dev, E, k):
    # integer-valued logits: many exact ties, within a lane's experts and across wave rows
    cfg = synth.tiny_config(T=64, d=64, E=E, k=k, d_ff=64, act="f32", w="f32", seed=10)
    rng = np.random.default_rng(10)
    lg = rng.integers(-1, 2, size=(cfg.T, cfg.E)).astype(np.float32)
    lg[lg == 0] = np.where(rng.random(np.count_nonzero(lg == 0)) < 0.5, -0.0, 0.0).astype(np.float32)
    run_full(cfg, dev, logits=lg)


def test_empty_batch(dev):
    cfg = synth.tiny_config(T=0, d=128, E=8, k=2, d_ff=256, act="bf16", w="bf16")
    W = H.DeviceWeights(cfg, dev, experts=[])
    logits = np.zeros((0, cfg.E), np.float32)
    x = np.zeros((0, cfg.d), np.uint16)
    got = H.run_layer(cfg, logits, x, W, dev)
    assert got["counts"].tolist() == [0] * 8 and got["offsets"].tolist() == [0] * 9


def test_golden_load_example_on_gpu(dev):
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "load_imbalance_example.json")))
    owners = [[e] for e, c in enumerate(g["counts"]) for _ in range(c)]
    np.random.default_rng(7).shuffle(owners)
    lg = torch.from_numpy(_onehot_logits(owners, g["experts"])).to(dev)
    T, E = lg.shape
    ids = torch.empty((T, 1), dtype=torch.int32, device=dev)
    gates = torch.empty((T, 1), dtype=torch.float32, device=dev)
    counts = torch.full((E,), -7, dtype=torch.int32, device=dev)
    moe.moe_route(lg, 1, ids, gates, counts)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == g["counts"]
    assert torch.all(gates == 1.0)
    # the permutation's scan reproduces the printed per-expert blocks
    x = torch.zeros((T, 8), dtype=torch.bfloat16, device=dev)
    out = layer_buffers(T, E, 1, 8, torch.bfloat16, device=dev)
    ws = moe.Workspace(moe.moe_permute_workspace_size(T, E, 1), device=dev)
    moe.moe_permute(x, ids, E, out["counts"], out["offsets"], out["sorted_to_flat"],
                    out["flat_to_sorted"], out["x_sorted"], ws)
    torch.cuda.synchronize()
    assert out["offsets"].cpu().tolist() == [0, 140, 235, 313, 375, 423, 463, 494, 512]
    c = out["counts"].cpu().numpy()
    assert f"{c.max() / (T // E):.1f}x" == g["hot_vs_balanced_printed"]


# ----------------------------------------------------------------------------------------
# each call on its own
# ----------------------------------------------------------------------------------------
@pytest.mark.parametrize("act,w", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "fp8_e4m3fn")])
def test_calls_separately(dev, act, w):
    cfg = synth.tiny_config(T=75, d=256, E=10, k=3, d_ff=256, act=act, w=w, zipf_s=1.2, seed=11)
    logits, x = synth.make_routing_inputs(cfg)
    W = H.DeviceWeights(cfg, dev)
    ref = oracle.layer(logits, x, act, W.raw, w, cfg.k)
    T, E, k, d = cfg.T, cfg.E, cfg.k, cfg.d
    lg = torch.from_numpy(logits).to(dev)
    out = layer_buffers(T, E, k, d, H.ACT_TORCH[act], device=dev)
    counts_route = torch.full((E,), 99, dtype=torch.int32, device=dev)
    moe.moe_route(lg, k, out["topk_ids"], out["topk_gates"], counts_route)
    ws = moe.Workspace(moe.moe_permute_workspace_size(T, E, k), device=dev)
    moe.moe_permute(H.to_dev(x, act, dev), out["topk_ids"], E, out["counts"], out["offsets"],
                    out["sorted_to_flat"], out["flat_to_sorted"], out["x_sorted"], ws)
    torch.cuda.synchronize()
    got = {n: H.to_host(t) for n, t in out.items()}
    H.check_routing_exact(got, ref, E)
    assert np.array_equal(H.to_host(counts_route), ref["counts"])
    H.check_gates(got["topk_gates"], ref["topk_gates"], k)
    assert np.array_equal(got["x_sorted"], ref["x_sorted"])
    # grouped FFN fed with the oracle's x_sorted and offsets
    xs = H.to_dev(ref["x_sorted"], act, dev)
    off = torch.from_numpy(ref["offsets"]).to(dev)
    ys = torch.empty((T * k, d), dtype=torch.float32, device=dev)
    wsf = moe.Workspace(moe.moe_ffn_workspace_size(T * k, E, d, cfg.d_ff, H.ACT_TORCH[act], H.W_TORCH[w]), device=dev)
    moe.moe_grouped_ffn(xs, off, W.gate, W.up, W.down, ys, wsf, **W.kwargs())
    # combine fed with the oracle's y_sorted (as fp32), map and gates
    y = torch.empty((T, d), dtype=torch.float32, device=dev)
    moe.moe_combine(torch.from_numpy(ref["y_sorted"].astype(np.float32)).to(dev),
                    torch.from_numpy(ref["flat_to_sorted"]).to(dev),
                    torch.from_numpy(ref["topk_gates"].astype(np.float32)).to(dev), y)
    torch.cuda.synchronize()
    assert oracle.rel_max_err(H.to_host(ys), ref["y_sorted"]) <= H.TOL[w]
    assert oracle.rel_max_err(H.to_host(y), ref["y"]) <= 1e-6


def test_identity_experts_through_permute_and_combine(dev):
    """moe_permute then y_sorted := x_sorted then moe_combine returns x (normalised gates)."""
    cfg = synth.tiny_config(T=500, d=512, E=32, k=6, d_ff=8, act="f32", w="f32", zipf_s=1.0, seed=12)
    logits, x = synth.make_routing_inputs(cfg)
    T, E, k, d = cfg.T, cfg.E, cfg.k, cfg.d
    out = layer_buffers(T, E, k, d, torch.float32, device=dev)
    moe.moe_route(torch.from_numpy(logits).to(dev), k, out["topk_ids"], out["topk_gates"])
    ws = moe.Workspace(moe.moe_permute_workspace_size(T, E, k), device=dev)
    xd = torch.from_numpy(x).to(dev)
    moe.moe_permute(xd, out["topk_ids"], E, out["counts"], out["offsets"], out["sorted_to_flat"],
                    out["flat_to_sorted"], out["x_sorted"], ws)
    moe.moe_combine(out["x_sorted"], out["flat_to_sorted"], out["topk_gates"], out["y"])
    torch.cuda.synchronize()
    assert oracle.rel_max_err(out["y"].cpu().numpy(), x.astype(np.float64)) <= 1e-6


@pytest.mark.parametrize("T,E,k", [(3, 4, 1), (16, 8, 2), (60, 2, 1)])
def test_decode_few_experts_long_contraction(dev, T, E, k):
    # one to a few experts and a long contraction on the decode-sized path with so few tiles
    # that each tile's contraction is cut into chunks on different workgroups (up to 16 chunks
    # of at least 2 steps) whose fp32 partials a second launch adds in chunk order; (60, 2, 1) routes 36
    # and 24 rows, so both 32-row halves of a tile carry rows. The result matches the oracle and
    # a second run bit for bit.
    cfg = synth.tiny_config(T=T, d=2048, E=E, k=k, d_ff=1024, act="bf16", w="bf16", seed=5)
    assert cfg.T * cfg.k < 32 * cfg.E
    got, _ = run_full(cfg, dev)
    logits, x = synth.make_routing_inputs(cfg)
    ids, _ = oracle.route(logits, cfg.k)
    W = H.DeviceWeights(cfg, dev, experts=H.active_experts(np.bincount(ids.ravel(), minlength=cfg.E)))
    again = H.run_layer(cfg, logits, x, W, dev)
    for n in got:
        assert np.array_equal(got[n].view(np.uint8), again[n].view(np.uint8)), n


@pytest.mark.parametrize("T,d,E,k,d_ff,act,w,zipf", [
    (5, 1024, 16, 2, 512, "bf16", "bf16", 1.0),        # decode, contraction split of both GEMMs
    (40, 512, 4, 2, 768, "bf16", "bf16", None),        # decode split, 14-27 rows per expert
    (200, 256, 6, 3, 384, "bf16", "bf16", 1.2),        # prefill, every tile in a split last round
    (300, 384, 5, 2, 640, "bf16", "bf16", None),       # prefill, last round split in 3
    (700, 512, 8, 2, 512, "bf16", "fp8_e4m3fn", 1.0),  # fp8 prefill, last round split
    (2048, 256, 64, 8, 384, "bf16", "bf16", None),     # prefill, near-uniform routing: most experts
    (2048, 256, 64, 8, 384, "bf16", "fp8_e4m3fn", None),  # 200-300 rows, split into balanced tiles
    (33, 200, 7, 3, 72, "f32", "f32", None),           # fp32 streaming
    (256, 512, 64, 4, 384, "bf16", "fp8_e4m3fn", 1.0),  # fp8, 16 rows per expert: the prefill kernel
    (128, 512, 64, 4, 384, "bf16", "fp8_e4m3fn", 1.0),  # fp8 decode (8 rows per expert): direct-to-LDS tiles
    (5, 1024, 16, 2, 512, "bf16", "fp8_e4m3fn", 1.0),   # tiny fp8 decode: streaming + direct-to-LDS tiles
])
def test_ffn_paths_and_splits(dev, T, d, E, k, d_ff, act, w, zipf):
    # the kernel paths the sizes select, including both contraction splits, against the oracle,
    # and a second run bit for bit (the split sums go in chunk order)
    cfg = synth.tiny_config(T=T, d=d, E=E, k=k, d_ff=d_ff, act=act, w=w, zipf_s=zipf, seed=21)
    got, _ = run_full(cfg, dev)
    logits, x = synth.make_routing_inputs(cfg)
    ids, _ = oracle.route(logits, cfg.k)
    W = H.DeviceWeights(cfg, dev, experts=H.active_experts(np.bincount(ids.ravel(), minlength=cfg.E)))
    again = H.run_layer(cfg, logits, x, W, dev)
    for n in got:
        assert np.array_equal(got[n].view(np.uint8), again[n].view(np.uint8)), n


def test_repeat_runs_bit_identical(dev):
    cfg = synth.CONFIGS["c2"]
    logits, x = synth.make_routing_inputs(cfg)
    ids, _ = oracle.route(logits, cfg.k)
    W = H.DeviceWeights(cfg, dev, experts=H.active_experts(np.bincount(ids.ravel(), minlength=cfg.E)))
    a = H.run_layer(cfg, logits, x, W, dev)
    b = H.run_layer(cfg, logits, x, W, dev)
    for n in a:
        assert np.array_equal(a[n].view(np.uint8), b[n].view(np.uint8)), n
