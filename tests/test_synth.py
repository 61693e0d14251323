"""The seeded input generator: format rounding against torch's conversions, determinism,
per-expert regeneration and the routing skew each workload is meant to have."""
import numpy as np
import torch

import oracle
import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 1e-30], np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.round_to_bf16(v), ref)


def test_e4m3fn_quantizer_matches_torch():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.uniform(-448, 448, 200000), rng.uniform(-0.05, 0.05, 50000),
                        [0.0, 448.0, -448.0, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -9 * 1.5]]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = synth.quantize_e4m3fn(v)
    # torch keeps the sign of a zero result; so do we
    assert np.array_equal(got, ref)
    assert np.array_equal(synth.quantize_e4m3fn_table(v), ref)


def test_block_quantisation_roundtrip_error():
    cfg = synth.tiny_config(T=1, d=256, E=1, k=1, d_ff=384, act="bf16", w="fp8_e4m3fn")
    w = synth.make_expert_weights(cfg, 0)
    assert w["gate"].dtype == np.uint8 and w["gate_scale"].shape == (3, 2)
    deq = oracle.decode_matrix(w["gate"], "fp8_e4m3fn", w["gate_scale"])
    assert np.max(np.abs(deq)) > 0
    # every block reaches its own amax exactly (448 * scale)
    for i in range(3):
        for j in range(2):
            blk = deq[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            assert np.isclose(np.max(np.abs(blk)), 448.0 * w["gate_scale"][i, j], rtol=1e-6)


def test_determinism_and_per_expert_streams():
    cfg = synth.tiny_config(T=9, d=32, E=6, k=2, d_ff=64, act="bf16", w="bf16", zipf_s=1.2, seed=4)
    a = synth.make_routing_inputs(cfg)
    b = synth.make_routing_inputs(cfg)
    assert all(np.array_equal(p, q) for p, q in zip(a, b))
    stacked = synth.make_all_weights(cfg)
    for e in (0, 3, 5):
        alone = synth.make_expert_weights(cfg, e)
        for key in ("gate", "up", "down"):
            assert np.array_equal(stacked[key][e], alone[key])
    partial = synth.make_all_weights(cfg, experts=[1])
    assert np.all(partial["gate"][0] == synth.BF16_NAN)
    assert np.array_equal(partial["gate"][1], stacked["gate"][1])


def test_zipf_bias_skews_routing():
    cfg = synth.CONFIGS["c2"]
    logits, x = synth.make_routing_inputs(cfg)
    assert logits.shape == (128, 128) and logits.dtype == np.float32
    assert x.shape == (128, 4096) and x.dtype == np.uint16
    ids = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :cfg.k]
    counts = np.bincount(ids.ravel(), minlength=cfg.E)
    assert counts.sum() == cfg.T * cfg.k
    active = int(np.count_nonzero(counts))
    assert 40 <= active <= 80
    assert counts.max() > 4 * counts[counts > 0].mean()


def test_layer_tokens_matches_layer():
    cfg = synth.tiny_config(T=11, d=24, E=5, k=3, d_ff=40, act="bf16", w="bf16", zipf_s=1.0, seed=2)
    logits, x = synth.make_routing_inputs(cfg)
    W = {e: synth.make_expert_weights(cfg, e) for e in range(cfg.E)}
    full = oracle.layer(logits, x, "bf16", lambda e: W[e], "bf16", cfg.k)
    toks = [0, 4, 10]
    y, rows = oracle.layer_tokens(toks, full["topk_ids"], full["topk_gates"], x, "bf16",
                                  lambda e: W[e], "bf16")
    assert np.allclose(y, full["y"][toks], rtol=1e-12, atol=1e-12)
    for (t, j), yr in rows.items():
        assert np.allclose(yr, full["y_sorted"][full["flat_to_sorted"][t * cfg.k + j]], rtol=1e-12, atol=1e-12)


def test_sampled_reference_matches_layer():
    # the GPU tests' per-token reference (every expert decoded once, both h roundings) is the
    # whole oracle's result on those tokens
    import types
    import gpu_harness as H
    cfg = synth.tiny_config(T=40, d=32, E=6, k=3, d_ff=48, act="bf16", w="bf16", zipf_s=1.2, seed=5)
    logits, x = synth.make_routing_inputs(cfg)
    Wd = {e: synth.make_expert_weights(cfg, e) for e in range(cfg.E)}
    W = types.SimpleNamespace(raw=lambda e: Wd[e])
    ids, gates = oracle.route(logits, cfg.k)
    perm = oracle.permute(ids, cfg.E)
    toks = H.covering_tokens(cfg, perm, 3, block=8, small=4)
    # every expert's first and last row and the first row of each 8-row block are owned by a
    # sampled token
    owned = {int(perm["flat_to_sorted"][t * cfg.k + j]) for t in toks for j in range(cfg.k)}
    for e in range(cfg.E):
        a, b = int(perm["offsets"][e]), int(perm["offsets"][e + 1])
        want = set(range(a, b)) if b - a <= 4 else set(range(a, b, 8)) | ({b - 1} if b > a else set())
        assert want <= owned
    # h from a bf16 implementation that rounds the fp64 h: its down projection is the bf16-h oracle
    full_h = oracle.layer(logits, x, "bf16", W.raw, "bf16", cfg.k, return_h=True)
    h_bits = {(t, j): synth.round_to_bf16(full_h["h"][full_h["flat_to_sorted"][t * cfg.k + j]].astype(np.float32))
              for t in toks for j in range(cfg.k)}
    ref = H.sampled_reference(toks, ids, gates, x, cfg, W, h_gpu=h_bits)
    for hr, suffix in ((None, ""), ("bf16", "_bf16h")):
        full = oracle.layer(logits, x, "bf16", W.raw, "bf16", cfg.k, h_round=hr)
        assert np.allclose(ref["y" + suffix], full["y"][toks], rtol=1e-12, atol=1e-12)
        for (t, j), yr in ref["rows" + suffix].items():
            assert np.allclose(yr, full["y_sorted"][full["flat_to_sorted"][t * cfg.k + j]], rtol=1e-12, atol=1e-12)
    for (t, j), h in ref["h64"].items():
        assert np.allclose(h, full_h["h"][full_h["flat_to_sorted"][t * cfg.k + j]], rtol=1e-12, atol=1e-14)
    # fp32 rounding of the fp64 h then RNE to bf16 is at most one double rounding away from the
    # bf16-h oracle's rounding: the rows agree within a bf16 unit's effect
    near = oracle.rel_max_err(ref["y_gpu_h"], ref["y_bf16h"])
    assert near <= 1e-2
    H.check_h_rounding_point(np.stack([h_bits[key] for key in sorted(h_bits)]),
                             np.stack([ref["h64"][key] for key in sorted(h_bits)]), "tiny")


def test_h_rounding_point_check_catches_mistakes():
    # the GPU tests' element-wise check of the implementation's bf16 h fails for an element two
    # bf16 units off, and for truncation in place of round-to-nearest
    import pytest
    import gpu_harness as H
    rng = np.random.default_rng(3)
    h64 = rng.standard_normal((64, 96)) * np.exp(rng.uniform(-3, 3, (64, 1)))
    good = synth.round_to_bf16(h64.astype(np.float32))
    H.check_h_rounding_point(good, h64, "good")
    bad = good.copy()
    i = np.unravel_index(np.argmax(np.abs(h64)), h64.shape)  # an element far above the allowance
    bad[i] = np.uint16(bad[i] + 2)
    with pytest.raises(AssertionError):
        H.check_h_rounding_point(bad, h64, "two units off")
    trunc = (h64.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    with pytest.raises(AssertionError):
        H.check_h_rounding_point(trunc, h64, "truncated")
