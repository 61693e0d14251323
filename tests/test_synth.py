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
    refs = H.sampled_reference(toks, ids, gates, x, cfg, W)
    for hr in (None, "bf16"):
        full = oracle.layer(logits, x, "bf16", W.raw, "bf16", cfg.k, h_round=hr)
        y, rows = refs[hr]
        assert np.allclose(y, full["y"][toks], rtol=1e-12, atol=1e-12)
        for (t, j), yr in rows.items():
            assert np.allclose(yr, full["y_sorted"][full["flat_to_sorted"][t * cfg.k + j]], rtol=1e-12, atol=1e-12)
