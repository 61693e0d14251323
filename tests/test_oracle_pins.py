"""Pins for the fp64 oracle, independent of the oracle's own code.

Each check ties the oracle to something other than itself: values the pages print for a
worked example (tests/golden/), library routines that compute the same definition (stable
argsort, bincount, cumsum, softmax, torch's format conversions), closed forms, invariants
and a dense all-experts brute force on tiny inputs. The mutation test at the end plants
plausible mistakes in the oracle (on the CPU) and checks that these pins catch every one.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import moe_oracle as om
import synth
from token_dispatch_expert_amd import traffic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------------------
# tiny workloads
# ----------------------------------------------------------------------------------------
def tiny_case(T, d, E, k, d_ff, seed, fmt="f32", ties=False):
    rng = np.random.default_rng(seed)
    if ties:
        logits = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
    else:
        logits = rng.standard_normal((T, E)).astype(np.float32)
    x = rng.standard_normal((T, d)).astype(np.float32)
    W = {e: dict(gate=(rng.standard_normal((d_ff, d)) / math.sqrt(d)).astype(np.float32),
                 up=(rng.standard_normal((d_ff, d)) / math.sqrt(d)).astype(np.float32),
                 down=(rng.standard_normal((d, d_ff)) / math.sqrt(d_ff)).astype(np.float32))
         for e in range(E)}
    return logits, x, W


def kept_by_capacity(ids, E, cap):
    """0/1 per flat assignment: kept iff fewer than `cap` earlier assignments (in flat order)
    went to the same expert, from a stable argsort and a running count per group."""
    flat = np.asarray(ids).reshape(-1)
    order = np.argsort(flat, kind="stable")
    starts = np.searchsorted(flat[order], np.arange(E))
    rank = np.empty(flat.size, dtype=np.int64)
    rank[order] = np.arange(flat.size) - starts[flat[order]]
    return rank < cap, rank


def brute_force_layer(logits, x, W, k, cap=None):
    """Dense all-experts-masked evaluation written independently of the oracle: every expert
    runs on every token (einsum over the stored layouts), a 0/1 mask from a stable argsort
    picks the top k, and the gates come from a full softmax renormalised over the top k. With
    a capacity, slots beyond it (kept_by_capacity) are masked out of the sum."""
    l = logits.astype(np.float64)
    T, E = l.shape
    order = np.argsort(-l, axis=1, kind="stable")[:, :k]
    p = scipy.special.softmax(l, axis=1)
    keep = np.ones((T, k), bool) if cap is None else kept_by_capacity(order, E, cap)[0].reshape(T, k)
    M = np.zeros((T, E))
    for t in range(T):
        sel = p[t, order[t]]
        M[t, order[t]] = np.where(keep[t], sel / sel.sum(), 0.0)
    X = x.astype(np.float64)
    y = np.zeros_like(X)
    for e in range(E):
        g = np.einsum("td,fd->tf", X, W[e]["gate"].astype(np.float64))
        u = np.einsum("td,fd->tf", X, W[e]["up"].astype(np.float64))
        hh = g * scipy.special.expit(g) * u
        ye = np.einsum("tf,df->td", hh, W[e]["down"].astype(np.float64))
        y += M[:, e:e + 1] * ye
    return y, order, M


def run_oracle(logits, x, W, k, cap=None):
    return oracle.layer(logits, x, "f32", lambda e: W[e], "f32", k, capacity=cap)


# ----------------------------------------------------------------------------------------
# checks (each returns normally or raises); collected so the mutation test can re-run them
# ----------------------------------------------------------------------------------------
def check_decode_bf16():
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.decode_bf16(bits)
    ok = np.isnan(ref) == np.isnan(got)
    assert ok.all()
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])


def check_decode_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode_e4m3fn(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def check_route_vs_stable_argsort():
    for seed, ties in [(0, False), (1, True), (2, True), (3, False)]:
        for (T, E, k) in [(9, 8, 1), (9, 8, 3), (5, 16, 16), (17, 33, 5)]:
            logits, _, _ = tiny_case(T, 4, E, k, 4, seed, ties=ties)
            ids, _ = oracle.route(logits, k)
            ref = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :k]
            assert np.array_equal(ids, ref)


def check_route_special_cases():
    # all-equal logits -> 0..k-1, equal gates
    ids, g = oracle.route(np.full((3, 6), 0.25, np.float32), 4)
    assert np.array_equal(ids, np.tile(np.arange(4), (3, 1)))
    assert np.allclose(g, 0.25, rtol=0, atol=1e-15)
    # +0.0 and -0.0 are equal: the lower index wins either way round
    lg = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], np.float32)
    ids, _ = oracle.route(lg, 2)
    assert np.array_equal(ids, [[0, 1], [0, 1]])
    # k = 1: gate is exactly 1
    logits, _, _ = tiny_case(11, 4, 7, 1, 4, 5)
    _, g = oracle.route(logits, 1)
    assert np.all(g == 1.0)
    # k = E: the gates are the full softmax, in descending order
    ids, g = oracle.route(logits, 7)
    full = scipy.special.softmax(logits.astype(np.float64), axis=1)
    assert np.allclose(g, np.take_along_axis(full, ids.astype(np.int64), axis=1), rtol=1e-13, atol=0)
    # gates sum to one and are non-increasing; ids are distinct
    ids, g = oracle.route(logits, 3)
    assert np.allclose(g.sum(1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(g, axis=1) <= 0)
    assert all(len(set(r)) == 3 for r in ids.tolist())
    # a constant added to a row changes neither ids nor gates (shift invariance)
    ids2, g2 = oracle.route(logits + np.float32(4.0), 3)
    assert np.array_equal(ids, ids2)
    assert np.allclose(g, g2, rtol=1e-6, atol=0)
    # a two-expert closed form: gates = sigmoid of the logit gap
    ids, g = oracle.route(np.array([[0.5, 2.0]], np.float32), 2)
    assert np.array_equal(ids, [[1, 0]])
    assert math.isclose(g[0, 1], 1.0 / (1.0 + math.exp(1.5)), rel_tol=1e-14)


def check_permute_vs_library():
    for seed, (T, E, k) in enumerate([(13, 8, 2), (40, 5, 5), (1, 4, 3), (64, 16, 1)]):
        logits, _, _ = tiny_case(T, 4, E, k, 4, seed, ties=True)
        ids, _ = oracle.route(logits, k)
        p = oracle.permute(ids, E)
        flat = ids.reshape(-1)
        assert np.array_equal(p["counts"], np.bincount(flat, minlength=E))
        assert np.array_equal(p["offsets"], np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
        assert np.array_equal(p["sorted_to_flat"], np.argsort(flat, kind="stable"))
        # bijection, inverse, contiguity, totals
        assert np.array_equal(np.sort(p["sorted_to_flat"]), np.arange(T * k))
        assert np.array_equal(p["flat_to_sorted"][p["sorted_to_flat"]], np.arange(T * k))
        assert p["counts"].sum() == T * k
        for e in range(E):
            a, b = p["offsets"][e], p["offsets"][e + 1]
            assert np.all(flat[p["sorted_to_flat"][a:b]] == e)


def check_golden_load_example():
    g = _golden("load_imbalance_example.json")
    E, T = g["experts"], g["tokens"]
    counts = np.array(g["counts"])
    assert counts.sum() == T
    # logits that make expert e the arg-max for exactly counts[e] tokens, in a scrambled order
    owner = np.repeat(np.arange(E), counts)
    np.random.default_rng(7).shuffle(owner)
    logits = np.random.default_rng(8).uniform(-1, 0, size=(T, E)).astype(np.float32)
    logits[np.arange(T), owner] = 1.0
    ids, gates = oracle.route(logits, 1)
    p = oracle.permute(ids, E)
    assert np.array_equal(p["counts"], counts)
    assert p["offsets"].tolist() == [0, 140, 235, 313, 375, 423, 463, 494, 512]
    ideal = T // E
    assert ideal == g["balanced_per_expert"]
    assert f"{p['counts'].max() / ideal:.1f}x" == g["hot_vs_balanced_printed"]
    assert round(100 * ideal / p["counts"].max()) == g["utilisation_printed_percent"]
    assert np.all(gates == 1.0)


def check_golden_volume_example():
    g = _golden("a2a_volume_example.json")
    per_layer = traffic.exchange_bytes_per_layer(g["tokens"], g["k"], g["d"], g["bytes_per_element"])
    assert per_layer == 2_097_152
    assert round(per_layer / 1e6, 1) == g["per_layer_printed_MB"]
    per_step = per_layer * g["layers"]
    assert round(per_step / 1e6) == g["per_step_printed_MB"]
    for link in g["links"]:
        ms = traffic.transfer_ms(per_step, link["GB_per_s"])
        digits = len(str(link["printed_ms"]).split(".")[1])
        assert round(ms, digits) == link["printed_ms"], (link, ms)


def check_swiglu_closed_form():
    # one expert, one token, d = d_ff = 1: y = c * silu(a x) * (b x)
    x = np.array([[2.0]], np.float32)
    W = {0: dict(gate=np.array([[0.5]], np.float32), up=np.array([[3.0]], np.float32),
                 down=np.array([[-1.0]], np.float32))}
    out = run_oracle(np.zeros((1, 1), np.float32), x, W, 1)
    expect = -1.0 * (1.0 / (1.0 + math.exp(-1.0))) * 6.0
    assert math.isclose(out["y"][0, 0], expect, rel_tol=1e-15)
    # gate and up are not interchangeable: silu sits on the gate branch only
    W2 = {0: dict(gate=np.array([[1.0, 0.0]], np.float32), up=np.array([[0.0, 1.0]], np.float32),
                  down=np.array([[1.0], [0.0]], np.float32))}
    out = run_oracle(np.zeros((1, 1), np.float32), np.array([[-1.0, 2.0]], np.float32), W2, 1)
    sil = -1.0 / (1.0 + math.exp(1.0))
    assert np.allclose(out["y"][0], [sil * 2.0, 0.0], rtol=1e-15, atol=0)


def check_brute_force_layer():
    shapes = [(7, 6, 5, 9), (16, 16, 8, 16), (3, 5, 4, 12), (10, 8, 8, 8)]
    for seed, (T, d, E, d_ff) in enumerate(shapes):
        for k in range(1, E + 1):
            logits, x, W = tiny_case(T, d, E, k, d_ff, 100 + seed, ties=(seed % 2 == 1))
            ref, order, _ = brute_force_layer(logits, x, W, k)
            out = run_oracle(logits, x, W, k)
            assert np.array_equal(out["topk_ids"], order)
            assert oracle.rel_max_err(out["y"], ref) < 1e-12, (T, d, E, d_ff, k)


def check_identity_experts_and_gather():
    logits, x, _ = tiny_case(12, 10, 6, 3, 4, 9)
    ids, gates = oracle.route(logits, 3)
    p = oracle.permute(ids, 6)
    xs = oracle.gather_rows(x, p["sorted_to_flat"], 3)
    # identity experts + normalised gates return the input
    y = oracle.combine(xs.astype(np.float64), p["flat_to_sorted"], gates)
    assert np.allclose(y, x.astype(np.float64), rtol=1e-14, atol=1e-14)
    # k = 1 puts every row back exactly
    ids1, g1 = oracle.route(logits, 1)
    p1 = oracle.permute(ids1, 6)
    xs1 = oracle.gather_rows(x, p1["sorted_to_flat"], 1)
    y1 = oracle.combine(xs1.astype(np.float64), p1["flat_to_sorted"], g1)
    assert np.array_equal(y1, x.astype(np.float64))
    # rows of x_sorted are copies of their token's row
    for r in range(len(xs)):
        assert np.array_equal(xs[r], x[p["sorted_to_flat"][r] // 3])


def check_fp8_dequant_blocks():
    # a 256x256 matrix in 2x2 blocks with distinct scales: value = code value * its block scale
    codes = np.full((256, 256), 0x38, np.uint8)  # 1.0
    codes[0, 0] = 0xB8  # -1.0
    scale = np.array([[2.0, 3.0], [5.0, 7.0]], np.float32)
    v = oracle.decode_matrix(codes, "fp8_e4m3fn", scale)
    assert v[0, 0] == -2.0 and v[1, 1] == 2.0 and v[0, 200] == 3.0 and v[200, 0] == 5.0 and v[255, 255] == 7.0


def check_bf16_layer_decodes_inputs():
    # the bf16 path decodes stored bit patterns exactly before any arithmetic
    cfg = synth.tiny_config(T=5, d=16, E=4, k=2, d_ff=32, act="bf16", w="bf16", seed=3)
    logits, xb = synth.make_routing_inputs(cfg)
    Wb = {e: synth.make_expert_weights(cfg, e) for e in range(cfg.E)}
    out = oracle.layer(logits, xb, "bf16", lambda e: Wb[e], "bf16", cfg.k)
    xf = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).float().numpy()
    Wf = {e: {n: torch.from_numpy(Wb[e][n].view(np.int16)).view(torch.bfloat16).float().numpy()
              for n in ("gate", "up", "down")} for e in range(cfg.E)}
    ref, _, _ = brute_force_layer(logits, xf, Wf, cfg.k)
    assert oracle.rel_max_err(out["y"], ref) < 1e-12


def check_bf16_value_rounding():
    # on fp32-representable inputs, rounding fp64 straight to bf16 must equal torch's fp32->bf16
    rng = np.random.default_rng(12)
    v = np.concatenate([rng.standard_normal(50000) * 3, [1.00390625, 1.01171875, -2.0 ** -20 * 1.00390625]]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_bf16_value(v.astype(np.float64)), ref)


def check_capacity_formula():
    # ceil(C * T * k / E) with C in percent, on values worked by hand
    assert oracle.expert_capacity(512, 8, 1, 125) == 80      # the page's example, C = 1.25
    assert oracle.expert_capacity(512, 8, 1, 100) == 64
    assert oracle.expert_capacity(10, 3, 1, 100) == 4        # 10/3 rounds up
    assert oracle.expert_capacity(128, 128, 8, 110) == 9     # 8.8 rounds up
    assert oracle.expert_capacity(128, 128, 8, 100) == 8     # exact, no round-up
    assert oracle.expert_capacity(64, 8, 2, 200) == 32


def check_capacity_golden_example():
    # the page's worked counts (section 5) under its typical C = 1.25: every expert keeps
    # min(count, 80), the hot expert's load falls to 1.25x the balanced 64
    g = _golden("load_imbalance_example.json")
    E, T = g["experts"], g["tokens"]
    counts = np.array(g["counts"])
    owner = np.repeat(np.arange(E), counts)
    np.random.default_rng(7).shuffle(owner)
    ids = owner.reshape(T, 1)
    cap = oracle.expert_capacity(T, E, 1, 125)
    p = oracle.permute(ids, E, cap)
    assert p["counts"].tolist() == [80, 80, 78, 62, 48, 40, 31, 18]
    assert p["offsets"][-1] == 437 and (p["flat_to_sorted"] < 0).sum() == 75
    assert p["counts"].max() / g["balanced_per_expert"] == 1.25
    kept, _ = kept_by_capacity(ids, E, cap)
    assert np.array_equal(p["flat_to_sorted"] >= 0, kept)


def check_capacity_vs_library():
    for seed, (T, E, k) in enumerate([(13, 8, 2), (40, 5, 5), (64, 16, 1), (30, 4, 3)]):
        logits, _, _ = tiny_case(T, 4, E, k, 4, 50 + seed, ties=True)
        ids, _ = oracle.route(logits, k)
        flat = ids.reshape(-1)
        n = np.bincount(flat, minlength=E)
        for cap in (0, 1, 2, 5, int(n.max()) - 1, int(n.max()), T):
            if cap < 0:
                continue
            p = oracle.permute(ids, E, cap)
            kept, rank = kept_by_capacity(ids, E, cap)
            c = np.minimum(n, cap)
            assert np.array_equal(p["counts"], c)
            assert np.array_equal(p["offsets"], np.concatenate([[0], np.cumsum(c)]))
            want = np.where(kept, np.concatenate([[0], np.cumsum(c)])[flat] + rank, -1)
            assert np.array_equal(p["flat_to_sorted"], want)
            assert np.array_equal(p["flat_to_sorted"][p["sorted_to_flat"]], np.arange(c.sum()))
            if cap >= n.max():  # a capacity nobody reaches changes nothing
                q = oracle.permute(ids, E)
                assert all(np.array_equal(p[key], q[key]) for key in q)


def check_capacity_brute_force_layer():
    for seed, (T, d, E, k, d_ff) in enumerate([(20, 6, 4, 2, 8), (33, 5, 6, 3, 7), (16, 8, 3, 1, 4)]):
        logits, x, W = tiny_case(T, d, E, k, d_ff, 300 + seed)
        for cap in (1, 3, 7, T, 0):
            ref, _, _ = brute_force_layer(logits, x, W, k, cap)
            out = run_oracle(logits, x, W, k, cap)
            if cap == 0:
                assert np.all(out["y"] == 0.0) and out["offsets"][-1] == 0
            else:
                assert oracle.rel_max_err(out["y"], ref) < 1e-12, (seed, cap)


def check_router_logits():
    rng = np.random.default_rng(41)
    # brute force (explicit sums over the contraction) and torch's fp64 matmul on tiny inputs
    for T, E, d in [(5, 3, 7), (9, 6, 32), (1, 4, 64)]:
        xb = synth.round_to_bf16(rng.standard_normal((T, d)).astype(np.float32))
        wb = synth.round_to_bf16((rng.standard_normal((E, d)) / math.sqrt(d)).astype(np.float32))
        got = oracle.router_logits(xb, "bf16", wb, "bf16")
        X, Wr = oracle.decode_bf16(xb), oracle.decode_bf16(wb)
        want = np.array([[math.fsum(X[t, i] * Wr[e, i] for i in range(d)) for e in range(E)] for t in range(T)])
        assert got.shape == (T, E)
        assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))
        tw = (torch.from_numpy(X) @ torch.from_numpy(Wr).T).numpy()
        assert np.allclose(got, tw, rtol=1e-12, atol=1e-14)
    # one-hot router rows pick single columns of x, exactly
    T, d, E = 8, 40, 5
    xb = synth.round_to_bf16(rng.standard_normal((T, d)).astype(np.float32))
    cols = [3, 0, 39, 17, 3]
    w = np.zeros((E, d), np.float32)
    w[np.arange(E), cols] = 1.0
    got = oracle.router_logits(xb, "bf16", synth.round_to_bf16(w), "bf16")
    assert np.array_equal(got, oracle.decode_bf16(xb)[:, cols])


def check_rel_max_err():
    # the error measure the tolerances are stated in: max|got - ref| / sqrt(mean(ref^2)),
    # worked by hand on inputs where max and mean error, and rms and max|ref|, all differ
    f = oracle.rel_max_err
    assert math.isclose(f(np.array([1.0, 2.0, 3.0]), np.array([1.0, 2.0, 4.0])), 1.0 / math.sqrt(7.0),
                        rel_tol=1e-15)
    assert math.isclose(f(np.array([0.0, 0.0, 3.0]), np.array([1.0, 1.0, 1.0])), 2.0, rel_tol=1e-15)
    # rms(ref) = sqrt((9 + 16) / 2) = 5 / sqrt(2); max|ref| = 4; the error is below the reference
    assert math.isclose(f(np.array([3.0, 3.0]), np.array([3.0, 4.0])), math.sqrt(2.0) / 5.0, rel_tol=1e-15)
    # 2-D inputs are measured over all elements; rms = sqrt(30 / 4), max|err| = 0.5
    got = np.array([[1.0, -2.0], [3.5, 4.0]])
    ref = np.array([[1.0, -2.0], [3.0, 4.0]])
    assert math.isclose(f(got, ref), 0.5 / math.sqrt(7.5), rel_tol=1e-15)
    # scale invariance, exact zero, and the all-zero reference (absolute error)
    assert math.isclose(f(8.0 * got, 8.0 * ref), f(got, ref), rel_tol=1e-15)
    assert f(ref, ref) == 0.0
    assert f(np.array([0.5, -2.0]), np.zeros(2)) == 2.0


CHECKS = [
    check_decode_bf16, check_decode_e4m3fn, check_route_vs_stable_argsort,
    check_route_special_cases, check_permute_vs_library, check_golden_load_example,
    check_golden_volume_example, check_swiglu_closed_form, check_brute_force_layer,
    check_identity_experts_and_gather, check_fp8_dequant_blocks, check_bf16_layer_decodes_inputs,
    check_bf16_value_rounding, check_capacity_formula, check_capacity_golden_example,
    check_capacity_vs_library, check_capacity_brute_force_layer, check_router_logits,
    check_rel_max_err,
]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_oracle_pin(check):
    check()


# ----------------------------------------------------------------------------------------
# the pins must catch plausible mistakes planted in the oracle
# ----------------------------------------------------------------------------------------
_ORIG = {n: getattr(om, n) for n in ("route", "permute", "combine", "decode_e4m3fn", "expert_ffn", "decode_bf16",
                                     "expert_capacity", "router_logits", "rel_max_err", "expert_down", "ffn",
                                     "make_weight_decoder")}


def _mut_route_tie_high(logits, k):
    lg = np.asarray(logits, np.float32).astype(np.float64)
    T, E = lg.shape
    ids = np.empty((T, k), np.int32)
    gates = np.empty((T, k))
    for t in range(T):
        row = lg[t].copy()
        ch = []
        for _ in range(k):
            e = E - 1 - int(np.argmax(row[::-1]))   # last occurrence wins ties
            ch.append(e)
            row[e] = -np.inf
        w = np.exp(lg[t, ch] - lg[t, ch[0]])
        ids[t], gates[t] = ch, w / w.sum()
    return ids, gates


def _mut_route_full_softmax(logits, k):
    ids, _ = _ORIG["route"](logits, k)
    lg = np.asarray(logits, np.float32).astype(np.float64)
    p = np.exp(lg - lg.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    return ids, np.take_along_axis(p, ids.astype(np.int64), 1)


def _mut_route_smallest(logits, k):
    ids, g = _ORIG["route"](-np.asarray(logits, np.float32), k)
    return ids, g


def _mut_route_no_max_shift_sign(logits, k):
    ids, _ = _ORIG["route"](logits, k)
    lg = np.asarray(logits, np.float32).astype(np.float64)
    sel = np.take_along_axis(lg, ids.astype(np.int64), 1)
    w = np.exp(sel[:, :1] - sel)       # wrong sign
    return ids, w / w.sum(1, keepdims=True)


def _mut_permute_unstable(topk_ids, E, capacity=None):
    p = _ORIG["permute"](topk_ids, E, capacity)
    s2f = p["sorted_to_flat"].copy()
    for e in range(E):
        a, b = p["offsets"][e], p["offsets"][e + 1]
        s2f[a:b] = s2f[a:b][::-1]
    f2s = np.full_like(p["flat_to_sorted"], -1)
    f2s[s2f] = np.arange(len(s2f))
    return dict(p, sorted_to_flat=s2f, flat_to_sorted=f2s.astype(np.int32))


def _mut_permute_inclusive_scan(topk_ids, E, capacity=None):
    p = _ORIG["permute"](topk_ids, E, capacity)
    off = p["offsets"].copy()
    off[:-1] = off[1:]
    return dict(p, offsets=off)


def _mut_permute_keep_last(topk_ids, E, capacity=None):
    # a capacity that keeps each expert's last assignments instead of its first
    if capacity is None:
        return _ORIG["permute"](topk_ids, E)
    R = np.asarray(topk_ids).size
    p = _ORIG["permute"](np.asarray(topk_ids).reshape(-1)[::-1].reshape(R, 1), E, capacity)
    f2s = p["flat_to_sorted"][::-1].copy()
    s2f = np.full_like(p["sorted_to_flat"], 0)
    s2f[f2s[f2s >= 0]] = np.nonzero(f2s >= 0)[0]
    return dict(p, sorted_to_flat=s2f.astype(np.int32), flat_to_sorted=f2s.astype(np.int32))


def _mut_permute_cap_plus_one(topk_ids, E, capacity=None):
    return _ORIG["permute"](topk_ids, E, None if capacity is None else capacity + 1)


def _mut_capacity_floor(T, E, k, factor_percent):
    return (factor_percent * T * k) // (100 * E)


def _mut_combine_keeps_dropped(y_sorted, flat_to_sorted, gates):
    # a dropped slot's -1 used as an index (the last row) instead of being skipped
    T, k = gates.shape
    y = np.zeros((T, y_sorted.shape[1]))
    for t in range(T):
        for j in range(k):
            y[t] += gates[t, j] * y_sorted[int(flat_to_sorted[t * k + j])]
    return y


def _mut_h_round(h, h_round):
    return om.round_bf16_value(h) if h_round == "bf16" else h


def _mut_ffn_silu_on_up(X, Wg, Wu, Wd, return_h=False, h_round=None):
    G, U = X @ Wg.T, X @ Wu.T
    h = _mut_h_round(om.silu(U) * G, h_round)
    y = h @ Wd.T
    return (y, h) if return_h else y


def _mut_ffn_sigmoid_only(X, Wg, Wu, Wd, return_h=False, h_round=None):
    G, U = X @ Wg.T, X @ Wu.T
    h = _mut_h_round((1.0 / (1.0 + np.exp(-G))) * U, h_round)
    y = h @ Wd.T
    return (y, h) if return_h else y


def _mut_ffn_down_untransposed(X, Wg, Wu, Wd, return_h=False, h_round=None):
    G, U = X @ Wg.T, X @ Wu.T
    h = _mut_h_round(om.silu(G) * U, h_round)
    y = h @ Wd if Wd.shape[0] == Wd.shape[1] else h @ Wd.T[:, ::-1]
    return (y, h) if return_h else y


def _mut_grouped_ffn_expert_shift(x_sorted, offsets, expert_weights, return_h=False, h_round=None):
    # each segment goes through the next expert's weights (segment index off by one)
    E = len(offsets) - 1
    return _ORIG["ffn"](x_sorted, offsets, lambda e: expert_weights((e + 1) % E), return_h, h_round)


def _mut_grouped_ffn_last_row_skipped(x_sorted, offsets, expert_weights, return_h=False, h_round=None):
    # every non-empty segment stops one row short (end taken as inclusive-minus-one)
    off = np.asarray(offsets).copy()
    out = _ORIG["ffn"](x_sorted, off, expert_weights, return_h, h_round)
    y = out[0] if return_h else out
    for e in range(len(off) - 1):
        if off[e + 1] > off[e]:
            y[off[e + 1] - 1] = 0.0
    return out


def _mut_decoder_gate_up_swapped(raw_weights, w_fmt):
    dec = _ORIG["make_weight_decoder"](raw_weights, w_fmt)
    def swapped(e):
        g, u, d = dec(e)
        return u, g, d
    return swapped


def _mut_combine_unweighted(y_sorted, flat_to_sorted, gates):
    return _ORIG["combine"](y_sorted, flat_to_sorted, np.ones_like(gates))


def _mut_combine_wrong_map(y_sorted, flat_to_sorted, gates):
    inv = np.empty_like(flat_to_sorted)
    inv[flat_to_sorted] = np.arange(len(flat_to_sorted))
    return _ORIG["combine"](y_sorted, inv, gates)


def _mut_decode_bf16_shift(bits):
    u32 = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(15)
    return u32.view(np.float32).astype(np.float64)


def _mut_decode_e4m3_bias8(codes):
    return _ORIG["decode_e4m3fn"](codes) / 2.0


def _mut_router_drop_last_term(x, x_fmt, w_router, w_fmt):
    X = om.decode_activations(x, x_fmt)[:, :-1]
    Wr = om.decode_matrix(w_router, w_fmt)[:, :-1]
    return X @ Wr.T


def _mut_router_untransposed_rows(x, x_fmt, w_router, w_fmt):
    X = om.decode_activations(x, x_fmt)
    Wr = om.decode_matrix(w_router, w_fmt)
    return X @ Wr[::-1].T


def _mut_down_reversed_inputs(h, Wd):
    # h's columns paired with the wrong rows of the stored down matrix
    return h[:, ::-1] @ Wd.T


def _mut_down_missing_last(h, Wd):
    return h[:, :-1] @ Wd[:, :-1].T


def _mut_err_mean(got, ref):
    # mean |error| in place of the largest
    ref, got = np.asarray(ref, np.float64), np.asarray(got, np.float64)
    return float(np.mean(np.abs(got - ref))) / float(np.sqrt(np.mean(ref * ref)))


def _mut_err_max_ref(got, ref):
    # the largest |ref| in place of the rms
    ref, got = np.asarray(ref, np.float64), np.asarray(got, np.float64)
    return float(np.max(np.abs(got - ref))) / float(np.max(np.abs(ref)))


def _mut_err_no_sqrt(got, ref):
    ref, got = np.asarray(ref, np.float64), np.asarray(got, np.float64)
    return float(np.max(np.abs(got - ref))) / float(np.mean(ref * ref))


def _mut_err_mean_abs_ref(got, ref):
    ref, got = np.asarray(ref, np.float64), np.asarray(got, np.float64)
    return float(np.max(np.abs(got - ref))) / float(np.mean(np.abs(ref)))


MUTANTS = {
    "route_tie_high": ("route", _mut_route_tie_high),
    "route_full_softmax": ("route", _mut_route_full_softmax),
    "route_smallest": ("route", _mut_route_smallest),
    "route_gate_sign": ("route", _mut_route_no_max_shift_sign),
    "permute_unstable": ("permute", _mut_permute_unstable),
    "permute_inclusive_scan": ("permute", _mut_permute_inclusive_scan),
    "permute_keep_last": ("permute", _mut_permute_keep_last),
    "permute_cap_plus_one": ("permute", _mut_permute_cap_plus_one),
    "capacity_floor": ("expert_capacity", _mut_capacity_floor),
    "combine_keeps_dropped": ("combine", _mut_combine_keeps_dropped),
    "router_drop_last_term": ("router_logits", _mut_router_drop_last_term),
    "router_reversed_experts": ("router_logits", _mut_router_untransposed_rows),
    "ffn_silu_on_up": ("expert_ffn", _mut_ffn_silu_on_up),
    "ffn_sigmoid_only": ("expert_ffn", _mut_ffn_sigmoid_only),
    "ffn_down_untransposed": ("expert_ffn", _mut_ffn_down_untransposed),
    "grouped_ffn_expert_shift": ("ffn", _mut_grouped_ffn_expert_shift),
    "grouped_ffn_last_row_skipped": ("ffn", _mut_grouped_ffn_last_row_skipped),
    "decoder_gate_up_swapped": ("make_weight_decoder", _mut_decoder_gate_up_swapped),
    "combine_unweighted": ("combine", _mut_combine_unweighted),
    "combine_wrong_map": ("combine", _mut_combine_wrong_map),
    "decode_bf16_shift": ("decode_bf16", _mut_decode_bf16_shift),
    "decode_e4m3_bias8": ("decode_e4m3fn", _mut_decode_e4m3_bias8),
    "down_reversed_inputs": ("expert_down", _mut_down_reversed_inputs),
    "down_missing_last": ("expert_down", _mut_down_missing_last),
    "rel_err_mean": ("rel_max_err", _mut_err_mean),
    "rel_err_max_ref": ("rel_max_err", _mut_err_max_ref),
    "rel_err_no_sqrt": ("rel_max_err", _mut_err_no_sqrt),
    "rel_err_mean_abs_ref": ("rel_max_err", _mut_err_mean_abs_ref),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    fn_name, mutant = MUTANTS[name]
    monkeypatch.setattr(om, fn_name, mutant)
    monkeypatch.setattr(oracle, fn_name, mutant, raising=False)
    failures = 0
    for check in CHECKS:
        try:
            check()
        except TypeError:
            raise  # a mutant whose signature does not fit its callers never ran: no catch
        except Exception:  # an assertion or a shape error both count as caught
            failures += 1
    assert failures > 0, f"no pin caught mutant {name}"
