"""GPU parity of the fused router (moe_route_gemm): the fp32 logits against the fp64 oracle
within the rounding bound of an fp32 dot product, and the top-k / gates against the oracle's
routing of the GPU's own fp32 logits (the selection is compared in the precision that made
it), bit for bit; also against moe_route on the same logits and with the logits not written."""
import numpy as np
import pytest
import torch

import gpu_harness as H
import oracle
import synth
import token_dispatch_expert_amd as moe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return H.require_gpu()


def make(T, E, d, seed, dup=None):
    rng = np.random.default_rng(seed)
    x = synth.round_to_bf16(rng.standard_normal((T, d)).astype(np.float32))
    w = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    if dup is not None:            # identical rows -> exactly equal logits -> ties
        for a, b in dup:
            w[b] = w[a]
    return x, synth.round_to_bf16(w)


def run(dev, x, w, k, with_logits=True):
    T, d = x.shape
    E = w.shape[0]
    xd, wd = H.to_dev(x, "bf16", dev), H.to_dev(w, "bf16", dev)
    ids = torch.full((T, k), -5, dtype=torch.int32, device=dev)
    ws = moe.Workspace(moe.moe_route_gemm_workspace_size(T, E, k), device=dev)
    gates = torch.full((T, k), float("nan"), device=dev)
    counts = torch.full((E,), -5, dtype=torch.int32, device=dev)
    lg = torch.full((T, E), float("nan"), device=dev) if with_logits else None
    moe.moe_route_gemm(xd, wd, k, ids, gates, counts, lg, workspace=ws)
    torch.cuda.synchronize()
    return (ids.cpu().numpy(), gates.cpu().numpy(), counts.cpu().numpy(),
            None if lg is None else lg.cpu().numpy())


@pytest.mark.parametrize("T,E,k,d,dup", [
    (128, 128, 8, 4096, None),        # decode-shape router (contraction split over workgroups)
    (2000, 96, 4, 256, None),         # one fused pass, 16-token tiles
    (8192, 256, 8, 7168, None),       # prefill DeepSeek-V3-shaped router (32-token tiles)
    (37, 40, 5, 96, None),            # ragged token tile, E not a multiple of 16
    (1, 8, 8, 32, None),              # k = E, one token
    (300, 64, 6, 128, [(5, 9), (9, 12), (0, 63)]),  # exact ties between experts
])
def test_route_gemm(dev, T, E, k, d, dup):
    x, w = make(T, E, d, seed=T + E + d, dup=dup)
    ids, gates, counts, lg = run(dev, x, w, k)
    # logits: |gpu - exact| <= gamma_d * (|x| |w|^T), gamma_d = d u / (1 - d u), u = 2^-24 (the
    # fp32 rounding bound of a d-term sum of exact products, whatever the summation order)
    X, Wr = oracle.decode_bf16(x), oracle.decode_bf16(w)
    ref = oracle.router_logits(x, "bf16", w, "bf16")
    u = 2.0 ** -24
    gamma = d * u / (1 - d * u)
    bound = gamma * (np.abs(X) @ np.abs(Wr).T)
    err = np.abs(lg.astype(np.float64) - ref)
    assert np.all(err <= bound), f"logit error {err.max():.3e} over the bound at {np.unravel_index(np.argmax(err - bound), err.shape)}"
    print(f"T={T} E={E} d={d}: logit rel err {oracle.rel_max_err(lg, ref):.2e}", flush=True)
    # selection and gates: the oracle's routing of these fp32 logits
    rid, rg = oracle.route(lg, k)
    assert np.array_equal(ids, rid), np.argwhere(ids != rid)[:5]
    H.check_gates(gates, rg, k)
    assert np.array_equal(counts, np.bincount(rid.ravel(), minlength=E))
    # moe_route on the same logits gives the same bits; so does the launch without logits
    ids2 = torch.empty((T, k), dtype=torch.int32, device=dev)
    g2 = torch.empty((T, k), dtype=torch.float32, device=dev)
    moe.moe_route(torch.from_numpy(lg).to(dev), k, ids2, g2)
    torch.cuda.synchronize()
    assert np.array_equal(ids2.cpu().numpy(), ids) and np.array_equal(g2.cpu().numpy().view(np.uint32), gates.view(np.uint32))
    ids3, gates3, _, _ = run(dev, x, w, k, with_logits=False)
    assert np.array_equal(ids3, ids) and np.array_equal(gates3.view(np.uint32), gates.view(np.uint32))
    if dup:
        for a, b in dup:   # the tied pair: the lower index is chosen first wherever both are
            both = np.isin(ids, [a, b]).sum(axis=1) == 2
            for t in np.nonzero(both)[0]:
                row = ids[t].tolist()
                assert row.index(min(a, b)) < row.index(max(a, b))


def test_route_gemm_empty(dev):
    x = np.zeros((0, 64), np.uint16)
    w = synth.round_to_bf16(np.ones((16, 64), np.float32))
    ids, gates, counts, lg = run(dev, x, w, 2)
    assert counts.tolist() == [0] * 16 and ids.shape == (0, 2)
