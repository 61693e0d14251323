"""GPU check of moe_permute_noalloc, the permutation for callers that cannot allocate: its
scratch is the library's static per-GPU array, not a workspace argument. Its outputs must be
bit-identical to moe_permute's (integer maps, counts, offsets and the x_sorted bytes) on two
calls in a row, the second with a smaller batch, both large enough for the multi-launch path
that uses the scratch, then on a batch small enough for the one-workgroup path."""
import numpy as np
import pytest
import torch

import oracle
import synth
import token_dispatch_expert_amd as moe
from token_dispatch_expert_amd import binding as B
from token_dispatch_expert_amd.binding import layer_buffers

import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return H.require_gpu()


def _permute_both(dev, T, E, k, d, seed):
    cfg = synth.tiny_config(T=T, d=d, E=E, k=k, d_ff=64, act="bf16", w="bf16", zipf_s=1.2, seed=seed)
    logits, x = synth.make_routing_inputs(cfg)
    ids, _ = oracle.route(logits, k)
    ids_d = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).to(dev)
    xd = H.to_dev(x, "bf16", dev)
    outs = []
    for noalloc in (False, True):
        out = layer_buffers(T, E, k, d, torch.bfloat16, device=dev)
        for t in out.values():
            t.fill_(float("nan")) if t.is_floating_point() else t.fill_(-7)
        args = (xd, ids_d, E, out["counts"], out["offsets"], out["sorted_to_flat"], out["flat_to_sorted"],
                out["x_sorted"])
        if noalloc:
            B.moe_permute_noalloc(*args)
        else:
            ws = moe.Workspace(moe.moe_permute_workspace_size(T, E, k), device=dev)
            ws.buf.fill_(0xFF)
            moe.moe_permute(*args, ws)
        torch.cuda.synchronize()
        outs.append({n: H.to_host(out[n]) for n in ("counts", "offsets", "sorted_to_flat",
                                                      "flat_to_sorted", "x_sorted")})
    ref = oracle.permute(ids, E)
    for n in ("counts", "offsets", "sorted_to_flat", "flat_to_sorted"):
        assert np.array_equal(outs[0][n], ref[n]), n
    for n in outs[0]:
        assert np.array_equal(outs[1][n], outs[0][n]), f"{n} differs between moe_permute_noalloc and moe_permute"
    print(f"noalloc permute T={T} E={E} k={k}: identical to moe_permute", flush=True)


def test_noalloc_permute_matches_workspace_permute(dev):
    # 1,000,000 assignments over 256 experts: 3,907 tiles x 256 experts, 3.8 MiB of the 4 MiB
    _permute_both(dev, T=125000, E=256, k=8, d=64, seed=1)
    # a smaller batch right after: the scratch keeps the first call's larger contents
    _permute_both(dev, T=1500, E=300, k=7, d=128, seed=2)
    # one workgroup path (no scratch)
    _permute_both(dev, T=300, E=64, k=4, d=64, seed=3)


def test_noalloc_permute_rejects_sizes_beyond_its_scratch(dev):
    T, E, k, d = (1 << 20) // 8 + 32, 256, 8, 8   # 4,097 tiles x 256 experts: just over 4 MiB
    assert moe.moe_permute_workspace_size(T, E, k) > B.PERMUTE_NOALLOC_SCRATCH_BYTES
    ids = torch.zeros((T, k), dtype=torch.int32, device=dev)
    x = torch.zeros((T, d), dtype=torch.bfloat16, device=dev)
    out = layer_buffers(T, E, k, d, torch.bfloat16, device=dev)
    with pytest.raises(B.MoeError) as ei:
        B.moe_permute_noalloc(x, ids, E, out["counts"], out["offsets"], out["sorted_to_flat"],
                              out["flat_to_sorted"], out["x_sorted"])
    assert ei.value.status == B.MOE_ERR_WORKSPACE
