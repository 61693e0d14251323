"""moe_layer captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library enqueues only kernels (no allocation, no memset, no synchronisation): on the
caller's stream, and for prefill-sized bf16 layers also on a second stream forked from it and
joined back with events, which a capture records as a branch of the graph. So a whole layer can
be captured once and replayed, which removes the host launch cost from decode steps. Each replay is checked bit for bit against the eager call on the
same inputs, with the outputs poisoned and other eager work on the device between replays."""
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


def _layer_fn(cfg, dev):
    logits, x = synth.make_routing_inputs(cfg)
    ids, _ = oracle.route(logits, cfg.k)
    W = H.DeviceWeights(cfg, dev, experts=H.active_experts(np.bincount(ids.ravel(), minlength=cfg.E)))
    lg = torch.from_numpy(logits).to(dev)
    xd = H.to_dev(x, cfg.act, dev)
    out = layer_buffers(cfg.T, cfg.E, cfg.k, cfg.d, H.ACT_TORCH[cfg.act], device=dev)
    ws = moe.Workspace(moe.moe_layer_workspace_size(cfg.T, cfg.E, cfg.k, cfg.d, cfg.d_ff,
                                                    H.ACT_TORCH[cfg.act], H.W_TORCH[cfg.w]), device=dev)
    skw = W.scales or {}

    def fn():
        moe.moe_layer(lg, xd, W.gate, W.up, W.down, cfg.k, out, ws, **skw)
    return fn, out


def _poison(out):
    for t in out.values():
        if t.is_floating_point():
            t.fill_(float("nan"))
        else:
            t.fill_(-7)


@pytest.mark.parametrize("cfg", [
    synth.CONFIGS["c2"],                                                   # decode: route, small permute, split-free tiles
    synth.tiny_config(T=5, d=1024, E=16, k=2, d_ff=512, act="bf16", w="bf16", zipf_s=1.0, seed=21),  # contraction split
    synth.tiny_config(T=700, d=192, E=40, k=2, d_ff=320, act="bf16", w="bf16", zipf_s=1.5, seed=13),  # prefill kernel, tail split
    # prefill kernel with the small experts on the second stream (the fork and join are captured;
    # the capture stream gets its own second stream, created during the capture)
    synth.tiny_config(T=4096, d=512, E=128, k=4, d_ff=384, act="bf16", w="bf16", zipf_s=2.0, seed=17),
    synth.tiny_config(T=128, d=512, E=64, k=4, d_ff=384, act="bf16", w="fp8_e4m3fn", zipf_s=1.0, seed=21),  # fp8 decode tiles
    synth.tiny_config(T=256, d=512, E=64, k=4, d_ff=384, act="bf16", w="fp8_e4m3fn", zipf_s=1.0, seed=21),  # fp8 prefill kernel
], ids=["c2", "decode-split", "prefill", "prefill-second-stream", "fp8-decode", "fp8-prefill"])
def test_layer_graph_replay_matches_eager(dev, cfg):
    fn, out = _layer_fn(cfg, dev)
    # every eager call runs on the stream the graph is captured on: the library keys its second
    # stream by the caller's stream, so eager calls and the capture take the same schedule
    s = torch.cuda.Stream()

    def eager():
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()

    eager()
    ref = {k: v.clone() for k, v in out.items()}
    # a second eager call gives the same bits (the reference is stable)
    _poison(out)
    eager()
    for k in out:
        assert torch.equal(out[k].view(torch.uint8), ref[k].view(torch.uint8)), k

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()

    other_fn, other_out = _layer_fn(synth.CONFIGS["c1"], dev)
    for rep in range(4):
        _poison(out)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in out:
            assert torch.equal(out[k].view(torch.uint8), ref[k].view(torch.uint8)), (rep, k)
        # unrelated eager work on the device between replays
        other_fn()
        torch.cuda.synchronize()
