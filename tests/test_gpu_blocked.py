"""Weights in the blocked layouts (8 rows x 128 bytes per block: 64 bf16 or 128 fp8 elements).

moe_block_weights is checked against the layouts' definition (a numpy reshape and transpose),
and whole layers with blocked weights against the same layers with row-major weights: where the
same kernels run, the arithmetic is the same, so every output must be bit-identical, on every
kernel path that reads bf16 weights (decode-sized tiles, their contraction split, the prefill
kernel's large tiles and streaming role, and the lean kernel on the second stream) and fp8
weights (decode-sized and prefill tiles), and the full-size c3-c5 layers as the benchmark
times them. The smallest fp8 launches, whose row-major weights stream their few-row experts on
another kernel (another summation order), are checked against the fp64 oracle."""
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


def _blocked_reference(w: np.ndarray, B: int) -> np.ndarray:
    """[E, N, K] -> [E][N/8][K/B][8][B], flattened back to [E, N, K] storage."""
    E, N, K = w.shape
    return w.reshape(E, N // 8, 8, K // B, B).transpose(0, 1, 3, 2, 4).reshape(E, N, K)


def test_block_weights_layout(dev):
    rng = np.random.default_rng(3)
    for E, N, K in ((1, 8, 64), (3, 24, 192), (2, 136, 320)):
        bits = rng.integers(0, 1 << 16, size=(E, N, K), dtype=np.uint16)
        src = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
        dst = torch.full_like(src, float("nan"))
        moe.moe_block_weights(src, dst)
        torch.cuda.synchronize()
        got = dst.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, _blocked_reference(bits, 64)), (E, N, K)
    for E, N, K in ((1, 8, 128), (3, 24, 384), (2, 136, 640)):
        codes = rng.integers(0, 256, size=(E, N, K), dtype=np.uint8)
        src = torch.from_numpy(codes).to(dev).view(torch.float8_e4m3fn)
        dst = torch.zeros_like(src.view(torch.uint8)).view(torch.float8_e4m3fn)
        moe.moe_block_weights(src, dst)
        torch.cuda.synchronize()
        got = dst.view(torch.uint8).cpu().numpy()
        assert np.array_equal(got, _blocked_reference(codes, 128)), (E, N, K)


def test_block_weights_beyond_2g_elements(dev):
    # a whole [E, N, K] tensor of more than 2^31 elements (the DeepSeek-V3 expert shape): every
    # element checked by the index formula at sampled positions and over the last block
    E, N, K = 147, 2048, 7168
    assert E * N * K > 2 ** 31
    g = torch.Generator(device=dev).manual_seed(5)
    src = torch.randint(-32768, 32767, (E, N, K), dtype=torch.int16, device=dev, generator=g)
    dst = torch.empty_like(src)
    moe.moe_block_weights(src.view(torch.bfloat16), dst.view(torch.bfloat16))
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    e = torch.from_numpy(rng.integers(0, E, 4096)).to(dev)
    n = torch.from_numpy(rng.integers(0, N, 4096)).to(dev)
    k = torch.from_numpy(rng.integers(0, K, 4096)).to(dev)
    e = torch.cat([e, torch.full((512,), E - 1, device=dev)])
    n = torch.cat([n, (N - 8 + torch.arange(512, device=dev) // 64)])
    k = torch.cat([k, (K - 64 + torch.arange(512, device=dev) % 64)])
    pos = ((e * (N // 8) + n // 8) * (K // 64) + k // 64) * 512 + (n % 8) * 64 + k % 64
    assert torch.equal(dst.view(-1)[pos], src[e, n, k])
    del src, dst


def test_block_weights_beyond_2p32_pieces(dev):
    # a tensor of more 16-byte pieces than one dispatch has threads (2^32): 2,400 experts of
    # 2048 x 7168 bf16, 70.5 GB each for source and destination
    E, N, K = 2400, 2048, 7168
    assert E * N * K * 2 // 16 > 2 ** 32
    need = 2 * E * N * K * 2
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info(dev)
    if free < need + (8 << 30):
        pytest.skip(f"needs {need / 2**30:.0f} GiB of free device memory, {free / 2**30:.0f} GiB free")
    src = torch.empty((E, N, K), dtype=torch.int16, device=dev)
    g = torch.Generator(device=dev).manual_seed(8)
    for e0 in range(0, E, 200):
        src[e0:e0 + 200].random_(-32768, 32767, generator=g)
    dst = torch.empty_like(src)
    moe.moe_block_weights(src.view(torch.bfloat16), dst.view(torch.bfloat16))
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    e = torch.from_numpy(rng.integers(0, E, 8192)).to(dev)
    n = torch.from_numpy(rng.integers(0, N, 8192)).to(dev)
    k = torch.from_numpy(rng.integers(0, K, 8192)).to(dev)
    # every element of the last block, and of the first block past 2^32 pieces (2^36 bytes)
    first = (2 ** 36) // 2 // 512 * 512                 # an element index at a block start
    blk = first // 512
    kb = blk % (K // 64); nb = blk // (K // 64) % (N // 8); eb = blk // (K // 64) // (N // 8)
    idx = torch.arange(512, device=dev)
    e = torch.cat([e, torch.full((512,), E - 1, device=dev), torch.full((512,), eb, device=dev)])
    n = torch.cat([n, N - 8 + idx // 64, nb * 8 + idx // 64])
    k = torch.cat([k, K - 64 + idx % 64, kb * 64 + idx % 64])
    pos = ((e * (N // 8) + n // 8) * (K // 64) + k // 64) * 512 + (n % 8) * 64 + k % 64
    assert int(pos.max()) == E * N * K - 1
    assert torch.equal(dst.view(-1)[pos], src[e, n, k])
    del src, dst
    torch.cuda.empty_cache()


def _run(cfg, dev, W, blocked):
    logits, x = synth.make_routing_inputs(cfg)
    lg = torch.from_numpy(logits).to(dev)
    xd = H.to_dev(x, cfg.act, dev)
    out = layer_buffers(cfg.T, cfg.E, cfg.k, cfg.d, torch.bfloat16, device=dev)
    ws = moe.Workspace(moe.moe_layer_workspace_size(cfg.T, cfg.E, cfg.k, cfg.d, cfg.d_ff,
                                                    torch.bfloat16, H.W_TORCH[cfg.w]), device=dev)
    for t in out.values():
        t.fill_(float("nan")) if t.is_floating_point() else t.fill_(-7)
    ws.buf.fill_(0xFF)
    gate, up, down, skw = W
    moe.moe_layer(lg, xd, gate, up, down, cfg.k, out, ws, weights_blocked=blocked, **skw)
    torch.cuda.synchronize()
    return {n: t.cpu() for n, t in out.items()}


@pytest.mark.parametrize("cfg", [
    synth.CONFIGS["c2"],                                                             # decode tiles
    synth.tiny_config(T=5, d=1024, E=16, k=2, d_ff=512, act="bf16", w="bf16", zipf_s=1.0, seed=21),   # split
    synth.tiny_config(T=700, d=192, E=40, k=2, d_ff=320, act="bf16", w="bf16", zipf_s=1.5, seed=13),  # prefill
    synth.tiny_config(T=4096, d=512, E=128, k=4, d_ff=384, act="bf16", w="bf16", zipf_s=0.9, seed=17),  # streaming role
    synth.tiny_config(T=4096, d=512, E=128, k=4, d_ff=384, act="bf16", w="bf16", zipf_s=2.0, seed=17),  # lean kernel
    synth.tiny_config(T=128, d=512, E=64, k=4, d_ff=384, act="bf16", w="fp8_e4m3fn", zipf_s=1.0, seed=21),  # fp8 decode
    synth.tiny_config(T=256, d=512, E=64, k=4, d_ff=384, act="bf16", w="fp8_e4m3fn", zipf_s=1.0, seed=21),  # fp8 prefill
], ids=["c2", "decode-split", "prefill", "prefill-streaming-role", "prefill-second-stream",
        "fp8-decode", "fp8-prefill"])
def test_blocked_layer_matches_row_major(dev, cfg):
    W, blocked = _weights_both(cfg, dev)
    ref = _run(cfg, dev, (W.gate, W.up, W.down, W.kwargs()), False)
    got = _run(cfg, dev, blocked, True)
    assert bool(torch.isfinite(ref["y"]).all())
    for n in ref:
        assert torch.equal(got[n].view(torch.uint8), ref[n].view(torch.uint8)), n


def _weights_both(cfg, dev):
    logits, _ = synth.make_routing_inputs(cfg)
    ids, _ = oracle.route(logits, cfg.k)
    W = H.DeviceWeights(cfg, dev, experts=H.active_experts(np.bincount(ids.ravel(), minlength=cfg.E)))
    blocked = []
    for w in (W.gate, W.up, W.down):
        b = torch.empty_like(w)
        moe.moe_block_weights(w, b)
        blocked.append(b)
    return W, (*blocked, W.kwargs())


def test_blocked_fp8_smallest_launch_against_oracle(dev):
    # a decode step of 5 tokens: with row-major fp8 weights the few-row experts stream on the
    # kernel that splits each item's contraction over its waves; blocked weights take the tiles
    cfg = synth.tiny_config(T=5, d=1024, E=16, k=2, d_ff=512, act="bf16", w="fp8_e4m3fn",
                            zipf_s=1.0, seed=21)
    W, blocked = _weights_both(cfg, dev)
    logits, x = synth.make_routing_inputs(cfg)
    got = _run(cfg, dev, blocked, True)
    ref = oracle.layer(logits, x, cfg.act, W.raw, cfg.w, cfg.k)
    assert np.array_equal(got["topk_ids"].numpy(), ref["topk_ids"])
    assert np.array_equal(got["offsets"].numpy(), ref["offsets"])
    err = oracle.rel_max_err(got["y"].numpy(), ref["y"])
    assert err <= H.TOL["fp8_e4m3fn"], err


def _device_weights(cfg, dev, seed=0):
    """Seeded weights drawn on the device for all E experts (no host copies: this comparison
    needs no oracle), in the row-major layout, and their blocked copies."""
    g = torch.Generator(device=dev).manual_seed(seed)
    fp8 = cfg.w == "fp8_e4m3fn"

    def mat(N, K):
        out = torch.empty((cfg.E, N, K), dtype=torch.float8_e4m3fn if fp8 else torch.bfloat16, device=dev)
        for e0 in range(0, cfg.E, 32):
            w = torch.randn((min(32, cfg.E - e0), N, K), generator=g, device=dev)
            out[e0:e0 + 32] = w.mul_(64.0).clamp_(-448, 448).to(out.dtype) if fp8 else w.div_(K ** 0.5).to(out.dtype)
        return out

    W = [mat(cfg.d_ff, cfg.d), mat(cfg.d_ff, cfg.d), mat(cfg.d, cfg.d_ff)]
    skw = {}
    if fp8:
        for n, (N, K) in zip(("s_gate", "s_up", "s_down"), ((cfg.d_ff, cfg.d), (cfg.d_ff, cfg.d), (cfg.d, cfg.d_ff))):
            skw[n] = torch.rand((cfg.E, N // 128, K // 128), generator=g, device=dev).add_(0.5).div_(64 * K ** 0.5)
    blocked = []
    for w in W:
        b = torch.empty_like(w)
        moe.moe_block_weights(w, b)
        blocked.append(b)
    torch.cuda.synchronize()
    return (*W, skw), (*blocked, skw)


@pytest.mark.parametrize("name", ["c3", "c4", "c5"])
def test_blocked_full_size_matches_row_major(dev, name):
    # the full-size decode (c3) and prefill layers in the configuration the benchmark times (blocked weights):
    # every output bit-identical to the same layer with row-major weights, whose parity against
    # the oracle the full-size sampled tests check
    cfg = synth.CONFIGS[name]
    row_major, blocked = _device_weights(cfg, dev)
    ref = _run(cfg, dev, row_major, False)
    got = _run(cfg, dev, blocked, True)
    assert bool(torch.isfinite(ref["y"]).all())
    for n in ref:
        assert torch.equal(got[n].view(torch.uint8), ref[n].view(torch.uint8)), n
    del row_major, blocked
    torch.cuda.empty_cache()
