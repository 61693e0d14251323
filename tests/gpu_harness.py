"""Shared helpers for the GPU parity tests: moving synthetic inputs to the device in their
stored formats, running the layer through the C ABI, and comparing with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
import token_dispatch_expert_amd as moe
from token_dispatch_expert_amd.binding import layer_buffers

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8_e4m3fn": 5e-2}
# Second, tighter bar for bf16 activations: against the oracle with h rounded to bf16 between
# the GEMMs (the implementation's documented rounding point). What remains is fp32 accumulation
# order and the rare h element whose fp32 and fp64 values round to different bf16 neighbours.
TOL_ROUNDING_POINT = 5e-3
ACT_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}
W_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3fn": torch.float8_e4m3fn}


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need an MI355X: torch.cuda.is_available() is False")
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, fmt: str, dev) -> torch.Tensor:
    if fmt == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    if fmt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    if fmt == "fp8_e4m3fn":
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev).view(torch.float8_e4m3fn)
    raise ValueError(fmt)


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


class DeviceWeights:
    """Expert weights on the device: experts in `experts` hold their seeded values, every other
    expert a NaN canary (so an expert read by mistake poisons the output). Host copies of the
    generated experts are kept for the oracle."""

    def __init__(self, cfg: synth.Config, dev, experts=None):
        self.cfg = cfg
        E, d, d_ff = cfg.E, cfg.d, cfg.d_ff
        wt = W_TORCH[cfg.w]
        nan_bits = {"f32": None, "bf16": int(synth.BF16_NAN), "fp8_e4m3fn": int(synth.FP8_NAN)}[cfg.w]

        def canary(shape):
            if cfg.w == "f32":
                return torch.full(shape, float("nan"), dtype=torch.float32, device=dev)
            if cfg.w == "bf16":
                return torch.full(shape, nan_bits, dtype=torch.int16, device=dev).view(torch.bfloat16)
            return torch.full(shape, nan_bits, dtype=torch.uint8, device=dev).view(torch.float8_e4m3fn)

        self.gate = canary((E, d_ff, d))
        self.up = canary((E, d_ff, d))
        self.down = canary((E, d, d_ff))
        self.scales = None
        if cfg.w == "fp8_e4m3fn":
            self.scales = dict(
                s_gate=torch.full((E, d_ff // 128, d // 128), float("nan"), device=dev),
                s_up=torch.full((E, d_ff // 128, d // 128), float("nan"), device=dev),
                s_down=torch.full((E, d // 128, d_ff // 128), float("nan"), device=dev))
        self.host = {}
        experts = range(E) if experts is None else sorted(experts)
        assert wt == self.gate.dtype
        for e, w in synth.iter_expert_weights(cfg, experts):
            self.host[e] = w
            self.gate[e].copy_(to_dev(w["gate"], cfg.w, dev))
            self.up[e].copy_(to_dev(w["up"], cfg.w, dev))
            self.down[e].copy_(to_dev(w["down"], cfg.w, dev))
            if self.scales is not None:
                for n in ("gate", "up", "down"):
                    self.scales["s_" + n][e].copy_(torch.from_numpy(w[n + "_scale"]).to(dev))
        torch.cuda.synchronize()

    def raw(self, e):
        return self.host[e]

    def kwargs(self):
        return dict(self.scales) if self.scales is not None else {}


def run_layer(cfg: synth.Config, logits: np.ndarray, x: np.ndarray, W: DeviceWeights, dev):
    lg = torch.from_numpy(logits).to(dev)
    xd = to_dev(x, cfg.act, dev)
    out = layer_buffers(cfg.T, cfg.E, cfg.k, cfg.d, ACT_TORCH[cfg.act], device=dev)
    ws = moe.Workspace(moe.moe_layer_workspace_size(cfg.T, cfg.E, cfg.k, cfg.d, cfg.d_ff,
                                                    ACT_TORCH[cfg.act], W_TORCH[cfg.w]), device=dev)
    # poison every output and the workspace: fresh allocations often reuse the blocks of the
    # previous run, whose values an unwritten output would otherwise inherit (and a repeat
    # comparison would then pass); the library must not rely on a cleared workspace either
    for t in out.values():
        t.fill_(float("nan")) if t.is_floating_point() else t.fill_(-7)
    ws.buf.fill_(0xFF)
    moe.moe_layer(lg, xd, W.gate, W.up, W.down, cfg.k, out, ws, **W.kwargs())
    torch.cuda.synchronize()
    return {n: to_host(t) for n, t in out.items()}


def check_routing_exact(got: dict, ref: dict, E: int):
    """ids, counts, offsets, both maps: bit-exact."""
    for n in ("topk_ids", "counts", "offsets", "sorted_to_flat", "flat_to_sorted"):
        g, r = np.asarray(got[n]), np.asarray(ref[n])
        assert g.shape == r.shape, n
        if not np.array_equal(g, r):
            bad = np.argwhere(g != r)[:5]
            raise AssertionError(f"{n} differs at {bad.tolist()}")


def check_gates(got_gates: np.ndarray, ref_gates: np.ndarray, k: int):
    err = oracle.rel_max_err(got_gates, ref_gates)
    assert err <= 1e-5, f"gate error {err:.3e}"
    s = got_gates.astype(np.float64).sum(axis=1)
    assert np.max(np.abs(s - 1.0)) <= k * 2.0 ** -23, np.max(np.abs(s - 1.0))


def active_experts(ref_counts: np.ndarray):
    return [int(e) for e in np.nonzero(ref_counts)[0]]


def covering_tokens(cfg, perm, n_random, seed=0, block=128, small=16):
    """Tokens whose rows reach every kernel role and every output tile of the full-size layer:
    n_random seeded tokens, plus the owners of every expert's first and last sorted row, of the
    first row of each of its 128-row blocks (so every row tile of 128 or 256 rows, the
    last-round split tiles included, holds a checked row; a y_sorted row spans every column
    tile of both GEMMs) and of every row of the experts with at most `small` rows (the
    streaming role's 16-row tiles)."""
    rng = np.random.default_rng(seed)
    toks = set(rng.choice(cfg.T, size=n_random, replace=False).tolist())
    off, s2f = perm["offsets"], perm["sorted_to_flat"]
    for e in range(cfg.E):
        a, b = int(off[e]), int(off[e + 1])
        if b == a:
            continue
        rows = range(a, b) if b - a <= small else list(range(a, b, block)) + [b - 1]
        toks.update(int(s2f[r]) // cfg.k for r in rows)
    return sorted(toks)


def sampled_reference(toks, ids, gates, x, cfg, W, h_rounds=(None, "bf16")):
    """The oracle's y rows and per-slot expert outputs for the listed tokens, for each h
    rounding in h_rounds, decoding every expert's weights once (oracle.layer_tokens per
    rounding would decode them twice). Returns {h_round: (y [len(toks), d], {(t, j): row})}."""
    k = cfg.k
    X = oracle.decode_activations(np.asarray(x)[toks], cfg.act)
    by_expert = {}
    for ti, t in enumerate(toks):
        for j in range(k):
            by_expert.setdefault(int(ids[t, j]), []).append((ti, j))
    dec = oracle.make_weight_decoder(W.raw, cfg.w)
    out = {}
    ys = {hr: np.zeros((len(toks) * k, cfg.d)) for hr in h_rounds}
    for e, items in sorted(by_expert.items()):
        Wg, Wu, Wd = dec(e)
        Xe = X[[ti for ti, _ in items]]
        for hr in h_rounds:
            Y = oracle.expert_ffn(Xe, Wg, Wu, Wd, h_round=hr)
            for (ti, j), yr in zip(items, Y):
                ys[hr][ti * k + j] = yr
    f2s = np.arange(len(toks) * k, dtype=np.int32)
    for hr in h_rounds:
        y = oracle.combine(ys[hr], f2s, np.asarray(gates)[toks])
        rows = {(t, j): ys[hr][ti * k + j] for ti, t in enumerate(toks) for j in range(k)}
        out[hr] = (y, rows)
    return out
