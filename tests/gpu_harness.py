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


def run_layer(cfg: synth.Config, logits: np.ndarray, x: np.ndarray, W: DeviceWeights, dev,
              h_rows=None):
    """moe_layer on the device; returns every output on the host. h_rows (optional, bf16
    activations): sorted rows whose h (the bf16 SwiGLU activations between the two GEMMs) is
    also returned, as bf16 bits under the key "h". h is read from the workspace, where the
    header places it: the grouped FFN's workspace follows the permutation's, and h
    [T*k, d_ff] opens it."""
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
    got = {n: to_host(t) for n, t in out.items()}
    if h_rows is not None:
        assert cfg.act == "bf16"
        off = moe.moe_permute_workspace_size(cfg.T, cfg.E, cfg.k)
        R = cfg.T * cfg.k
        h = ws.buf[off:off + R * cfg.d_ff * 2].view(torch.int16).view(R, cfg.d_ff)
        idx = torch.as_tensor(np.asarray(h_rows, np.int64), device=dev)
        got["h"] = h.index_select(0, idx).cpu().numpy().view(np.uint16)
    return got


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


def sampled_reference(toks, ids, gates, x, cfg, W, h_gpu=None):
    """The oracle on the listed tokens only, decoding every expert's weights once. Returns a
    dict with
      y, rows        : y [len(toks), d] and {(t, j): y_sorted row} of the plain fp64 oracle;
      y_bf16h, rows_bf16h : the same with h rounded to bf16 between the GEMMs (rounding point);
      h64            : {(t, j): the slot's fp64 h row};
    and, when h_gpu ({(t, j): the implementation's bf16 h row, as bits}) is given,
      y_gpu_h, rows_gpu_h : the down projection and combine applied to those h rows."""
    k = cfg.k
    X = oracle.decode_activations(np.asarray(x)[toks], cfg.act)
    by_expert = {}
    for ti, t in enumerate(toks):
        for j in range(k):
            by_expert.setdefault(int(ids[t, j]), []).append((ti, j))
    dec = oracle.make_weight_decoder(W.raw, cfg.w)
    modes = ["plain", "bf16h"] + (["gpu_h"] if h_gpu is not None else [])
    ys = {m: np.zeros((len(toks) * k, cfg.d)) for m in modes}
    h64 = {}
    for e, items in sorted(by_expert.items()):
        Wg, Wu, Wd = dec(e)
        Xe = X[[ti for ti, _ in items]]
        Y, H64 = oracle.expert_ffn(Xe, Wg, Wu, Wd, return_h=True)
        Yr = oracle.expert_ffn(Xe, Wg, Wu, Wd, h_round="bf16")
        Yg = None
        if h_gpu is not None:
            Hg = oracle.decode_bf16(np.stack([h_gpu[(toks[ti], j)] for ti, j in items]))
            Yg = oracle.expert_down(Hg, Wd)
        for n, (ti, j) in enumerate(items):
            ys["plain"][ti * k + j] = Y[n]
            ys["bf16h"][ti * k + j] = Yr[n]
            if Yg is not None:
                ys["gpu_h"][ti * k + j] = Yg[n]
            h64[(toks[ti], j)] = H64[n]
    f2s = np.arange(len(toks) * k, dtype=np.int32)
    out = {"h64": h64}
    for m, suffix in (("plain", ""), ("bf16h", "_bf16h"), ("gpu_h", "_gpu_h")):
        if m not in ys:
            continue
        out["y" + suffix] = oracle.combine(ys[m], f2s, np.asarray(gates)[toks])
        out["rows" + suffix] = {(t, j): ys[m][ti * k + j] for ti, t in enumerate(toks) for j in range(k)}
    return out


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values (8 significant bits) at the magnitude of each fp64 value."""
    _, e = np.frexp(np.asarray(v, np.float64))  # v = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(1.0, e - 8)


def check_h_rounding_point(h_gpu_bits: np.ndarray, h64: np.ndarray, name: str):
    """The implementation's bf16 h against the fp64 h: every element within one bf16 unit of the
    fp64 value (round to nearest of the fp32 result) plus an absolute allowance of 1e-4 rms(h)
    for the fp32 accumulation of dot products that cancel to near zero, and at least 99% of the
    elements exactly the nearest bf16 of the fp64 value."""
    hg = oracle.decode_bf16(h_gpu_bits)
    err = np.abs(hg - h64)
    rms = float(np.sqrt(np.mean(h64 * h64)))
    bound = bf16_ulp(h64) + 1e-4 * rms
    worst = float(np.max(err / bound))
    exact = float(np.mean(hg == oracle.round_bf16_value(h64)))
    print(f"{name}: h vs fp64 h: worst |err| / (1 bf16 unit + 1e-4 rms) = {worst:.3f}; "
          f"{exact:.5%} exactly the nearest bf16", flush=True)
    assert worst <= 1.0, f"h element off by more than one bf16 unit ({worst:.3f} of the bound)"
    assert exact >= 0.99, f"only {exact:.3%} of h elements are the nearest bf16 of the fp64 value"
