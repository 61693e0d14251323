"""Seeded synthetic inputs for the MoE layer (shared by the HIP path's tests/bench and the oracle).

This module holds *input preparation only*: random draws, rounding of fp32 draws to the
stored formats (bf16 round-to-nearest-even, fp8 e4m3fn block quantisation) and the workload
table. It contains none of the layer's arithmetic (no top-k, gating, sorting, FFN or combine),
and imports nothing from the oracle or from the HIP package.

Workloads (the synthetic stand-ins for the recorded routing that the expert-parallelism pages
measure on; shapes after the DeepSeek-V3 / Qwen3-235B MoE layers those pages discuss):

    name  T     d     E    k  d_ff  activations  weights              logit bias
    c1    64    128   8    2  256   fp32         fp32                 none
    c2    128   4096  128  8  1536  bf16         bf16                 Zipf s=1.2
    c3    256   7168  256  8  2048  bf16         bf16                 Zipf s=1.0
    c4    8192  7168  256  8  2048  bf16         bf16                 Zipf s=1.2
    c5    4096  7168  256  8  2048  bf16         fp8 e4m3fn + fp32    Zipf s=1.5
                                                 per-128x128 scales

Value recipe (seed 0 unless stated):
  * one main PCG64 stream (SeedSequence([seed, 0])) draws, in this order: a random expert
    ranking (a permutation of E; only when a bias is used), the logits' N(0,1) part [T, E]
    in fp64, and x ~ N(0,1) [T, d] in fp32;
  * logits = fp32(N(0,1) + b_e) with b_e = -s * ln(rank_e), rank_e = 1 + position of e in the
    ranking, so expert popularity follows a Zipf-like law of exponent s;
  * expert weights come from one PCG64 stream per (seed, matrix, expert)
    (SeedSequence([seed, 1 + matrix, e]), matrix 0 = gate, 1 = up, 2 = down), so any expert
    can be regenerated alone: fp32 N(0,1) scaled by 1/sqrt(d) (gate, up) or 1/sqrt(d_ff)
    (down), then rounded to the stored format.

Storage layout (the layout the C ABI takes): every weight matrix is stored with its
contraction axis contiguous, i.e. as the transpose of the math-side matrix:
  gate, up : [E, d_ff, d]   (row n holds the d inputs of output feature n)
  down     : [E, d, d_ff]
fp8 scales tile each stored matrix in 128x128 blocks: gate/up scales [E, d_ff/128, d/128],
down scales [E, d/128, d_ff/128]; scale = amax(|block|)/448 (1.0 for an all-zero block),
code = round-to-nearest-even(W/scale) in OCP e4m3fn, saturating at 448.

Formats in the returned arrays: fp32 as float32; bf16 as uint16 bit patterns; fp8 as uint8
e4m3fn codes.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

F32, BF16, FP8 = "f32", "bf16", "fp8_e4m3fn"

# bf16 bit pattern of a quiet NaN: used as a canary for experts a test leaves unset.
BF16_NAN = np.uint16(0x7FC0)
FP8_NAN = np.uint8(0x7F)


@dataclass(frozen=True)
class Config:
    name: str
    T: int
    d: int
    E: int
    k: int
    d_ff: int
    act: str
    w: str
    zipf_s: float | None
    seed: int = 0
    note: str = ""

    @property
    def rows(self) -> int:
        return self.T * self.k

    def with_(self, **kw) -> "Config":
        f = dict(self.__dict__)
        f.update(kw)
        return Config(**f)


CONFIGS = {
    "c1": Config("c1", 64, 128, 8, 2, 256, F32, F32, None,
                 note="tiny fp32 MoE layer"),
    "c2": Config("c2", 128, 4096, 128, 8, 1536, BF16, BF16, 1.2,
                 note="decode-shape Qwen3-235B-like MoE layer"),
    "c3": Config("c3", 256, 7168, 256, 8, 2048, BF16, BF16, 1.0,
                 note="mixed-regime DeepSeek-V3-shaped decode MoE layer"),
    "c4": Config("c4", 8192, 7168, 256, 8, 2048, BF16, BF16, 1.2,
                 note="prefill DeepSeek-V3-shaped MoE layer"),
    "c5": Config("c5", 4096, 7168, 256, 8, 2048, BF16, FP8, 1.5,
                 note="extreme-skew fp8-weight DeepSeek-V3-shaped MoE layer"),
}


# ----------------------------------------------------------------------------------------
# format rounding (input preparation)
# ----------------------------------------------------------------------------------------
def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round-to-nearest-even (inputs are finite)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _e4m3fn_table() -> np.ndarray:
    """Magnitudes of the 127 finite non-negative e4m3fn codes 0x00..0x7E (1 sign, 4 exponent
    bits with bias 7, 3 mantissa bits; exponent field 0 is subnormal; 0x7F is NaN)."""
    v = np.empty(127, dtype=np.float64)
    for c in range(127):
        e, m = c >> 3, c & 7
        v[c] = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return v


_E4M3_MAG = _e4m3fn_table()


def quantize_e4m3fn_table(v: np.ndarray) -> np.ndarray:
    """Round fp32 values to OCP e4m3fn codes by search over the code table: nearest finite
    value, ties to the even code, saturating at +-448 (slow; the cross-check of the fast
    version below)."""
    a = np.abs(v.astype(np.float64))
    idx = np.searchsorted(_E4M3_MAG, a, side="left")
    hi = np.minimum(idx, 126)
    lo = np.maximum(idx - 1, 0)
    dhi = np.abs(_E4M3_MAG[hi] - a)
    dlo = np.abs(a - _E4M3_MAG[lo])
    pick_lo = (dlo < dhi) | ((dlo == dhi) & ((lo & 1) == 0))
    code = np.where(pick_lo, lo, hi).astype(np.uint8)
    code = np.where(a >= 448.0, np.uint8(126), code)
    return (code | (np.signbit(v).astype(np.uint8) << np.uint8(7))).astype(np.uint8)


def quantize_e4m3fn(v: np.ndarray) -> np.ndarray:
    """Round fp32 values to OCP e4m3fn codes (round-to-nearest-even, saturating at +-448).

    Normal range (|v| >= 2^-6): round the fp32 significand to 3 bits (add 0x7FFFF plus the
    kept LSB, truncate) and rebias the exponent from 127 to 7. Subnormal range: multiples of
    2^-9, rounded half-to-even. Results above 448 saturate to code 0x7E."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v)
    u = a.view(np.uint32)
    r = (u + np.uint32(0x7FFFF) + ((u >> np.uint32(20)) & np.uint32(1))) & np.uint32(0xFFF00000)
    code_n = (((r >> np.uint32(23)).astype(np.int32) - 120) << 3) | ((r >> np.uint32(20)) & np.uint32(7)).astype(np.int32)
    code_s = np.rint(a.astype(np.float64) * 512.0).astype(np.int32)
    code = np.minimum(np.where(a < np.float32(2.0 ** -6), code_s, code_n), 126)
    return code.astype(np.uint8) | (np.signbit(v).astype(np.uint8) << np.uint8(7))


def quantize_blocks_e4m3fn(w: np.ndarray, block: int = 128):
    """Per-(block x block) quantisation of a stored fp32 matrix [N, K] -> (codes u8 [N, K],
    scales f32 [ceil(N/block), ceil(K/block)]); scale = amax/448 (1.0 for an all-zero block)."""
    n, kk = w.shape
    nb, kb = -(-n // block), -(-kk // block)
    wp = np.zeros((nb * block, kb * block), dtype=np.float32)
    wp[:n, :kk] = w
    blocks = wp.reshape(nb, block, kb, block)
    amax = np.max(np.abs(blocks), axis=(1, 3)).astype(np.float32)
    scales = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = quantize_e4m3fn((blocks / scales[:, None, :, None]).astype(np.float32))
    return np.ascontiguousarray(q.reshape(nb * block, kb * block)[:n, :kk]), scales


# ----------------------------------------------------------------------------------------
# draws
# ----------------------------------------------------------------------------------------
def _main_rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0])))


def expert_bias(cfg: Config, rng: np.random.Generator | None = None) -> np.ndarray:
    """Per-expert logit bias -s*ln(rank) over a random ranking (zeros when no bias)."""
    if cfg.zipf_s is None:
        return np.zeros(cfg.E)
    rng = rng or _main_rng(cfg.seed)
    perm = rng.permutation(cfg.E)
    rank = np.empty(cfg.E, dtype=np.int64)
    rank[perm] = np.arange(1, cfg.E + 1)
    return -cfg.zipf_s * np.log(rank.astype(np.float64))


def make_routing_inputs(cfg: Config):
    """(logits f32 [T, E], x [T, d] in the activation format)."""
    rng = _main_rng(cfg.seed)
    bias = expert_bias(cfg, rng)
    logits = (rng.standard_normal((cfg.T, cfg.E)) + bias[None, :]).astype(np.float32)
    x = rng.standard_normal((cfg.T, cfg.d), dtype=np.float32)
    if cfg.act == BF16:
        x = round_to_bf16(x)
    return logits, x


def _expert_rng(seed: int, matrix: int, e: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1 + matrix, e])))


def make_expert_weights(cfg: Config, e: int) -> dict:
    """Stored weights of expert e: keys gate, up, down (+ gate_scale, up_scale, down_scale
    for fp8)."""
    out = {}
    shapes = {"gate": (cfg.d_ff, cfg.d), "up": (cfg.d_ff, cfg.d), "down": (cfg.d, cfg.d_ff)}
    stds = {"gate": 1.0 / math.sqrt(cfg.d), "up": 1.0 / math.sqrt(cfg.d),
            "down": 1.0 / math.sqrt(cfg.d_ff)}
    for mi, name in enumerate(("gate", "up", "down")):
        w = _expert_rng(cfg.seed, mi, e).standard_normal(shapes[name], dtype=np.float32)
        w *= np.float32(stds[name])
        if cfg.w == F32:
            out[name] = w
        elif cfg.w == BF16:
            out[name] = round_to_bf16(w)
        else:
            out[name], out[name + "_scale"] = quantize_blocks_e4m3fn(w)
    return out


def weight_dtype_np(cfg: Config):
    return {F32: np.float32, BF16: np.uint16, FP8: np.uint8}[cfg.w]


def iter_expert_weights(cfg: Config, experts, threads: int | None = None):
    """Yield (e, weights dict) for the given experts, generated on a thread pool."""
    threads = threads or min(16, os.cpu_count() or 1)
    experts = list(experts)
    with ThreadPoolExecutor(threads) as ex:
        # bounded look-ahead so that large configs never hold every expert on the host
        futs = {}
        nxt = 0
        for i in range(len(experts)):
            while nxt < len(experts) and nxt < i + 2 * threads:
                futs[nxt] = ex.submit(make_expert_weights, cfg, experts[nxt])
                nxt += 1
            yield experts[i], futs.pop(i).result()


def make_all_weights(cfg: Config, experts=None, threads: int | None = None) -> dict:
    """Stacked stored weights [E, ...] on the host. Experts not listed in `experts` are
    filled with a NaN canary (a correct kernel never reads an expert with no rows)."""
    wdt = weight_dtype_np(cfg)
    nan = {F32: np.float32(np.nan), BF16: BF16_NAN, FP8: FP8_NAN}[cfg.w]
    E = cfg.E
    out = {
        "gate": np.full((E, cfg.d_ff, cfg.d), nan, dtype=wdt),
        "up": np.full((E, cfg.d_ff, cfg.d), nan, dtype=wdt),
        "down": np.full((E, cfg.d, cfg.d_ff), nan, dtype=wdt),
    }
    if cfg.w == FP8:
        out["gate_scale"] = np.full((E, -(-cfg.d_ff // 128), -(-cfg.d // 128)), np.nan, np.float32)
        out["up_scale"] = np.full((E, -(-cfg.d_ff // 128), -(-cfg.d // 128)), np.nan, np.float32)
        out["down_scale"] = np.full((E, -(-cfg.d // 128), -(-cfg.d_ff // 128)), np.nan, np.float32)
    experts = range(E) if experts is None else experts
    for e, w in iter_expert_weights(cfg, experts, threads):
        for key, arr in w.items():
            out[key][e] = arr
    return out


def tiny_config(T=7, d=32, E=5, k=2, d_ff=48, act=F32, w=F32, zipf_s=None, seed=0, name="tiny"):
    """A small workload for brute-force and edge-case tests."""
    return Config(name, T, d, E, k, d_ff, act, w, zipf_s, seed)
