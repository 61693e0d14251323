"""fp64 CPU oracle for one GPU's share of an expert-parallel MoE layer.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and its Python
binding) imports, calls or links this module; only the tests, the smoke check and the
benchmark's CPU-baseline leg use it. It shares no code, tables or helpers with the HIP path.

What it computes (cited to the pages by title and section):
  * "Expert Parallelism" tutorial, section 1 (What is it?): each MoE layer has E expert FFNs
    and each token goes to k of them.
  * same page, section 4 (The All-to-All), dispatch: the router names each token's experts;
    tokens are sorted by destination expert, counted, and every expert ends up with a
    contiguous block of rows.
  * same page, section 4, compute: each expert processes its rows (one grouped GEMM).
  * same page, section 4, combine: results return in the original order and each token's k
    expert outputs are summed with their gate weights.
The pages leave the gate formula, the FFN form, tie-breaks and number formats open; this
oracle takes the readings listed below (each is also listed in the design notes):
  R1 top-k: k passes of arg-max over the not-yet-chosen experts; equal logits go to the lower
     expert index (+0.0 and -0.0 are equal); slot order = selection order; selection is on
     the fp32 logits promoted exactly to fp64.
  R2 gates: softmax restricted to the k chosen logits (the same as a full softmax
     renormalised over the top k), g_j = exp(l_j - l_max) / sum_i exp(l_i - l_max).
  R3 order inside an expert: stable in the flat index i = t*k + j.
  R4, R5 expert FFN: SwiGLU, y = (silu(x Wg) * (x Wu)) Wd with silu(z) = z / (1 + exp(-z)),
     no biases; weights are stored with the contraction axis contiguous (gate/up as
     [d_ff, d], down as [d, d_ff]), so x Wg is x @ gate.T here.
  R6 fp8 weights: OCP e4m3fn codes times an fp32 scale per 128x128 block of the stored
     matrix, decoded exactly to fp64.
  R7 (optional, off by default) h_round="bf16": h is rounded to the nearest bf16 between the
     two GEMMs, the rounding point of a bf16 implementation; tests use it as a second,
     tighter comparison next to the plain fp64 one.
  R8 combine: fp64, summed in slot order j = 0..k-1.
  R9 capacity factor (optional; same page, section 5, mitigation 1, and section 10, exercise
     D): each expert keeps at most `capacity` assignments and the excess is dropped. The page
     states capacity = C * tokens / E; with k > 1 the count is of assignments, so
     capacity = ceil(C * T * k / E). The kept assignments of an expert are its first
     `capacity` in flat order (the stable order of R3); a dropped assignment gets no row
     (flat_to_sorted = -1) and adds nothing in the combine (the token passes the expert by,
     the residual connection being outside the layer); the gates are not renormalised. The
     factor is taken in percent, so the capacity is exact integer arithmetic.
  R14 router scores (the fused router's input side; same page, section 4: the router decides
     each token's experts): logits[t, e] = sum_i x[t, i] * w_router[e, i], one weight row per
     expert, no bias or scaling; exact decode, fp64. The top-k of the fused GPU router is
     checked by routing the GPU's own fp32 logits with `route` (a selection decided in floating
     point is compared in the precision that decided it), and those logits against these.
Everything is fp64 after an exact decode of the stored inputs; there is no blocking, fusion
or reordering beyond the steps above. Library primitives used as steps: numpy argmax (first
occurrence of the maximum), fp64 matrix products (BLAS) and exp.
"""
from __future__ import annotations

import numpy as np

F32, BF16, FP8 = "f32", "bf16", "fp8_e4m3fn"


# ----------------------------------------------------------------------------------------
# exact decoders of the stored formats
# ----------------------------------------------------------------------------------------
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64, exactly: a bf16 is the top half of an fp32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """OCP e4m3fn codes (uint8) -> fp64, exactly. Layout: sign, 4 exponent bits (bias 7),
    3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2^-6; the all-ones pattern
    S.1111.111 is NaN and there is no infinity."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = sign * np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def decode_matrix(w: np.ndarray, fmt: str, scale: np.ndarray | None = None,
                  block: int = 128) -> np.ndarray:
    """Stored matrix -> fp64 values (reading R6 for fp8: code value times its block's scale)."""
    if fmt == F32:
        return np.asarray(w, dtype=np.float32).astype(np.float64)
    if fmt == BF16:
        return decode_bf16(w)
    if fmt == FP8:
        vals = decode_e4m3fn(w)
        s = np.asarray(scale, dtype=np.float32).astype(np.float64)
        n, kk = vals.shape
        full = np.repeat(np.repeat(s, block, axis=0), block, axis=1)[:n, :kk]
        return vals * full
    raise ValueError(f"unknown format {fmt}")


def decode_activations(x: np.ndarray, fmt: str) -> np.ndarray:
    return decode_matrix(x, fmt)


# ----------------------------------------------------------------------------------------
# route: top-k selection and gates (tutorial section 4, router output; section 1, k of E)
# ----------------------------------------------------------------------------------------
def route(logits: np.ndarray, k: int):
    """Per token: the k largest logits, in selection order, and their gate weights.

    Returns (topk_ids int32 [T, k], topk_gates fp64 [T, k]). Readings R1, R2."""
    lg = np.asarray(logits, dtype=np.float32).astype(np.float64)
    T, E = lg.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    if not np.all(np.isfinite(lg)):
        raise ValueError("logits must be finite")
    ids = np.empty((T, k), dtype=np.int32)
    gates = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        row = lg[t].copy()
        chosen = []
        for _ in range(k):
            e = int(np.argmax(row))          # first index holding the maximum
            chosen.append(e)
            row[e] = -np.inf                 # chosen experts drop out of later passes
        sel = lg[t, chosen]
        w = np.exp(sel - sel[0])             # sel[0] is the largest chosen logit
        ids[t] = chosen
        gates[t] = w / np.sum(w)
    return ids, gates


def router_logits(x: np.ndarray, x_fmt: str, w_router: np.ndarray, w_fmt: str) -> np.ndarray:
    """Router scores [T, E] = X W_r^T in fp64 from the exactly decoded stored values (R14)."""
    X = decode_activations(x, x_fmt)
    Wr = decode_matrix(w_router, w_fmt)
    return X @ Wr.T


# ----------------------------------------------------------------------------------------
# permute: count, exclusive scan, stable scatter, row copy (tutorial section 4, dispatch)
# ----------------------------------------------------------------------------------------
def expert_capacity(T: int, E: int, k: int, factor_percent: int) -> int:
    """capacity = ceil(C * T * k / E) assignments per expert (reading R9), with the factor
    C given in percent (C = 1.25 -> 125) so that the value is exact integer arithmetic."""
    return -(-(int(factor_percent) * T * k) // (100 * E))


def permute(topk_ids: np.ndarray, E: int, capacity: int | None = None):
    """Stable counting sort of the flat assignments i = t*k + j by expert id (reading R3);
    with a capacity, each expert keeps only its first `capacity` assignments (reading R9).

    Returns dict(counts int32 [E] (kept assignments), offsets int32 [E+1],
    sorted_to_flat int32 [offsets[E]], flat_to_sorted int32 [R], -1 where dropped)."""
    flat = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    R = flat.size
    counts = np.zeros(E, dtype=np.int64)
    for i in range(R):
        counts[flat[i]] += 1
    if capacity is not None:
        counts = np.minimum(counts, capacity)
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = offsets[:E].copy()
    s2f = np.empty(int(offsets[E]), dtype=np.int64)
    f2s = np.full(R, -1, dtype=np.int64)
    for i in range(R):
        e = flat[i]
        pos = fill[e]
        if pos == offsets[e + 1]:
            continue  # this expert is full: the assignment is dropped
        fill[e] += 1
        s2f[pos] = i
        f2s[i] = pos
    return dict(counts=counts.astype(np.int32), offsets=offsets.astype(np.int32),
                sorted_to_flat=s2f.astype(np.int32), flat_to_sorted=f2s.astype(np.int32))


def gather_rows(x: np.ndarray, sorted_to_flat: np.ndarray, k: int) -> np.ndarray:
    """x_sorted[r] = x[sorted_to_flat[r] // k]: a copy of the stored rows (any format)."""
    R = len(sorted_to_flat)
    out = np.empty((R,) + x.shape[1:], dtype=x.dtype)
    for r in range(R):
        out[r] = x[int(sorted_to_flat[r]) // k]
    return out


# ----------------------------------------------------------------------------------------
# expert FFN (tutorial section 4, compute; reading R4)
# ----------------------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def round_bf16_value(v: np.ndarray) -> np.ndarray:
    """Nearest bf16 value of each fp64 value (8 significant bits, ties to even), as fp64.
    Used only for the optional rounding-point mode below (finite, normal-range inputs)."""
    m, e = np.frexp(np.asarray(v, dtype=np.float64))   # v = m * 2^e with 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)


def expert_ffn(X: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray,
               return_h: bool = False, h_round: str | None = None):
    """SwiGLU of one expert over its rows X [n, d] (fp64); Wg, Wu stored [d_ff, d], Wd
    stored [d, d_ff]. h_round="bf16" rounds h to bf16 before the down projection (the
    rounding point a bf16 implementation has between its two GEMMs); default: none."""
    G = X @ Wg.T
    U = X @ Wu.T
    h = silu(G) * U
    if h_round == "bf16":
        h = round_bf16_value(h)
    elif h_round is not None:
        raise ValueError(h_round)
    y = expert_down(h, Wd)
    return (y, h) if return_h else y


def expert_down(h: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """The down projection of one expert alone, y = h Wd (fp64; Wd stored [d, d_ff]): the
    second GEMM of expert_ffn, also applied by the tests to another implementation's own h."""
    return h @ Wd.T


def ffn(x_sorted: np.ndarray, offsets: np.ndarray, expert_weights, return_h: bool = False,
        h_round: str | None = None):
    """Grouped FFN: rows offsets[e]..offsets[e+1] go through expert e.

    x_sorted: fp64 [R, d]. expert_weights(e) -> (Wg, Wu, Wd) in fp64. Experts with no rows
    are never asked for their weights."""
    R, d = x_sorted.shape
    E = len(offsets) - 1
    y = np.zeros((R, d), dtype=np.float64)
    h_all = None
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        Wg, Wu, Wd = expert_weights(e)
        y_e, h_e = expert_ffn(x_sorted[a:b], Wg, Wu, Wd, return_h=True, h_round=h_round)
        y[a:b] = y_e
        if return_h:
            if h_all is None:
                h_all = np.zeros((R, h_e.shape[1]), dtype=np.float64)
            h_all[a:b] = h_e
    return (y, h_all) if return_h else y


# ----------------------------------------------------------------------------------------
# combine (tutorial section 4, combine; reading R8)
# ----------------------------------------------------------------------------------------
def combine(y_sorted: np.ndarray, flat_to_sorted: np.ndarray, gates: np.ndarray) -> np.ndarray:
    """y[t] = sum_j gates[t, j] * y_sorted[flat_to_sorted[t*k + j]], slot order, fp64; a
    dropped slot (flat_to_sorted = -1, reading R9) adds nothing."""
    T, k = gates.shape
    y = np.zeros((T, y_sorted.shape[1]), dtype=np.float64)
    for t in range(T):
        acc = np.zeros(y_sorted.shape[1], dtype=np.float64)
        for j in range(k):
            pos = int(flat_to_sorted[t * k + j])
            if pos < 0:
                continue
            acc = acc + gates[t, j] * y_sorted[pos]
        y[t] = acc
    return y


# ----------------------------------------------------------------------------------------
# whole layer and per-token evaluation
# ----------------------------------------------------------------------------------------
def make_weight_decoder(raw_weights, w_fmt: str):
    """raw_weights(e) -> dict(gate, up, down[, *_scale]) in the stored formats; returns a
    function e -> (Wg, Wu, Wd) in fp64."""
    def dec(e):
        w = raw_weights(e)
        return tuple(decode_matrix(w[n], w_fmt, w.get(n + "_scale")) for n in ("gate", "up", "down"))
    return dec


def layer(logits, x, x_fmt: str, raw_weights, w_fmt: str, k: int, return_h: bool = False,
          h_round: str | None = None, capacity: int | None = None):
    """The whole layer: route -> permute (optionally capped, R9) -> grouped FFN -> combine.
    Returns every intermediate."""
    T, E = np.asarray(logits).shape
    ids, gates = route(logits, k)
    p = permute(ids, E, capacity)
    x_sorted = gather_rows(np.asarray(x), p["sorted_to_flat"], k)
    xs = decode_activations(x_sorted, x_fmt)
    dec = make_weight_decoder(raw_weights, w_fmt)
    if return_h:
        y_sorted, h = ffn(xs, p["offsets"], dec, return_h=True, h_round=h_round)
    else:
        y_sorted, h = ffn(xs, p["offsets"], dec, h_round=h_round), None
    y = combine(y_sorted, p["flat_to_sorted"], gates)
    out = dict(topk_ids=ids, topk_gates=gates, x_sorted=x_sorted, y_sorted=y_sorted, y=y, **p)
    if return_h:
        out["h"] = h
    return out


def layer_tokens(tokens, topk_ids, topk_gates, x, x_fmt: str, raw_weights, w_fmt: str,
                 h_round: str | None = None):
    """y[t] for the listed tokens only, from their own routing (used to check large layers
    on a sample: a token's output depends only on its own row, ids and gates). Returns
    (y [len(tokens), d], y_rows dict (t, j) -> that slot's expert output)."""
    dec = make_weight_decoder(raw_weights, w_fmt)
    tokens = list(tokens)
    k = topk_ids.shape[1]
    X = decode_activations(np.asarray(x)[tokens], x_fmt)
    by_expert = {}
    for ti, t in enumerate(tokens):
        for j in range(k):
            by_expert.setdefault(int(topk_ids[t, j]), []).append((ti, j))
    rows = {}
    for e, items in sorted(by_expert.items()):
        Wg, Wu, Wd = dec(e)
        Y = expert_ffn(X[[ti for ti, _ in items]], Wg, Wu, Wd, h_round=h_round)
        for (ti, j), yr in zip(items, Y):
            rows[(tokens[ti], j)] = yr
    y = np.zeros((len(tokens), X.shape[1]), dtype=np.float64)
    for ti, t in enumerate(tokens):
        acc = np.zeros(X.shape[1], dtype=np.float64)
        for j in range(k):
            acc = acc + topk_gates[t, j] * rows[(t, j)]
        y[ti] = acc
    return y, rows


def rel_max_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max|got - ref| / sqrt(mean(ref^2)): the error measure the tolerances are stated in."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / rms if rms > 0 else float(np.max(np.abs(got - ref)))
