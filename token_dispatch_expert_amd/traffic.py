"""Algorithmic byte and flop counts of the MoE layer's steps (host-side arithmetic only).

These are the bytes each step *must* move and the flops it must do, independent of how a
kernel is written; achieved bandwidth / MFMA rate are these divided by measured time.

The dispatch volume follows the "Expert Parallelism" tutorial page, section 4 (The
All-to-All, communication volume): every token sends k rows of d elements one way and gets
k rows back, so one direction moves tokens * k * d * bytes.
"""
from __future__ import annotations

ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8_e4m3fn": 1}


def dispatch_bytes(tokens: int, k: int, d: int, elem_bytes: int) -> int:
    """One direction of the dispatch (or combine) exchange: tokens * k * d * bytes."""
    return tokens * k * d * elem_bytes


def exchange_bytes_per_layer(tokens: int, k: int, d: int, elem_bytes: int) -> int:
    """Dispatch plus combine for one MoE layer."""
    return 2 * dispatch_bytes(tokens, k, d, elem_bytes)


def transfer_ms(nbytes: float, gb_per_s: float) -> float:
    return nbytes / (gb_per_s * 1e9) * 1e3


def route_bytes(T: int, E: int, k: int) -> int:
    """logits f32 [T,E] read; ids i32 and gates f32 [T,k] written."""
    return T * E * 4 + T * k * 8


def permute_bytes(T: int, E: int, k: int, d: int, a: int) -> int:
    """x read once per token, x_sorted written once per assignment, ids read, both index maps
    written, counts and offsets written."""
    R = T * k
    return T * d * a + R * d * a + R * 4 + 2 * R * 4 + (2 * E + 1) * 4


def scatter_copy_bytes(T: int, k: int, d: int, a: int) -> int:
    """The row-copy part of the permutation: x read once, x_sorted written k times."""
    return T * d * a + T * k * d * a


def gate_up_bytes(active: int, R: int, d: int, d_ff: int, w: float, a: int, h: int,
                  scale_bytes: int = 0) -> int:
    """Gate/up pass: gate and up weights of every expert with rows, x_sorted read, h written."""
    return int(active * 2 * d * d_ff * w) + active * 2 * scale_bytes + R * d * a + R * d_ff * h


def down_bytes(active: int, R: int, d: int, d_ff: int, w: float, h: int,
               scale_bytes: int = 0) -> int:
    """Down pass: down weights of every expert with rows, h read, y_sorted (fp32) written."""
    return int(active * d * d_ff * w) + active * scale_bytes + R * d_ff * h + R * d * 4


def ffn_bytes(active: int, R: int, d: int, d_ff: int, w: float, a: int,
              scale_bytes_per_matrix: int = 0) -> int:
    """Layer-level FFN bytes: weights of active experts, x_sorted read, y_sorted (fp32) written
    (the h round trip between the two GEMMs is not counted: it is an implementation choice)."""
    return int(active * 3 * d * d_ff * w) + active * 3 * scale_bytes_per_matrix + R * d * a + R * d * 4


def fp8_scale_bytes(d: int, d_ff: int) -> int:
    return -(-d // 128) * -(-d_ff // 128) * 4


def ffn_flops(R: int, d: int, d_ff: int) -> int:
    """Three GEMMs of R x d x d_ff: gate, up and down."""
    return 6 * R * d * d_ff


def gate_up_flops(R: int, d: int, d_ff: int) -> int:
    return 4 * R * d * d_ff


def down_flops(R: int, d: int, d_ff: int) -> int:
    return 2 * R * d * d_ff


def combine_bytes(T: int, k: int, d: int, out_bytes: int = 4) -> int:
    """y_sorted (fp32) rows read, flat_to_sorted and gates read, y written."""
    R = T * k
    return R * d * 4 + R * 8 + T * d * out_bytes


def prefill_schedule_fills(counts, K: int, N: int, gated: bool, cus: int = 256, group_rows: int = 4,
                           small_rows: int = 16, stream_cu_gbps: float = 30.0,
                           tile_cu_tflops: float = 4.0) -> dict:
    """A model of the L2 fills (bytes fetched past the L2) of one prefill-kernel GEMM launch.

    It follows the large-tile schedule: experts with more than `small_rows` rows in 256-row tiles
    (rows dealt in 16-row fragments), `cols` output columns per tile (128 gated, 256 plain), item
    order by expert, then groups of `group_rows` row tiles with the column blocks outer; X
    streaming CUs (the kernel's balance rule) leave cus - X ranks; each round's items go to the 8
    XCDs in runs of consecutive items. Within a round an XCD fetches every distinct A tile (an
    expert's row tile, rows x K x 2 bytes) and B tile (256 weight rows x K x 2 bytes) it needs
    once over the whole contraction, and nothing outlives the round (a K-panel is MBs, the L2 per
    XCD 4 MB). The streaming role reads its experts' weights once. bf16 operands."""
    import math
    cols = 128 if gated else 256
    nt_per_expert = N // cols
    w_bytes = (2 if gated else 1) * N * K * 2
    hot = [(e, int(n)) for e, n in enumerate(counts) if n > small_rows]
    n_small = sum(1 for n in counts if 0 < n <= small_rows)
    tc = n_small * w_bytes / (stream_cu_gbps * 1e9)
    th = sum(2 * math.ceil(n / 256) * 256 * K * (2 * N if gated else N) for _, n in hot) / (tile_cu_tflops * 1e12)
    X = 0
    if tc > 0:
        X = int(cus * tc / (tc + th) / 8 + 0.5) * 8 if th > 0 else cus
        X = max(X, min(8, cus))
        if th > 0:
            X = min(X, cus - 8)
    ranks = cus - X
    items = []
    for e, n in hot:
        mt_count = math.ceil(n / 256)
        frags = math.ceil(n / 16)
        q, rem = divmod(frags, mt_count)
        tile_rows = []
        for mt in range(mt_count):
            first = 16 * (mt * q + min(mt, rem))
            tile_rows.append(min(16 * (q + (1 if mt < rem else 0)), n - first))
        for local in range(mt_count * nt_per_expert):
            g = local // (group_rows * nt_per_expert)
            gm = min(group_rows, mt_count - g * group_rows)
            j = local - g * group_rows * nt_per_expert
            items.append((e, g * group_rows + j % gm, j // gm, tile_rows[g * group_rows + j % gm]))
    fills = 0
    if ranks > 0:
        for base in range(0, len(items), ranks):
            n = min(ranks, len(items) - base)
            run = math.ceil(n / 8)
            for x in range(8):
                its = items[base + x * run: base + min(n, (x + 1) * run)]
                a_tiles = {(e, mt): r for e, mt, _, r in its}
                b_tiles = {(e, nt) for e, _, nt, _ in its}
                fills += sum(a_tiles.values()) * K * 2 + len(b_tiles) * 256 * K * 2
    return {"streaming_cus": X, "tile_items": len(items), "tile_fills": fills,
            "streamed": n_small * w_bytes, "fills": fills + n_small * w_bytes,
            "algorithmic": sum(n for _, n in hot) * K * 2 + len(hot) * w_bytes + n_small * w_bytes}
