"""Host-only checks of the C ABI: the library loads, exports every symbol include/moe.h declares,
and rejects invalid arguments with the documented status before making any HIP call (so these
run without a GPU: every call below fails validation and enqueues nothing)."""
import ctypes
import os
import re
import subprocess

import pytest

from token_dispatch_expert_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

# plausible-looking, suitably aligned device addresses; never dereferenced because every call
# here fails host-side validation first
P = 0x7F0000000000
P2 = 0x7F0000100000
P3 = 0x7F0000200000
MIS = 0x7F0000000002  # misaligned


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status_t|size_t|int|const char\s*\*)\s*(moe_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    path = B.library_path()
    if not os.path.exists(path):
        pytest.fail(f"{path} missing: run __graft_entry__.build()")
    return B.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(B.ENTRY_POINTS)
    nm = subprocess.run(["nm", "-D", "--defined-only", B.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (moe_\w+)$", nm, re.M))
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_status_strings(lib):
    for s in range(5):
        assert lib.moe_status_string(s).decode()
    assert lib.moe_status_string(99).decode() == "unknown status"


def test_route_rejects_bad_arguments(lib):
    r = lib.moe_route
    assert r(None, 4, 8, 2, P, P2, None, None) == B.MOE_ERR_INVALID_ARG          # null logits
    assert r(P, 4, 8, 9, P2, P3, None, None) == B.MOE_ERR_INVALID_ARG            # k > E
    assert r(P, 4, 8, 0, P2, P3, None, None) == B.MOE_ERR_INVALID_ARG            # k = 0
    assert r(P, -1, 8, 2, P2, P3, None, None) == B.MOE_ERR_INVALID_ARG           # T < 0
    assert r(P, 4, 2048, 2, P2, P3, None, None) == B.MOE_ERR_UNSUPPORTED         # E > 1024
    assert r(P, 4, 64, 33, P2, P3, None, None) == B.MOE_ERR_UNSUPPORTED          # k > 32
    assert r(MIS, 4, 8, 2, P2, P3, None, None) == B.MOE_ERR_INVALID_ARG          # misaligned
    assert r(P, 4, 8, 2, P2, P3, MIS, None) == B.MOE_ERR_INVALID_ARG             # misaligned counts
    assert r(P, 1 << 30, 8, 4, P2, P3, None, None) == B.MOE_ERR_INVALID_ARG      # T*k overflows


def test_permute_rejects_bad_arguments(lib):
    pm = lib.moe_permute
    T, E, k, d = 64, 8, 2, 128
    ws = lib.moe_permute_workspace_size(T, E, k)
    assert ws == 256  # one tile of 8 int32 histograms, rounded to 256 bytes
    ok = [P, B.MOE_BF16, P2, T, E, k, d, P3, P3, P3, P3, P, P2, ws, None]

    def call(**kw):
        a = list(ok)
        names = ["x", "dt", "ids", "T", "E", "k", "d", "counts", "offsets", "s2f", "f2s", "xs", "ws", "wsb", "s"]
        for n, v in kw.items():
            a[names.index(n)] = v
        return pm(*a)

    assert call(ws=None) == B.MOE_ERR_WORKSPACE
    assert call(wsb=ws - 4) == B.MOE_ERR_WORKSPACE
    assert call(dt=B.MOE_FP8_E4M3FN, ws=None) == B.MOE_ERR_UNSUPPORTED
    assert call(d=12, ws=None) == B.MOE_ERR_UNSUPPORTED      # 24-byte rows are not 16-byte multiples
    assert call(x=None, ws=None) == B.MOE_ERR_INVALID_ARG
    assert call(xs=MIS, ws=None) == B.MOE_ERR_INVALID_ARG
    assert call(k=9, ws=None) == B.MOE_ERR_INVALID_ARG


def test_capacity_entry_points(lib):
    cap = lib.moe_expert_capacity
    assert cap(512, 8, 1, 125) == 80          # the tutorial's worked counts at C = 1.25
    assert cap(10, 3, 1, 100) == 4 and cap(128, 128, 8, 110) == 9 and cap(128, 128, 8, 100) == 8
    assert cap(0, 8, 2, 150) == 0
    assert cap(-1, 8, 2, 100) == -1 and cap(8, 0, 2, 100) == -1 and cap(8, 8, 0, 100) == -1
    assert cap(8, 8, 2, -5) == -1
    assert cap(1 << 30, 1, 1, 1000) == 2**31 - 1  # saturates
    T, E, k, d = 64, 8, 2, 128
    ws = lib.moe_permute_workspace_size(T, E, k)
    a = [P, B.MOE_BF16, P2, T, E, k, d, 5, P3, P3, P3, P3, P, P2, ws, None]
    a[7] = -1
    assert lib.moe_permute_capped(*a) == B.MOE_ERR_INVALID_ARG
    a[7] = 5
    a[-3] = None
    assert lib.moe_permute_capped(*a) == B.MOE_ERR_WORKSPACE
    d_ff = 256
    need = lib.moe_layer_workspace_size(T, E, k, d, d_ff, B.MOE_BF16, B.MOE_BF16)
    la = [P, P2, B.MOE_BF16, T, E, k, d, d_ff, -3, P, P2, P3, B.MOE_BF16, None, None, None,
          P, P2, P3, P, P2, P3, P, P2, P3, B.MOE_F32, P, need, None]
    assert lib.moe_layer_capped(*la) == B.MOE_ERR_INVALID_ARG
    la[8], la[-2] = 4, need - 16
    assert lib.moe_layer_capped(*la) == B.MOE_ERR_WORKSPACE


def test_ffn_rejects_bad_arguments(lib):
    f = lib.moe_grouped_ffn
    rows, E, d, d_ff = 128, 8, 256, 384
    wsb = lib.moe_ffn_workspace_size(rows, E, d, d_ff, B.MOE_BF16, B.MOE_BF16)
    # decode-sized bf16 launch with at most 256 tiles whatever the routing: 6 column tiles of 64
    # h columns x (2 row tiles + 8 experts) = 60, so the partial tiles (512 x 64 x 128 fp32)
    # follow h
    split = 512 * 64 * 128 * 4
    assert wsb == rows * d_ff * 2 + split
    base = dict(x=P, act=B.MOE_BF16, off=P2, rows=rows, E=E, d=d, d_ff=d_ff, wg=P, wu=P2, wd=P3,
                wdt=B.MOE_BF16, sg=None, su=None, sd=None, y=P, ws=P2, wsb=wsb, s=None)

    def call(**kw):
        a = dict(base, **kw)
        return f(*a.values())

    assert call(act=B.MOE_F32, ws=None) == B.MOE_ERR_UNSUPPORTED                 # f32 act + bf16 w
    assert call(act=B.MOE_FP8_E4M3FN, ws=None) == B.MOE_ERR_UNSUPPORTED
    assert call(wdt=B.MOE_FP8_E4M3FN, d_ff=320, ws=None) == B.MOE_ERR_UNSUPPORTED  # d_ff not /128
    assert call(wdt=B.MOE_FP8_E4M3FN, d_ff=512, ws=None) == B.MOE_ERR_INVALID_ARG  # scales missing
    assert call(sg=P, ws=None) == B.MOE_ERR_INVALID_ARG                          # scales with bf16
    assert call(d=100, ws=None) == B.MOE_ERR_UNSUPPORTED                         # d not /8
    assert call(ws=None) == B.MOE_ERR_WORKSPACE
    assert call(wsb=wsb - 1) == B.MOE_ERR_WORKSPACE
    assert call(rows=-1, ws=None) == B.MOE_ERR_INVALID_ARG
    assert call(wg=MIS, ws=None) == B.MOE_ERR_INVALID_ARG
    # blocked bf16 weights: bf16 activations, d and d_ff multiples of 64, the bf16 workspace
    assert lib.moe_ffn_workspace_size(rows, E, d, d_ff, B.MOE_BF16, B.MOE_BF16_BLOCKED) == wsb
    assert call(wdt=B.MOE_BF16_BLOCKED, ws=None) == B.MOE_ERR_WORKSPACE          # accepted
    assert call(wdt=B.MOE_BF16_BLOCKED, d_ff=320 + 8, ws=None) == B.MOE_ERR_UNSUPPORTED
    assert call(wdt=B.MOE_BF16_BLOCKED, act=B.MOE_F32, ws=None) == B.MOE_ERR_UNSUPPORTED
    assert call(wdt=B.MOE_BF16_BLOCKED, sg=P, ws=None) == B.MOE_ERR_INVALID_ARG
    # blocked fp8: d and d_ff multiples of 128 and at most 65536, scales required
    assert call(wdt=B.MOE_FP8_E4M3FN_BLOCKED, d_ff=512, ws=None) == B.MOE_ERR_INVALID_ARG   # no scales
    assert call(wdt=B.MOE_FP8_E4M3FN_BLOCKED, d_ff=320, ws=None) == B.MOE_ERR_UNSUPPORTED
    assert call(wdt=B.MOE_FP8_E4M3FN_BLOCKED, d=65536 + 128, ws=None) == B.MOE_ERR_UNSUPPORTED


def test_block_weights_rejects_bad_arguments(lib):
    # every case fails validation before anything is enqueued (no call here has valid arguments)
    f = lib.moe_block_weights
    big = 1 << 40  # an aligned address far from P
    bf, f8 = B.MOE_BF16, B.MOE_FP8_E4M3FN
    assert f(P, big, B.MOE_F32, 2, 16, 128, None) == B.MOE_ERR_UNSUPPORTED
    assert f(P, big, B.MOE_BF16_BLOCKED, 2, 16, 128, None) == B.MOE_ERR_UNSUPPORTED
    assert f(P, big, bf, 0, 16, 128, None) == B.MOE_ERR_INVALID_ARG            # E < 1
    assert f(P, big, bf, 2, 12, 128, None) == B.MOE_ERR_INVALID_ARG            # N not /8
    assert f(P, big, bf, 2, 16, 96, None) == B.MOE_ERR_INVALID_ARG             # K not /64
    assert f(P, big, f8, 2, 16, 192, None) == B.MOE_ERR_INVALID_ARG            # fp8 K not /128
    assert f(None, big, bf, 2, 16, 128, None) == B.MOE_ERR_INVALID_ARG         # null
    assert f(MIS, big, bf, 2, 16, 128, None) == B.MOE_ERR_INVALID_ARG          # misaligned
    assert f(P, P + 64, bf, 2, 16, 128, None) == B.MOE_ERR_INVALID_ARG         # overlapping
    assert f(P, big, bf, 1, 1 << 15, 1 << 15, None) == B.MOE_ERR_INVALID_ARG   # a 2 GiB matrix
    assert f(P, big, f8, 1, 1 << 16, 1 << 15, None) == B.MOE_ERR_INVALID_ARG   # a 2 GiB fp8 matrix
    assert f(P, big, bf, 1 << 20, 1 << 10, 1 << 10, None) == B.MOE_ERR_INVALID_ARG  # 2^40 elements


def test_combine_and_layer_reject_bad_arguments(lib):
    c = lib.moe_combine
    assert c(P, P2, P3, 4, 2, 6, P, B.MOE_F32, None) == B.MOE_ERR_UNSUPPORTED   # d not /4
    assert c(None, P2, P3, 4, 2, 8, P, B.MOE_F32, None) == B.MOE_ERR_INVALID_ARG
    assert c(P, P2, P3, 4, 0, 8, P, B.MOE_F32, None) == B.MOE_ERR_INVALID_ARG
    assert c(P, P2, P3, 4, 2, 8, P, B.MOE_FP8_E4M3FN, None) == B.MOE_ERR_UNSUPPORTED  # fp8 output
    assert c(P, P2, P3, 4, 2, 8, P, 7, None) == B.MOE_ERR_INVALID_ARG                 # no such format
    assert c(P, P2, P3, 4, 2, 8, MIS, B.MOE_BF16, None) == B.MOE_ERR_INVALID_ARG      # y misaligned
    T, E, k, d, d_ff = 16, 8, 2, 128, 256
    need = lib.moe_layer_workspace_size(T, E, k, d, d_ff, B.MOE_BF16, B.MOE_BF16)
    assert need == lib.moe_permute_workspace_size(T, E, k) + lib.moe_ffn_workspace_size(T * k, E, d, d_ff, B.MOE_BF16, B.MOE_BF16)
    args = [P, P2, B.MOE_BF16, T, E, k, d, d_ff, P, P2, P3, B.MOE_BF16, None, None, None,
            P, P2, P3, P, P2, P3, P, P2, P3, B.MOE_F32, P, need - 16, None]
    assert lib.moe_layer(*args) == B.MOE_ERR_WORKSPACE
    args[-2] = need
    args[-4] = 9
    assert lib.moe_layer(*args) == B.MOE_ERR_INVALID_ARG     # no such output format
    args[-4] = B.MOE_BF16
    args[2] = B.MOE_FP8_E4M3FN
    assert lib.moe_layer(*args) == B.MOE_ERR_UNSUPPORTED


def test_ffn_workspace_split_rule(lib):
    f = lib.moe_ffn_workspace_size
    split = 512 * 64 * 128 * 4
    # one decode token routed to 8 of 128 experts (d=4096, d_ff=1536): gate/up has at most
    # 24 x (1 + 8) = 216 tiles -> split
    assert f(8, 128, 4096, 1536, B.MOE_BF16, B.MOE_BF16) == 8 * 1536 * 2 + split
    # 1024 rows over 128 experts: up to 24 x (16 + 128) tiles -> no split
    assert f(1024, 128, 4096, 1536, B.MOE_BF16, B.MOE_BF16) == 1024 * 1536 * 2
    # decode-sized fp8 weights and fp32 never split
    assert f(8, 128, 4096, 1536, B.MOE_BF16, B.MOE_FP8_E4M3FN) == 8 * 1536 * 2
    assert f(8, 128, 4096, 1536, B.MOE_F32, B.MOE_F32) == 8 * 1536 * 4
    # prefill-sized (rows >= 32 E): a 256-byte header and 256 partial tiles of the hot tile
    # (256 x 256 fp32 with bf16 weights, 128 x 256 with fp8) for the last round's split tiles
    assert f(4096, 8, 4096, 1536, B.MOE_BF16, B.MOE_BF16) == 4096 * 1536 * 2 + 256 + 256 * 256 * 256 * 4
    assert f(4096, 8, 4096, 1536, B.MOE_BF16, B.MOE_FP8_E4M3FN) == 4096 * 1536 * 2 + 256 + 256 * 128 * 256 * 4


def test_workspace_sizes(lib):
    # one int32 per (tile of 256 assignments, expert), rounded up to 256 bytes
    assert lib.moe_permute_workspace_size(8192, 256, 8) == 256 * 256 * 4
    assert lib.moe_permute_workspace_size(0, 256, 8) == 0
    assert lib.moe_permute_workspace_size(5, 4, 9) == 0           # invalid -> 0
    assert lib.moe_ffn_workspace_size(65536, 256, 7168, 2048, B.MOE_BF16, B.MOE_FP8_E4M3FN) == \
        65536 * 2048 * 2 + 256 + 256 * 128 * 256 * 4
    assert lib.moe_ffn_workspace_size(128, 8, 128, 256, B.MOE_F32, B.MOE_F32) == 128 * 256 * 4


def test_route_gemm_rejects_bad_arguments(lib):
    f = lib.moe_route_gemm
    wsb = lib.moe_route_gemm_workspace_size(16, 8, 2)
    assert wsb == 16 * 16 * 8 * 4                          # 16 contraction chunks of fp32 partials
    assert lib.moe_route_gemm_workspace_size(4096, 8, 2) == 0
    ok = [P, B.MOE_BF16, P2, B.MOE_BF16, 16, 8, 2, 64, None, P3, P, None, P2, wsb, None]

    def call(**kw):
        a = list(ok)
        names = ["x", "xdt", "w", "wdt", "T", "E", "k", "d", "logits", "ids", "gates", "counts", "ws", "wsb", "s"]
        for n, v in kw.items():
            a[names.index(n)] = v
        return f(*a)

    assert call(xdt=B.MOE_F32) == B.MOE_ERR_UNSUPPORTED
    assert call(wdt=B.MOE_FP8_E4M3FN) == B.MOE_ERR_UNSUPPORTED
    assert call(E=300) == B.MOE_ERR_UNSUPPORTED            # more experts than one tile row holds
    assert call(d=48) == B.MOE_ERR_UNSUPPORTED             # not a multiple of 32
    assert call(k=9) == B.MOE_ERR_INVALID_ARG
    assert call(x=None) == B.MOE_ERR_INVALID_ARG
    assert call(logits=MIS) == B.MOE_ERR_INVALID_ARG
    assert call(ws=None) == B.MOE_ERR_WORKSPACE
    assert call(wsb=wsb - 4) == B.MOE_ERR_WORKSPACE


def test_noalloc_permute_rejects_bad_arguments(lib):
    f = lib.moe_permute_noalloc
    # the per-tile counts of 4,097 tiles x 256 experts exceed the 4 MiB static scratch
    T, E, k, d = (1 << 20) // 8 + 32, 256, 8, 8
    assert lib.moe_permute_workspace_size(T, E, k) > B.PERMUTE_NOALLOC_SCRATCH_BYTES
    assert f(P, B.MOE_BF16, P2, T, E, k, d, P3, P3, P3, P3, P, None) == B.MOE_ERR_WORKSPACE
    assert f(None, B.MOE_BF16, P2, 64, 8, 2, 128, P3, P3, P3, P3, P, None) == B.MOE_ERR_INVALID_ARG
    assert f(P, B.MOE_FP8_E4M3FN, P2, 64, 8, 2, 128, P3, P3, P3, P3, P, None) == B.MOE_ERR_UNSUPPORTED
    assert f(P, B.MOE_BF16, P2, 64, 8, 9, 128, P3, P3, P3, P3, P, None) == B.MOE_ERR_INVALID_ARG

