"""C ABI contract on the CPU: the library loads, exports what include/attn.h and
include/attn_block.h, include/attn_decode.h, include/attn_dropout.h and include/attn_rope.h
declare, and rejects every invalid argument before
touching the GPU.

Every call below fails validation, and validation happens before any HIP
call, so none of them launches anything (no GPU is needed or used).
"""
import ctypes
import os
import re

import pytest

import tiled_attention_memory_amd as tam

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("attn.h", "attn_block.h", "attn_decode.h", "attn_dropout.h",
                                                         "attn_rope.h")]

A = 1 << 20          # fake, 16-byte aligned, far-apart "device" addresses (never dereferenced)
GOOD = dict(B=1, Hq=4, Hkv=2, S=128, D=128, causal=1, scale=0.125)


def declared_functions():
    src = "\n".join(open(h).read() for h in HEADERS)
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_exports():
    assert declared_functions() == sorted(tam.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(tam.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    assert tam.attn_version() == 1
    for code in range(11):
        assert tam.attn_status_string(code) and tam.attn_status_string(code) != "unknown status"
    assert tam.attn_status_string(99) == "unknown status"


def fwd(**kw):
    args = dict(GOOD)
    ptrs = dict(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A)
    for key in list(kw):
        if key in ptrs:
            ptrs[key] = kw.pop(key)
    args.update(kw)
    return tam.attn_fwd_raw(ptrs["q"], ptrs["k"], ptrs["v"], ptrs["o"], ptrs["lse"], args["B"],
                            args["Hq"], args["Hkv"], args["S"], args["D"], args["causal"],
                            args["scale"])


def ws_bytes(**kw):
    a = dict(GOOD, **kw)
    return tam.attn_bwd_workspace_bytes(a["B"], a["Hq"], a["Hkv"], a["S"], a["D"])


def bwd(ws_size=None, **kw):
    args = dict(GOOD)
    ptrs = dict(q=A, k=2 * A, v=3 * A, o=4 * A, dout=5 * A, lse=6 * A, dq=7 * A, dk=8 * A,
                dv=9 * A, ws=10 * A)
    for key in list(kw):
        if key in ptrs:
            ptrs[key] = kw.pop(key)
    args.update(kw)
    if ws_size is None:
        ws_size = 0   # default: too small, so a fully valid call still cannot launch
    return tam.attn_bwd_raw(ptrs["q"], ptrs["k"], ptrs["v"], ptrs["o"], ptrs["dout"], ptrs["lse"],
                            ptrs["dq"], ptrs["dk"], ptrs["dv"], ptrs["ws"], ws_size, args["B"],
                            args["Hq"], args["Hkv"], args["S"], args["D"], args["causal"],
                            args["scale"])


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "lse"])
def test_fwd_null_pointer(name):
    assert fwd(**{name: 0}) == 1


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), 2), (dict(Hq=0), 2), (dict(Hkv=0), 2), (dict(S=0), 2), (dict(S=-5), 2),
    (dict(Hq=6, Hkv=4), 2), (dict(S=(1 << 22) + 1), 2), (dict(B=1 << 20, Hq=1 << 5), 2),
    (dict(D=96), 3), (dict(D=256), 3), (dict(D=0), 3),
    (dict(scale=float("nan")), 4), (dict(scale=float("inf")), 4), (dict(scale=float("-inf")), 4),
    (dict(causal=2), 8), (dict(causal=-1), 8),
])
def test_fwd_bad_arguments(kw, code):
    assert fwd(**kw) == code


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "lse"])
def test_fwd_misaligned(name):
    base = dict(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A)
    assert fwd(**{name: base[name] + 8}) == 5


def test_fwd_aliasing():
    assert fwd(o=A) == 9                 # o on top of q
    assert fwd(lse=4 * A + 64) == 9      # lse inside o
    assert fwd(o=2 * A + 4096) == 9      # o overlapping k


def test_workspace_query():
    n = ws_bytes()
    assert n >= 2 * 4 * 128 * 4           # Delta and scaled LSE, one float each per query row
    assert n % 256 == 0
    with pytest.raises(tam.AttnError):
        ws_bytes(D=80)
    with pytest.raises(tam.AttnError):
        ws_bytes(Hq=3, Hkv=2)
    lib = tam.load()
    assert lib.attn_bwd_workspace_bytes(1, 4, 2, 128, 128, None) == 1
    # grows with the sequence: per query row two floats, an fp16 copy of its Q and dO rows and
    # (every 32 rows) three exponents; per key an fp16 copy of its K row and (every 64 keys) two
    # exponents; plus dK/dV partials when the heads are split
    B, Hq, Hkv, S, D = 1, 8, 1, 81920, 128
    rows = B * Hq * S
    per_rows = (rows * (2 * 4 + 2 * D * 2) + 3 * 4 * B * Hq * ((S + 31) // 32)
                + B * Hkv * S * D * 2 + 2 * 4 * B * Hkv * ((S + 63) // 64))
    n = ws_bytes(Hq=Hq, Hkv=Hkv, S=S)
    assert per_rows <= n <= per_rows + 8 * 2 * B * Hkv * S * D * 4 + 12 * 256


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv"])
def test_bwd_null_pointer(name):
    assert bwd(**{name: 0}) == 1


def test_bwd_workspace_checks():
    need = ws_bytes()
    assert bwd(ws_size=need - 1) == 6
    assert bwd(ws=0, ws_size=need) == 6
    assert bwd(ws=10 * A + 8, ws_size=need) == 5


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=5, Hkv=2), 2), (dict(D=32), 3), (dict(scale=float("nan")), 4), (dict(causal=3), 8),
])
def test_bwd_bad_arguments(kw, code):
    assert bwd(**kw) == code


def test_bwd_aliasing():
    need = ws_bytes()
    assert bwd(ws_size=need, dq=A) == 9                    # dq on q
    assert bwd(ws_size=need, dk=7 * A + 128) == 9          # dk inside dq
    assert bwd(ws_size=need, ws=6 * A, ) == 9              # workspace on lse
    assert bwd(ws_size=need, dv=5 * A) == 9                # dv on dout


# ---------------------------------------------------------------------------
# context-parallel building block (attn_block.h): validation only
# ---------------------------------------------------------------------------
def fwd_block(**kw):
    a = dict(B=1, Hq=4, Hkv=2, Sq=100, Sk=70, D=128, causal=1, q0=0, k0=0, scale=0.125)
    ptrs = dict(q=A, k=2 * A, v=3 * A, o=4 * A, lse=8 * A)
    for key in list(kw):
        if key in ptrs:
            ptrs[key] = kw.pop(key)
    a.update(kw)
    return tam.load().attn_fwd_block(ptrs["q"], ptrs["k"], ptrs["v"], ptrs["o"], ptrs["lse"], a["B"], a["Hq"],
                                     a["Hkv"], a["Sq"], a["Sk"], a["D"], a["causal"], a["q0"], a["k0"], a["scale"],
                                     None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), 1), (dict(lse=0), 1),
    (dict(Sq=0), 2), (dict(Sk=0), 2), (dict(Sk=(1 << 22) + 1), 2), (dict(Hq=3), 2),
    (dict(D=96), 3), (dict(scale=float("inf")), 4), (dict(k=2 * A + 8), 5), (dict(causal=2), 8),
    (dict(q0=(1 << 62) + 1), 2), (dict(k0=-(1 << 62) - 1), 2),
    (dict(o=A + 4096), 9),          # o_part on top of q
    (dict(lse=4 * A + 100 * 128), 9),  # lse_part inside o_part (o_part is 4*100*128*4 bytes)
])
def test_fwd_block_rejects(kw, status):
    assert fwd_block(**kw) == status


def test_merge_rejects():
    lib = tam.load()
    arr = ctypes.c_void_p * 2
    ok = (arr(A, 2 * A), arr(3 * A, 5 * A))
    assert lib.attn_merge(*ok, 0, 6 * A, 7 * A, 1, 4, 64, 128, None) == 2           # n = 0
    assert lib.attn_merge(*ok, 17, 6 * A, 7 * A, 1, 4, 64, 128, None) == 2          # n > ATTN_MAX_MERGE
    assert lib.attn_merge(arr(A, 0), ok[1], 2, 6 * A, 7 * A, 1, 4, 64, 128, None) == 1
    assert lib.attn_merge(*ok, 2, 6 * A, 7 * A, 1, 4, 64, 96, None) == 3
    assert lib.attn_merge(*ok, 2, A + 64, 7 * A, 1, 4, 64, 128, None) == 9          # o on top of a part
    assert lib.attn_merge(arr(A + 4, 2 * A), ok[1], 2, 6 * A, 7 * A, 1, 4, 64, 128, None) == 5


def test_block_backward_rejects():
    lib = tam.load()
    B, Hq, Hkv, Sq, Sk, D = 1, 4, 2, 64, 96, 128
    need = tam.attn_bwd_block_workspace_bytes(B, Hq, Hkv, Sq, Sk, D)
    assert need >= tam.attn_bwd_block_workspace_bytes(B, Hq, Hkv, Sq, 32, D)
    W = 64 * A
    assert lib.attn_bwd_block_begin(A, 2 * A, 3 * A, W, need - 1, B, Hq, Hkv, Sq, Sk, D, None) == 6
    assert lib.attn_bwd_block_begin(A, 2 * A, 3 * A, 0, need, B, Hq, Hkv, Sq, Sk, D, None) == 6
    assert lib.attn_bwd_block_begin(A, 2 * A, 3 * A, A + 256, need, B, Hq, Hkv, Sq, Sk, D, None) == 9
    assert lib.attn_bwd_block_dq(A, 2 * A, 3 * A, 4 * A, W, need, B, Hq, Hkv, Sq, Sk, D, 3, 0, 0, 0.1, None) == 8
    assert lib.attn_bwd_block_dq(A, 2 * A, 3 * A, 4 * A, W, need, B, Hq, Hkv, Sq, Sk, D, 1, (1 << 62) + 1, 0, 0.1,
                                 None) == 2
    assert lib.attn_bwd_block_dq_end(0, W, need, B, Hq, Hkv, Sq, Sk, D, 0.1, None) == 1
    assert lib.attn_bwd_block_dq_end(A, W, need, B, Hq, Hkv, Sq, Sk, D, float("nan"), None) == 4
    assert lib.attn_bwd_block_dkdv(A, 2 * A, 3 * A, 4 * A, 5 * A, 5 * A, W, need, B, Hq, Hkv, Sq, Sk, D, 1, 0, 0,
                                   0.1, None) == 9    # dk and dv overlap
    assert lib.attn_bwd_block_dkdv(A, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A, W, need, B, Hq, Hkv, Sq, Sk + 512, D, 1,
                                   0, 0, 0.1, None) == 6    # workspace sized for a smaller key block


@pytest.mark.parametrize("shape", [
    # B, Hq, Hkv, Sq, largest key block, D: shapes where a shorter key block splits
    # the group's heads more finely than the longest one
    (1, 64, 8, 4096, 16384, 128),
    (1, 8, 1, 10240, 131072, 128),
    (1, 4, 2, 64, 96, 128),
])
def test_block_workspace_covers_every_shorter_key_block(shape):
    """The size for the largest key block passes the workspace check of every call with a
    shorter one. dk and dv overlap in these calls, an error checked after the workspace,
    so a call that passes the workspace check returns ATTN_ERR_ALIAS and launches nothing."""
    lib = tam.load()
    B, Hq, Hkv, Sq, Sk_max, D = shape
    need = tam.attn_bwd_block_workspace_bytes(B, Hq, Hkv, Sq, Sk_max, D)
    W = 1 << 44
    for sk in sorted({1, 63, 64, 127, 128, 129, 1000, 1024, 4096, 8192, 10240, Sk_max - 1, Sk_max}):
        if sk > Sk_max:
            continue
        assert lib.attn_bwd_block_dkdv(A, 2 * A, 3 * A, 4 * A, 5 * A, 5 * A, W, need, B, Hq, Hkv, Sq, sk, D, 1,
                                       0, 0, 0.1, None) == 9, sk
        assert lib.attn_bwd_block_dq(A, 2 * A, 3 * A, 4 * A, A + 256, need, B, Hq, Hkv, Sq, sk, D, 1, 0, 0, 0.1,
                                     None) == 9, sk


def test_noalloc_rejects_before_touching_the_gpu():
    """attn_bwd_noalloc validates like attn_bwd, and rejects sizes whose workspace exceeds its
    fixed scratch (ATTN_ERR_SCRATCH_LIMIT) before looking the scratch up."""
    lib = tam.load()
    p = [A, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A, 7 * A, 8 * A, 9 * A]
    assert lib.attn_bwd_noalloc(*p, 1, 32, 8, 32768, 128, 1, 0.1, None) == 10
    assert tam.attn_bwd_workspace_bytes(1, 32, 8, 32768, 128) > tam.NOALLOC_SCRATCH_BYTES
    assert lib.attn_bwd_noalloc(0, *p[1:], 1, 4, 2, 128, 128, 1, 0.1, None) == 1
    assert lib.attn_bwd_noalloc(*p, 1, 4, 3, 128, 128, 1, 0.1, None) == 2
    assert lib.attn_bwd_noalloc(*p, 1, 4, 2, 128, 96, 1, 0.1, None) == 3
    assert lib.attn_bwd_noalloc(*p, 1, 4, 2, 128, 128, 1, float("inf"), None) == 4
    assert lib.attn_bwd_noalloc(*p[:6], A + 8, *p[7:], 1, 4, 2, 128, 128, 1, 0.1, None) == 5
    assert lib.attn_bwd_noalloc(*p, 1, 4, 2, 128, 128, 2, 0.1, None) == 8
    assert lib.attn_bwd_noalloc(*p[:6], A + 64, *p[7:], 1, 4, 2, 128, 128, 1, 0.1, None) == 9   # dq on q
    assert lib.attn_bwd_noalloc(*p[:8], 8 * A + 64, 1, 4, 2, 128, 128, 1, 0.1, None) == 9       # dv on dk


# ---------------------------------------------------------------------------
# decode (attn_decode.h): validation only
# ---------------------------------------------------------------------------
def test_decode_rejects():
    lib = tam.load()
    B, Hq, Hkv, Sq, Sk, D = 2, 8, 2, 4, 1000, 128
    need = tam.attn_decode_workspace_bytes(B, Hq, Hkv, Sq, Sk, D)
    W = 64 * A
    ok = (A, 2 * A, 3 * A, 4 * A, 5 * A, W, need)
    assert lib.attn_decode(*ok, B, Hq, Hkv, 33, Sk, D, 1, 0.1, None) == 2        # g * Sq = 132 > 128
    assert lib.attn_decode(*ok, B, Hq, Hkv, Sq, 3, D, 1, 0.1, None) == 2         # Sq > Sk
    assert lib.attn_decode(*ok, B, 6, 4, Sq, Sk, D, 1, 0.1, None) == 2           # Hq % Hkv
    assert lib.attn_decode(*ok, B, Hq, Hkv, Sq, Sk, 80, 1, 0.1, None) == 3
    assert lib.attn_decode(*ok, B, Hq, Hkv, Sq, Sk, D, 5, 0.1, None) == 8
    assert lib.attn_decode(*ok, B, Hq, Hkv, Sq, Sk, D, 1, float("inf"), None) == 4
    assert lib.attn_decode(A, 2 * A, 3 * A, 4 * A, 5 * A, W, need - 1, B, Hq, Hkv, Sq, Sk, D, 1, 0.1, None) == 6
    assert lib.attn_decode(A, 2 * A, 3 * A, A + 64, 5 * A, W, need, B, Hq, Hkv, Sq, Sk, D, 1, 0.1, None) == 9
    assert lib.attn_decode(A, 2 * A + 2, 3 * A, 4 * A, 5 * A, W, need, B, Hq, Hkv, Sq, Sk, D, 1, 0.1, None) == 5
    assert lib.attn_decode(0, 2 * A, 3 * A, 4 * A, 5 * A, W, need, B, Hq, Hkv, Sq, Sk, D, 1, 0.1, None) == 1
    with pytest.raises(tam.AttnError):
        tam.attn_decode_workspace_bytes(B, Hq, Hkv, 33, Sk, D)                    # g * Sq = 132 > 128
    assert tam.attn_decode_workspace_bytes(1, 64, 8, 16, 4096, 128) > 0


# ---------------------------------------------------------------------------
# dropout (attn_dropout.h): validation only
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("p", [-0.1, 0.999, 1.0, float("nan"), float("inf")])
def test_dropout_rejects_bad_probability(p):
    lib = tam.load()
    assert lib.attn_fwd_dropout(A, 2 * A, 3 * A, 4 * A, 5 * A, 1, 4, 2, 128, 128, 1, 0.1, p, 7, None) == 4
    need = tam.attn_bwd_workspace_bytes(1, 4, 2, 128, 128)
    assert lib.attn_bwd_dropout(A, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A, 7 * A, 8 * A, 9 * A, 16 * A, need, 1, 4, 2, 128,
                                128, 1, 0.1, p, 7, None) == 4


def test_dropout_other_errors_match_attn_fwd():
    lib = tam.load()
    assert lib.attn_fwd_dropout(0, 2 * A, 3 * A, 4 * A, 5 * A, 1, 4, 2, 128, 128, 1, 0.1, 0.2, 7, None) == 1
    assert lib.attn_fwd_dropout(A, 2 * A, 3 * A, 4 * A, 5 * A, 1, 4, 3, 128, 128, 1, 0.1, 0.2, 7, None) == 2
    assert lib.attn_fwd_dropout(A, 2 * A, 3 * A, A, 5 * A, 1, 4, 2, 128, 128, 1, 0.1, 0.2, 7, None) == 9


# ---------------------------------------------------------------------------
# rotary embedding (attn_rope.h): validation only
# ---------------------------------------------------------------------------
def test_rope_rejects():
    lib = tam.load()
    B, Hq, Hkv, S, D = 1, 4, 2, 128, 128
    need = tam.attn_rope_workspace_bytes(B, Hq, Hkv, S, D)
    assert need > tam.attn_bwd_workspace_bytes(B, Hq, Hkv, S, D)
    W = 64 * A
    for base in (0.0, -1.0, float("nan"), float("inf")):
        assert lib.attn_fwd_rope(A, 2 * A, 3 * A, 4 * A, 5 * A, W, need, B, Hq, Hkv, S, D, 1, 0.1, base, None) == 4
        assert lib.attn_bwd_rope(A, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A, 7 * A, 8 * A, 9 * A, W, need, B, Hq, Hkv, S, D,
                                 1, 0.1, base, None) == 4
    assert lib.attn_fwd_rope(A, 2 * A, 3 * A, 4 * A, 5 * A, W, need - 1, B, Hq, Hkv, S, D, 1, 0.1, 1e4, None) == 6
    assert lib.attn_fwd_rope(A, 2 * A, 3 * A, 4 * A, 5 * A, A + 128, need, B, Hq, Hkv, S, D, 1, 0.1, 1e4, None) == 9
    assert lib.attn_bwd_rope(A, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A, 7 * A, 8 * A, 9 * A, W, 16, B, Hq, Hkv, S, D, 1, 0.1,
                             1e4, None) == 6
    assert lib.attn_fwd_rope(A, 2 * A, 3 * A, 4 * A, 5 * A, W, need, B, Hq, Hkv, S, 96, 1, 0.1, 1e4, None) == 3
