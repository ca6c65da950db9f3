"""C-ABI tests that need no GPU: the library loads, exports every symbol the
header declares, plans sensible geometry, and rejects invalid arguments
before touching the HIP runtime (no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dyt.h")


@pytest.fixture(scope="module")
def dyt():
    import __graft_entry__ as ge
    ge._ensure_built()
    import bwd_dyt_forward_amd as m
    return m


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(dyt_[a-z_]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_expected_entry_points():
    assert _declared_functions() == sorted([
        "dyt_forward", "dyt_backward", "dyt_backward_partials", "dyt_backward_finish",
        "dyt_backward_workspace_size", "dyt_status_string", "dyt_abi_version", "dyt_get_plan",
        "dyt_forward_residual", "dyt_backward_residual", "dyt_backward_residual_partials",
        "dyt_get_forward_plan", "dyt_forward_strided", "dyt_backward_strided",
        "dyt_get_forward_residual_plan", "dyt_build_id", "dyt_backward_noalloc",
        "dyt_xcd_hint", "dyt_set_xcd_flip_override"])


def test_xcd_flip_override_accepts_only_a_parity_or_minus_one(dyt):
    """Host-only: the override takes -1, 0 or 1; anything else is rejected."""
    for v in (2, -2, 7):
        assert dyt.lib.dyt_set_xcd_flip_override(v) == 1   # DYT_ERR_INVALID_ARG
    for v in (0, 1, -1):
        assert dyt.lib.dyt_set_xcd_flip_override(v) == 0


def test_library_exports_every_declared_symbol(dyt):
    for name in _declared_functions():
        assert hasattr(dyt.lib, name), name
    # and they are real dynamic symbols of the .so
    out = os.popen(f"nm -D --defined-only {dyt.LIB_FILE}").read()
    for name in _declared_functions():
        assert re.search(rf"\bT {name}\b", out), f"{name} not exported"


def test_no_cpu_fallback_in_product_path():
    """The package's Python code calls only the C ABI (no oracle, no numpy math)."""
    pkg = os.path.join(ROOT, "bwd_dyt_forward_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            src = open(os.path.join(pkg, fn)).read()
            assert "oracle" not in src.replace("oracle/", ""), fn
            assert "torch.tanh" not in src and "np.tanh" not in src, fn


def test_version_and_status_strings(dyt):
    assert dyt.dyt_abi_version() == 7
    names = [dyt.dyt_status_string(i) for i in range(6)]
    assert names == ["DYT_OK", "DYT_ERR_INVALID_ARG", "DYT_ERR_UNSUPPORTED_DTYPE",
                     "DYT_ERR_WORKSPACE_TOO_SMALL", "DYT_ERR_MISALIGNED", "DYT_ERR_HIP"]
    assert dyt.dyt_status_string(99) == "DYT_ERR_UNKNOWN"


CONFIG_SHAPES = [
    (1024, 64, "f32"), (65537, 16, "bf16"), (100003, 17, "f32"), (100003, 100, "f32"),
    (100003, 255, "f32"), (32768, 4096, "bf16"), (4194304, 32, "bf16"),
    (65537, 16, "f16"), (32768, 4096, "f16"), (1031, 300, "f16"),
]


RAGGED_SHAPES = [(5, 4095, "bf16"), (3, 10001, "bf16"), (2, 2051, "f32"), (9, 3001, "f16"),
                 (40, 4097, "f32"), (9, 20003, "bf16")]


@pytest.mark.parametrize("M,N,xdt", CONFIG_SHAPES)
@pytest.mark.parametrize("vec", [True, False])
def test_plan_invariants(dyt, M, N, xdt, vec):
    p = dyt.dyt_get_plan(M, N, xdt, "f32", vec)
    sx = 4 if xdt == "f32" else 2       # bf16 and f16 are both 2 bytes
    cap = p["block"] * p["vec"] * p["slots"]
    assert p["block"] == 256
    assert p["vec"] == (16 // sx if vec else 1)
    # tiling and workspace layout do not depend on the kernel variant
    q = dyt.dyt_get_plan(M, N, xdt, "f32", not vec)
    for key in ("packed", "rows_per_tile", "tile_elems", "col_blocks", "tiles", "fwd_grid",
                "bwd_grid", "ws_row", "ws_bytes"):
        assert p[key] == q[key], key
    assert 1 <= p["tile_elems"] <= cap <= 8192
    assert p["slots"] in ((1, 2, 3, 4) if vec else (16, 32))
    if p["packed"]:
        R = p["rows_per_tile"]
        assert p["tile_elems"] == R * N and p["col_blocks"] == 1
        assert p["tiles"] == -(-M // R)
        # every tile starts at the same column phase of a 16-byte vector
        assert (R * N * sx) % 16 == 0
    else:
        assert p["rows_per_tile"] == 1
        assert p["col_blocks"] * p["tile_elems"] >= N > (p["col_blocks"] - 1) * p["tile_elems"]
        assert p["tiles"] == M * p["col_blocks"]
        assert p["bwd_grid"] % p["col_blocks"] == 0 and p["fwd_grid"] % p["col_blocks"] == 0
        # pass 1 writes whole column groups of its partial row as 16-byte stores
        assert p["tile_elems"] % 4 == 0 and p["tile_elems"] % p["vec"] == 0
    # fwd_grid is the forward plan's grid, over the forward's own tiles
    f = dyt.dyt_get_forward_plan(M, N, xdt, "f32", vec)
    assert 1 <= p["fwd_grid"] <= f["tiles"] and 1 <= p["bwd_grid"] <= p["tiles"]
    wcols = N if p["packed"] else p["tile_elems"]
    assert p["ws_row"] >= 2 * wcols + 1 and p["ws_row"] % 32 == 0   # whole 128-byte lines
    assert p["ws_bytes"] == p["bwd_grid"] * p["ws_row"] * 4
    assert p["fin_grid"] == -(-(2 * N + 1) // 64)
    ws = dyt.dyt_backward_workspace_size(M, N, xdt, "f32")
    assert ws == -(-p["ws_bytes"] // 16) * 16


def test_plan_uses_1d_grid_beyond_65535_rows(dyt):
    """More than 65,535 rows: still one grid dimension, tiles cover every row."""
    p = dyt.dyt_get_plan(65537, 16, "bf16", "f32")
    assert p["tiles"] * p["rows_per_tile"] >= 65537
    p = dyt.dyt_get_plan(10 ** 7, 4096, "bf16", "f32")
    assert p["tiles"] == 10 ** 7 and p["bwd_grid"] <= 4096


@pytest.mark.parametrize("M,N,xdt", CONFIG_SHAPES + RAGGED_SHAPES + [(7, 5000, "f32"), (3, 20000, "bf16"),
                                                     (1, 1, "f16")])
@pytest.mark.parametrize("vec", [True, False])
def test_forward_plan_invariants(dyt, M, N, xdt, vec):
    """The forward tiles independently of the backward, with the same rules."""
    p = dyt.dyt_get_forward_plan(M, N, xdt, "f32", vec)
    b = dyt.dyt_get_plan(M, N, xdt, "f32", vec)
    sx = 4 if xdt == "f32" else 2
    assert p["fwd_grid"] == b["fwd_grid"] and p["ws_bytes"] == 0 and p["bwd_grid"] == 0
    assert p["packed"] == b["packed"] and p["vec"] == b["vec"]
    assert 1 <= p["tile_elems"] <= p["block"] * p["vec"] * p["slots"] <= 8192
    if p["packed"]:
        R = p["rows_per_tile"]
        assert p["tile_elems"] == R * N and p["tiles"] == -(-M // R)
        assert (R * N * sx) % 16 == 0
    else:
        assert p["col_blocks"] * p["tile_elems"] >= N > (p["col_blocks"] - 1) * p["tile_elems"]
        assert p["tiles"] == M * p["col_blocks"] and p["fwd_grid"] % p["col_blocks"] == 0
    assert 1 <= p["fwd_grid"] <= p["tiles"]


@pytest.mark.parametrize("M,N,xdt", RAGGED_SHAPES)
def test_ragged_rows_take_the_vector_kernels(dyt, M, N, xdt):
    """Rows whose length is not a multiple of the vector width are cut into
    whole-vector column blocks (the kernels shift each row's last vector)."""
    v = 4 if xdt == "f32" else 8
    for p in (dyt.dyt_get_plan(M, N, xdt, "f32"), dyt.dyt_get_forward_plan(M, N, xdt, "f32")):
        assert not p["packed"] and p["vec"] == v and N % v != 0
        assert p["tile_elems"] % v == 0 and p["tile_elems"] <= p["block"] * v * p["slots"]
        last = N - (p["col_blocks"] - 1) * p["tile_elems"]
        assert 1 <= last <= p["tile_elems"]


@pytest.mark.parametrize("M,N,xdt", [(3, 261121, "f32"), (3, 522241, "bf16"), (2, 522242, "f16")])
def test_short_last_block_shapes(dyt, M, N, xdt):
    """The GPU tests' shapes whose last column block is shorter than one
    vector in the backward or forward plan (the shifted vector then reaches
    into the previous block)."""
    v = 4 if xdt == "f32" else 8
    lasts = []
    for p in (dyt.dyt_get_plan(M, N, xdt, "f32"), dyt.dyt_get_forward_plan(M, N, xdt, "f32")):
        assert not p["packed"]
        lasts.append(N - (p["col_blocks"] - 1) * p["tile_elems"])
    assert min(lasts) >= 1 and any(last < v for last in lasts)


def _occ(p, N):
    cap = p["block"] * p["vec"] * p["slots"]
    return p["tile_elems"] / cap if p["packed"] else N / (p["col_blocks"] * cap)


# (M, N, x dtype, layout, K) of the backward and forward plans after
# occupancy re-tiling (the GPU tests run these shapes)
RETILED = [(2800, 1500, "bf16", "packed", 3), (1100, 5120, "bf16", "segments", 3),
           (2000, 2560, "bf16", "packed", 4), (1700, 2560, "f32", "segments", 3),
           (2100, 4104, "f32", "segments", 3), (1400, 3072, "bf16", "packed", 3)]


@pytest.mark.parametrize("M,N,xdt,layout,k", RETILED)
def test_occupancy_retiling(dyt, M, N, xdt, layout, k):
    """Widths that fill the default tiles poorly are re-tiled: K >= 2 slots,
    at least as many slots carrying data as the default tiling would."""
    p = dyt.dyt_get_plan(M, N, xdt, "f32")
    assert p["slots"] == k and bool(p["packed"]) == (layout == "packed")
    assert _occ(p, N) >= 0.66 and p["tile_elems"] <= 8192


def test_headline_plans_unchanged(dyt):
    """The measured plans of 32,768 x 4,096 and 4,194,304 x 32 bfloat16."""
    b = dyt.dyt_get_plan(32768, 4096, "bf16", "f32")
    f = dyt.dyt_get_forward_plan(32768, 4096, "bf16", "f32")
    assert (b["packed"], b["slots"], b["tile_elems"], b["col_blocks"], b["bwd_grid"]) == (0, 2, 4096, 1, 256)
    assert (f["packed"], f["slots"], f["tile_elems"], f["col_blocks"], f["fwd_grid"]) == (0, 1, 2048, 2, 1024)
    b = dyt.dyt_get_plan(4194304, 32, "bf16", "f32")
    f = dyt.dyt_get_forward_plan(4194304, 32, "bf16", "f32")
    assert (b["packed"], b["slots"], b["rows_per_tile"], b["tile_elems"], b["bwd_grid"]) == (1, 2, 128, 4096, 256)
    assert (f["packed"], f["slots"], f["rows_per_tile"], f["tile_elems"], f["fwd_grid"]) == (1, 2, 128, 4096, 256)
    # the 4,194,304 x 32 forward walks flat (packed 2-byte tiles of two slots)
    # from any base; its tiles are what row-strided launches run
    assert f["flat"] == 1 and f["flat_grid"] == 256 and f["flat_aligned_only"] == 0
    assert dyt.dyt_get_forward_plan(32768, 4096, "bf16", "f32")["flat"] == 0


def test_tile_table_covers_every_dtype_width_and_size():
    """Every (x dtype, N, M*N) resolves to exactly one row of the measured table."""
    import re
    src = open(os.path.join(ROOT, "bwd_dyt_forward_amd", "csrc", "dyt_tune_table.inc")).read()
    rows = re.findall(r"\{(DYT_\w+), (\d+), (\d+), (\d+), (\d+), \{(\d+), (\d+), (\d+)\}, "
                      r"\{(\d+), (\d+), (\d+)\}, \{(\d+), (\d+), (\d+)\}\}", src)
    assert rows
    for dt in ("DYT_F32", "DYT_BF16", "DYT_F16"):
        mine = [r for r in rows if r[0] == dt]
        spans = sorted({(int(r[1]), int(r[2])) for r in mine})
        assert spans[0][0] == 1 and spans[-1][1] >= 1 << 30
        for (a, b), (c, d) in zip(spans, spans[1:]):
            assert c == b + 1, (dt, b, c)
        for lo, hi in spans:
            sizes = sorted((int(r[3]), int(r[4])) for r in mine if (int(r[1]), int(r[2])) == (lo, hi))
            assert sizes[0][0] <= 1 and sizes[-1][1] >= 1 << 62
            for (a, b), (c, d) in zip(sizes, sizes[1:]):
                assert c == b + 1, (dt, lo, b, c)
    for r in rows:
        v = list(map(int, r[5:]))
        for mt, kc, g in (v[0:3], v[3:6], v[6:9]):
            assert mt >= 1 and kc in (0, 1, 2, 4) and 64 <= g <= 4096


def test_plan_narrow_rows_are_packed(dyt):
    for N in (1, 2, 3, 16, 17, 32, 64, 100, 255, 256):
        p = dyt.dyt_get_plan(100003, N, "bf16", "f32")
        assert p["packed"] == 1 and p["rows_per_tile"] >= 2, N
    p = dyt.dyt_get_plan(32768, 4096, "bf16", "f32")
    assert p["packed"] == 0 and p["col_blocks"] == 1
    p = dyt.dyt_get_plan(64, 20000, "bf16", "f32")
    assert p["packed"] == 0 and p["col_blocks"] >= 5


def test_workspace_size_empty_and_invalid(dyt):
    assert dyt.dyt_backward_workspace_size(0, 64, "f32", "f32") == 0
    assert dyt.dyt_backward_workspace_size(64, 0, "f32", "f32") == 0
    assert dyt.dyt_backward_workspace_size(-1, 64, "f32", "f32") == 0
    assert dyt.dyt_backward_workspace_size(4, 4, 7, 0) == 0


# ----------------------------------------------------- error paths (no HIP)
# Pointer values below are never dereferenced: validation fails first.
A16 = 0x10000          # a 16-byte aligned fake device address
F32, BF16 = 0, 1
E_OK, E_ARG, E_DT, E_WS, E_AL = 0, 1, 2, 3, 4


def _fwd(dyt, x=A16, a=A16 + 0x100000, g=A16 + 0x200000, b=A16 + 0x300000, y=A16 + 0x400000,
         M=4, N=4, xdt=F32, pdt=F32):
    return dyt.lib.dyt_forward(x, a, g, b, y, M, N, xdt, pdt, None)


def _bwd(dyt, x=A16, dy=A16 + 0x100000, a=A16 + 0x200000, g=A16 + 0x300000, dx=A16 + 0x400000,
         da=A16 + 0x500000, dg=A16 + 0x600000, db=A16 + 0x700000, ws=A16 + 0x800000,
         wsb=1 << 20, M=4, N=4, xdt=F32, pdt=F32):
    return dyt.lib.dyt_backward(x, dy, a, g, dx, da, dg, db, ws, wsb, M, N, xdt, pdt, None)


def test_forward_error_codes(dyt):
    assert _fwd(dyt, xdt=3) == E_DT
    assert _fwd(dyt, pdt=-1) == E_DT
    assert _fwd(dyt, M=-1) == E_ARG
    assert _fwd(dyt, N=-3) == E_ARG
    assert _fwd(dyt, M=2 ** 62, N=2 ** 10) == E_ARG                # size overflow
    for kw in ("x", "a", "g", "b", "y"):
        assert _fwd(dyt, **{kw: None}) == E_ARG, kw
    assert _fwd(dyt, x=A16 + 2) == E_AL                            # f32 needs 4-byte alignment
    assert _fwd(dyt, y=A16 + 1, xdt=BF16) == E_AL
    assert _fwd(dyt, g=A16 + 0x200002) == E_AL
    assert _fwd(dyt, y=A16 + 8) == E_ARG                           # y overlaps x
    assert _fwd(dyt, y=A16 + 0x200000 - 8) == E_ARG                # y overlaps gamma
    # empty problems enqueue nothing and accept NULL pointers
    assert _fwd(dyt, x=None, a=None, g=None, b=None, y=None, M=0) == E_OK
    assert _fwd(dyt, x=None, a=None, g=None, b=None, y=None, N=0) == E_OK


def test_backward_error_codes(dyt):
    need = dyt.dyt_backward_workspace_size(4, 4, F32, F32)
    assert need > 0
    assert _bwd(dyt, xdt=5) == E_DT
    assert _bwd(dyt, M=-1) == E_ARG
    for kw in ("x", "dy", "a", "g", "dx", "da", "dg", "db", "ws"):
        assert _bwd(dyt, **{kw: None}) == E_ARG, kw
    assert _bwd(dyt, wsb=need - 1) == E_WS
    assert _bwd(dyt, ws=A16 + 0x800004) == E_AL                    # workspace needs 16 bytes
    assert _bwd(dyt, dx=A16 + 0x400002) == E_AL
    assert _bwd(dyt, da=A16 + 0x500001, pdt=BF16) == E_AL
    assert _bwd(dyt, dx=A16 + 0x100000) == E_ARG                   # dx aliases dy
    assert _bwd(dyt, dg=A16 + 0x700000) == E_ARG                   # dgamma aliases dbeta
    assert _bwd(dyt, ws=A16) == E_ARG                              # workspace aliases x
    # dalpha is always written, so it is always required
    assert _bwd(dyt, da=None, M=0) == E_ARG


def test_split_backward_error_codes(dyt):
    L = dyt.lib
    need = dyt.dyt_backward_workspace_size(4, 4, F32, F32)
    ws = A16 + 0x800000
    # pass 1: x, dy, alpha, gamma, dx and workspace required; no param grads involved
    assert L.dyt_backward_partials(None, A16 + 0x100000, A16 + 0x200000, A16 + 0x300000,
                                   A16 + 0x400000, ws, need, 4, 4, F32, F32, None) == E_ARG
    assert L.dyt_backward_partials(A16, A16 + 0x100000, A16 + 0x200000, A16 + 0x300000,
                                   A16 + 0x400000, ws, need - 1, 4, 4, F32, F32, None) == E_WS
    assert L.dyt_backward_partials(A16, A16 + 0x100000, A16 + 0x200000, A16 + 0x300000,
                                   A16 + 0x100000, ws, need, 4, 4, F32, F32, None) == E_ARG
    # pass 2: workspace and the three gradient outputs
    assert L.dyt_backward_finish(ws, need, None, A16, A16 + 64, 4, 4, F32, F32, None) == E_ARG
    assert L.dyt_backward_finish(ws, need, A16 + 128, None, A16 + 64, 4, 4, F32, F32, None) == E_ARG
    assert L.dyt_backward_finish(ws, need - 16, A16 + 128, A16, A16 + 64, 4, 4, F32, F32, None) == E_WS
    assert L.dyt_backward_finish(ws, need, A16 + 128, A16, A16 + 8, 4, 4, F32, F32, None) == E_ARG
    assert L.dyt_backward_finish(ws, need, A16 + 128, A16, A16 + 64, 4, 4, 9, F32, None) == E_DT


def _fres(dyt, x=A16, r=A16 + 0x100000, a=A16 + 0x200000, g=A16 + 0x300000, b=A16 + 0x400000,
          h=A16 + 0x500000, y=A16 + 0x600000, M=4, N=4, xdt=F32, pdt=F32):
    return dyt.lib.dyt_forward_residual(x, r, a, g, b, h, y, M, N, xdt, pdt, None)


def _bres(dyt, h=A16, dy=A16 + 0x100000, dres=A16 + 0x200000, a=A16 + 0x300000,
          g=A16 + 0x400000, dh=A16 + 0x500000, da=A16 + 0x600000, dg=A16 + 0x700000,
          db=A16 + 0x800000, ws=A16 + 0x900000, wsb=1 << 20, M=4, N=4, xdt=F32, pdt=F32):
    return dyt.lib.dyt_backward_residual(h, dy, dres, a, g, dh, da, dg, db, ws, wsb, M, N, xdt, pdt,
                                         None)


def test_strided_error_codes(dyt):
    L = dyt.lib
    x, a, g, b, y = A16, A16 + 0x100000, A16 + 0x200000, A16 + 0x300000, A16 + 0x400000
    # pitch below N or not positive
    assert L.dyt_forward_strided(x, 3, a, g, b, y, 4, 4, 4, F32, F32, None) == E_ARG
    assert L.dyt_forward_strided(x, 4, a, g, b, y, 0, 4, 4, F32, F32, None) == E_ARG
    # a strided x whose span reaches y: overlap (4 rows of pitch 0x10000 floats)
    assert L.dyt_forward_strided(x, 0x10000, a, g, b, A16 + 0x80000, 4, 4, 4, F32, F32, None) == E_ARG
    assert L.dyt_forward_strided(x + 2, 8, a, g, b, y, 4, 4, 4, F32, F32, None) == E_AL
    assert L.dyt_forward_strided(None, 8, a, g, b, y, 4, 4, 4, F32, F32, None) == E_ARG
    assert L.dyt_forward_strided(None, 8, None, None, None, None, 4, 0, 4, F32, F32, None) == E_OK
    need = dyt.dyt_backward_workspace_size(4, 4, F32, F32)
    args = [A16, 8, A16 + 0x100000, 8, A16 + 0x200000, A16 + 0x300000, A16 + 0x400000, 8,
            A16 + 0x500000, A16 + 0x600000, A16 + 0x700000, A16 + 0x800000, need, 4, 4, F32, F32, None]
    bad = list(args); bad[3] = 2
    assert L.dyt_backward_strided(*bad) == E_ARG                     # dy pitch < N
    bad = list(args); bad[6] = A16 + 0x100010
    assert L.dyt_backward_strided(*bad) == E_ARG                     # dx inside dy's span
    bad = list(args); bad[12] = need - 1
    assert L.dyt_backward_strided(*bad) == E_WS


def test_residual_forward_error_codes(dyt):
    assert _fres(dyt, xdt=3) == E_DT
    assert _fres(dyt, M=-1) == E_ARG
    for kw in ("x", "r", "a", "g", "b", "h", "y"):
        assert _fres(dyt, **{kw: None}) == E_ARG, kw
    assert _fres(dyt, r=A16 + 0x100002) == E_AL
    assert _fres(dyt, h=A16 + 0x500001, xdt=BF16) == E_AL
    assert _fres(dyt, h=A16) == E_ARG                              # h aliases x (no in-place)
    assert _fres(dyt, h=A16 + 0x100000) == E_ARG                   # h aliases r
    assert _fres(dyt, y=A16 + 0x500000) == E_ARG                   # y aliases h
    assert _fres(dyt, y=A16 + 0x100008) == E_ARG                   # y overlaps r
    assert _fres(dyt, x=None, r=None, a=None, g=None, b=None, h=None, y=None, M=0) == E_OK


def test_residual_backward_error_codes(dyt):
    need = dyt.dyt_backward_workspace_size(4, 4, F32, F32)
    assert _bres(dyt, xdt=5) == E_DT
    for kw in ("h", "dy", "dres", "a", "g", "dh", "da", "dg", "db", "ws"):
        assert _bres(dyt, **{kw: None}) == E_ARG, kw
    assert _bres(dyt, wsb=need - 1) == E_WS
    assert _bres(dyt, dres=A16 + 0x200002) == E_AL
    assert _bres(dyt, dh=A16 + 0x200000) == E_ARG                  # dh aliases dres (no in-place)
    assert _bres(dyt, ws=A16 + 0x200000) == E_ARG                  # workspace aliases dres
    L = dyt.lib
    assert L.dyt_backward_residual_partials(A16, A16 + 0x100000, None, A16 + 0x300000,
                                            A16 + 0x400000, A16 + 0x500000, A16 + 0x900000, need,
                                            4, 4, F32, F32, None) == E_ARG
    assert L.dyt_backward_residual_partials(A16, A16 + 0x100000, A16 + 0x200000, A16 + 0x300000,
                                            A16 + 0x400000, A16 + 0x200000, A16 + 0x900000, need,
                                            4, 4, F32, F32, None) == E_ARG


def test_module_constructs_on_cpu(dyt):
    """The nn.Module drop-in builds its parameters without a GPU."""
    layer = dyt.DyT(16, alpha_init=0.25)
    assert layer.alpha.shape == (1,) and float(layer.alpha[0]) == 0.25
    assert layer.weight.shape == (16,) and bool((layer.weight == 1).all())
    assert layer.bias.shape == (16,) and not layer.bias.any()
    assert "16" in repr(layer)


def test_residual_module_constructs_on_cpu(dyt):
    layer = dyt.DyTResidual(8, alpha_init=0.5)
    assert layer.weight.shape == (8,) and isinstance(layer, dyt.DyT)


def test_c_caller_builds_links_and_runs(tmp_path):
    """The header is plain C99 and the library is callable from C without
    Python (only calls that never reach the GPU)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    pkg = os.path.join(ROOT, "bwd_dyt_forward_amd")
    exe = str(tmp_path / "abi_check")
    src = os.path.join(ROOT, "tests", "c_abi", "abi_check.c")
    cc = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                         f"-I{os.path.join(ROOT, 'include')}", src, "-o", exe, f"-L{pkg}", "-ldyt",
                         f"-Wl,-rpath,{pkg}"], capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "FAIL" not in run.stdout and run.stdout.count("ok ") == 10


def test_library_build_id_matches_current_sources(dyt):
    """The library under test was built from exactly these sources: the id
    it returns, the id embedded in the file and the hash of the sources next
    to it agree (the binding refuses to load otherwise)."""
    from bwd_dyt_forward_amd import build
    want = build.source_hash()
    assert dyt.lib.dyt_build_id().decode() == want
    assert build.built_id() == want
    assert not build.is_stale()


def test_loader_checks_the_build_id_unless_told_otherwise(dyt):
    """_load refuses the in-tree library when told to expect a variant build
    (other flags, so another id), and loads it with any_sources (how
    bench.py --variants lib:PATH compares prebuilt libraries from other
    sources); the ABI version is checked either way."""
    from bwd_dyt_forward_amd import _lib, build
    with pytest.raises(ImportError, match="build id"):
        _lib._load(build.LIB_PATH, ["-DDYT_FWD_U=1"])
    lib = _lib._load(build.LIB_PATH, ["-DDYT_FWD_U=1"], any_sources=True)
    assert lib.dyt_abi_version() == _lib.ABI_VERSION
    assert lib.dyt_build_id().decode() == build.source_hash()


def test_source_hash_follows_code_and_flags_not_comments(tmp_path, monkeypatch):
    from bwd_dyt_forward_amd import build
    src = tmp_path / "k.hpp"
    src.write_text("int a = 1;  // one\n")
    monkeypatch.setattr(build, "DEPENDS", [str(src)])
    h0 = build.source_hash()
    src.write_text("/* one */ int a =\n 1;\n\n")
    assert build.source_hash() == h0
    src.write_text("int a = 2;\n")
    h1 = build.source_hash()
    assert h1 != h0
    monkeypatch.setattr(build, "HIPCC_FLAGS", [*build.HIPCC_FLAGS, "-ffast-math"])
    assert build.source_hash() != h1
    # a library file carrying another id is stale
    lib = tmp_path / "libx.so"
    lib.write_bytes(b"\x7fELF..." + build.BUILD_ID_MARK + b"0123456789abcdef" + b"\0")
    assert build.built_id(str(lib)) == "0123456789abcdef"
    assert build.is_stale(str(lib))
    assert build.built_id(str(tmp_path / "missing.so")) is None


def test_noalloc_size_limit_is_checked_before_any_hip_call(dyt):
    """dyt_backward_noalloc refuses a problem whose partial rows exceed its
    static scratch with DYT_ERR_WORKSPACE_TOO_SMALL, before touching the GPU
    (so this runs without one); rows of up to 20,480 columns fit."""
    limit = dyt._lib.NOALLOC_SCRATCH_BYTES
    assert dyt.dyt_backward_workspace_size(1, 1 << 22, "f32", "f32") > limit
    st = dyt.lib.dyt_backward_noalloc(None, None, None, None, None, None, None, None, 1, 1 << 22,
                                      dyt.DYT_F32, dyt.DYT_F32, None)
    assert st == 3
    assert dyt.lib.dyt_backward_noalloc(None, None, None, None, None, None, None, None, 4, 4, 99,
                                        dyt.DYT_F32, None) == 2
    for xdt in ("f32", "bf16", "f16"):
        for N in list(range(1, 20481, 7)) + [4096, 8192, 16384, 20480]:
            for M in (1000, 100003, 1 << 22):
                assert dyt.dyt_backward_workspace_size(M, N, xdt, "f32") <= 13 << 20, (M, N, xdt)
