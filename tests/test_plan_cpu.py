"""Launch plans over random shapes (pure host functions, no GPU): the tiling
invariants the kernels rely on, for the forward and backward plans and the
element-wise variant, and the slot rule of the row-segment kernels (each
slot's vector lies inside the row; every column of a segment is owned by
exactly one slot's own elements), restated from the kernels' documentation:
slot k of thread t starts at o = (k * 256 + t) * V; a slot is used if
o < segment length L; a used slot that would run past L is shifted back to
end at L (its first lo = o - (L - V) elements are another slot's); unused
slots recompute the segment's first whole vector."""
import numpy as np
import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

VEC = {"f32": 4, "bf16": 8, "f16": 8}


@pytest.fixture(scope="module")
def dyt():
    import __graft_entry__ as ge
    ge._ensure_built()
    import bwd_dyt_forward_amd as m
    return m


def _check_tiling(p, M, N, v, vector):
    cap = p["block"] * p["vec"] * p["slots"]
    assert p["block"] == 256
    if vector:
        assert p["vec"] == v and p["slots"] in (1, 2, 3, 4)
    else:
        assert p["vec"] == 1 and p["slots"] in (16, 32)
    assert 1 <= p["tile_elems"] <= cap <= 8192
    grid = p["fwd_grid"] if p["bwd_grid"] == 0 else p["bwd_grid"]
    if p["packed"]:
        R = p["rows_per_tile"]
        assert R >= 1 and p["tile_elems"] == R * N and (R * N) % v == 0
        assert p["col_blocks"] == 1 and p["tiles"] == -(-M // R)
        assert 1 <= grid <= p["tiles"]
    else:
        T, nb = p["tile_elems"], p["col_blocks"]
        assert p["rows_per_tile"] == 1 and T % v == 0
        last = N - (nb - 1) * T
        assert 1 <= last <= T
        assert p["tiles"] == M * nb and grid % nb == 0 and nb <= grid <= p["tiles"]


def _slot_rule(L, V, K):
    """(used, off, lo) arrays over all (k, t) for a segment of length L."""
    o = (np.arange(K)[:, None] * 256 + np.arange(256)[None, :]).ravel() * V
    last = min(max(L - V, 1 - V), 8192 - V)
    used = o < L
    full = o + V <= L
    off = np.where(~used, min(last, 0), np.where(full, o, last))
    lo = np.where(used & ~full, o - last, 0)
    return used, off, lo


def _check_segments(p, N):
    V, K, T, nb = p["vec"], p["slots"], p["tile_elems"], p["col_blocks"]
    for b in {0, nb - 1}:
        col_base = b * T
        L = T if b < nb - 1 else N - (nb - 1) * T
        used, off, lo = _slot_rule(L, V, K)
        cols = col_base + off[:, None] + np.arange(V)[None, :]
        assert cols.min() >= 0 and cols.max() < N, "a slot's vector leaves the row"
        own = np.zeros(L, dtype=np.int64)
        for e in range(V):
            sel = used & (e >= lo)
            np.add.at(own, (off[sel] + e), 1)
        assert (own == 1).all(), "a column is not owned exactly once"


def _occupancy(p, N):
    cap = p["block"] * p["vec"] * p["slots"]
    return p["tile_elems"] / cap if p["packed"] else N / (p["col_blocks"] * cap)


def _check_flat(f, M, N, xdt, residual=False):
    """The forward walks flat exactly for rows of a whole number of 16-byte
    vectors, at most 20,480 long, that its tiles fit poorly: filled below
    0.9 (float32 x); for 2-byte x, packed tiles or row segments filled below
    0.85; the residual-fused forward, for rows of at most 8,192, whenever its
    tiles leave a slot empty or are 2-byte packed tiles of two or more
    slots. The grid is one workgroup
    per 1,024 vectors (at least one), at most 256. Only the plain forward's
    2-byte packed tiles of one slot filled at least 0.85 walk flat at
    aligned bases alone. Rows that are not a whole number of vectors walk
    flat (plain and residual forward) when N + V rounded up to 4 is at most 3,584
    (2-byte x, always) or 5,120 (float32 x, below 0.9): four copies of both
    parameters in at most 160 KB of LDS. Float32 rows of the plain forward
    count as filled poorly at any fill beyond 2^26 elements."""
    v = VEC[xdt]
    occ = _occupancy(f, N)
    k2 = xdt != "f32" and f["packed"] and f["slots"] >= 2
    big = not residual and xdt == "f32" and M * N > (1 << 26)
    if residual:
        poor = occ < 1 - 1e-9 or k2
    else:
        poor = (occ < 0.9 or big) if xdt == "f32" else (occ < 0.85 or bool(f["packed"]))
    if N % v:
        fits = -(-(N + v) // 4) * 4 <= (5120 if xdt == "f32" else 3584)
        want = fits and (xdt != "f32" or occ < 0.9 or big)
    else:
        want = N <= (8192 if residual else 20480) and poor
    assert f["flat"] == int(want)
    if want:
        assert f["flat_grid"] == max(1, min(256, -(-(M * N // v) // 1024)))
    else:
        assert f["flat_grid"] == 0
    aligned_only = (want and not residual and N % v == 0 and xdt != "f32" and f["packed"] and f["slots"] == 1
                    and occ >= 0.85)
    assert f["flat_aligned_only"] == int(aligned_only)


@settings(max_examples=300, deadline=None)
@given(M=st.integers(1, 1 << 22), N=st.integers(1, 1 << 20), xdt=st.sampled_from(["f32", "bf16", "f16"]))
def test_plans_hold_their_invariants(dyt, M, N, xdt):
    if M * N > (1 << 36):
        return
    v = VEC[xdt]
    b = dyt.dyt_get_plan(M, N, xdt, "f32")
    f = dyt.dyt_get_forward_plan(M, N, xdt, "f32")
    for p in (b, f):
        _check_tiling(p, M, N, v, True)
        if not p["packed"]:
            _check_segments(p, N)
    _check_flat(f, M, N, xdt)
    assert (b["flat"], b["flat_grid"], b["flat_aligned_only"]) == (f["flat"], f["flat_grid"], f["flat_aligned_only"])
    r = dyt.dyt_get_forward_residual_plan(M, N, xdt, "f32")
    _check_tiling(r, M, N, v, True)
    _check_flat(r, M, N, xdt, residual=True)
    e = dyt.dyt_get_plan(M, N, xdt, "f32", False)
    _check_tiling(e, M, N, v, False)
    assert e["flat"] == 0 and e["flat_grid"] == 0 and e["flat_aligned_only"] == 0
    for key in ("packed", "rows_per_tile", "tile_elems", "col_blocks", "tiles", "bwd_grid", "ws_row", "ws_bytes"):
        assert e[key] == b[key], key
    assert b["ws_row"] >= 2 * (N if b["packed"] else b["tile_elems"]) + 1 and b["ws_row"] % 4 == 0
    assert b["ws_bytes"] == b["bwd_grid"] * b["ws_row"] * 4
    assert dyt.dyt_backward_workspace_size(M, N, xdt, "f32") == -(-b["ws_bytes"] // 16) * 16


@pytest.mark.parametrize("N,xdt", [(261121, "f32"), (522241, "bf16"), (4095, "bf16"), (10001, "f32")])
def test_slot_rule_on_short_and_ragged_segments(dyt, N, xdt):
    """Segments shorter than a vector and ragged row ends keep the rule."""
    for M in (1, 3, 1000):
        for p in (dyt.dyt_get_plan(M, N, xdt, "f32"), dyt.dyt_get_forward_plan(M, N, xdt, "f32")):
            assert not p["packed"]
            _check_segments(p, N)


def test_slot_rule_rejects_the_old_short_segment_offsets():
    """The check above fails for the earlier rule (unused slots at offset 0
    even in a segment shorter than a vector), which wrote past the row end."""
    L, V, K, N, col_base = 1, 4, 1, 261121, 261120
    o = np.arange(256) * V
    used = o < L
    last = L - V
    off = np.where(~used, 0, np.where(o + V <= L, o, last))
    cols = col_base + off[:, None] + np.arange(V)[None, :]
    assert cols.max() >= N
    used2, off2, _ = _slot_rule(L, V, K)
    assert (col_base + off2[:, None] + np.arange(V)[None, :]).max() < N


@pytest.mark.parametrize("N,xdt,flat", [
    (2560, "bf16", 1), (4104, "bf16", 1), (1536, "bf16", 1), (768, "bf16", 1), (2048, "bf16", 1),
    (3072, "bf16", 1), (5120, "bf16", 1), (32, "bf16", 1), (64, "bf16", 1), (4096, "bf16", 0),
    (7168, "bf16", 0), (6144, "bf16", 0), (8192, "bf16", 0),
    (2560, "f32", 1), (4104, "f32", 1), (5120, "f32", 1), (4096, "f32", 1), (10000, "f32", 1),
    (9216, "f32", 1), (13312, "f32", 1), (17408, "f32", 1), (18432, "f32", 1), (20480, "f32", 1),
    (8200, "bf16", 1), (11264, "bf16", 0), (24576, "f32", 0),
    (2560, "f16", 1),
    # rows that are not a whole number of vectors
    (1500, "bf16", 1), (1001, "bf16", 1), (255, "bf16", 1), (17, "bf16", 1), (3, "bf16", 1),
    (2039, "bf16", 1), (2047, "bf16", 1), (3071, "bf16", 1), (3575, "bf16", 1), (3577, "bf16", 0),
    (4095, "bf16", 0), (5111, "bf16", 0),
    (8183, "bf16", 0), (1500, "f16", 1),
    (1501, "f32", 1), (3001, "f32", 1), (5113, "f32", 1), (5117, "f32", 0), (255, "f32", 1), (17, "f32", 1),
    (2043, "f32", 1)])
def test_flat_forward_choice(dyt, N, xdt, flat):
    """Just under 2^27 elements (M = 2^27 // N) the measured choice: for
    2-byte x the flat walk for widths the tiles fill poorly and for rows that
    are not a whole number of vectors, the tiles where they fill; float32
    rows walk flat at any fill beyond 2^26 elements (x larger than the
    last-level cache). Rows whose gamma/beta would not fit the LDS copy
    (24,576 wide, 5,117 wide with its shifted copies) keep the tiles."""
    M = (1 << 27) // N
    f = dyt.dyt_get_forward_plan(M, N, xdt, "f32")
    assert f["flat"] == flat
    _check_flat(f, M, N, xdt)
    assert dyt.dyt_get_forward_plan(M, N, xdt, "f32", False)["flat"] == 0


@pytest.mark.parametrize("N,xdt,flat", [
    (2560, "bf16", 1), (3072, "bf16", 1), (4104, "bf16", 1), (1536, "bf16", 1),
    (4096, "bf16", 0), (32, "bf16", 1), (4095, "bf16", 0), (1500, "bf16", 1), (17, "bf16", 1),
    (2560, "f32", 1), (4104, "f32", 1), (1501, "f32", 1), (255, "f32", 0)])
def test_flat_residual_forward_choice(dyt, N, xdt, flat):
    """The residual-fused forward at 2^27 elements: flat unless its tiles are
    full (and then not 2-byte packed tiles of two or more slots); rows that
    are not a whole number of vectors as in the plain forward."""
    M = (1 << 27) // N
    r = dyt.dyt_get_forward_residual_plan(M, N, xdt, "f32")
    assert r["flat"] == flat
    _check_flat(r, M, N, xdt, residual=True)


@pytest.mark.parametrize("M,N,xdt", [(33, 20000, "f32"), (100, 19456, "f32"), (33, 8200, "bf16"),
                                     (41, 13312, "f32")])
def test_wide_residual_forward_keeps_its_tiles(dyt, M, N, xdt):
    """Rows over 8,192 columns: the plain forward may walk flat (gamma/beta in
    up to 160 KB of LDS), the residual-fused one keeps its tiles, the range
    its flat walk was measured on ending at 8,192."""
    assert dyt.dyt_get_forward_residual_plan(M, N, xdt, "f32")["flat"] == 0
    assert dyt.dyt_get_forward_residual_plan(M, 8192, xdt, "f32")["flat"] in (0, 1)
