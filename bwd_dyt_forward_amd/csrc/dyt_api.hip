// dyt_api.hip - C ABI of the fused DyT layer (declared in include/dyt.h):
// argument validation, launch planning and kernel dispatch on gfx950.
//
// The plan is a pure function of (M, N, dtypes), so the order of every
// floating-point sum, and with it every result bit, is reproducible run to
// run and device to device. The kernel instances are launched from
// dyt_launch_{fwd,bwd}_<dtype>.hip (see dyt_launch.hpp).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <type_traits>

#include "dyt.h"
#include "dyt_launch.hpp"

// Default persistent-grid sizes (workgroups): one 256-thread workgroup per
// compute unit of MI355X (256 CUs). Measured on the 32768 x 4096
// and 4194304 x 32 bfloat16 workloads, one workgroup per CU streamed HBM
// faster than 2-8 per CU (fewer concurrent streams), and grids that are not
// a multiple of the CU count lose to load imbalance. The constants are not
// queried from the device so that the summation order - and every result
// bit - depends on the problem shape only.
#ifndef DYT_FWD_GRID
#define DYT_FWD_GRID 256
#endif
#ifndef DYT_BWD_GRID
#define DYT_BWD_GRID 256
#endif
// Tiles wanted before a packed plan stops shrinking K for more parallelism.
#ifndef DYT_MIN_TILES
#define DYT_MIN_TILES 1024
#endif
// Largest K for row segments (0: the tile capacity's).
#ifndef DYT_WIDE_KCAP
#define DYT_WIDE_KCAP 0
#endif
// The constants above are the defaults; the measured table below overrides
// them per (x dtype, row length) unless built with DYT_TUNE_TABLE=0 (the
// tuner's candidate builds).
#ifndef DYT_TUNE_TABLE
#define DYT_TUNE_TABLE 1
#endif

namespace {

// One row of the offline-measured tile table (bwd_dyt_forward_amd/tune.py
// writes dyt_tune_table.inc): for x dtype `xdt`, row lengths
// n_lo <= N <= n_hi and problem sizes e_lo <= M * N <= e_hi, one setting
// each for the forward, the backward and the residual forward.
// A packed plan takes the largest K that still yields min_tiles tiles, row
// segments use at most kcap slots (0: no cap), and the grid has `grid`
// workgroups. The forward's tiling is independent of the backward's (it has
// no workspace), so the two are tuned separately. A static table keeps each
// plan a pure function of the shape: the summation order, and every result
// bit, never depends on a run-time measurement.
struct TuneDir {
    int64_t min_tiles;
    int kcap;
    int grid;
};
struct TuneEntry {
    int xdt;
    int64_t n_lo, n_hi;
    int64_t e_lo, e_hi;
    TuneDir fwd, bwd, res_fwd;   // plain forward, backward (both kinds), residual forward
};

// Which kernel a plan is for. The backward with and without the residual
// gradient share one plan, so their parameter gradients are bitwise equal.
enum class Dir { Fwd, Bwd, ResFwd };

const TuneEntry kTuneTable[] = {
#include "dyt_tune_table.inc"
};

TuneDir tune_for(int xdt, int64_t M, int64_t N, Dir d) {
    if (DYT_TUNE_TABLE) {
        const int64_t elems = M * N;
        for (const TuneEntry& e : kTuneTable)
            if (e.xdt == xdt && e.n_lo <= N && N <= e.n_hi && e.e_lo <= elems && elems <= e.e_hi)
                return d == Dir::Fwd ? e.fwd : d == Dir::Bwd ? e.bwd : e.res_fwd;
    }
    return TuneDir{DYT_MIN_TILES, DYT_WIDE_KCAP, d == Dir::Bwd ? DYT_BWD_GRID : DYT_FWD_GRID};
}

using dyt::Geo;
using dyt::host::BwdPtrs;
using dyt::host::FwdPtrs;
using dyt::host::Plan;
using dyt::FinGeo;
using dyt::FlatGeo;
using dyt::bf16_t;
using dyt::kBlock;


bool dtype_ok(int d) { return d == DYT_F32 || d == DYT_BF16 || d == DYT_F16; }
int64_t dtype_size(int d) { return d == DYT_F32 ? 4 : 2; }

// Calls f.template operator()<T>() with T the storage type of dtype code d.
template <typename F>
bool with_dtype(int d, F&& f) {
    switch (d) {
        case DYT_F32: return f(float{});
        case DYT_BF16: return f(dyt::bf16_t{});
        case DYT_F16: return f(dyt::f16_t{});
        default: return false;
    }
}
int64_t gcd64(int64_t a, int64_t b) {
    while (b) {
        const int64_t t = a % b;
        a = b;
        b = t;
    }
    return a;
}
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

constexpr int64_t kMaxN = (int64_t)1 << 30;   // row length limit (int32 in-tile offsets)

// Tiling helpers: packed tiles of r whole rows, or row segments in nb column
// blocks, with k vector slots per thread.
void fill_packed(Plan& p, int64_t M, int64_t N, int vec, int k, int64_t r, int64_t grid) {
    p.packed = true;
    p.vec = vec;
    p.slots = k;
    p.R = r;
    p.T = r * N;
    p.nb = 1;
    p.last_len = p.T;
    p.tiles = ceil_div(M, r);
    p.wcols = N;
    p.grid = std::min<int64_t>(p.tiles, grid);
}

void fill_segments(Plan& p, int64_t M, int64_t N, int vec, int k, int64_t grid) {
    const int64_t cap = (int64_t)kBlock * vec * k;
    p.packed = false;
    p.vec = vec;
    p.slots = k;
    p.nb = ceil_div(N, cap);
    p.T = round_up(ceil_div(N, p.nb), vec);
    while (p.nb > 1 && (p.nb - 1) * p.T >= N) --p.nb;   // no empty last block
    p.last_len = N - (p.nb - 1) * p.T;
    p.R = 1;
    p.tiles = M * p.nb;
    p.wcols = p.T;
    p.grid = p.nb * std::min<int64_t>(M, std::max<int64_t>(1, grid / p.nb));
}

// Fraction of the vector slots that carry data (row segments: averaged over
// the column blocks).
double occupancy(const Plan& p, int64_t N) {
    const double cap = (double)kBlock * p.vec * p.slots;
    return p.packed ? (double)p.T / cap : (double)N / ((double)p.nb * cap);
}

// Pure host: validates sizes/dtypes and fills the plan. The plan depends
// only on (M, N, x dtype); pointer alignment and row pitches never change
// it. The one launch that cannot use 16-byte vectors (row-strided packed
// rows whose length is not a multiple of V) runs the same tiles with the
// element-wise kernel variant (V = 1, K = 16 or 32: a capacity that holds
// the tile), so the partial-row layout - and with it dyt_backward_finish -
// is the same for every launch of a shape.
//
// The default tiling uses tiles of up to kTileCap elements with K a power of
// two (the measured tile table picks K and the grid). Widths that fill those
// tiles poorly (fewer than DYT_OCC_MIN of the slots carry data, e.g. rows of
// 2,560 or 5,120 bf16 elements; DYT_OCC_MIN_FWD for the forward) are
// re-tiled for occupancy: K = 2 .. 4 slots
// (tiles up to kTileMax elements), packed rows or row segments, whichever
// fills the most slots (ties: the bigger tile), if that beats the default by
// DYT_OCC_GAIN. Backward throughput follows slot occupancy almost linearly
// on MI355X (wasted slots still load and compute); measured at 2^27
// elements, re-tiling lifts the backward by 10-35% at N = 2,560 ... 6,144
// (bf16) and 2,560 ... 5,120 (f32) and never lost beyond noise, while
// re-tiling to K = 1 (tiles of 256 vectors) lost up to 19%, hence
// DYT_OCC_KMIN. Widths that fill the default tiles keep the measured plan.
#ifndef DYT_OCC_MIN
#define DYT_OCC_MIN 0.9
#endif
// The forward (half the arithmetic per byte) is re-tiled only below this
// occupancy: from 0.63 and less it gained up to 26% (f32 rows of 2,560 to
// 5,120), while bf16 rows of 1,500 (0.73 -> 0.98) lost 4%.
#ifndef DYT_OCC_MIN_FWD
#define DYT_OCC_MIN_FWD 0.7
#endif
#ifndef DYT_OCC_GAIN
#define DYT_OCC_GAIN 0.05
#endif
#ifndef DYT_OCC_KMIN
#define DYT_OCC_KMIN 2
#endif
// The flat forward (dyt_fwd_flat_kernel) serves contiguous rows whose length
// is a multiple of the vector width and at most kFlatMaxN (gamma and beta as
// float32 in at most 160 KB of LDS) when the tiles fit the rows poorly: for
// 2-byte x, packed tiles (several rows each) at any fill and row segments
// filled below DYT_FLAT_OCC_2B; for float32 x, tiles filled below
// DYT_FLAT_OCC_4B. Measured on MI355X at 2^27 elements (interleaved medians
// of 20-launch means, outputs bit-identical): the 2-byte flat walk (plain
// stores, dyt_kernels.hpp fwd_flat_store_nt) against the tiles it replaces,
// bf16 rows of 32 / 64 (packed, full): 81.4 / 81.4 against 83.7 / 85.4 us;
// 768 / 1,536 / 2,048 (packed): 82.0 / 82.8 / 82.9 against 90-95 us; row
// segments 3,072 / 5,120 filled 0.75 / 0.83: 84.5 / 87.1 against 85.8 /
// 89.9 us; 2,560 / 4,104 (0.62 / 0.67): 84.0 / 85.6 against 97 / 95 us;
// while row segments filled 0.88 or fully keep the lead (7,168: 85.6
// against 89.0; 4,096 / 6,144 / 8,192: 82.0 / 82.4 / 85.3 against 84.9 /
// 87.8 / 90.6 us). float32 flat rows of 2,560 / 4,104 / 5,120: 181-183 us
// against 199-236 us tiled. At bases one element off 16-byte alignment the
// packed one-slot tiles of full rows keep the lead (bf16 32 / 64 wide: 89.5 /
// 90.9 against 92.3 / 92.6 us flat), while the flat walk keeps its own
// (768 / 2,048 / 3,072 wide: 94.0-96.4 against 105.9-106.6 us), so the
// former walk flat only from aligned bases or from bases where the walk can
// start aligned (DYT_FLAT_SHIFT; Plan::flat_aligned_only).
// Rows that are not a whole number of vectors walk flat in the plain and
// the residual forward (the LDS copy then holds 4 shifted copies per
// parameter, N + V up to DYT_FLAT_RAG_MAX_LEN / _4B) for 2-byte x at any
// fill and for float32 x below DYT_FLAT_OCC_4B: bf16 rows of 3 / 17 / 100 /
// 255 / 511 / 1,001 / 1,500 / 2,039: 81.9-88.4 us against 89.2-113.2 us for
// the shifted-slot tiles (1,500 at a base one element off: 99.3 against
// 118.2); float32 1,501 (0.73 filled): 192.9 against 236.0 us, while full
// float32 tiles win at 100,003 x 255 (37.3 against 41.2 us); beyond 2^26
// elements float32 rows walk flat at any fill (DYT_FLAT_BIG_4B).
// The residual-fused forward (two inputs, two outputs) walks flat whenever
// its tiles leave any slot empty or are 2-byte packed tiles of K >= 2: there
// the flat walk measured as fast as full tiles (4,096 and 32 wide bf16:
// 181.6 / 179.7 against 180.9 / 180.6 us) and faster everywhere else (bf16
// 1,536 / 2,560 / 3,072 / 4,104: 181-182 us against 191-227 us; f32 2,560 /
// 4,104 / 5,120: 370-380 us against 402-512 us).
// The fill is that of the tiles the tile table sizes for the shape: where
// it gives float32 row segments of one slot (1,024 columns), rows such as
// 5,120 or 3,001 wide fill them and keep the tiles.
// The forward has no reduction, so the choice changes no result bit.
#ifndef DYT_FLAT_OCC_2B
#define DYT_FLAT_OCC_2B 0.85
#endif
#ifndef DYT_FLAT_OCC_4B
#define DYT_FLAT_OCC_4B 0.9
#endif
// Rows that are not a whole number of vectors (0 keeps the shifted-slot
// tiles there).
#ifndef DYT_FLAT_RAG
#define DYT_FLAT_RAG 1
#endif
// Float32 rows walk flat above DYT_FLAT_BIG_4B elements however full their
// tiles are: x then exceeds the 256 MB last-level cache, which the tiles'
// write-back stores profit from in back-to-back calls. Measured on MI355X
// (bench.py --flat-crossover, contiguous forwards, interleaved medians,
// outputs bit-identical): row segments 3,072 / 4,096 / 5,120 wide at
// 8.0e7-1.3e8 elements took 0.92-0.97 of the tiles' time flat, packed rows
// 64 / 100 / 255 / 1,000 wide 0.67-0.97 of it; at 2^26 elements and below
// the flat walk took 1.05-1.60 of the tiles' time (255 wide at 2^26: 0.89,
// 1,000 wide at 2^24: 0.97).
#ifndef DYT_FLAT_BIG_4B
#define DYT_FLAT_BIG_4B (int64_t(1) << 26)
#endif
// The residual-fused forward as well, with the same rule: bf16 rows of 17 /
// 255 / 1,001 / 1,500 / 3,071 181-186 us against 214-234 us tiled, float32
// 1,501 / 3,001 (0.73 filled) 384 / 387 against 516 / 502, float32 255
// (full tiles) 429 against 428.
#ifndef DYT_FLAT_RAG_RES
#define DYT_FLAT_RAG_RES 1
#endif
// Tensors that start off the 16-byte grid (all by the same amount): the flat
// walk starts, with the ragged layout, at their first element on the
// 128-byte line grid (else on the 16-byte grid). bf16 at +1 element: 2,560 /
// 1,500 / 32 wide 87.6-87.9 / 85.4-85.5 / 81.7 us, against 95.5-96.0 / 99.1
// for the unaligned walk and 89.9 for the 32-wide tiles (89.7 / 88.3 when
// starting on the 16-byte grid).
#ifndef DYT_FLAT_SHIFT
#define DYT_FLAT_SHIFT 1
#endif
// Workgroups of the flat forward (one per CU measured fastest, 4 vectors
// per thread and step; on 4,194,304 x 32 bf16 two or four per CU, or 8
// vectors per step, took 82.1-83.3 us against 81.6 us: bench.py --variants
// flat_grid_512,flat_grid_1024,flat_u8).
#ifndef DYT_FLAT_GRID
#define DYT_FLAT_GRID 256
#endif
// Share (x 1024) of the groups that the forward's workgroups on even XCDs
// take where the forward streams with write-back stores; 512 would be an
// even deal, 0 deals round-robin. With round-robin tiles of one slot the
// odd XCDs' workgroups end 12-14% after the even ones on MI355X (32,768 x
// 4,096 bf16: median exits 61 against 70 us). 543 (53%) measured best there:
// forward 82.6 -> 79.9 us, step 218.7 -> 213.5 us; 100,003 x 255 float32
// forward 37.6 -> 36.8 us; 573 (56%) over-corrects (81.1 us). Which
// workgroups run on the even XCDs depends on the hardware queue (XCD of
// workgroup w = (w + k) mod 8, k 0 in a one-stream process and 5 in one
// that had captured graphs on six more streams), so the launch follows the
// XCD parity hint below; with k odd and no hint the weighted deal measured
// 84.0 against 82.2 us round-robin.
#ifndef DYT_XCD_EVEN_SHARE_Q
#define DYT_XCD_EVEN_SHARE_Q 543
#endif
// Share (x 1024) of those groups that the first half of a grid of two
// workgroups per CU takes (the half dispatched first; its workgroups ended
// their loops at 61 against 70 us for the second half at 32,768 x 4,096
// bf16, bench.py --wg-timeline --timeline-raw); 0: both halves alike.
// Measured at 52-55%: 0.7-0.9 us faster there, 0.3-1.7 us slower on the
// float32 100,003-row forwards (HBM stays saturated while the second half
// finishes), so it is off.
#ifndef DYT_ROUND0_SHARE_Q
#define DYT_ROUND0_SHARE_Q 0
#endif
// The same for the 2-byte flat walk, whose odd/even gap is about half the
// tiles' (69.8 against 74.3 us median exits at 4,194,304 x 32): 53% over-
// corrected it (forward 81.2 -> 82.0 us, even XCDs now last); with the XCD
// parity hint, 51.5-53% stay within 0.6 us of round-robin, so the flat walk
// keeps the round-robin deal.
#ifndef DYT_XCD_EVEN_SHARE_FLAT_Q
#define DYT_XCD_EVEN_SHARE_FLAT_Q 0
#endif
// The same for backward pass 1 (nontemporal stores; its XCDs end within
// about 1 us of each other at 32,768 x 4,096). A constant of the build, so
// the rows summed into each partial row still depend on the shape only.
#ifndef DYT_XCD_EVEN_SHARE_BWD_Q
#define DYT_XCD_EVEN_SHARE_BWD_Q 0
#endif
// Widest rows of the flat forward (gamma and beta as float32 in the 160 KB
// of LDS a gfx950 workgroup may hold; 0 turns the flat walk off). Above
// 8,192 columns, measured at 2^27 elements: float32 9,216 / 10,240 / 13,312
// / 14,336 wide (tiles 0.75 / 0.83 / 0.81 / 0.88 filled) 187.5-189.7 us
// against 191.5-207.8 tiled; bf16 8,200 (0.80) 89.3 against 92.5.
#ifndef DYT_FLAT_MAX_N
#define DYT_FLAT_MAX_N 20480
#endif
static_assert(DYT_FLAT_MAX_N <= 20480, "the flat forward stages 2 N floats in at most 160 KB of LDS");
constexpr int64_t kFlatMaxN = DYT_FLAT_MAX_N;
// The residual-fused forward walks flat only up to 8,192 columns, the range
// its flat-against-tiles measurements cover; wider rows keep its tiles.
#ifndef DYT_FLAT_MAX_N_RES
#define DYT_FLAT_MAX_N_RES 8192
#endif
// Rows that are not whole vectors: longest copy (flat_rag_len words; 8 of
// them, the four shifted copies of gamma and beta, in the 160 KB of LDS a
// gfx950 workgroup may hold), for 2-byte and for float32 x. Measured at
// 2^27 elements, flat against tiles: bf16 2,047 / 3,071 wide 85.8-86.8 /
// 89.1 against 97.6-98.0 / 93.8-94.2 us, but 4,095 / 5,111 wide 91.2-92.4 /
// 94.2-94.4 against 89.9 / 92.0-92.1; float32 3,001 / 5,113 wide (tiles 0.73
// / 0.83 filled) 188.4 / 192.6 against 214.7 / 233.2.
#ifndef DYT_FLAT_RAG_MAX_LEN
#define DYT_FLAT_RAG_MAX_LEN 3584
#endif
#ifndef DYT_FLAT_RAG_MAX_LEN_4B
#define DYT_FLAT_RAG_MAX_LEN_4B 5120
#endif
static_assert(8 * DYT_FLAT_RAG_MAX_LEN * 4 <= 160 * 1024 && 8 * DYT_FLAT_RAG_MAX_LEN_4B * 4 <= 160 * 1024,
              "four copies of gamma and beta exceed 160 KB of LDS");

int make_plan(int64_t M, int64_t N, int xdt, int pdt, Dir dir, Plan& p) {
    if (!dtype_ok(xdt) || !dtype_ok(pdt)) return DYT_ERR_UNSUPPORTED_DTYPE;
    if (M < 0 || N < 0 || N > kMaxN) return DYT_ERR_INVALID_ARG;
    const int64_t sx = dtype_size(xdt);
    if (N > 0 && M > INT64_MAX / N / 16) return DYT_ERR_INVALID_ARG;
    p = Plan();
    const int vmax = (int)(16 / sx);           // elements per 16 bytes
    const int kmax = dyt::kTileCap / (kBlock * vmax);
    const TuneDir tune = tune_for(xdt, M, N, dir);
    if (M == 0 || N == 0) {
        p.fin_grid = ceil_div(2 * N + 1, 64);
        return DYT_OK;
    }
    // packed tiles: R >= 2 whole rows, R a multiple of r0 (the rows that make
    // R * N a multiple of V), within kTileCap elements
    const int64_t r0 = 16 / gcd64(N * sx, 16);
    const int64_t rcap = (dyt::kTileCap / N) / r0 * r0;
    if (rcap >= 2) {
        // largest K (biggest tiles) that still yields DYT_MIN_TILES tiles,
        // else the smallest K that holds an aligned row group
        int chosen = 0;
        for (int k = kmax; k >= 1; k /= 2) {
            const int64_t r = ((int64_t)kBlock * vmax * k / N) / r0 * r0;
            if (r < 1) break;
            chosen = k;
            if (ceil_div(M, r) >= tune.min_tiles) break;
        }
        const int64_t r = ((int64_t)kBlock * vmax * chosen / N) / r0 * r0;
        fill_packed(p, M, N, vmax, chosen, r, tune.grid);
    } else {
        // row segments: vectors from each row's start; with N not a multiple
        // of V the kernels shift each row's last vector back (RAG)
        const int kbig = tune.kcap > 0 ? std::min(kmax, tune.kcap) : kmax;
        int k = 1;
        while (k < kbig && (int64_t)kBlock * vmax * k < N) k *= 2;
        fill_segments(p, M, N, vmax, k, tune.grid);
    }
    const double occ = occupancy(p, N);
    if (occ < (dir == Dir::Bwd ? DYT_OCC_MIN : DYT_OCC_MIN_FWD)) {
        const int kalt = std::min(dyt::kSlotsMax, dyt::kTileMax / (kBlock * vmax));
        const int khi = tune.kcap > 0 ? std::min(kalt, std::max(tune.kcap, (int)p.slots)) : kalt;
        Plan best = p;
        double best_occ = occ;
        for (int k = DYT_OCC_KMIN; k <= khi; ++k) {
            const int64_t cap = (int64_t)kBlock * vmax * k;
            Plan c;
            const int64_t r = (cap / N) / r0 * r0;
            if (r >= 2) {
                fill_packed(c, M, N, vmax, k, r, tune.grid);
            } else {
                fill_segments(c, M, N, vmax, k, tune.grid);
            }
            const double co = occupancy(c, N);
            if (co > best_occ + 1e-9 || (co > best_occ - 1e-9 && c.T > best.T)) {
                best = c;
                best_occ = co;
            }
        }
        if (best_occ >= occ + DYT_OCC_GAIN) p = best;
    }
    // The forward's XCD-weighted deal pairs neighbouring workgroups of one
    // column block (make_walk): row segments keep an even number of
    // workgroups per block (1,020 rather than 1,023 for three blocks).
    if (dir == Dir::Fwd && !p.packed && p.nb > 1 && (p.grid / p.nb) % 2 == 1 && p.grid / p.nb > 1)
        p.grid -= p.nb;
    const double fill = occupancy(p, N);
    const bool k2 = sx == 2 && p.packed && p.slots >= 2;
    const bool big_4b = dir == Dir::Fwd && sx == 4 && M * N > DYT_FLAT_BIG_4B;
    const bool poor_fit =
        dir == Dir::Fwd ? (sx == 2 ? fill < DYT_FLAT_OCC_2B || p.packed : fill < DYT_FLAT_OCC_4B || big_4b)
                        : fill < 1.0 - 1e-9 || k2;
    const bool rag = N % vmax != 0;
    const bool rag_fits = kFlatMaxN > 0 && N <= kFlatMaxN &&
                          dyt::flat_rag_len((int)N, (int)vmax) <=
                              (sx == 2 ? DYT_FLAT_RAG_MAX_LEN : DYT_FLAT_RAG_MAX_LEN_4B);
    const bool rag_dir = dir == Dir::Fwd || (dir == Dir::ResFwd && DYT_FLAT_RAG_RES);
    const int64_t max_n = dir == Dir::ResFwd ? std::min<int64_t>(kFlatMaxN, DYT_FLAT_MAX_N_RES) : kFlatMaxN;
    const bool flat_ok = rag ? rag_dir && DYT_FLAT_RAG && rag_fits && N <= max_n &&
                                   (sx == 2 || fill < DYT_FLAT_OCC_4B || big_4b)
                             : dir != Dir::Bwd && N <= max_n && poor_fit;
    if (flat_ok) {
        const int64_t groups = ceil_div(M * N / vmax, (int64_t)DYT_FLAT_U * kBlock);
        p.flat = true;
        p.flat_grid = std::max<int64_t>(1, std::min<int64_t>(groups, DYT_FLAT_GRID));
        p.flat_aligned_only = !rag && dir == Dir::Fwd && sx == 2 && p.packed && p.slots == 1 &&
                              fill >= DYT_FLAT_OCC_2B;
        p.flat_shift = rag_fits && DYT_FLAT_SHIFT;
    }
    // Partial rows are a whole number of 128-byte lines apart: pass 2 reads
    // 64 consecutive floats of each row per workgroup, two lines instead of
    // three when rows start on the line grid (a 16-byte multiple fetched
    // 1.44x the workspace at 4,096 columns).
    p.ld = round_up(2 * p.wcols + 1, 32);
    p.fin_grid = ceil_div(2 * N + 1, 64);
    p.ws_bytes = p.grid * p.ld * (int64_t)sizeof(float);
#if DYT_FUSED_FIN
#ifndef DYT_FUSED_FIN_MAX
#define DYT_FUSED_FIN_MAX (1 << 20)
#endif
    if (dir == Dir::Bwd && p.nb == 1 && p.ws_bytes <= DYT_FUSED_FIN_MAX) {
        p.fused = true;
        p.ctr_off = round_up(p.ws_bytes, 128);
        p.ws_bytes = p.ctr_off + 128;
    }
#endif
    return DYT_OK;
}

// Kernel variant of a launch: the plan's vector width, or element-wise
// access (see vector_ok).
Plan variant_for(const Plan& p, bool vector) {
    Plan q = p;
    if (!vector && q.vec != 1) {
        q.vec = 1;
        q.slots = q.T <= 16 * kBlock ? 16 : 32;
    }
    return q;
}

#if DYT_WG_TIMELINE
// Workgroup timeline buffer of the next launches (measurement builds only;
// set by dyt_timeline_set).
uint64_t* g_stamps = nullptr;
#endif

Geo make_geo(const Plan& p, int64_t M, int64_t N) {
    Geo g;
#if DYT_WG_TIMELINE
    g.stamps = g_stamps;
#endif
#if DYT_FUSED_FIN
    g.fin_out[0] = g.fin_out[1] = g.fin_out[2] = nullptr;
    g.ctr = nullptr;
#endif
    g.total = M * N;
    g.ntiles = p.tiles;
    g.N = N;
    g.T = (int32_t)p.T;
    g.R = (int32_t)p.R;
    g.nb = (int32_t)p.nb;
    g.last_len = (int32_t)p.last_len;
    g.ld = (int32_t)p.ld;
    g.wcols = (int32_t)p.wcols;
    g.pitch[0] = g.pitch[1] = g.pitch[2] = N;
    g.even_share_q = 0;
    g.xcd_flip = 0;
    g.xcd_seen = nullptr;
    g.round0_q = 0;
    g.buf_store = 0;
    return g;
}

bool aligned(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr % a) == 0; }

struct Range {
    const char* lo;
    const char* hi;
};
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }
Range range(const void* p, int64_t bytes) {
    const char* c = static_cast<const char*>(p);
    return Range{c, c + bytes};
}

// ------------------------------------------------------------- dispatch

int64_t pitch_or(int64_t ld, int64_t N) { return ld == 0 ? N : ld; }

// Bytes a row-pitched M x N tensor spans (0 when empty).
int64_t span_bytes(int64_t M, int64_t N, int64_t ld, int64_t sx) {
    return (M > 0 && N > 0) ? ((M - 1) * ld + N) * sx : 0;
}

// Pitches valid: each at least N and small enough that every element offset
// fits in int64 (checked like M * N).
bool pitches_ok(int64_t M, int64_t N, std::initializer_list<int64_t> lds) {
    for (int64_t ld : lds)
        if (ld < N || (M > 0 && ld > INT64_MAX / M / 16)) return false;
    return true;
}

// The vector kernels take any element-aligned base and any row pitch; only a
// row-strided launch of packed tiles needs N to be a multiple of the vector
// width, so that no slot straddles the gap between two rows.
bool vector_ok(const Plan& p, int64_t N, int64_t sx, bool strided) {
    return !(strided && p.packed && N % (16 / sx) != 0);
}


template <typename PT>
void launch_finish(const Plan& p, int64_t N, const float* ws, void* dg, void* db, void* da,
                   hipStream_t s) {
    FinGeo f;
    f.P = p.grid;
    f.N = N;
    f.nb = (int32_t)p.nb;
    f.wc = (int32_t)p.T;
    f.wcols = (int32_t)p.wcols;
    f.ld = (int32_t)p.ld;
    f.packed = p.packed ? 1 : 0;
    hipLaunchKernelGGL((dyt::dyt_bwd_finish_kernel<PT>), dim3((unsigned)p.fin_grid),
                       dim3(dyt::kFinBlock), 0, s, ws, (PT*)dg, (PT*)db, (PT*)da, f);
}

int hip_status() { return hipGetLastError() == hipSuccess ? DYT_OK : DYT_ERR_HIP; }

// Shared validation of the backward entry points. Pointers a pass does not
// use are passed as nullptr with use_* = false.
int validate_backward(const void* x, const void* dy, const void* dres, bool use_dres,
                      const void* alpha, const void* gamma, void* dx, void* dalpha, void* dgamma,
                      void* dbeta, const void* workspace, size_t workspace_bytes, int64_t M,
                      int64_t N, int x_dtype, int param_dtype, bool use_pass1, bool use_pass2,
                      Plan& base, int64_t ldx = 0, int64_t lddy = 0, int64_t lddx = 0) {
    int st = make_plan(M, N, x_dtype, param_dtype, Dir::Bwd, base);
    if (st != DYT_OK) return st;
    const int64_t sx = dtype_size(x_dtype), sp = dtype_size(param_dtype);
    const bool any = M > 0 && N > 0;
    const bool p1 = use_pass1 && any;
    if (use_pass2) {
        if (!dalpha) return DYT_ERR_INVALID_ARG;
        if (N > 0 && (!dgamma || !dbeta)) return DYT_ERR_INVALID_ARG;
    }
    if (p1 && (!x || !dy || !alpha || !gamma || !dx || (use_dres && !dres))) return DYT_ERR_INVALID_ARG;
    ldx = pitch_or(ldx, N);
    lddy = pitch_or(lddy, N);
    lddx = pitch_or(lddx, N);
    if (!pitches_ok(M, N, {ldx, lddy, lddx})) return DYT_ERR_INVALID_ARG;
    const size_t need = (size_t)round_up(base.ws_bytes, 16);
    if (workspace_bytes < need) return DYT_ERR_WORKSPACE_TOO_SMALL;
    if (need > 0 && !workspace) return DYT_ERR_INVALID_ARG;
    if (need > 0 && !aligned(workspace, 16)) return DYT_ERR_MISALIGNED;
    if (use_pass2 && (!aligned(dalpha, sp) || (N > 0 && (!aligned(dgamma, sp) || !aligned(dbeta, sp)))))
        return DYT_ERR_MISALIGNED;
    if (p1 && (!aligned(x, sx) || !aligned(dy, sx) || !aligned(dx, sx) || !aligned(alpha, sp) ||
               !aligned(gamma, sp) || (use_dres && !aligned(dres, sx))))
        return DYT_ERR_MISALIGNED;
    // outputs (and the workspace) must not overlap inputs or each other
    // (strided tensors: over the bytes from their first to their last element)
    const int64_t mx = p1 ? span_bytes(M, N, ldx, sx) : 0;
    const Range outs[5] = {range(dx, p1 ? span_bytes(M, N, lddx, sx) : 0),
                           range(dalpha, use_pass2 ? sp : 0),
                           range(dgamma, use_pass2 ? N * sp : 0), range(dbeta, use_pass2 ? N * sp : 0),
                           range(workspace, (int64_t)need)};
    const Range ins[5] = {range(x, mx), range(dy, p1 ? span_bytes(M, N, lddy, sx) : 0),
                          range(dres, use_dres ? mx : 0), range(alpha, p1 ? sp : 0),
                          range(gamma, p1 ? N * sp : 0)};
    for (int a = 0; a < 5; ++a) {
        if (outs[a].lo == outs[a].hi) continue;
        for (const Range& i : ins)
            if (i.lo != i.hi && overlap(outs[a], i)) return DYT_ERR_INVALID_ARG;
        for (int b = a + 1; b < 5; ++b)
            if (outs[b].lo != outs[b].hi && overlap(outs[a], outs[b])) return DYT_ERR_INVALID_ARG;
    }
    return DYT_OK;
}

int enqueue_pass1(const Plan& base, const BwdPtrs& a, int64_t M, int64_t N, int x_dtype,
                  int param_dtype, hipStream_t s, void* const* fin_out = nullptr) {
    if (M == 0 || N == 0) return DYT_OK;
    const bool res = a.dres != nullptr;
    const int64_t ldx = pitch_or(a.ldx, N), lddy = pitch_or(a.lddy, N), lddx = pitch_or(a.lddx, N);
    const bool strided = ldx != N || lddy != N || lddx != N;
    const int64_t sx = dtype_size(x_dtype);
    const Plan p = variant_for(base, vector_ok(base, N, sx, strided));
    Geo g = make_geo(p, M, N);
    g.pitch[0] = ldx;
    g.pitch[1] = lddy;
    g.pitch[2] = lddx;
    if (p.vec > 1 && p.tiles >= 8 * p.grid) g.even_share_q = DYT_XCD_EVEN_SHARE_BWD_Q;
    // every vector of dx on the 16-byte grid (as for the forward's y)
    g.buf_store = !strided && !res && p.vec > 1 && aligned(a.dx, 16) && p.T % p.vec == 0 &&
                  (p.packed || N % p.vec == 0);
#if DYT_FUSED_FIN
    g.fin_out[0] = g.fin_out[1] = g.fin_out[2] = nullptr;
    g.ctr = nullptr;
    if (fin_out && base.fused) {
        for (int k = 0; k < 3; ++k) g.fin_out[k] = fin_out[k];
        g.ctr = reinterpret_cast<unsigned*>(reinterpret_cast<char*>(a.ws) + base.ctr_off);
    }
#else
    (void)fin_out;
#endif
    const bool ok = with_dtype(x_dtype, [&](auto xt) {
        return dyt::host::launch_backward<decltype(xt)>(param_dtype, res, strided, p, g, a, s);
    });
    if (!ok) return DYT_ERR_INVALID_ARG;
    return hip_status();
}

int enqueue_pass2(const Plan& base, const void* workspace, void* dalpha, void* dgamma,
                  void* dbeta, int64_t N, int param_dtype, hipStream_t s) {
    const float* ws = static_cast<const float*>(workspace);
    with_dtype(param_dtype, [&](auto pt) {
        launch_finish<decltype(pt)>(base, N, ws, dgamma, dbeta, dalpha, s);
        return true;
    });
    return hip_status();
}

// ------------------------------------------------------- XCD parity hint
// The forward's XCD-weighted deal gives the larger share to the class of
// workgroups expected on the even XCDs; which class that is depends on the
// hardware queue the stream runs on (the XCD of its workgroup 0). Each
// weighted launch records the XCD its workgroup 0 ran on in a slot of
// coherent pinned host memory, and the next launch on that stream reads the
// slot to choose its flip. The value is only a hint: flip is a kernel
// argument, the same for the whole launch, and every flip covers every
// group exactly once; a stale or raced slot costs time, never results. The
// slots (64 per device, chosen by the stream's address) are allocated by
// the device's first weighted forward outside stream capture and kept
// until the process ends; without them flip is 0.
constexpr int kHintDevices = 64;
constexpr int kHintSlots = 64;
struct XcdHint {
    std::mutex mu;
    std::atomic<int32_t*> host{nullptr};
    int32_t* dev = nullptr;   // device address of host[0]
    int xccs = 0;             // XCDs of the device, 0 if unknown
    bool tried = false;
};
XcdHint g_xcd_hint[kHintDevices];
std::atomic<int> g_flip_override{-1};   // dyt_set_xcd_flip_override
std::atomic<int> g_cus[kHintDevices];     // compute units per device: 0 unknown, -1 no answer

// Compute units of the current device (0 if the runtime does not say).
int device_cus() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kHintDevices) {
        (void)hipGetLastError();
        return 0;
    }
    int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) {
            c = n;
        } else {
            (void)hipGetLastError();
            c = -1;
        }
        g_cus[dev].store(c, std::memory_order_relaxed);
    }
    return c > 0 ? c : 0;
}

// The hint slot of stream s on the current device (host and device
// addresses) and the device's XCD count; false when there are no slots.
bool xcd_hint_slot(hipStream_t s, int32_t** host_slot, int32_t** dev_slot, int* xccs) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kHintDevices) {
        (void)hipGetLastError();
        return false;
    }
    XcdHint& h = g_xcd_hint[dev];
    int32_t* host = h.host.load(std::memory_order_acquire);
    if (host == nullptr) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
            (void)hipGetLastError();
            return false;   // no allocation while a graph is being captured
        }
        std::lock_guard<std::mutex> lock(h.mu);
        if (!h.tried) {
            h.tried = true;
            int n = 0;
            if (hipDeviceGetAttribute(&n, hipDeviceAttributeNumberOfXccs, dev) == hipSuccess) h.xccs = n;
            void* p = nullptr;
            if (hipHostMalloc(&p, kHintSlots * sizeof(int32_t), hipHostMallocCoherent) == hipSuccess &&
                p != nullptr) {
                void* d = nullptr;
                if (hipHostGetDevicePointer(&d, p, 0) == hipSuccess && d != nullptr) {
                    int32_t* q = static_cast<int32_t*>(p);
                    for (int i = 0; i < kHintSlots; ++i) q[i] = -1;
                    h.dev = static_cast<int32_t*>(d);
                    h.host.store(q, std::memory_order_release);
                } else {
                    (void)hipHostFree(p);
                }
            }
            (void)hipGetLastError();   // a failure here is not the launch's error
        }
        host = h.host.load(std::memory_order_acquire);
        if (host == nullptr) return false;
    }
    const size_t i = ((uintptr_t)s >> 4) % kHintSlots;
    *host_slot = host + i;
    *dev_slot = h.dev + i;
    *xccs = h.xccs;
    return true;
}

// The XCD parity of a weighted forward launch on stream s: share_q is
// cleared on devices that report another XCD count than 8; flip and seen
// follow the stream's hint slot and dyt_set_xcd_flip_override.
void apply_xcd_hint(hipStream_t s, int32_t& share_q, int32_t& flip, int32_t*& seen) {
    flip = 0;
    seen = nullptr;
    if (share_q == 0) return;
    int32_t *hs = nullptr, *ds = nullptr;
    int xccs = 0;
    if (xcd_hint_slot(s, &hs, &ds, &xccs)) {
        if (xccs != 0 && xccs != 8) {
            share_q = 0;   // the deal is measured for eight XCDs
            return;
        }
        const int32_t v = *static_cast<volatile int32_t*>(hs);
        flip = v >= 0 ? (v & 1) : 0;
        seen = ds;
    }
    const int ov = g_flip_override.load(std::memory_order_relaxed);
    if (ov >= 0) flip = ov;
}

// Forward with or without the fused residual add: validation, then launch.
int forward_impl(const FwdPtrs& a, bool res, int64_t M, int64_t N, int x_dtype, int param_dtype,
                 hipStream_t s) {
    Plan base;
    int st = make_plan(M, N, x_dtype, param_dtype, res ? Dir::ResFwd : Dir::Fwd, base);
    if (st != DYT_OK) return st;
    if (M == 0 || N == 0) return DYT_OK;
    if (!a.x || !a.alpha || !a.gamma || !a.beta || !a.y || (res && (!a.r || !a.h)))
        return DYT_ERR_INVALID_ARG;
    const int64_t ldx = pitch_or(a.ldx, N), ldy = pitch_or(a.ldy, N);
    if (!pitches_ok(M, N, {ldx, ldy})) return DYT_ERR_INVALID_ARG;
    const bool strided = ldx != N || ldy != N;
    if (strided && res) return DYT_ERR_INVALID_ARG;   // not offered by any entry point
    const int64_t sx = dtype_size(x_dtype), sp = dtype_size(param_dtype);
    if (!aligned(a.x, sx) || !aligned(a.y, sx) || !aligned(a.alpha, sp) || !aligned(a.gamma, sp) ||
        !aligned(a.beta, sp) || (res && (!aligned(a.r, sx) || !aligned(a.h, sx))))
        return DYT_ERR_MISALIGNED;
    // outputs must not overlap inputs or each other (strided tensors: over the
    // bytes from their first to their last element)
    const int64_t mx = span_bytes(M, N, ldx, sx), my = span_bytes(M, N, ldy, sx);
    const Range outs[2] = {range(a.y, my), range(a.h, res ? my : 0)};
    const Range ins[5] = {range(a.x, mx), range(a.r, res ? mx : 0), range(a.alpha, sp),
                          range(a.gamma, N * sp), range(a.beta, N * sp)};
    for (const Range& o : outs) {
        if (o.lo == o.hi) continue;
        for (const Range& i : ins)
            if (i.lo != i.hi && overlap(o, i)) return DYT_ERR_INVALID_ARG;
    }
    if (res && overlap(outs[0], outs[1])) return DYT_ERR_INVALID_ARG;
    // Off the 16-byte grid, the flat walk starts at the first element on the
    // 128-byte (cache line) grid when every operand is off it by the same
    // amount, else at the first element on the 16-byte grid when they agree
    // on that (head: the elements before it).
    auto off = [&](uintptr_t m) {
        const uintptr_t o = (uintptr_t)a.x % m;
        const bool same = (uintptr_t)a.y % m == o &&
                          (!res || ((uintptr_t)a.r % m == o && (uintptr_t)a.h % m == o));
        return same ? (int64_t)((m - o) % m) : (int64_t)-1;
    };
    int64_t head = 0;
    if (base.flat && !strided && (uintptr_t)a.x % 16 != 0 && base.flat_shift) {
        const int64_t line = off(128), vec = off(16);
        head = line >= 0 ? line / sx : vec > 0 ? vec / sx : 0;
        head = std::min<int64_t>(head, M * N);
    }
    const bool bases16 = aligned(a.x, 16) && aligned(a.y, 16);
    if (base.flat && !strided && (bases16 || head > 0 || !base.flat_aligned_only)) {
        FlatGeo f;
#if DYT_WG_TIMELINE
        f.stamps = g_stamps;
#endif
        f.head = (int32_t)head;
        f.total = M * N - head;
        f.nvec = f.total / (16 / sx);
        f.N = (int32_t)N;
        // the XCD-weighted deal where the walk stores with write-back stores
        // (2-byte x, no residual add) and each class gets several groups
        const int64_t fgroups = f.nvec / (DYT_FLAT_U * kBlock);
        const bool weigh = DYT_XCD_EVEN_SHARE_FLAT_Q != 0 && sx == 2 && !res && base.flat_grid % 2 == 0 &&
                           fgroups >= 4 * base.flat_grid;
        f.even_share_q = weigh ? DYT_XCD_EVEN_SHARE_FLAT_Q : 0;
        apply_xcd_hint(s, f.even_share_q, f.xcd_flip, f.xcd_seen);   // may clear the share
        f.buf_store = aligned(static_cast<const char*>(a.y) + head * sx, 16);
        const int64_t fstride = f.even_share_q != 0 ? base.flat_grid / 2 : base.flat_grid;
        f.cstep = (int32_t)((fstride * DYT_FLAT_U * kBlock * (16 / sx)) % N);
        const bool ok = with_dtype(x_dtype, [&](auto xt) {
            return dyt::host::launch_forward_flat<decltype(xt)>(param_dtype, res, base, f, a, s);
        });
        if (!ok) return DYT_ERR_INVALID_ARG;   // not reachable: the plan checked N
        return hip_status();
    }
    const Plan p = variant_for(base, vector_ok(base, N, sx, strided));
    Geo g = make_geo(p, M, N);
    g.pitch[0] = ldx;
    g.pitch[1] = ldy;
    // the XCD-weighted deal for tiles of one vector slot (write-back stores),
    // plain forward, enough groups per workgroup
    if (!res && p.slots == 1 && p.vec > 1 && p.tiles >= 8 * p.grid) {
        g.even_share_q = DYT_XCD_EVEN_SHARE_Q;
        apply_xcd_hint(s, g.even_share_q, g.xcd_flip, g.xcd_seen);
        if (g.even_share_q != 0 && DYT_ROUND0_SHARE_Q != 0 && p.grid == 2 * (int64_t)device_cus())
            g.round0_q = DYT_ROUND0_SHARE_Q;   // two workgroups per CU
    }
    // every vector of y on the 16-byte grid: y aligned, tiles (and, for row
    // segments, rows) a whole number of vectors
    g.buf_store = !strided && p.vec > 1 && aligned(a.y, 16) && p.T % p.vec == 0 &&
                  (p.packed || N % p.vec == 0);
    const bool ok = with_dtype(x_dtype, [&](auto xt) {
        return dyt::host::launch_forward<decltype(xt)>(param_dtype, res, strided, p, g, a, s);
    });
    if (!ok) return DYT_ERR_INVALID_ARG;   // no kernel instance for this plan (not reachable)
    return hip_status();
}

// Both passes, with or without the residual gradient (res: a.dres is used).
int backward_impl(const BwdPtrs& a, bool res, void* dalpha, void* dgamma, void* dbeta,
                  size_t workspace_bytes, int64_t M, int64_t N, int x_dtype, int param_dtype,
                  hipStream_t s) {
    Plan base;
    int st = validate_backward(a.x, a.dy, a.dres, res, a.alpha, a.gamma, a.dx, dalpha, dgamma,
                               dbeta, a.ws, workspace_bytes, M, N, x_dtype, param_dtype, true,
                               true, base, a.ldx, a.lddy, a.lddx);
    if (st != DYT_OK) return st;
#if DYT_FUSED_FIN
    if (base.fused && M > 0 && N > 0) {
        void* outs[3] = {dgamma, dbeta, dalpha};
        return enqueue_pass1(base, a, M, N, x_dtype, param_dtype, s, outs);
    }
#endif
    st = enqueue_pass1(base, a, M, N, x_dtype, param_dtype, s);
    if (st != DYT_OK) return st;
    return enqueue_pass2(base, a.ws, dalpha, dgamma, dbeta, N, param_dtype, s);
}

void fill_plan(const Plan& p, dyt_plan* out) {
    out->packed = p.packed ? 1 : 0;
    out->vec = p.vec;
    out->slots = p.slots;
    out->block = kBlock;
    out->rows_per_tile = p.R;
    out->tile_elems = p.T;
    out->col_blocks = p.nb;
    out->tiles = p.tiles;
    out->flat = 0;
    out->flat_grid = 0;
    out->flat_aligned_only = 0;
}

// ------------------------------------------------ allocation-free backward
// dyt_backward_noalloc keeps its partial rows in `scratch`, a file-scope
// device array of DYT_NOALLOC_SCRATCH_BYTES that every GPU the library runs
// on holds until the process ends. In host code `scratch` names a host-side
// stand-in, not device memory: its device address is looked up once per
// device (with that device current) and only that address is handed to
// kernels. Nothing in it has to start at zero: pass 1 writes every entry
// pass 2 reads. Calls that overlap on one GPU share the array and race.
}  // namespace

static __device__ __align__(256) float scratch[DYT_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
struct ScratchSlot {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call per device).
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DYT_ERR_HIP;
    ScratchSlot& slot = g_scratch[dev];
    std::call_once(slot.once, [&slot] {
        slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch));
    });
    if (slot.err != hipSuccess || slot.ptr == nullptr) return DYT_ERR_HIP;
    *out = slot.ptr;
    return DYT_OK;
}

// The build id, after a marker that lets a build step find it in the file
// without loading the library.
#ifndef DYT_BUILD_ID
#define DYT_BUILD_ID "unknown"
#endif
__attribute__((used)) const char kBuildId[] = "DYT_BUILD_ID=" DYT_BUILD_ID;
constexpr int kBuildIdSkip = sizeof("DYT_BUILD_ID=") - 1;

}  // namespace

extern "C" {

int dyt_abi_version(void) { return DYT_ABI_VERSION; }

const char* dyt_build_id(void) { return kBuildId + kBuildIdSkip; }

int dyt_xcd_hint(void* stream) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kHintDevices) {
        (void)hipGetLastError();
        return -1;
    }
    const int32_t* host = g_xcd_hint[dev].host.load(std::memory_order_acquire);
    if (host == nullptr) return -1;
    const size_t i = ((uintptr_t)stream >> 4) % kHintSlots;
    return *static_cast<const volatile int32_t*>(host + i);
}

int dyt_set_xcd_flip_override(int flip) {
    if (flip < -1 || flip > 1) return DYT_ERR_INVALID_ARG;
    g_flip_override.store(flip, std::memory_order_relaxed);
    return DYT_OK;
}

#if DYT_WG_TIMELINE
// Measurement builds only (not part of the ABI in dyt.h): the device buffer
// (4 words per workgroup, large enough for the grid) that the forward and
// backward pass-1 launches enqueued after this call record their workgroup
// timeline into; NULL stops recording.
int dyt_timeline_set(void* device_buffer) {
    g_stamps = static_cast<uint64_t*>(device_buffer);
    return DYT_OK;
}
#endif

const char* dyt_status_string(int status) {
    switch (status) {
        case DYT_OK: return "DYT_OK";
        case DYT_ERR_INVALID_ARG: return "DYT_ERR_INVALID_ARG";
        case DYT_ERR_UNSUPPORTED_DTYPE: return "DYT_ERR_UNSUPPORTED_DTYPE";
        case DYT_ERR_WORKSPACE_TOO_SMALL: return "DYT_ERR_WORKSPACE_TOO_SMALL";
        case DYT_ERR_MISALIGNED: return "DYT_ERR_MISALIGNED";
        case DYT_ERR_HIP: return "DYT_ERR_HIP";
        default: return "DYT_ERR_UNKNOWN";
    }
}

int dyt_get_plan(int64_t M, int64_t N, int x_dtype, int param_dtype, int vector_access,
                 dyt_plan* out) {
    if (!out) return DYT_ERR_INVALID_ARG;
    Plan base, fbase;
    int st = make_plan(M, N, x_dtype, param_dtype, Dir::Bwd, base);
    if (st != DYT_OK) return st;
    st = make_plan(M, N, x_dtype, param_dtype, Dir::Fwd, fbase);
    if (st != DYT_OK) return st;
    const Plan p = variant_for(base, vector_access != 0);
    fill_plan(p, out);
    out->flat = fbase.flat && vector_access != 0;
    out->flat_grid = out->flat ? fbase.flat_grid : 0;
    out->flat_aligned_only = out->flat && fbase.flat_aligned_only;
    out->fwd_grid = fbase.grid;
    out->bwd_grid = p.grid;
    out->ws_row = p.ld;
    out->fin_grid = p.fin_grid;
    out->ws_bytes = p.ws_bytes;
    return DYT_OK;
}

int dyt_get_forward_plan(int64_t M, int64_t N, int x_dtype, int param_dtype, int vector_access,
                         dyt_plan* out) {
    if (!out) return DYT_ERR_INVALID_ARG;
    Plan base;
    const int st = make_plan(M, N, x_dtype, param_dtype, Dir::Fwd, base);
    if (st != DYT_OK) return st;
    const Plan p = variant_for(base, vector_access != 0);
    fill_plan(p, out);
    out->flat = base.flat && vector_access != 0;
    out->flat_grid = out->flat ? base.flat_grid : 0;
    out->flat_aligned_only = out->flat && base.flat_aligned_only;
    out->fwd_grid = p.grid;
    out->bwd_grid = 0;
    out->ws_row = 0;
    out->fin_grid = 0;
    out->ws_bytes = 0;
    return DYT_OK;
}

int dyt_get_forward_residual_plan(int64_t M, int64_t N, int x_dtype, int param_dtype,
                                  dyt_plan* out) {
    if (!out) return DYT_ERR_INVALID_ARG;
    Plan p;
    const int st = make_plan(M, N, x_dtype, param_dtype, Dir::ResFwd, p);
    if (st != DYT_OK) return st;
    fill_plan(p, out);
    out->flat = p.flat;
    out->flat_grid = p.flat_grid;
    out->flat_aligned_only = p.flat_aligned_only;
    out->fwd_grid = p.grid;
    out->bwd_grid = 0;
    out->ws_row = 0;
    out->fin_grid = 0;
    out->ws_bytes = 0;
    return DYT_OK;
}

size_t dyt_backward_workspace_size(int64_t M, int64_t N, int x_dtype, int param_dtype) {
    Plan p;
    if (make_plan(M, N, x_dtype, param_dtype, Dir::Bwd, p) != DYT_OK) return 0;
    return (size_t)round_up(p.ws_bytes, 16);
}

int dyt_forward(const void* x, const void* alpha, const void* gamma, const void* beta, void* y,
                int64_t M, int64_t N, int x_dtype, int param_dtype, void* stream) {
    return forward_impl(FwdPtrs{x, nullptr, alpha, gamma, beta, y, nullptr}, false, M, N, x_dtype,
                        param_dtype, static_cast<hipStream_t>(stream));
}

int dyt_forward_strided(const void* x, int64_t ldx, const void* alpha, const void* gamma,
                        const void* beta, void* y, int64_t ldy, int64_t M, int64_t N, int x_dtype,
                        int param_dtype, void* stream) {
    if (ldx <= 0 || ldy <= 0) return DYT_ERR_INVALID_ARG;
    return forward_impl(FwdPtrs{x, nullptr, alpha, gamma, beta, y, nullptr, ldx, ldy}, false, M, N,
                        x_dtype, param_dtype, static_cast<hipStream_t>(stream));
}

int dyt_backward_strided(const void* x, int64_t ldx, const void* dy, int64_t lddy,
                         const void* alpha, const void* gamma, void* dx, int64_t lddx,
                         void* dalpha, void* dgamma, void* dbeta, void* workspace,
                         size_t workspace_bytes, int64_t M, int64_t N, int x_dtype,
                         int param_dtype, void* stream) {
    if (ldx <= 0 || lddy <= 0 || lddx <= 0) return DYT_ERR_INVALID_ARG;
    return backward_impl(BwdPtrs{x, dy, nullptr, alpha, gamma, dx, static_cast<float*>(workspace),
                                 ldx, lddy, lddx},
                         false, dalpha, dgamma, dbeta, workspace_bytes, M, N, x_dtype,
                         param_dtype, static_cast<hipStream_t>(stream));
}

int dyt_forward_residual(const void* x, const void* r, const void* alpha, const void* gamma,
                         const void* beta, void* h, void* y, int64_t M, int64_t N, int x_dtype,
                         int param_dtype, void* stream) {
    return forward_impl(FwdPtrs{x, r, alpha, gamma, beta, y, h}, true, M, N, x_dtype, param_dtype,
                        static_cast<hipStream_t>(stream));
}

int dyt_backward_partials(const void* x, const void* dy, const void* alpha, const void* gamma,
                          void* dx, void* workspace, size_t workspace_bytes, int64_t M, int64_t N,
                          int x_dtype, int param_dtype, void* stream) {
    Plan base;
    int st = validate_backward(x, dy, nullptr, false, alpha, gamma, dx, nullptr, nullptr, nullptr,
                               workspace, workspace_bytes, M, N, x_dtype, param_dtype, true, false,
                               base);
    if (st != DYT_OK) return st;
    return enqueue_pass1(base, BwdPtrs{x, dy, nullptr, alpha, gamma, dx, static_cast<float*>(workspace)},
                         M, N, x_dtype, param_dtype, static_cast<hipStream_t>(stream));
}

int dyt_backward_residual_partials(const void* h, const void* dy, const void* dres,
                                   const void* alpha, const void* gamma, void* dh, void* workspace,
                                   size_t workspace_bytes, int64_t M, int64_t N, int x_dtype,
                                   int param_dtype, void* stream) {
    Plan base;
    int st = validate_backward(h, dy, dres, true, alpha, gamma, dh, nullptr, nullptr, nullptr,
                               workspace, workspace_bytes, M, N, x_dtype, param_dtype, true, false,
                               base);
    if (st != DYT_OK) return st;
    return enqueue_pass1(base, BwdPtrs{h, dy, dres, alpha, gamma, dh, static_cast<float*>(workspace)},
                         M, N, x_dtype, param_dtype, static_cast<hipStream_t>(stream));
}

int dyt_backward_finish(const void* workspace, size_t workspace_bytes, void* dalpha,
                        void* dgamma, void* dbeta, int64_t M, int64_t N, int x_dtype,
                        int param_dtype, void* stream) {
    Plan base;
    int st = validate_backward(nullptr, nullptr, nullptr, false, nullptr, nullptr, nullptr, dalpha,
                               dgamma, dbeta, workspace, workspace_bytes, M, N, x_dtype,
                               param_dtype, false, true, base);
    if (st != DYT_OK) return st;
    return enqueue_pass2(base, workspace, dalpha, dgamma, dbeta, N, param_dtype,
                         static_cast<hipStream_t>(stream));
}

int dyt_backward(const void* x, const void* dy, const void* alpha, const void* gamma, void* dx,
                 void* dalpha, void* dgamma, void* dbeta, void* workspace,
                 size_t workspace_bytes, int64_t M, int64_t N, int x_dtype, int param_dtype,
                 void* stream) {
    return backward_impl(BwdPtrs{x, dy, nullptr, alpha, gamma, dx, static_cast<float*>(workspace)},
                         false, dalpha, dgamma, dbeta, workspace_bytes, M, N, x_dtype, param_dtype,
                         static_cast<hipStream_t>(stream));
}

int dyt_backward_noalloc(const void* x, const void* dy, const void* alpha, const void* gamma,
                         void* dx, void* dalpha, void* dgamma, void* dbeta, int64_t M, int64_t N,
                         int x_dtype, int param_dtype, void* stream) {
    // sizes first (pure host): a problem whose partial rows exceed the
    // static scratch is refused before any HIP call
    Plan p;
    const int st = make_plan(M, N, x_dtype, param_dtype, Dir::Bwd, p);
    if (st != DYT_OK) return st;
    if (round_up(p.ws_bytes, 16) > (int64_t)DYT_NOALLOC_SCRATCH_BYTES) return DYT_ERR_WORKSPACE_TOO_SMALL;
    void* ws = nullptr;
    const int sa = scratch_address(&ws);
    if (sa != DYT_OK) return sa;
    return backward_impl(BwdPtrs{x, dy, nullptr, alpha, gamma, dx, static_cast<float*>(ws)}, false,
                         dalpha, dgamma, dbeta, DYT_NOALLOC_SCRATCH_BYTES, M, N, x_dtype,
                         param_dtype, static_cast<hipStream_t>(stream));
}

int dyt_backward_residual(const void* h, const void* dy, const void* dres, const void* alpha,
                          const void* gamma, void* dh, void* dalpha, void* dgamma, void* dbeta,
                          void* workspace, size_t workspace_bytes, int64_t M, int64_t N,
                          int x_dtype, int param_dtype, void* stream) {
    return backward_impl(BwdPtrs{h, dy, dres, alpha, gamma, dh, static_cast<float*>(workspace)},
                         true, dalpha, dgamma, dbeta, workspace_bytes, M, N, x_dtype, param_dtype,
                         static_cast<hipStream_t>(stream));
}

}  // extern "C"
