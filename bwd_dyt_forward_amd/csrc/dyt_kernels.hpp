// dyt_kernels.hpp - HIP kernels of the fused DyT layer for CDNA4 (gfx950).
//
// Work decomposition (shared by the forward and the first backward pass)
// ----------------------------------------------------------------------
// The M x N row-major tensor is cut into tiles that a 256-thread workgroup
// streams with one 16-byte access per thread and "slot" (K slots per
// thread, V elements per slot, so a tile holds at most 256*V*K elements):
//
//  * packed tiles (several whole rows; used whenever two or more rows fit a
//    4096-element tile): tile t is the contiguous run of R rows starting at
//    row t*R, i.e. elements [t*R*N, (t+1)*R*N). R*N is a multiple of V, so
//    the element at tile offset o always sits in column o mod N and a
//    vector never needs columns from two rows' worth of parameters in a
//    different order. Each thread therefore owns the same columns in every
//    tile: its gamma/beta values live in registers for the whole kernel and
//    its backward accumulators are per (slot, lane).
//  * row segments (wide rows): tile t is row t / nb, column block t % nb of
//    width Wc (a multiple of V). The grid size is a multiple of nb, so a
//    workgroup always sees the same column block. When N is not a multiple
//    of V, the last vector of every row is shifted back to end at the row's
//    end (see Slots).
//
// Memory accesses assume only element alignment: gfx9 and later GPUs run
// global memory instructions in unaligned mode under ROCm (the compiler
// assumes it for HSA code objects and emits the same 16-byte instructions),
// so tensors at any element-aligned address, and rows of any length or
// pitch, take the 16-byte vector path.
//
// The grid is one-dimensional and persistent (one workgroup per CU): groups
// of U adjacent tiles are dealt round-robin to the workgroups, and each
// workgroup pipelines its groups through two register buffers. Rows never
// map to a grid dimension, so there is no 65,535 limit on M (the
// Liger-Kernel pull request "fix(dyt): use a 1D grid and tile small-width
// rows", Summary, "Launch limit" and "Small widths" bullets, describes both
// problems for its Triton kernels; this is the CDNA4 design, not a
// translation).
//
// Every tile except possibly the last (packed) takes an unmasked path. The
// last tile masks lanes past the end of the data; the backward computes
// those lanes and then removes them with a select, after the arithmetic,
// so zeros loaded for missing lanes cannot inject tanh(inf * 0) = NaN into
// the sums (same pull request, Summary, "Padding" bullet).
//
// Backward reduction (deterministic, no atomics)
// ----------------------------------------------
// Pass 1 keeps float32 accumulators per thread, then reduces them once per
// workgroup in a fixed order: dalpha by a wavefront butterfly and a fixed
// sum over the 4 waves; dgamma/dbeta columns through LDS (packed tiles) or
// directly (row segments, where every column belongs to one thread). Each
// workgroup writes one partial row [dgamma(Wcols) | dbeta(Wcols) | dalpha]
// to the workspace. Pass 2 sums the partial rows column by column in a
// fixed order (16 contiguous segments, then the 16 segment sums in order)
// and rounds to the parameter dtype.
#pragma once

#include <type_traits>

#include "dyt_math.hpp"

namespace dyt {

#ifndef DYT_BLOCK
#define DYT_BLOCK 256
#endif
#ifndef DYT_TILE_CAP
#define DYT_TILE_CAP 4096
#endif
constexpr int kBlock = DYT_BLOCK;       // threads per workgroup (wave64s x 64)
constexpr int kTileCap = DYT_TILE_CAP;  // elements per tile of the default tiling
constexpr int kTileMax = 8192;          // largest tile of any plan (occupancy re-tiling)
constexpr int kSlotsMax = 4;            // largest K of the vector kernels
constexpr int kFinBlock = 1024;   // pass-2 threads: 64 outputs x 16 segments
constexpr int kFinSegs = kFinBlock / 64;

// Workgroup timeline, compiled in only for measurement builds
// (-DDYT_WG_TIMELINE=1): thread 0 of each workgroup of the forward kernels
// and of backward pass 1 records the constant-rate real-time counter at
// entry (word 0), at the end of its streaming loop (word 1) and at exit
// (word 2), and the XCD and hardware ids it ran on (word 3: XCC_ID << 32 |
// HW_ID), at 4 words per workgroup of a buffer the host supplies (null: no
// record). Default builds carry none of it.
#ifndef DYT_WG_TIMELINE
#define DYT_WG_TIMELINE 0
#endif
#ifndef DYT_FUSED_FIN
#define DYT_FUSED_FIN 0
#endif
#if DYT_WG_TIMELINE
#define DYT_STAMPS_FIELD uint64_t* stamps;
__device__ __forceinline__ void wg_stamp(uint64_t* s, int k) {
    if (s && threadIdx.x == 0) s[blockIdx.x * 4 + k] = __builtin_amdgcn_s_memrealtime();
}
__device__ __forceinline__ void wg_stamp_exit(uint64_t* s) {
    if (s && threadIdx.x == 0) {
        uint32_t xcc, hw;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
        s[blockIdx.x * 4 + 2] = __builtin_amdgcn_s_memrealtime();
        s[blockIdx.x * 4 + 3] = ((uint64_t)xcc << 32) | hw;
    }
}
#define DYT_STAMP(G, k) wg_stamp((G).stamps, (k))
#define DYT_STAMP_EXIT(G) wg_stamp_exit((G).stamps)
#else
#define DYT_STAMPS_FIELD
#define DYT_STAMP(G, k) ((void)0)
#define DYT_STAMP_EXIT(G) ((void)0)
#endif

struct Geo {
    int64_t total;     // M * N
    int64_t ntiles;
    int64_t N;         // row length (elements)
    int32_t T;         // packed: R*N elements per tile; wide: Wc
    int32_t R;         // packed: rows per tile; wide: 1
    int32_t nb;        // wide: column blocks per row; packed: 1
    int32_t last_len;  // wide: columns in the last block; packed: T
    int32_t ld;        // floats per workspace partial row
    int32_t wcols;     // packed: N; wide: Wc (dgamma/dbeta entries per row)
    // Row pitches (elements) of the activations of a strided launch: forward
    // x (and r), y (and h); backward x (and dres), dy, dx. N when contiguous.
    int64_t pitch[3];
    // Forward only: the share (x 1024) of each column block's groups that
    // the workgroups on even XCDs take (make_walk); 0: round-robin.
    int32_t even_share_q;
    // Forward only: 1 when the workgroups of odd index are expected on the
    // even XCDs (make_walk); xcd_seen, when not null, receives the XCD that
    // workgroup 0 ran on (a hint for the next launch's xcd_flip).
    int32_t xcd_flip;
    int32_t* xcd_seen;
    // Forward only, with even_share_q: the share (x 1024) of each column
    // block's groups that the first G / 2 workgroups take (make_walk); 0:
    // no split by dispatch round.
    int32_t round0_q;
    // Forward only: 1 when every 16-byte vector of y lies on the 16-byte grid
    // (y aligned, rows a whole number of vectors), so its write-back stores
    // may go through store_with_policy.
    int32_t buf_store;
    DYT_STAMPS_FIELD
#if DYT_FUSED_FIN
    // Fused finish (backward pass 1 only): when fin_out[0] is set, the
    // workgroup that finishes last sums the partial rows and writes dgamma,
    // dbeta, dalpha (fin_out[0..2], parameter dtype); ctr is the workspace's
    // arrival counter (zero on entry, left zero).
    void* fin_out[3];
    unsigned* ctr;
#endif
};

struct FinGeo {
    int64_t P;         // partial rows
    int64_t N;
    int32_t nb;
    int32_t wc;        // wide: block width
    int32_t wcols;
    int32_t ld;
    int32_t packed;
};

// ---------------------------------------------------------------- memory IO
// Raw<XT, V>: the V elements of one access as loaded from memory (one
// 16-byte vector, or one element). Loads return raw registers so that every
// load of a tile is issued before any value is needed. x, dy, y and dx are
// each touched exactly once, so the loads and the backward's stores carry
// the nontemporal hint (streaming through the caches instead of displacing
// other data; on MI355X this lifts a plain 16-byte copy from ~5.7 to ~6.4
// TB/s); the forward's stores take the hint only where it measured faster
// (fwd_tile_store_nt, fwd_flat_store_nt).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// The same vectors as seen in memory: only element alignment is assumed.
typedef uint32_t u32x4_m __attribute__((ext_vector_type(4), aligned(2)));
typedef float f32x4_m __attribute__((ext_vector_type(4), aligned(4)));

#ifndef DYT_FWD_NT
#define DYT_FWD_NT 1
#endif
// The persistent loops load group i + 1 while computing group i, two
// register buffers in turn. With an even number of groups the last pair is
// done without a second load; 1 restores the earlier form, whose last load
// re-read the previous group (valid memory, never computed).
#ifndef DYT_TAIL_PREFETCH
#define DYT_TAIL_PREFETCH 0
#endif
#ifndef DYT_BWD_NT
#define DYT_BWD_NT 1
#endif
// Store kind of the residual-fused pass 1's dh (1: nontemporal, as the plain
// pass 1's dx; 0: write-back). Its three input streams and one output
// stream run faster with write-back stores on MI355X: at 32,768 x 4,096
// bf16 the residual backward took 172.9 against 184.3 us, and a residual
// step (forward then backward) 357.1 against 368.8 us (bench.py --variants
// bwd_res_nt reproduces the nontemporal form); a reference stream of three
// inputs and one output measured fastest with write-back stores too.
#ifndef DYT_BWD_RES_NT
#define DYT_BWD_RES_NT 0
#endif
// Measurement builds only: pass 1 writes dx through a buffer descriptor with
// these cache-policy bits (contiguous, 16-byte aligned, no residual) instead
// of the stores above; 0 keeps them. Measured on MI355X (bench.py --variants
// bwd_store_sc0,bwd_store_sc1,bwd_store_sc1_nt): sc0, sc1 and sc1 +
// nontemporal made the 32,768 x 4,096 bf16 backward 23-26% slower (162-166
// against 131.6 us) and the float32 100,003-row ones 4-16% slower.
#ifndef DYT_BWD_STORE_POL
#define DYT_BWD_STORE_POL 0
#endif
template <bool NT, typename T>
__device__ __forceinline__ T stream_load(const T* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT, typename T>
__device__ __forceinline__ void stream_store(T v, T* p) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}
// 16-byte vectors at element-aligned addresses. Not deduced from the pointer
// type: template deduction would drop the reduced alignment of the typedef
// and the access would be declared 16-byte aligned.
template <bool NT>
__device__ __forceinline__ u32x4 stream_load_v(const u32x4_m* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT>
__device__ __forceinline__ f32x4 stream_load_v(const f32x4_m* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT>
__device__ __forceinline__ void stream_store_v(u32x4 v, u32x4_m* p) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}
template <bool NT>
__device__ __forceinline__ void stream_store_v(f32x4 v, f32x4_m* p) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

template <typename XT, int V> struct Raw;
// Each Raw<XT, V> has: load (raw registers), unpack (to float32), pack (float32
// to raw registers, rounding to nearest even), store_raw, and store = pack +
// store_raw. pack followed by unpack yields the values as stored.

template <> struct Raw<float, 4> {
    using T = f32x4;
    template <bool NT = true>
    static __device__ __forceinline__ T load(const float* p) {
        return stream_load_v<NT>(reinterpret_cast<const f32x4_m*>(p));
    }
    static __device__ __forceinline__ void unpack(const T& r, float (&v)[4]) {
        v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
    }
    static __device__ __forceinline__ T pack(const float (&v)[4]) {
        const f32x4 t = {v[0], v[1], v[2], v[3]};
        return t;
    }
    template <bool NT = true>
    static __device__ __forceinline__ void store_raw(float* p, const T& t) {
        stream_store_v<NT>(t, reinterpret_cast<f32x4_m*>(p));
    }
    template <bool NT = true>
    static __device__ __forceinline__ void store(float* p, const float (&v)[4]) {
        store_raw<NT>(p, pack(v));
    }
};

template <> struct Raw<bf16_t, 8> {
    using T = u32x4;
    template <bool NT = true>
    static __device__ __forceinline__ T load(const bf16_t* p) {
        return stream_load_v<NT>(reinterpret_cast<const u32x4_m*>(p));
    }
    static __device__ __forceinline__ void unpack(const T& r, float (&v)[8]) {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __builtin_bit_cast(float, w[i] << 16);
            v[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ T pack(const float (&v)[8]) {
        const u32x4 t = {pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]), pack2_bf16(v[4], v[5]),
                         pack2_bf16(v[6], v[7])};
        return t;
    }
    template <bool NT = true>
    static __device__ __forceinline__ void store_raw(bf16_t* p, const T& t) {
        stream_store_v<NT>(t, reinterpret_cast<u32x4_m*>(p));
    }
    template <bool NT = true>
    static __device__ __forceinline__ void store(bf16_t* p, const float (&v)[8]) {
        store_raw<NT>(p, pack(v));
    }
};

template <> struct Raw<f16_t, 8> {
    using T = u32x4;
    template <bool NT = true>
    static __device__ __forceinline__ T load(const f16_t* p) {
        return stream_load_v<NT>(reinterpret_cast<const u32x4_m*>(p));
    }
    static __device__ __forceinline__ void unpack(const T& r, float (&v)[8]) {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xffffu));
            v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
        }
    }
    static __device__ __forceinline__ T pack(const float (&v)[8]) {
        const u32x4 t = {pack2_f16(v[0], v[1]), pack2_f16(v[2], v[3]), pack2_f16(v[4], v[5]),
                         pack2_f16(v[6], v[7])};
        return t;
    }
    template <bool NT = true>
    static __device__ __forceinline__ void store_raw(f16_t* p, const T& t) {
        stream_store_v<NT>(t, reinterpret_cast<u32x4_m*>(p));
    }
    template <bool NT = true>
    static __device__ __forceinline__ void store(f16_t* p, const float (&v)[8]) {
        store_raw<NT>(p, pack(v));
    }
};

template <> struct Raw<f16_t, 1> {
    using T = uint16_t;
    template <bool NT = true>
    static __device__ __forceinline__ T load(const f16_t* p) {
        return stream_load<NT>(reinterpret_cast<const uint16_t*>(p));
    }
    static __device__ __forceinline__ void unpack(const T& r, float (&v)[1]) {
        v[0] = (float)__builtin_bit_cast(_Float16, r);
    }
    static __device__ __forceinline__ T pack(const float (&v)[1]) { return from_f32<f16_t>(v[0]).bits; }
    template <bool NT = true>
    static __device__ __forceinline__ void store_raw(f16_t* p, const T& t) {
        stream_store<NT>(t, reinterpret_cast<uint16_t*>(p));
    }
    template <bool NT = true>
    static __device__ __forceinline__ void store(f16_t* p, const float (&v)[1]) {
        store_raw<NT>(p, pack(v));
    }
};

template <> struct Raw<float, 1> {
    using T = float;
    template <bool NT = true>
    static __device__ __forceinline__ T load(const float* p) { return stream_load<NT>(p); }
    static __device__ __forceinline__ void unpack(const T& r, float (&v)[1]) { v[0] = r; }
    static __device__ __forceinline__ T pack(const float (&v)[1]) { return v[0]; }
    template <bool NT = true>
    static __device__ __forceinline__ void store_raw(float* p, const T& t) { stream_store<NT>(t, p); }
    template <bool NT = true>
    static __device__ __forceinline__ void store(float* p, const float (&v)[1]) {
        store_raw<NT>(p, pack(v));
    }
};

template <> struct Raw<bf16_t, 1> {
    using T = uint16_t;
    template <bool NT = true>
    static __device__ __forceinline__ T load(const bf16_t* p) {
        return stream_load<NT>(reinterpret_cast<const uint16_t*>(p));
    }
    static __device__ __forceinline__ void unpack(const T& r, float (&v)[1]) {
        v[0] = __builtin_bit_cast(float, (uint32_t)r << 16);
    }
    static __device__ __forceinline__ T pack(const float (&v)[1]) { return from_f32<bf16_t>(v[0]).bits; }
    template <bool NT = true>
    static __device__ __forceinline__ void store_raw(bf16_t* p, const T& t) {
        stream_store<NT>(t, reinterpret_cast<uint16_t*>(p));
    }
    template <bool NT = true>
    static __device__ __forceinline__ void store(bf16_t* p, const float (&v)[1]) {
        store_raw<NT>(p, pack(v));
    }
};

// First n (< V) elements only; the rest read as 0 and are not written.
template <typename XT, int V>
__device__ __forceinline__ void load_partial(const XT* p, int n, float (&v)[V]) {
#pragma unroll
    for (int e = 0; e < V; ++e) v[e] = (e < n) ? to_f32(p[e < n ? e : 0]) : 0.0f;
}
template <typename XT, int V>
__device__ __forceinline__ void store_partial(XT* p, int n, const float (&v)[V]) {
#pragma unroll
    for (int e = 0; e < V; ++e)
        if (e < n) p[e] = from_f32<XT>(v[e]);
}

// ------------------------------------------------------------ tile geometry
// Per-thread constants of the persistent loop. Slot k of thread tid covers
// tile offsets o = (k * kBlock + tid) * V + [0, V). A slot is "used" if its
// vector starts inside the workgroup's tiles (packed: o < T; row segments:
// o < this block's length). An unused slot is pointed at the tile's first
// whole vector (offset 0, or the shifted one below when a row segment is
// shorter than V) and given that vector's parameters, so it recomputes it
// and rewrites exactly the bytes its owner writes there. A
// used slot that would run past the end of a row segment (N not a multiple
// of V) is shifted back to end there: its first `lo` elements belong to the
// slot before it (or, in a segment shorter than V, to the previous column
// block), are recomputed from the same data and parameters, and so rewrite
// the same bytes; the backward leaves them out of its sums. Loads
// and stores therefore carry no branches, and the compiler can keep the
// next tile's loads in flight across this tile's stores (a conditional
// store makes it wait for every outstanding access at the loop back-edge).
template <int V, int K>
struct Slots {
    int off[K];     // element offset of the slot inside the tile (0 if unused)
    int lo[K];      // elements of the slot before this one's own (shifted slot), else 0
    bool used[K];
};

// SHIFT: row segments whose length may not be a multiple of V.
template <int V, int K, bool SHIFT>
__device__ __forceinline__ Slots<V, K> make_slots(int tid, int seg_len) {
    Slots<V, K> s;
    // 1 <= seg_len <= kTileMax; the clamp only tells the compiler the range
    // of the offsets. A segment shorter than V (the last of several column
    // blocks) has its one vector reach back into the previous block of the
    // same row: columns another workgroup owns and writes identically.
    const int last = min(max(seg_len - V, 1 - V), kTileMax - V);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int o = (k * kBlock + tid) * V;
        s.used[k] = o < seg_len;
        if constexpr (!SHIFT) {       // segment length a multiple of V
            s.off[k] = s.used[k] ? o : 0;
            s.lo[k] = 0;
        } else {
            // unused slots recompute the segment's first whole vector: the
            // one at offset 0, or the shifted one if the segment is shorter
            // than V (offset 0 would then run past the row's end)
            const bool full = o + V <= seg_len;
            s.off[k] = !s.used[k] ? min(last, 0) : full ? o : last;
            s.lo[k] = s.used[k] && !full ? o - last : 0;
        }
    }
    return s;
}

// Work of one workgroup. The data is cut into "units" of equal shape:
// whole tiles (packed) or rows (row segments; the workgroup owns one column
// block of every row). Units are taken in groups of U adjacent units, so a
// group is one contiguous run of memory (packed) or U row segments one row
// apart; groups are dealt round-robin to the gcount workgroups that share a
// column block: group index gw, gw + gcount, ... Units left over after the
// last whole group (fewer than U) are dealt the same way one by one, and a
// packed problem whose size is not a multiple of T has one partial tile
// (index units) that workgroup units % gcount handles with masks.
struct TileWalk {
    int64_t units;     // whole units
    int64_t unit;      // elements between consecutive units (T or N)
    int64_t gw;        // this workgroup's index among those of its column block
    int64_t gcount;    // workgroups per column block (G / nb)
    int64_t col_base;  // first column of this workgroup's block (0 when packed)
    int seg_len;       // elements (packed) or columns (row segments) per tile
    bool tail;         // this workgroup also owns the partial packed tile
    // The groups of U units of the main loop: g_first, g_first + g_stride,
    // ... below g_end.
    int64_t g_first, g_stride, g_end;
};

// Groups of ng that the even-XCD class takes at share share_q / 1024.
__host__ __device__ __forceinline__ int64_t even_groups(int64_t ng, int share_q) {
    return (ng * share_q + 512) >> 10;
}

//
// XCD-weighted deal (share_q != 0, the forward's write-back-store kernels).
// The hardware hands workgroup w to XCD (w + k) mod 8, k fixed per hardware
// queue (0 in a process that uses one stream; other values once more
// streams than hardware queues exist), and on MI355X workgroups on the odd
// XCDs stream with write-back (plain) stores 12-14% slower than those on
// the even XCDs, which end early and idle (bench.py --wg-timeline). With
// share_q the workgroups form two classes by the parity of w, each pair
// 2i, 2i + 1 sharing column block i mod nb; in every block the class
// expected on the even XCDs (even w, or odd w when flip = 1, i.e. k odd)
// takes the first share_q / 1024 of the groups and the other class the rest,
// each round-robin among its members. Every group is covered once whatever
// flip is, as long as it is the same for the whole launch (a kernel
// argument). Needs G a multiple of 2 nb, else (and with share_q = 0) every
// group is dealt round-robin to all of the block's workgroups.
// With round_q as well (G a multiple of 4 nb), the grid is first cut into
// its halves, the workgroups dispatched in the first and in the second
// round onto CUs that host two: each block's first round_q / 1024 of the
// groups go to the first half, the rest to the second, and within each half
// the two XCD classes split that half's range as above. The forward has no
// reduction: the deal changes which workgroup computes an element, never
// its bits.
template <int U>
__device__ __forceinline__ TileWalk make_walk(const Geo& g, bool packed, int64_t wg, int64_t G,
                                              int share_q, int flip, int round_q) {
    TileWalk w;
    const int64_t nb = packed ? 1 : g.nb;
    const bool weighted = share_q != 0 && G % (2 * nb) == 0;
    const bool rounds = weighted && round_q != 0 && G % (4 * nb) == 0;
    const int64_t H = rounds ? G / 2 : G;                 // workgroups per half
    const int64_t half = (rounds && wg >= H) ? 1 : 0;
    const int64_t wl = wg - half * H;                     // index within the half
    const int64_t pair = wl >> 1, odd = wl & 1;
    const int64_t b = weighted ? pair % nb : wg % nb;
    w.gw = weighted ? 2 * (pair / nb) + odd + half * (H / nb) : wg / nb;
    w.gcount = G / nb;
    if (packed) {
        w.units = g.total / g.T;
        w.unit = g.T;
        w.col_base = 0;
        w.seg_len = g.T;
        w.tail = (w.units * (int64_t)g.T < g.total) && (wg == w.units % G);
    } else {
        w.units = g.ntiles / g.nb;   // rows
        w.unit = g.N;
        w.col_base = b * g.T;
        w.seg_len = (b == g.nb - 1) ? g.last_len : g.T;
        w.tail = false;
    }
    const int64_t ng = w.units / U;
    if (weighted) {
        const int64_t n0 = rounds ? even_groups(ng, round_q) : ng;   // the first half's groups
        const int64_t lo = half ? n0 : 0, nr = half ? ng - n0 : n0;
        const int64_t ne = even_groups(nr, share_q);
        const int64_t cls = odd ^ (int64_t)(flip & 1);   // 1: the class expected on odd XCDs
        w.g_first = lo + (cls ? ne : 0) + pair / nb;
        w.g_stride = H / nb / 2;
        w.g_end = lo + (cls ? nr : ne);
    } else {
        w.g_first = w.gw;
        w.g_stride = w.gcount;
        w.g_end = ng;
    }
    return w;
}

// Addressing of one tensor in this workgroup's walk: unit u starts at
// element col_base + u * upitch, and slot k lies `off[k]` elements after it.
// Contiguous tensors share one Addr (upitch = T or N, off = the slot's tile
// offset). A tensor with row pitch ld (strided launch) has upitch = R * ld
// (packed) or ld (row segments), and a packed slot at tile offset o lies at
// (o / N) * ld + o mod N: with N a multiple of V the slot's V elements stay
// in one row.
template <int K, bool STRIDED>
struct Addr {
    using Off = typename std::conditional<STRIDED, int64_t, int>::type;
    int64_t upitch;
    Off off[K];
};

template <int V, int K, bool PACKED, bool STRIDED>
__device__ __forceinline__ Addr<K, STRIDED> make_addr(const Slots<V, K>& sl, const TileWalk& w,
                                                      const Geo& g, int64_t ld) {
    Addr<K, STRIDED> a;
    if constexpr (!STRIDED) {
        a.upitch = w.unit;
#pragma unroll
        for (int k = 0; k < K; ++k) a.off[k] = sl.off[k];
    } else {
        a.upitch = PACKED ? (int64_t)g.R * ld : ld;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int o = sl.off[k];
            a.off[k] = PACKED ? (int64_t)(o / (int)g.N) * ld + o % (int)g.N : (int64_t)o;
        }
    }
    return a;
}

// Offset of tile offset o (a natural slot position, for the masked tail).
template <bool PACKED, bool STRIDED>
__device__ __forceinline__ int64_t tile_off(int o, const Geo& g, int64_t ld) {
    if constexpr (STRIDED && PACKED) return (int64_t)(o / (int)g.N) * ld + o % (int)g.N;
    else return o;
}

template <bool ACC>
__device__ __forceinline__ float dyt_tanh(float u) {
    if constexpr (ACC) return tanh_fwd_f32(u);
    else return tanh_fast(u);
}
template <bool ACC>
__device__ __forceinline__ void dyt_tanh_sech2(float xv, float alpha, float& t, float& d) {
    if constexpr (ACC) tanh_sech2_accurate(xv, alpha, t, d);
    else tanh_sech2_fast(alpha * xv, t, d);
}

// Loads of U consecutive tiles of this workgroup (all K slots, raw
// registers; tile j of the input sits at bi + j * pi) and the forward
// arithmetic and stores of such a loaded group (outputs at bo + j * po).
// With RES the residual r is loaded beside x, h = x + r is rounded to the
// storage type and stored, and y is computed from the stored h.
template <typename XT, int V, int K, int U, bool RES, typename AD>
__device__ __forceinline__ void fwd_load(const XT* __restrict__ x, const XT* __restrict__ r,
                                         int64_t bi, const AD& ai,
                                         typename Raw<XT, V>::T (&rx)[U][K],
                                         typename Raw<XT, V>::T (&rr)[U][K]) {
#pragma unroll
    for (int j = 0; j < U; ++j)
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int64_t at = bi + j * ai.upitch + ai.off[k];
            rx[j][k] = Raw<XT, V>::template load<DYT_FWD_NT>(x + at);
            if constexpr (RES) rr[j][k] = Raw<XT, V>::template load<DYT_FWD_NT>(r + at);
        }
}

// Store hint of the forward's outputs (y, and h with the residual add).
// Loads always stream nontemporally. Stores: plain write-back stores where
// each thread stores one vector per tile (K = 1) and in the flat walk over
// 2-byte data, nontemporal otherwise. Measured on MI355X, alone and in
// back-to-back forward + backward steps, bit-identical outputs: float16
// 32768 x 4096 (K = 1 tiles) 93.9 -> 82.0 us alone, step 236.6 -> 225.8 us;
// the flat walk over bfloat16 / float16 rows of 2,560 89.1 / 86.4 -> 83.6 /
// 83.5 us alone, step -2.7% / -2.2%; but float32 flat rows of 5,120 182.0 ->
// 189.2 us and the residual-fused forward at K = 2 178.4 -> 185.5 us with
// plain stores, so those keep the hint. (For the bfloat16 and float32 K = 1
// tiles the compiler had already emitted plain stores.)
template <typename XT, int K>
constexpr bool fwd_tile_store_nt() { return DYT_FWD_NT && K >= 2; }
template <typename XT, bool RES>
constexpr bool fwd_flat_store_nt() { return DYT_FWD_NT && (RES || sizeof(XT) == 4); }

// Cache policy of the plain forward's write-back stores above (contiguous
// launches with 16-byte vectors), per x dtype size: 0 keeps ordinary
// stores; a nonzero value sends each such store through a buffer descriptor
// based at the workgroup-uniform start of its tile with those cache-policy
// bits (16: sc1, written through to device scope instead of staying dirty
// in its XCD's L2). Measured on MI355X (bench.py --variants
// fwd_store_f32_plain,fwd_store_sc1_all): sc1 made the float32 100,003 x
// 100 and x 255 forwards 4-10% faster and the bfloat16 32,768 x 4,096 and
// 4,194,304 x 32 forwards 9-13% slower.
#ifndef DYT_FWD_STORE_POL_F32
#define DYT_FWD_STORE_POL_F32 16
#endif
#ifndef DYT_FWD_STORE_POL_2B
#define DYT_FWD_STORE_POL_2B 0
#endif
template <typename XT>
constexpr int fwd_store_pol() { return sizeof(XT) == 4 ? DYT_FWD_STORE_POL_F32 : DYT_FWD_STORE_POL_2B; }

// 16-byte store of raw (one vector) at byte_off from a workgroup-uniform
// base, through a raw buffer descriptor of span_bytes (stores past the span
// are dropped by the hardware's range check; callers stay inside it), with
// cache-policy bits POL.
template <int POL, typename T>
__device__ __forceinline__ void store_with_policy(void* uniform_base, uint32_t span_bytes,
                                                  uint32_t byte_off, const T& raw) {
    static_assert(sizeof(T) == 16, "one 16-byte vector");
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(uniform_base, (short)0, (int)span_bytes, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, raw), rs, (int)byte_off, 0, POL);
}

// v = x (+ r, rounded to XT and stored to h when RES; store hint ST_NT)
template <typename XT, int V, bool RES, bool ST_NT>
__device__ __forceinline__ void fwd_input(const typename Raw<XT, V>::T& rx,
                                          const typename Raw<XT, V>::T& rr, XT* __restrict__ h,
                                          float (&v)[V]) {
    using R = Raw<XT, V>;
    R::unpack(rx, v);
    if constexpr (RES) {
        float rv[V];
        R::unpack(rr, rv);
#pragma unroll
        for (int e = 0; e < V; ++e) v[e] += rv[e];
        const typename R::T hr = R::pack(v);
        R::template store_raw<ST_NT>(h, hr);
        R::unpack(hr, v);
    }
}

// BUF: y's stores go through store_with_policy when span_bytes, the tile's
// bytes, is nonzero (bo, the tile's start, is workgroup-uniform); else, and
// without BUF, plain stores.
template <typename XT, int V, int K, int U, bool ACC, bool RES, bool BUF, typename AD>
__device__ __forceinline__ void fwd_tile(const typename Raw<XT, V>::T (&rx)[U][K],
                                         const typename Raw<XT, V>::T (&rr)[U][K],
                                         XT* __restrict__ y, XT* __restrict__ h, int64_t bo,
                                         const AD& ao, const float (&gm)[K][V],
                                         const float (&bt)[K][V], float alpha,
                                         uint32_t span_bytes) {
#pragma unroll
    for (int j = 0; j < U; ++j)
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int64_t at = bo + j * ao.upitch + ao.off[k];
            constexpr bool kStNt = fwd_tile_store_nt<XT, K>();
            float v[V];
            fwd_input<XT, V, RES, kStNt>(rx[j][k], rr[j][k], h + at, v);
#pragma unroll
            for (int e = 0; e < V; ++e)
                v[e] = __builtin_fmaf(gm[k][e], dyt_tanh<ACC>(alpha * v[e]), bt[k][e]);
            bool done = false;
            if constexpr (BUF) {
                if (span_bytes != 0) {
                    store_with_policy<fwd_store_pol<XT>()>(y + bo + j * ao.upitch, span_bytes,
                                                         (uint32_t)(ao.off[k] * (int)sizeof(XT)),
                                                         Raw<XT, V>::pack(v));
                    done = true;
                }
            }
            if (!done) Raw<XT, V>::template store<kStNt>(y + at, v);
        }
}

// ---------------------------------------------------------------- forward
// y = gamma * tanh(alpha * x) + beta; with RES (residual add fused in front)
// h = x + r and y = gamma * tanh(alpha * h) + beta. Loads of the next tile
// are issued before the current tile is computed (register double
// buffering). r and h are unused (null) without RES. STRIDED: x and y have
// row pitches g.pitch[0] and g.pitch[1] (no RES). RAG: row segments whose
// length N is not a multiple of V (shifted slots).
template <typename XT, typename PT, int V, int K, int U, bool PACKED, bool RES, bool STRIDED,
          bool RAG>
__global__ void __launch_bounds__(kBlock)
dyt_fwd_kernel(const XT* __restrict__ x, const XT* __restrict__ r,
               const PT* __restrict__ alpha_p, const PT* __restrict__ gamma,
               const PT* __restrict__ beta, XT* __restrict__ y, XT* __restrict__ h,
               const Geo g) {
    static_assert(!(RES && STRIDED), "the residual layer takes contiguous tensors");
    static_assert(!(RAG && PACKED), "packed tiles hold whole vectors");
    using R = Raw<XT, V>;
    constexpr bool ACC = std::is_same<XT, float>::value;
    const int tid = threadIdx.x;
    const int64_t wg = blockIdx.x;
    const int64_t G = gridDim.x;
    const float alpha = to_f32(alpha_p[0]);
    const TileWalk w = make_walk<U>(g, PACKED, wg, G, g.even_share_q, g.xcd_flip, g.round0_q);
    const Slots<V, K> sl = make_slots<V, K, RAG>(tid, w.seg_len);
    const Addr<K, STRIDED> ai = make_addr<V, K, PACKED, STRIDED>(sl, w, g, g.pitch[0]);
    const Addr<K, STRIDED> ao = STRIDED ? make_addr<V, K, PACKED, STRIDED>(sl, w, g, g.pitch[1]) : ai;
    DYT_STAMP(g, 0);
    if (g.xcd_seen != nullptr && wg == 0 && tid == 0) {
        uint32_t xcc;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
        *g.xcd_seen = (int32_t)(xcc & 0xFu);
    }

    float gm[K][V], bt[K][V];
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const int o = sl.off[k] + e;   // unused slots: tile offsets 0..V-1
            const int64_t c = PACKED ? (int64_t)(o % (int)g.N) : w.col_base + o;
            gm[k][e] = to_f32(gamma[c]);
            bt[k][e] = to_f32(beta[c]);
        }
    // write-back stores of y with a cache policy (see fwd_store_pol)
    constexpr bool BUF = fwd_store_pol<XT>() != 0 && !STRIDED && !RES && V > 1 &&
                         !fwd_tile_store_nt<XT, K>();
    const uint32_t span = g.buf_store ? (uint32_t)w.seg_len * (uint32_t)sizeof(XT) : 0u;

    // Persistent loop over this workgroup's groups of U adjacent units,
    // alternating between two register buffers (A and B): the loads of one
    // group are in flight while the other group is computed. Each step's
    // loads are pinned above the compute that follows them by a scheduling
    // barrier. With an even number of groups the last pair is done without
    // a further load (DYT_TAIL_PREFETCH).
    const int64_t ng = w.units / U;
    const int64_t iters = w.g_first < w.g_end ? (w.g_end - w.g_first + w.g_stride - 1) / w.g_stride : 0;
    const int64_t ustep = w.g_stride * U;        // units between this workgroup's groups
    const int64_t gsi = ustep * ai.upitch, gso = ustep * ao.upitch;
    if (iters > 0) {
        typename R::T xa[U][K], xb[U][K], ra[U][K], rb[U][K];
        int64_t bia = w.col_base + w.g_first * U * ai.upitch;   // input / output bases of group A
        int64_t boa = STRIDED ? w.col_base + w.g_first * U * ao.upitch : bia;
        fwd_load<XT, V, K, U, RES>(x, r, bia, ai, xa, ra);
        const int64_t npairs = iters / 2;
        const int64_t nfull = (DYT_TAIL_PREFETCH || (iters & 1)) ? npairs : npairs - 1;
        for (int64_t pi = 0; pi < nfull; ++pi) {
            const int64_t bib = bia + gsi, bob = STRIDED ? boa + gso : bib;
            fwd_load<XT, V, K, U, RES>(x, r, bib, ai, xb, rb);
            __builtin_amdgcn_sched_barrier(0);
            fwd_tile<XT, V, K, U, ACC, RES, BUF>(xa, ra, y, h, boa, ao, gm, bt, alpha, span);
            __builtin_amdgcn_sched_barrier(0);
            const bool more = 2 * pi + 2 < iters;
            const int64_t bin = more ? bib + gsi : bib;
            const int64_t bon = STRIDED ? (more ? bob + gso : bob) : bin;
            fwd_load<XT, V, K, U, RES>(x, r, bin, ai, xa, ra);
            __builtin_amdgcn_sched_barrier(0);
            fwd_tile<XT, V, K, U, ACC, RES, BUF>(xb, rb, y, h, bob, ao, gm, bt, alpha, span);
            __builtin_amdgcn_sched_barrier(0);
            bia = bin;
            boa = bon;
        }
        if (!DYT_TAIL_PREFETCH && !(iters & 1)) {   // the last pair (iters >= 2)
            const int64_t bib = bia + gsi, bob = STRIDED ? boa + gso : bib;
            fwd_load<XT, V, K, U, RES>(x, r, bib, ai, xb, rb);
            __builtin_amdgcn_sched_barrier(0);
            fwd_tile<XT, V, K, U, ACC, RES, BUF>(xa, ra, y, h, boa, ao, gm, bt, alpha, span);
            __builtin_amdgcn_sched_barrier(0);
            fwd_tile<XT, V, K, U, ACC, RES, BUF>(xb, rb, y, h, bob, ao, gm, bt, alpha, span);
        }
        if (iters & 1) fwd_tile<XT, V, K, U, ACC, RES, BUF>(xa, ra, y, h, boa, ao, gm, bt, alpha, span);
    }
    // units after the last whole group (fewer than U in total)
    for (int64_t u = ng * U + w.gw; u < w.units; u += w.gcount) {
        typename R::T x1[1][K], r1[1][K];
        fwd_load<XT, V, K, 1, RES>(x, r, w.col_base + u * ai.upitch, ai, x1, r1);
        fwd_tile<XT, V, K, 1, ACC, RES, BUF>(x1, r1, y, h, w.col_base + u * ao.upitch, ao, gm, bt, alpha,
                                             span);
    }
    DYT_STAMP(g, 1);

    if (PACKED && w.tail) {
        const int64_t ti = w.units * ai.upitch;   // the partial tile, input side
        const int64_t to = w.units * ao.upitch;   // and output side
        const int len = (int)(g.total - w.units * (int64_t)g.T);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int o = (k * kBlock + tid) * V;
            const int n = len - o;
            if (n > 0) {
                const int64_t oi = ti + tile_off<PACKED, STRIDED>(o, g, g.pitch[0]);
                const int64_t oo = to + tile_off<PACKED, STRIDED>(o, g, g.pitch[1]);
                float v[V];
                if (n >= V) {
                    typename R::T rr{};
                    if constexpr (RES) rr = R::load(r + oi);
                    fwd_input<XT, V, RES, fwd_tile_store_nt<XT, K>()>(R::load(x + oi), rr, h + oo, v);
                } else {
                    load_partial<XT, V>(x + oi, n, v);
                    if constexpr (RES) {
                        float rv[V];
                        load_partial<XT, V>(r + oi, n, rv);
#pragma unroll
                        for (int e = 0; e < V; ++e) v[e] = to_f32(from_f32<XT>(v[e] + rv[e]));
                        store_partial<XT, V>(h + oo, n, v);
                    }
                }
#pragma unroll
                for (int e = 0; e < V; ++e)
                    v[e] = __builtin_fmaf(gm[k][e], dyt_tanh<ACC>(alpha * v[e]), bt[k][e]);
                if (n >= V) R::template store<fwd_tile_store_nt<XT, K>()>(y + oo, v);
                else store_partial<XT, V>(y + oo, n, v);
            }
        }
    }
    DYT_STAMP_EXIT(g);
}

// ------------------------------------------------------------ flat forward
// The forward over contiguous rows that the slot tiles fit poorly (e.g.
// 2,560 bfloat16 columns: 62% of the slots of two 2,048-element row
// segments) or whose length N is not a multiple of V (RAG: the tiles then
// shift their slots row by row). The problem is walked as one run of
// nvec = floor(M*N/V) vectors, so every access carries data; vector q
// covers elements q*V .. q*V+V-1, whose columns are c .. c+V-1 taken mod N
// with c = (q*V) mod N, and gamma/beta come from a float32 copy of both in
// LDS instead of per-thread registers: 2*N floats. With RAG, c is any
// column and the entries c .. c+V-1 may run past column N - 1 (no vector
// straddles a row when N is a multiple of V), so each parameter is kept as
// 4 copies of N+V entries running on with columns 0, 1, ... again, copy s
// shifted left by s words: entry c then sits at the multiple of 4 c - s of
// copy s = c mod 4, and every read is a 16-byte LDS read as without RAG.
// The last M*N mod V elements (RAG only) are done by one thread of
// workgroup 0. With RAG the walk may also start head elements in, at the
// first element whose address is a multiple of 128 bytes (a cache line; 16
// bytes if the tensors are not all off the line grid by the same amount)
// when the tensors start off that grid: every wave access then covers whole
// lines, the head elements are done one per thread of the last workgroup,
// and vector q covers elements head + q*V ... with columns from
// (q*V + head) mod N.
// The vectors are cut into groups of
// B = U * kBlock (one contiguous run); workgroup w of G takes groups w,
// w + G, ..., and thread tid vectors tid, tid + kBlock, ... of each, so
// every wave access covers 64 adjacent vectors. A thread's U columns each
// advance by cstep = (G*B*V) mod N from one of its groups to the next. The
// last, partial group (nvec mod B vectors) goes to workgroup
// (nvec / B) mod G, with a bounds check per vector. Loads, arithmetic,
// rounding and stores per element are those of dyt_fwd_kernel: both give
// the same bits.
// Words per copy of the RAG layout: entries 0 .. N+V-1, rounded up to a
// multiple of 4 (every copy starts 16-byte aligned). 4 copies per parameter.
__host__ __device__ constexpr int flat_rag_len(int N, int V) {
    return (N + V + 3) / 4 * 4;
}

struct FlatGeo {
    int64_t nvec;      // whole vectors of the walk (floor(total / V))
    int64_t total;     // elements of the walk (M * N - head)
    int32_t N;         // row length
    int32_t cstep;     // (G * U * kBlock * V) mod N
    int32_t head;      // RAG only: elements before the walk (< 128 bytes), one per thread
    int32_t even_share_q;  // share (x 1024) of the groups the even-XCD workgroups take; 0: round-robin
    int32_t xcd_flip;      // 1: odd workgroups expected on the even XCDs (as in Geo)
    int32_t* xcd_seen;     // not null: receives the XCD of workgroup 0 (as in Geo)
    int32_t buf_store;     // 1: y + head on the 16-byte grid (store_with_policy allowed)
    DYT_STAMPS_FIELD
};

template <typename XT, int U, bool RES>
__device__ __forceinline__ void flat_load(const XT* __restrict__ x, const XT* __restrict__ r,
                                          int64_t q, typename Raw<XT, 16 / sizeof(XT)>::T (&rx)[U],
                                          typename Raw<XT, 16 / sizeof(XT)>::T (&rr)[U]) {
    constexpr int V = 16 / sizeof(XT);
#pragma unroll
    for (int j = 0; j < U; ++j) {
        const int64_t at = (q + j * kBlock) * V;
        rx[j] = Raw<XT, V>::template load<DYT_FWD_NT>(x + at);
        if constexpr (RES) rr[j] = Raw<XT, V>::template load<DYT_FWD_NT>(r + at);
    }
}

// Computes and stores vector q + j*kBlock (column col[j]) of a loaded group.
// BUF: y's store goes through store_with_policy at byte bo_bytes from yb,
// the workgroup-uniform start of the group, when span_bytes (one group) is
// nonzero.
template <typename XT, bool ACC, bool RES, bool RAG, bool BUF = false>
__device__ __forceinline__ void flat_vec(const typename Raw<XT, 16 / sizeof(XT)>::T& rx,
                                         const typename Raw<XT, 16 / sizeof(XT)>::T& rr,
                                         XT* __restrict__ y, XT* __restrict__ h, int64_t at,
                                         int col, const float* sg, const float* sb, float alpha,
                                         int L, XT* yb = nullptr, uint32_t bo_bytes = 0,
                                         uint32_t span_bytes = 0) {
    constexpr int V = 16 / sizeof(XT);
    float v[V], gm[V], bt[V];
    constexpr bool kStNt = fwd_flat_store_nt<XT, RES>();
    fwd_input<XT, V, RES, kStNt>(rx, rr, h + at, v);
    // Without RAG col is a multiple of V (and so of 4); with RAG copy s =
    // col mod 4 holds entry col at the multiple of 4 col - s. Either way the
    // V entries from col on are 16-byte LDS reads.
    int base = col;
    if constexpr (RAG) {
        const int s = col & 3;
        base = (col - s) + s * L;
    }
#pragma unroll
    for (int e = 0; e < V; e += 4) {
        const float4 g4 = *reinterpret_cast<const float4*>(sg + base + e);
        const float4 b4 = *reinterpret_cast<const float4*>(sb + base + e);
        gm[e] = g4.x; gm[e + 1] = g4.y; gm[e + 2] = g4.z; gm[e + 3] = g4.w;
        bt[e] = b4.x; bt[e + 1] = b4.y; bt[e + 2] = b4.z; bt[e + 3] = b4.w;
    }
#pragma unroll
    for (int e = 0; e < V; ++e) v[e] = __builtin_fmaf(gm[e], dyt_tanh<ACC>(alpha * v[e]), bt[e]);
    bool done = false;
    if constexpr (BUF) {
        if (span_bytes != 0) {
            store_with_policy<fwd_store_pol<XT>()>(yb, span_bytes, bo_bytes, Raw<XT, V>::pack(v));
            done = true;
        }
    }
    if (!done) Raw<XT, V>::template store<kStNt>(y + at, v);
}

// Computes and stores a loaded group, then moves each column on to this
// thread's next group.
// q: this thread's first vector of the group, q0: the group's first vector
// (workgroup-uniform).
template <typename XT, int U, bool ACC, bool RES, bool RAG>
__device__ __forceinline__ void flat_group(const typename Raw<XT, 16 / sizeof(XT)>::T (&rx)[U],
                                           const typename Raw<XT, 16 / sizeof(XT)>::T (&rr)[U],
                                           XT* __restrict__ y, XT* __restrict__ h, int64_t q,
                                           int64_t q0, int (&col)[U], const float* sg,
                                           const float* sb, float alpha, int N, int cstep, int L,
                                           bool buf) {
    constexpr int V = 16 / sizeof(XT);
    // write-back stores of y with a cache policy (see fwd_store_pol)
    constexpr bool BUF = fwd_store_pol<XT>() != 0 && !fwd_flat_store_nt<XT, RES>();
    XT* const yb = y + q0 * V;
#pragma unroll
    for (int j = 0; j < U; ++j) {
        flat_vec<XT, ACC, RES, RAG, BUF>(rx[j], rr[j], y, h, (q + j * kBlock) * V, col[j], sg, sb, alpha,
                                         L, yb, (uint32_t)((q - q0 + j * kBlock) * 16),
                                         buf ? (uint32_t)(U * kBlock * 16) : 0u);
        const int c = col[j] + cstep;
        col[j] = c >= N ? c - N : c;
    }
}

// Dynamic LDS: 2 * N floats (gamma, then beta), with RAG 8 * flat_rag_len.
// r and h as in dyt_fwd_kernel (null without RES).
template <typename XT, typename PT, int U, bool RES, bool RAG>
__global__ void __launch_bounds__(kBlock)
dyt_fwd_flat_kernel(const XT* __restrict__ x, const XT* __restrict__ r,
                    const PT* __restrict__ alpha_p, const PT* __restrict__ gamma,
                    const PT* __restrict__ beta, XT* __restrict__ y, XT* __restrict__ h,
                    const FlatGeo f) {
    constexpr int V = 16 / sizeof(XT);
    constexpr int64_t B = (int64_t)U * kBlock;   // vectors per group
    using R = Raw<XT, V>;
    constexpr bool ACC = std::is_same<XT, float>::value;
    extern __shared__ float4 flat_lds[];
    DYT_STAMP(f, 0);
    const int N = f.N;
    const int L = RAG ? flat_rag_len(N, V) : N;         // words per copy
    const int NW = RAG ? 4 * L : N;                     // LDS words per parameter
    float* const sg = reinterpret_cast<float*>(flat_lds);
    float* const sb = sg + NW;
    const int tid = threadIdx.x;
    if constexpr (RAG) {
        // word k of copy s is column (k + s) mod N: column c, read once,
        // goes to words c - s + m*N (m >= 0) of copy s that lie in [0, L)
        for (int c = tid; c < N; c += kBlock) {
            const float gv = to_f32(gamma[c]);
            const float bv = to_f32(beta[c]);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                for (int k = c - s; k < L; k += N)
                    if (k >= 0) {
                        sg[s * L + k] = gv;
                        sb[s * L + k] = bv;
                    }
        }
    } else {
        for (int c = tid; c < N; c += kBlock) {
            sg[c] = to_f32(gamma[c]);
            sb[c] = to_f32(beta[c]);
        }
    }
    __syncthreads();
    const float alpha = to_f32(alpha_p[0]);
    const int64_t w = blockIdx.x;
    const int64_t G = gridDim.x;
    const int hd = RAG ? f.head : 0;
    if (RAG && hd > 0 && w == G - 1 && tid < hd) {
        // the head, one element per thread: column tid mod N (copy 0: word c
        // is column c mod N)
        const int c = tid % N;
        float v = to_f32(x[tid]);
        if constexpr (RES) {
            v = to_f32(from_f32<XT>(v + to_f32(r[tid])));
            h[tid] = from_f32<XT>(v);
        }
        y[tid] = from_f32<XT>(__builtin_fmaf(sg[c], dyt_tanh<ACC>(alpha * v), sb[c]));
    }
    // the walk, from element hd on
    x += hd;
    y += hd;
    if constexpr (RES) {
        r += hd;
        h += hd;
    }
    const int64_t ngroups = f.nvec / B;                 // whole groups
    // The groups of this workgroup: round-robin over all workgroups, or with
    // even_share_q (G even) the XCD-weighted deal of make_walk: the class
    // expected on the even XCDs (even w, or odd w with xcd_flip) takes the
    // first even_groups(ngroups) groups, the other class the rest, each
    // round-robin among the G / 2 of its class.
    const bool weighted = f.even_share_q != 0;
    const int64_t cls = (w & 1) ^ (int64_t)(f.xcd_flip & 1);
    const int64_t ne = weighted ? even_groups(ngroups, f.even_share_q) : ngroups;
    const int64_t g_stride = weighted ? G / 2 : G;
    const int64_t g_first = weighted ? (cls ? ne : 0) + (w >> 1) : w;
    const int64_t g_end = weighted && cls ? ngroups : ne;
    if (weighted && f.xcd_seen != nullptr && w == 0 && tid == 0) {
        uint32_t xcc;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
        *f.xcd_seen = (int32_t)(xcc & 0xFu);
    }
    const int64_t iters = g_first < g_end ? (g_end - g_first + g_stride - 1) / g_stride : 0;
    int col[U];
#pragma unroll
    for (int j = 0; j < U; ++j) col[j] = (int)(((g_first * B + j * kBlock + tid) * V + hd) % N);

    // Same two-buffer loop as dyt_fwd_kernel (no load past this workgroup's
    // groups, see DYT_TAIL_PREFETCH). f.cstep advances the columns by
    // g_stride groups.
    const int64_t gstep = g_stride * B;
    if (iters > 0) {
        typename R::T xa[U], xb[U], ra[U], rb[U];
        int64_t qa0 = g_first * B;                       // group starts (uniform)
        int64_t qa = qa0 + tid;
        flat_load<XT, U, RES>(x, r, qa, xa, ra);
        const int64_t npairs = iters / 2;
        const int64_t nfull = (DYT_TAIL_PREFETCH || (iters & 1)) ? npairs : npairs - 1;
        for (int64_t pi = 0; pi < nfull; ++pi) {
            const int64_t qb0 = qa0 + gstep, qb = qa + gstep;
            flat_load<XT, U, RES>(x, r, qb, xb, rb);
            __builtin_amdgcn_sched_barrier(0);
            flat_group<XT, U, ACC, RES, RAG>(xa, ra, y, h, qa, qa0, col, sg, sb, alpha, N, f.cstep, L,
                                             f.buf_store != 0);
            __builtin_amdgcn_sched_barrier(0);
            const bool more = 2 * pi + 2 < iters;
            const int64_t qn0 = more ? qb0 + gstep : qb0, qn = more ? qb + gstep : qb;
            flat_load<XT, U, RES>(x, r, qn, xa, ra);
            __builtin_amdgcn_sched_barrier(0);
            flat_group<XT, U, ACC, RES, RAG>(xb, rb, y, h, qb, qb0, col, sg, sb, alpha, N, f.cstep, L,
                                             f.buf_store != 0);
            __builtin_amdgcn_sched_barrier(0);
            qa0 = qn0;
            qa = qn;
        }
        if (!DYT_TAIL_PREFETCH && !(iters & 1)) {   // the last pair (iters >= 2)
            const int64_t qb0 = qa0 + gstep, qb = qa + gstep;
            flat_load<XT, U, RES>(x, r, qb, xb, rb);
            __builtin_amdgcn_sched_barrier(0);
            flat_group<XT, U, ACC, RES, RAG>(xa, ra, y, h, qa, qa0, col, sg, sb, alpha, N, f.cstep, L,
                                             f.buf_store != 0);
            __builtin_amdgcn_sched_barrier(0);
            flat_group<XT, U, ACC, RES, RAG>(xb, rb, y, h, qb, qb0, col, sg, sb, alpha, N, f.cstep, L,
                                             f.buf_store != 0);
        }
        if (iters & 1)
            flat_group<XT, U, ACC, RES, RAG>(xa, ra, y, h, qa, qa0, col, sg, sb, alpha, N, f.cstep, L,
                                             f.buf_store != 0);
    }
    DYT_STAMP(f, 1);
    // The partial group (index ngroups) goes to the workgroup whose sequence
    // reaches it; its columns have advanced to that group.
    const bool owns_partial = weighted ? (cls && (w >> 1) == (ngroups - ne) % g_stride)
                                       : w == ngroups % G;
    if (ngroups * B < f.nvec && owns_partial) {
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int64_t q = ngroups * B + j * kBlock + tid;
            if (q < f.nvec) {
                typename R::T x1, r1{};
                x1 = R::template load<DYT_FWD_NT>(x + q * V);
                if constexpr (RES) r1 = R::template load<DYT_FWD_NT>(r + q * V);
                flat_vec<XT, ACC, RES, RAG>(x1, r1, y, h, q * V, col[j], sg, sb, alpha, L);
            }
        }
    }
    // RAG: the last total - nvec*V (< V) elements, columns c0 .. c0+n-1 mod N.
    if constexpr (RAG) {
        const int64_t t0 = f.nvec * V;
        if (t0 < f.total && w == 0 && tid == 0) {
            const int n = (int)(f.total - t0);
            const int c0 = (int)((t0 + hd) % N);
            float v[V];
            load_partial<XT, V>(x + t0, n, v);
            if constexpr (RES) {
                float rv[V];
                load_partial<XT, V>(r + t0, n, rv);
#pragma unroll
                for (int e = 0; e < V; ++e) v[e] = to_f32(from_f32<XT>(v[e] + rv[e]));
                store_partial<XT, V>(h + t0, n, v);
            }
#pragma unroll
            for (int e = 0; e < V; ++e)   // copy 0: word c is column c mod N
                v[e] = __builtin_fmaf(sg[c0 + e], dyt_tanh<ACC>(alpha * v[e]), sb[c0 + e]);
            store_partial<XT, V>(y + t0, n, v);
        }
    }
    DYT_STAMP_EXIT(f);
}

#if DYT_FUSED_FIN
// The finish of pass 2 done by one workgroup of kBlock threads, in pass 2's
// summation order (16 contiguous row segments, each summed in row order from
// 0, then the 16 segment sums in order), so the results equal pass 2's bit
// for bit. Output j < N sits at column j of the partial rows (dgamma),
// N <= j < 2N at wcols + j - N (dbeta), j = 2N at 2 wcols (dalpha). Threads
// take 16 outputs x 16 segments per round, several rounds in flight.
template <typename PT>
__device__ void finish_in_workgroup(const float* __restrict__ ws, int64_t P, int ld, int64_t N,
                                    int wcols, PT* __restrict__ dg, PT* __restrict__ db,
                                    PT* __restrict__ da) {
    constexpr int kR = 4;                       // rounds in flight
    __shared__ float seg_sum[kR][16][16];
    const int tid = threadIdx.x;
    const int seg = tid >> 4, c = tid & 15;
    const int64_t nout = 2 * N + 1;
    const int64_t i0 = seg * P / 16, i1 = (seg + 1) * P / 16;
    for (int64_t base = 0; base < nout; base += 16 * kR) {
        float acc[kR];
#pragma unroll
        for (int r = 0; r < kR; ++r) {
            const int64_t j = base + r * 16 + c;
            int64_t off = 0;
            if (j < N) off = j;
            else if (j < 2 * N) off = wcols + (j - N);
            else off = 2 * (int64_t)wcols;
            acc[r] = 0.0f;
            const bool ok = j < nout;
            const float* __restrict__ p = ws + i0 * ld + off;
            int64_t i = i0;
            for (; i + 16 <= i1; i += 16, p += 16 * (int64_t)ld) {
                float v[16];
#pragma unroll
                for (int q = 0; q < 16; ++q) v[q] = ok ? p[q * (int64_t)ld] : 0.0f;
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[r] += v[q];
            }
            for (; i < i1; ++i, p += ld) acc[r] += ok ? *p : 0.0f;
        }
#pragma unroll
        for (int r = 0; r < kR; ++r) seg_sum[r][seg][c] = acc[r];
        __syncthreads();
        if (tid < 16 * kR) {
            const int r = tid >> 4, cc = tid & 15;
            const int64_t j = base + r * 16 + cc;
            if (j < nout) {
                float t = seg_sum[r][0][cc];
#pragma unroll
                for (int q = 1; q < 16; ++q) t += seg_sum[r][q][cc];
                const PT out = from_f32<PT>(t);
                if (j < N) dg[j] = out;
                else if (j < 2 * N) db[j - N] = out;
                else da[0] = out;
            }
        }
        __syncthreads();
    }
}
#endif

// ---------------------------------------------------------------- backward
// Pass 1: dx, plus one float32 partial row per workgroup.
// RAG (row segments with N not a multiple of V): elements e < lo of a
// shifted slot are another slot's; they stay out of dalpha here and out of
// the partial row at the end (dgamma/dbeta: not written).
template <typename XT, int V, int K, bool ACC, bool RAG>
__device__ __forceinline__ void bwd_slot(const float (&xv)[V], const float (&dv)[V],
                                         const float (&gm)[V], float alpha, int lo,
                                         float (&out)[V], float (&ag)[V], float (&ab)[V],
                                         float& aa) {
#pragma unroll
    for (int e = 0; e < V; ++e) {
        float th, sd;
        dyt_tanh_sech2<ACC>(xv[e], alpha, th, sd);
        const float gd = (dv[e] * gm[e]) * sd;     // dy * gamma * sech^2
        out[e] = gd * alpha;
        ag[e] = __builtin_fmaf(dv[e], th, ag[e]);
        ab[e] += dv[e];
        if constexpr (RAG) aa = __builtin_fmaf(e >= lo ? gd : 0.0f, xv[e], aa);
        else aa = __builtin_fmaf(gd, xv[e], aa);
    }
}

// With RES the residual gradient dres is loaded beside x and dy and added
// (in float32) to dx before the one rounding to the storage type. x (and
// dres) are addressed by ax, dy by ad, dx by ao; unit bases bx, bd, bo.
template <typename XT, int V, int K, int U, bool RES, typename AD>
__device__ __forceinline__ void bwd_load(const XT* __restrict__ x, const XT* __restrict__ dy,
                                         const XT* __restrict__ dres, int64_t bx, const AD& ax,
                                         int64_t bd, const AD& ad,
                                         typename Raw<XT, V>::T (&rx)[U][K],
                                         typename Raw<XT, V>::T (&rd)[U][K],
                                         typename Raw<XT, V>::T (&rr)[U][K]) {
#pragma unroll
    for (int j = 0; j < U; ++j)
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int64_t atx = bx + j * ax.upitch + ax.off[k];
            rx[j][k] = Raw<XT, V>::template load<DYT_BWD_NT>(x + atx);
            rd[j][k] = Raw<XT, V>::template load<DYT_BWD_NT>(dy + bd + j * ad.upitch + ad.off[k]);
            if constexpr (RES) rr[j][k] = Raw<XT, V>::template load<DYT_BWD_NT>(dres + atx);
        }
}

template <typename XT, int V, int K, int U, bool ACC, bool RES, bool RAG, typename AD>
__device__ __forceinline__ void bwd_tile(const typename Raw<XT, V>::T (&rx)[U][K],
                                         const typename Raw<XT, V>::T (&rd)[U][K],
                                         const typename Raw<XT, V>::T (&rr)[U][K],
                                         XT* __restrict__ dx, int64_t bo, const AD& ao,
                                         const float (&gm)[K][V], float alpha, const int (&lo)[K],
                                         float (&ag)[K][V], float (&ab)[K][V], float (&aa)[K],
                                         uint32_t span_bytes = 0) {
#pragma unroll
    for (int j = 0; j < U; ++j)
#pragma unroll
        for (int k = 0; k < K; ++k) {
            float xv[V], dv[V], out[V];
            Raw<XT, V>::unpack(rx[j][k], xv);
            Raw<XT, V>::unpack(rd[j][k], dv);
            bwd_slot<XT, V, K, ACC, RAG>(xv, dv, gm[k], alpha, lo[k], out, ag[k], ab[k], aa[k]);
            if constexpr (RES) {
                float rv[V];
                Raw<XT, V>::unpack(rr[j][k], rv);
#pragma unroll
                for (int e = 0; e < V; ++e) out[e] += rv[e];
            }
            if constexpr (DYT_BWD_STORE_POL != 0 && !RES && !RAG && V > 1) {
                if (span_bytes != 0) {
                    store_with_policy<DYT_BWD_STORE_POL>(dx + bo + j * ao.upitch, span_bytes,
                                                         (uint32_t)(ao.off[k] * (int)sizeof(XT)),
                                                         Raw<XT, V>::pack(out));
                    continue;
                }
            }
            Raw<XT, V>::template store<(RES ? DYT_BWD_RES_NT : DYT_BWD_NT) != 0>(
                dx + bo + j * ao.upitch + ao.off[k], out);
        }
}

// x is the layer input (h of the residual forward); dres and RES as above.
// STRIDED: x, dy, dx have row pitches g.pitch[0], g.pitch[1], g.pitch[2]
// (no RES). The tiling - and so every partial row - is the contiguous one.
// RAG: row segments whose length N is not a multiple of V (shifted slots).
template <typename XT, typename PT, int V, int K, int U, bool PACKED, bool RES, bool STRIDED,
          bool RAG>
__global__ void __launch_bounds__(kBlock)
dyt_bwd_partial_kernel(const XT* __restrict__ x, const XT* __restrict__ dy,
                       const XT* __restrict__ dres, const PT* __restrict__ alpha_p,
                       const PT* __restrict__ gamma, XT* __restrict__ dx,
                       float* __restrict__ ws, const Geo g) {
    static_assert(!(RES && STRIDED), "the residual layer takes contiguous tensors");
    static_assert(!(RAG && PACKED), "packed tiles hold whole vectors");
    using R = Raw<XT, V>;
    constexpr bool ACC = std::is_same<XT, float>::value;
    const int tid = threadIdx.x;
    const int64_t wg = blockIdx.x;
    const int64_t G = gridDim.x;
    const float alpha = to_f32(alpha_p[0]);
    // the deal (round-robin, or XCD-weighted with g.even_share_q) depends
    // on the shape only, so do the rows summed into each partial row
    const TileWalk w = make_walk<U>(g, PACKED, wg, G, g.even_share_q, g.xcd_flip, 0);
    const Slots<V, K> sl = make_slots<V, K, RAG>(tid, w.seg_len);
    const Addr<K, STRIDED> ax = make_addr<V, K, PACKED, STRIDED>(sl, w, g, g.pitch[0]);
    const Addr<K, STRIDED> ad = STRIDED ? make_addr<V, K, PACKED, STRIDED>(sl, w, g, g.pitch[1]) : ax;
    const Addr<K, STRIDED> ao = STRIDED ? make_addr<V, K, PACKED, STRIDED>(sl, w, g, g.pitch[2]) : ax;
    DYT_STAMP(g, 0);

    float gm[K][V], ag[K][V], ab[K][V];
    float aa[K];     // dalpha partial per slot: unused slots are dropped at the end
#pragma unroll
    for (int k = 0; k < K; ++k) {
        aa[k] = 0.0f;
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const int o = sl.off[k] + e;   // unused slots: tile offsets 0..V-1
            const int64_t c = PACKED ? (int64_t)(o % (int)g.N) : w.col_base + o;
            ag[k][e] = 0.0f;
            ab[k][e] = 0.0f;
            gm[k][e] = to_f32(gamma[c]);
        }
    }

    // Same two-buffer persistent loop over groups of U adjacent units as the
    // forward.
    const uint32_t span = (DYT_BWD_STORE_POL != 0 && g.buf_store) ? (uint32_t)w.seg_len * (uint32_t)sizeof(XT) : 0u;
    const int64_t ng = w.units / U;
    const int64_t iters = w.g_first < w.g_end ? (w.g_end - w.g_first + w.g_stride - 1) / w.g_stride : 0;
    const int64_t ustep = w.g_stride * U;
    const int64_t cb = w.col_base;
    const int64_t gsx = ustep * ax.upitch, gsd = ustep * ad.upitch, gso = ustep * ao.upitch;
    if (iters > 0) {
        typename R::T xa[U][K], da[U][K], ra[U][K], xb[U][K], db[U][K], rb[U][K];
        const int64_t u0 = w.g_first * U;
        // without row pitches all three operands share one offset
        int64_t bxa = cb + u0 * ax.upitch;
        int64_t bda = STRIDED ? cb + u0 * ad.upitch : bxa, boa = STRIDED ? cb + u0 * ao.upitch : bxa;
        bwd_load<XT, V, K, U, RES>(x, dy, dres, bxa, ax, bda, ad, xa, da, ra);
        const int64_t npairs = iters / 2;
        const int64_t nfull = (DYT_TAIL_PREFETCH || (iters & 1)) ? npairs : npairs - 1;
        for (int64_t pi = 0; pi < nfull; ++pi) {
            const int64_t bxb = bxa + gsx;
            const int64_t bdb = STRIDED ? bda + gsd : bxb, bob = STRIDED ? boa + gso : bxb;
            bwd_load<XT, V, K, U, RES>(x, dy, dres, bxb, ax, bdb, ad, xb, db, rb);
            __builtin_amdgcn_sched_barrier(0);
            bwd_tile<XT, V, K, U, ACC, RES, RAG>(xa, da, ra, dx, boa, ao, gm, alpha, sl.lo, ag, ab, aa, span);
            __builtin_amdgcn_sched_barrier(0);
            const bool more = 2 * pi + 2 < iters;
            const int64_t bxn = more ? bxb + gsx : bxb;
            const int64_t bdn = STRIDED ? (more ? bdb + gsd : bdb) : bxn;
            const int64_t bon = STRIDED ? (more ? bob + gso : bob) : bxn;
            bwd_load<XT, V, K, U, RES>(x, dy, dres, bxn, ax, bdn, ad, xa, da, ra);
            __builtin_amdgcn_sched_barrier(0);
            bwd_tile<XT, V, K, U, ACC, RES, RAG>(xb, db, rb, dx, bob, ao, gm, alpha, sl.lo, ag, ab, aa, span);
            __builtin_amdgcn_sched_barrier(0);
            bxa = bxn;
            bda = bdn;
            boa = bon;
        }
        if (!DYT_TAIL_PREFETCH && !(iters & 1)) {   // the last pair (iters >= 2)
            const int64_t bxb = bxa + gsx;
            const int64_t bdb = STRIDED ? bda + gsd : bxb, bob = STRIDED ? boa + gso : bxb;
            bwd_load<XT, V, K, U, RES>(x, dy, dres, bxb, ax, bdb, ad, xb, db, rb);
            __builtin_amdgcn_sched_barrier(0);
            bwd_tile<XT, V, K, U, ACC, RES, RAG>(xa, da, ra, dx, boa, ao, gm, alpha, sl.lo, ag, ab, aa, span);
            __builtin_amdgcn_sched_barrier(0);
            bwd_tile<XT, V, K, U, ACC, RES, RAG>(xb, db, rb, dx, bob, ao, gm, alpha, sl.lo, ag, ab, aa, span);
        }
        if (iters & 1) bwd_tile<XT, V, K, U, ACC, RES, RAG>(xa, da, ra, dx, boa, ao, gm, alpha, sl.lo, ag, ab, aa, span);
    }
    for (int64_t u = ng * U + w.gw; u < w.units; u += w.gcount) {
        typename R::T x1[1][K], d1[1][K], r1[1][K];
        bwd_load<XT, V, K, 1, RES>(x, dy, dres, cb + u * ax.upitch, ax, cb + u * ad.upitch, ad, x1, d1, r1);
        bwd_tile<XT, V, K, 1, ACC, RES, RAG>(x1, d1, r1, dx, cb + u * ao.upitch, ao, gm, alpha, sl.lo, ag,
                                             ab, aa, span);
    }

    if (PACKED && w.tail) {
        const int len = (int)(g.total - w.units * (int64_t)g.T);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int o = (k * kBlock + tid) * V;
            const int n = len - o;
            if (n > 0) {
                const int64_t ox = w.units * ax.upitch + tile_off<PACKED, STRIDED>(o, g, g.pitch[0]);
                const int64_t od = w.units * ad.upitch + tile_off<PACKED, STRIDED>(o, g, g.pitch[1]);
                const int64_t oo = w.units * ao.upitch + tile_off<PACKED, STRIDED>(o, g, g.pitch[2]);
                float xv[V], dv[V], rv[V], out[V];
                if (n >= V) {
                    R::unpack(R::load(x + ox), xv);
                    R::unpack(R::load(dy + od), dv);
                    if constexpr (RES) R::unpack(R::load(dres + ox), rv);
                } else {
                    load_partial<XT, V>(x + ox, n, xv);
                    load_partial<XT, V>(dy + od, n, dv);
                    if constexpr (RES) load_partial<XT, V>(dres + ox, n, rv);
                }
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    float th, sd;
                    dyt_tanh_sech2<ACC>(xv[e], alpha, th, sd);
                    const float gd = (dv[e] * gm[k][e]) * sd;
                    out[e] = gd * alpha;
                    if constexpr (RES) out[e] += rv[e];
                    // Mask after the arithmetic: a lane past the end computed on
                    // zeros (tanh(inf * 0) = NaN when alpha = inf); the select
                    // drops whatever it produced.
                    const bool ok = e < n;
                    const float cg = dv[e] * th;
                    const float ca = gd * xv[e];
                    ag[k][e] += ok ? cg : 0.0f;
                    ab[k][e] += ok ? dv[e] : 0.0f;
                    aa[k] += ok ? ca : 0.0f;
                }
                if (n >= V) R::store(dx + oo, out);
                else store_partial<XT, V>(dx + oo, n, out);
            }
        }
    }

    DYT_STAMP(g, 1);

    // ---- workgroup reduction into one partial row
    float* __restrict__ wrow = ws + wg * (int64_t)g.ld;
    __shared__ float red[kBlock / 64];
    float v = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) v += sl.used[k] ? aa[k] : 0.0f;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    if ((tid & 63) == 0) red[tid >> 6] = v;

    if constexpr (PACKED) {
        // Column sums over the tile's R rows, dgamma and dbeta together. The
        // tile goes to LDS as laid out in memory (element o = row o / N,
        // column o mod N). With N <= block size, thread (j, c) = (tid / N,
        // tid mod N) sums rows j, j + G2, j + 2 G2, ... of column c in that
        // order (G2 = block / N groups), then thread c adds the G2 group sums
        // in group order; wider packed rows sum all R rows per column in row
        // order. Loads are issued eight at a time ahead of the additions,
        // which keep their fixed order (bitwise the same as one at a time).
        constexpr int kTile = K * kBlock * V;
        __shared__ float4 shg4[kTile / 4], shb4[kTile / 4];
        __shared__ float s2g[kBlock], s2b[kBlock];
        float* const shg = reinterpret_cast<float*>(shg4);
        float* const shb = reinterpret_cast<float*>(shb4);
        const int N = (int)g.N;
        const int Rr = g.R;
        const int T = g.T;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int o = (k * kBlock + tid) * V;
            if constexpr (V % 4 == 0) {
                if (o + V <= T) {
#pragma unroll
                    for (int e = 0; e < V; e += 4) {
                        shg4[(o + e) / 4] = make_float4(ag[k][e], ag[k][e + 1], ag[k][e + 2], ag[k][e + 3]);
                        shb4[(o + e) / 4] = make_float4(ab[k][e], ab[k][e + 1], ab[k][e + 2], ab[k][e + 3]);
                    }
                    continue;
                }
            }
#pragma unroll
            for (int e = 0; e < V; ++e)
                if (o + e < T) {
                    shg[o + e] = ag[k][e];
                    shb[o + e] = ab[k][e];
                }
        }
        __syncthreads();
        // sa += a[(first + i * step) * stride] for i = 0 .. count-1 in that
        // order (sb likewise from b)
        auto ordered_sum = [](const float* __restrict__ a, const float* __restrict__ b, int first,
                              int step, int count, int stride, float& sa, float& sb) {
            for (int i0 = 0; i0 < count; i0 += 8) {
                float va[8], vb[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int idx = (i0 + i < count) ? (first + (i0 + i) * step) * stride : 0;
                    va[i] = a[idx];
                    vb[i] = b[idx];
                }
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    if (i0 + i < count) {
                        sa += va[i];
                        sb += vb[i];
                    }
            }
        };
        if (N <= kBlock) {
            const int G2 = kBlock / N;
            if (tid < G2 * N) {
                const int c = tid % N;
                const int j = tid / N;
                const int nrow = j < Rr ? (Rr - j + G2 - 1) / G2 : 0;
                float sg = 0.0f, sb = 0.0f;
                ordered_sum(shg + c, shb + c, j, G2, nrow, N, sg, sb);
                s2g[tid] = sg;
                s2b[tid] = sb;
            }
            __syncthreads();
            if (tid < N) {
                float sg = s2g[tid], sb = s2b[tid];
                ordered_sum(s2g + tid, s2b + tid, 1, 1, G2 - 1, N, sg, sb);
                wrow[tid] = sg;
                wrow[g.wcols + tid] = sb;
            }
        } else {
            for (int c = tid; c < N; c += kBlock) {
                float sg = 0.0f, sb = 0.0f;
                ordered_sum(shg + c, shb + c, 0, 1, Rr, N, sg, sb);
                wrow[c] = sg;
                wrow[g.wcols + c] = sb;
            }
        }
    } else {
        // Each thread owns V consecutive columns per slot: whole in-range
        // groups go out as 16-byte stores (the partial row, ld and the column
        // block width are all multiples of 4 floats, the workspace 16-byte
        // aligned); only the ragged end of the last column block is written
        // element by element. Element-wise stores here, lanes 4*V bytes
        // apart, cost about 2% of the pass at N = 4096.
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int o = (k * kBlock + tid) * V;
            if constexpr (V % 4 == 0) {
                if (o + V <= w.seg_len) {
#pragma unroll
                    for (int e = 0; e < V; e += 4) {
                        *reinterpret_cast<float4*>(wrow + o + e) =
                            make_float4(ag[k][e], ag[k][e + 1], ag[k][e + 2], ag[k][e + 3]);
                        *reinterpret_cast<float4*>(wrow + g.wcols + o + e) =
                            make_float4(ab[k][e], ab[k][e + 1], ab[k][e + 2], ab[k][e + 3]);
                    }
                    continue;
                }
            }
            if constexpr (RAG) {
                // the slot's registers hold columns off + e; a shifted slot
                // writes only its own ones (e >= lo)
                if (!sl.used[k]) continue;
#pragma unroll
                for (int e = 0; e < V; ++e)
                    if (e >= sl.lo[k]) {
                        wrow[sl.off[k] + e] = ag[k][e];
                        wrow[g.wcols + sl.off[k] + e] = ab[k][e];
                    }
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e)
                    if (o + e < w.seg_len) {
                        wrow[o + e] = ag[k][e];
                        wrow[g.wcols + o + e] = ab[k][e];
                    }
            }
        }
    }
    __syncthreads();
    if (tid == 0) {
        float s = red[0];
#pragma unroll
        for (int q = 1; q < kBlock / 64; ++q) s += red[q];
        wrow[2 * g.wcols] = s;
    }
#if DYT_FUSED_FIN
    if (g.fin_out[0] != nullptr) {
        // publish this workgroup's partial row at device scope, then count it
        __threadfence();
        __syncthreads();
        __shared__ unsigned ticket;
        if (tid == 0)
            ticket = __hip_atomic_fetch_add(g.ctr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (ticket == (unsigned)(G - 1)) {
            __threadfence();   // every workgroup's row is visible to every thread here
            finish_in_workgroup<PT>(ws, G, g.ld, g.N, g.wcols, (PT*)g.fin_out[0],
                                    (PT*)g.fin_out[1], (PT*)g.fin_out[2]);
            if (tid == 0) __hip_atomic_store(g.ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
#endif
    DYT_STAMP_EXIT(g);
}


// Pass 2: out[j] = fixed-order sum of the partial rows' column j, rounded to
// the parameter dtype. Outputs j < N are dgamma, N <= j < 2N dbeta, j = 2N
// dalpha. Lane = output, wave = one of 16 contiguous row segments.
template <typename PT>
__global__ void __launch_bounds__(kFinBlock)
dyt_bwd_finish_kernel(const float* __restrict__ ws, PT* __restrict__ dgamma,
                      PT* __restrict__ dbeta, PT* __restrict__ dalpha, const FinGeo f) {
    const int lane = threadIdx.x & 63;
    const int seg = threadIdx.x >> 6;
    const int64_t j = (int64_t)blockIdx.x * 64 + lane;
    const int64_t nout = 2 * f.N + 1;
    float acc = 0.0f;
    if (j < nout) {
        int64_t row0 = 0, step = 1, nrows = f.P, off;
        if (j < 2 * f.N) {
            const bool isb = j >= f.N;
            const int64_t c = isb ? j - f.N : j;
            if (f.packed) {
                off = (isb ? f.wcols : 0) + c;
            } else {
                const int64_t b = c / f.wc;
                row0 = b;
                step = f.nb;
                nrows = f.P / f.nb;
                off = (isb ? f.wc : 0) + (c - b * f.wc);
            }
        } else {
            off = 2 * (int64_t)f.wcols;
        }
        const int64_t i0 = seg * nrows / kFinSegs;
        const int64_t i1 = (seg + 1) * nrows / kFinSegs;
        const int64_t stride = step * f.ld;
        const float* __restrict__ p = ws + (row0 + i0 * step) * f.ld + off;
        // 16 loads in flight per step (one round trip for the usual 256
        // partial rows), summed in row order
        int64_t i = i0;
        for (; i + 16 <= i1; i += 16, p += 16 * stride) {
            float v[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) v[q] = p[q * stride];
#pragma unroll
            for (int q = 0; q < 16; ++q) acc += v[q];
        }
        for (; i < i1; ++i, p += stride) acc += *p;
    }
    __shared__ float red[kFinSegs][64];
    red[seg][lane] = acc;
    __syncthreads();
    if (seg == 0 && j < nout) {
        float s = red[0][lane];
#pragma unroll
        for (int q = 1; q < kFinSegs; ++q) s += red[q][lane];
        const PT out = from_f32<PT>(s);
        if (j < f.N) dgamma[j] = out;
        else if (j < 2 * f.N) dbeta[j - f.N] = out;
        else dalpha[0] = out;
    }
}

}  // namespace dyt
