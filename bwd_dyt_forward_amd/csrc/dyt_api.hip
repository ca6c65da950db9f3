// dyt_api.hip - C ABI of the fused DyT layer (declared in include/dyt.h):
// argument validation, launch planning and kernel dispatch on gfx950.
//
// The plan is a pure function of (M, N, dtypes, 16-byte alignment class), so
// the order of every floating-point sum, and with it every result bit, is
// reproducible run to run and device to device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "dyt.h"
#include "dyt_kernels.hpp"

// Persistent-grid sizes (workgroups): one 256-thread workgroup per compute
// unit of MI355X (256 CUs) for every kernel. Measured on the 32768 x 4096
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
#ifndef DYT_BWD_GRID_WIDE
#define DYT_BWD_GRID_WIDE 256
#endif
// Tiles per pipeline buffer (loads in flight per wave = U * K per input):
// the forward has one input stream and needs two tiles in flight, the
// backward's two input streams already keep enough bytes in flight.
#ifndef DYT_FWD_U
#define DYT_FWD_U 2
#endif
#ifndef DYT_BWD_U
#define DYT_BWD_U 1
#endif
// Tiles wanted before a packed plan stops shrinking K for more parallelism.
#ifndef DYT_MIN_TILES
#define DYT_MIN_TILES 1024
#endif

namespace {

using dyt::Geo;
using dyt::FinGeo;
using dyt::bf16_t;
using dyt::kBlock;

struct Plan {
    bool packed = true;
    int vec = 1;
    int slots = 1;
    int64_t R = 1;
    int64_t T = 0;
    int64_t nb = 1;
    int64_t last_len = 0;
    int64_t tiles = 0;
    int64_t fwd_grid = 0;
    int64_t bwd_grid = 0;
    int64_t ld = 0;
    int64_t wcols = 0;
    int64_t fin_grid = 1;
    int64_t ws_bytes = 0;
};

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

// Pure host: validates sizes/dtypes and fills the plan. The plan depends
// only on (M, N, x dtype): tensors whose bases are not 16-byte aligned run
// the same tiles with the element-wise kernel variant (V = 1, K = 16, whose
// 4096-element capacity holds any tile), so the partial-row layout - and
// with it dyt_backward_finish - does not depend on pointer alignment.
int make_plan(int64_t M, int64_t N, int xdt, int pdt, Plan& p) {
    if (!dtype_ok(xdt) || !dtype_ok(pdt)) return DYT_ERR_UNSUPPORTED_DTYPE;
    if (M < 0 || N < 0 || N > kMaxN) return DYT_ERR_INVALID_ARG;
    const int64_t sx = dtype_size(xdt);
    if (N > 0 && M > INT64_MAX / N / 16) return DYT_ERR_INVALID_ARG;
    p = Plan();
    const int vmax = (int)(16 / sx);           // elements per 16 bytes
    const int kmax = dyt::kTileCap / (kBlock * vmax);
    if (M == 0 || N == 0) {
        p.fin_grid = ceil_div(2 * N + 1, 64);
        return DYT_OK;
    }
    // packed tiles: R >= 2 whole rows, R a multiple of r0 (the rows that keep
    // each tile 16-byte aligned), within kTileCap elements
    const int64_t r0 = 16 / gcd64(N * sx, 16);
    const int64_t rcap = (dyt::kTileCap / N) / r0 * r0;
    if (rcap >= 2) {
        p.packed = true;
        p.vec = vmax;
        // largest K (biggest tiles) that still yields DYT_MIN_TILES tiles,
        // else the smallest K that holds an aligned row group
        int chosen = 0;
        for (int k = kmax; k >= 1; k /= 2) {
            const int64_t r = ((int64_t)kBlock * vmax * k / N) / r0 * r0;
            if (r < 1) break;
            chosen = k;
            if (ceil_div(M, r) >= DYT_MIN_TILES) break;
        }
        const int64_t r = ((int64_t)kBlock * vmax * chosen / N) / r0 * r0;
        p.slots = chosen;
        p.R = r;
        p.T = r * N;
        p.nb = 1;
        p.last_len = p.T;
        p.tiles = ceil_div(M, r);
        p.wcols = N;
        p.fwd_grid = std::min<int64_t>(p.tiles, DYT_FWD_GRID);
        p.bwd_grid = std::min<int64_t>(p.tiles, DYT_BWD_GRID);
    } else {
        p.packed = false;
        const bool v = (N * sx) % 16 == 0;     // rows start 16-byte aligned
        p.vec = v ? vmax : 1;
        const int kbig = v ? kmax : 16;
        int k = v ? 1 : 16;
        while (k < kbig && (int64_t)kBlock * p.vec * k < N) k *= 2;
        p.slots = k;
        const int64_t cap = (int64_t)kBlock * p.vec * k;
        p.nb = ceil_div(N, cap);
        p.T = round_up(ceil_div(N, p.nb), p.vec);
        while (p.nb > 1 && (p.nb - 1) * p.T >= N) --p.nb;   // no empty last block
        p.last_len = N - (p.nb - 1) * p.T;
        p.R = 1;
        p.tiles = M * p.nb;
        p.wcols = p.T;
        p.fwd_grid = p.nb * std::min<int64_t>(M, std::max<int64_t>(1, DYT_FWD_GRID / p.nb));
        p.bwd_grid = p.nb * std::min<int64_t>(M, std::max<int64_t>(1, DYT_BWD_GRID_WIDE / p.nb));
    }
    p.ld = round_up(2 * p.wcols + 1, 4);
    p.fin_grid = ceil_div(2 * N + 1, 64);
    p.ws_bytes = p.bwd_grid * p.ld * (int64_t)sizeof(float);
    return DYT_OK;
}

// Kernel variant for the actual pointers: the plan's vector width when every
// activation pointer is 16-byte aligned, else element-wise access.
Plan variant_for(const Plan& p, bool vec_aligned) {
    Plan q = p;
    if (!vec_aligned && q.vec != 1) {
        q.vec = 1;
        q.slots = 16;
    }
    return q;
}

Geo make_geo(const Plan& p, int64_t M, int64_t N) {
    Geo g;
    g.total = M * N;
    g.ntiles = p.tiles;
    g.N = N;
    g.T = (int32_t)p.T;
    g.R = (int32_t)p.R;
    g.nb = (int32_t)p.nb;
    g.last_len = (int32_t)p.last_len;
    g.ld = (int32_t)p.ld;
    g.wcols = (int32_t)p.wcols;
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
template <typename XT, typename PT, int V, int K>
void launch_fwd_vk(const Plan& p, const Geo& g, const void* x, const void* a, const void* gm,
                   const void* bt, void* y, hipStream_t s) {
    const dim3 grid((unsigned)p.fwd_grid), block(kBlock);
    if (p.packed)
        hipLaunchKernelGGL((dyt::dyt_fwd_kernel<XT, PT, V, K, DYT_FWD_U, true>), grid, block, 0, s,
                           (const XT*)x, (const PT*)a, (const PT*)gm, (const PT*)bt, (XT*)y, g);
    else
        hipLaunchKernelGGL((dyt::dyt_fwd_kernel<XT, PT, V, K, DYT_FWD_U, false>), grid, block, 0, s,
                           (const XT*)x, (const PT*)a, (const PT*)gm, (const PT*)bt, (XT*)y, g);
}

template <typename XT, typename PT, int V, int K>
void launch_bwd_vk(const Plan& p, const Geo& g, const void* x, const void* dy, const void* a,
                   const void* gm, void* dx, float* ws, hipStream_t s) {
    const dim3 grid((unsigned)p.bwd_grid), block(kBlock);
    if (p.packed)
        hipLaunchKernelGGL((dyt::dyt_bwd_partial_kernel<XT, PT, V, K, DYT_BWD_U, true>), grid, block, 0, s,
                           (const XT*)x, (const XT*)dy, (const PT*)a, (const PT*)gm, (XT*)dx, ws, g);
    else
        hipLaunchKernelGGL((dyt::dyt_bwd_partial_kernel<XT, PT, V, K, DYT_BWD_U, false>), grid, block, 0, s,
                           (const XT*)x, (const XT*)dy, (const PT*)a, (const PT*)gm, (XT*)dx, ws, g);
}

// Kernel instances: vector access at K in {1, 2, ..., 4096 / (256 V)}, and
// the element-wise variant (V = 1) at K = 16.
template <typename XT, typename PT>
bool launch_fwd(const Plan& p, const Geo& g, const void* x, const void* a, const void* gm,
                const void* bt, void* y, hipStream_t s) {
    constexpr int VV = 16 / sizeof(XT);
    if (p.vec == 1 && p.slots == 16) { launch_fwd_vk<XT, PT, 1, 16>(p, g, x, a, gm, bt, y, s); return true; }
    if (p.vec != VV) return false;
    switch (p.slots) {
        case 1: launch_fwd_vk<XT, PT, VV, 1>(p, g, x, a, gm, bt, y, s); return true;
        case 2: launch_fwd_vk<XT, PT, VV, 2>(p, g, x, a, gm, bt, y, s); return true;
        case 4:
            if constexpr (VV == 4) { launch_fwd_vk<XT, PT, VV, 4>(p, g, x, a, gm, bt, y, s); return true; }
            return false;
        default: return false;
    }
}

template <typename XT, typename PT>
bool launch_bwd(const Plan& p, const Geo& g, const void* x, const void* dy, const void* a,
                const void* gm, void* dx, float* ws, hipStream_t s) {
    constexpr int VV = 16 / sizeof(XT);
    if (p.vec == 1 && p.slots == 16) { launch_bwd_vk<XT, PT, 1, 16>(p, g, x, dy, a, gm, dx, ws, s); return true; }
    if (p.vec != VV) return false;
    switch (p.slots) {
        case 1: launch_bwd_vk<XT, PT, VV, 1>(p, g, x, dy, a, gm, dx, ws, s); return true;
        case 2: launch_bwd_vk<XT, PT, VV, 2>(p, g, x, dy, a, gm, dx, ws, s); return true;
        case 4:
            if constexpr (VV == 4) { launch_bwd_vk<XT, PT, VV, 4>(p, g, x, dy, a, gm, dx, ws, s); return true; }
            return false;
        default: return false;
    }
}

template <typename PT>
void launch_finish(const Plan& p, int64_t N, const float* ws, void* dg, void* db, void* da,
                   hipStream_t s) {
    FinGeo f;
    f.P = p.bwd_grid;
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
int validate_backward(const void* x, const void* dy, const void* alpha, const void* gamma,
                      void* dx, void* dalpha, void* dgamma, void* dbeta, const void* workspace,
                      size_t workspace_bytes, int64_t M, int64_t N, int x_dtype, int param_dtype,
                      bool use_pass1, bool use_pass2, Plan& base) {
    int st = make_plan(M, N, x_dtype, param_dtype, base);
    if (st != DYT_OK) return st;
    const int64_t sx = dtype_size(x_dtype), sp = dtype_size(param_dtype);
    const bool any = M > 0 && N > 0;
    const bool p1 = use_pass1 && any;
    if (use_pass2) {
        if (!dalpha) return DYT_ERR_INVALID_ARG;
        if (N > 0 && (!dgamma || !dbeta)) return DYT_ERR_INVALID_ARG;
    }
    if (p1 && (!x || !dy || !alpha || !gamma || !dx)) return DYT_ERR_INVALID_ARG;
    const size_t need = (size_t)round_up(base.ws_bytes, 16);
    if (workspace_bytes < need) return DYT_ERR_WORKSPACE_TOO_SMALL;
    if (need > 0 && !workspace) return DYT_ERR_INVALID_ARG;
    if (need > 0 && !aligned(workspace, 16)) return DYT_ERR_MISALIGNED;
    if (use_pass2 && (!aligned(dalpha, sp) || (N > 0 && (!aligned(dgamma, sp) || !aligned(dbeta, sp)))))
        return DYT_ERR_MISALIGNED;
    if (p1 && (!aligned(x, sx) || !aligned(dy, sx) || !aligned(dx, sx) || !aligned(alpha, sp) ||
               !aligned(gamma, sp)))
        return DYT_ERR_MISALIGNED;
    // outputs (and the workspace) must not overlap inputs or each other
    const int64_t mn = p1 ? M * N * sx : 0;
    const Range outs[5] = {range(dx, mn), range(dalpha, use_pass2 ? sp : 0),
                           range(dgamma, use_pass2 ? N * sp : 0), range(dbeta, use_pass2 ? N * sp : 0),
                           range(workspace, (int64_t)need)};
    const Range ins[4] = {range(x, mn), range(dy, mn), range(alpha, p1 ? sp : 0),
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

int enqueue_pass1(const Plan& base, const void* x, const void* dy, const void* alpha,
                  const void* gamma, void* dx, void* workspace, int64_t M, int64_t N,
                  int x_dtype, int param_dtype, hipStream_t s) {
    if (M == 0 || N == 0) return DYT_OK;
    const Plan p = variant_for(base, aligned(x, 16) && aligned(dy, 16) && aligned(dx, 16));
    const Geo g = make_geo(p, M, N);
    float* ws = static_cast<float*>(workspace);
    const bool ok = with_dtype(x_dtype, [&](auto xt) {
        return with_dtype(param_dtype, [&](auto pt) {
            return launch_bwd<decltype(xt), decltype(pt)>(p, g, x, dy, alpha, gamma, dx, ws, s);
        });
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

}  // namespace

extern "C" {

int dyt_abi_version(void) { return DYT_ABI_VERSION; }

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

int dyt_get_plan(int64_t M, int64_t N, int x_dtype, int param_dtype, int vector_aligned,
                 dyt_plan* out) {
    if (!out) return DYT_ERR_INVALID_ARG;
    Plan base;
    const int st = make_plan(M, N, x_dtype, param_dtype, base);
    if (st != DYT_OK) return st;
    const Plan p = variant_for(base, vector_aligned != 0);
    out->packed = p.packed ? 1 : 0;
    out->vec = p.vec;
    out->slots = p.slots;
    out->block = kBlock;
    out->rows_per_tile = p.R;
    out->tile_elems = p.T;
    out->col_blocks = p.nb;
    out->tiles = p.tiles;
    out->fwd_grid = p.fwd_grid;
    out->bwd_grid = p.bwd_grid;
    out->ws_row = p.ld;
    out->fin_grid = p.fin_grid;
    out->ws_bytes = p.ws_bytes;
    return DYT_OK;
}

size_t dyt_backward_workspace_size(int64_t M, int64_t N, int x_dtype, int param_dtype) {
    Plan p;
    if (make_plan(M, N, x_dtype, param_dtype, p) != DYT_OK) return 0;
    return (size_t)round_up(p.ws_bytes, 16);
}

int dyt_forward(const void* x, const void* alpha, const void* gamma, const void* beta, void* y,
                int64_t M, int64_t N, int x_dtype, int param_dtype, void* stream) {
    Plan base;
    int st = make_plan(M, N, x_dtype, param_dtype, base);
    if (st != DYT_OK) return st;
    if (M == 0 || N == 0) return DYT_OK;
    if (!x || !alpha || !gamma || !beta || !y) return DYT_ERR_INVALID_ARG;
    const int64_t sx = dtype_size(x_dtype), sp = dtype_size(param_dtype);
    if (!aligned(x, sx) || !aligned(y, sx) || !aligned(alpha, sp) || !aligned(gamma, sp) ||
        !aligned(beta, sp))
        return DYT_ERR_MISALIGNED;
    const Range ry = range(y, M * N * sx);
    if (overlap(ry, range(x, M * N * sx)) || overlap(ry, range(alpha, sp)) ||
        overlap(ry, range(gamma, N * sp)) || overlap(ry, range(beta, N * sp)))
        return DYT_ERR_INVALID_ARG;
    const Plan p = variant_for(base, aligned(x, 16) && aligned(y, 16));
    const Geo g = make_geo(p, M, N);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool ok = with_dtype(x_dtype, [&](auto xt) {
        return with_dtype(param_dtype, [&](auto pt) {
            return launch_fwd<decltype(xt), decltype(pt)>(p, g, x, alpha, gamma, beta, y, s);
        });
    });
    if (!ok) return DYT_ERR_INVALID_ARG;   // no kernel instance for this plan (not reachable)
    return hip_status();
}


int dyt_backward_partials(const void* x, const void* dy, const void* alpha, const void* gamma,
                          void* dx, void* workspace, size_t workspace_bytes, int64_t M, int64_t N,
                          int x_dtype, int param_dtype, void* stream) {
    Plan base;
    int st = validate_backward(x, dy, alpha, gamma, dx, nullptr, nullptr, nullptr, workspace,
                               workspace_bytes, M, N, x_dtype, param_dtype, true, false, base);
    if (st != DYT_OK) return st;
    return enqueue_pass1(base, x, dy, alpha, gamma, dx, workspace, M, N, x_dtype, param_dtype,
                         static_cast<hipStream_t>(stream));
}

int dyt_backward_finish(const void* workspace, size_t workspace_bytes, void* dalpha,
                        void* dgamma, void* dbeta, int64_t M, int64_t N, int x_dtype,
                        int param_dtype, void* stream) {
    Plan base;
    int st = validate_backward(nullptr, nullptr, nullptr, nullptr, nullptr, dalpha, dgamma, dbeta,
                               workspace, workspace_bytes, M, N, x_dtype, param_dtype, false, true,
                               base);
    if (st != DYT_OK) return st;
    return enqueue_pass2(base, workspace, dalpha, dgamma, dbeta, N, param_dtype,
                         static_cast<hipStream_t>(stream));
}

int dyt_backward(const void* x, const void* dy, const void* alpha, const void* gamma, void* dx,
                 void* dalpha, void* dgamma, void* dbeta, void* workspace,
                 size_t workspace_bytes, int64_t M, int64_t N, int x_dtype, int param_dtype,
                 void* stream) {
    Plan base;
    int st = validate_backward(x, dy, alpha, gamma, dx, dalpha, dgamma, dbeta, workspace,
                               workspace_bytes, M, N, x_dtype, param_dtype, true, true, base);
    if (st != DYT_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = enqueue_pass1(base, x, dy, alpha, gamma, dx, workspace, M, N, x_dtype, param_dtype, s);
    if (st != DYT_OK) return st;
    return enqueue_pass2(base, workspace, dalpha, dgamma, dbeta, N, param_dtype, s);
}

}  // extern "C"
