// dyt_launch.hpp - internal interface between the host logic of the C ABI
// (dyt_api.hip: validation and planning) and the kernel instances, which
// are compiled per x dtype and direction in dyt_launch_{fwd,bwd}_<dtype>.hip
// (so the library's translation units build in parallel).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "dyt.h"
#include "dyt_kernels.hpp"

// Vectors per thread and step of the flat forward (U * kBlock vectors per
// workgroup step); the host plan and the kernel instances share it.
#ifndef DYT_FLAT_U
#define DYT_FLAT_U 4
#endif

namespace dyt {
namespace host {

// Launch geometry of one direction: tiles (packed rows or row segments),
// vector width and slots, grid, and the backward's workspace layout.
struct Plan {
    bool packed = true;
    int vec = 1;
    int slots = 1;
    int64_t R = 1;
    int64_t T = 0;
    int64_t nb = 1;
    int64_t last_len = 0;
    int64_t tiles = 0;
    int64_t grid = 0;      // workgroups of this direction's kernel (pass 1 for the backward)
    int64_t ld = 0;
    int64_t wcols = 0;
    int64_t fin_grid = 1;
    int64_t ws_bytes = 0;
    // Forward only: the contiguous launch walks the problem as one run of
    // vectors (dyt_fwd_flat_kernel) on flat_grid workgroups; row-strided
    // launches keep the tiles above.
    bool flat = false;
    int64_t flat_grid = 0;
    // The flat walk only where x and y start 16-byte aligned or can start it
    // at an aligned element (2-byte packed tiles of one full slot, which stay
    // ahead of an unaligned walk).
    bool flat_aligned_only = false;
    // The four shifted gamma/beta copies fit in LDS: the flat walk can start
    // at the first 16-byte-aligned element when the tensors do not.
    bool flat_shift = false;
#if DYT_FUSED_FIN
    // Backward: pass 1's last workgroup does the finish (no pass-2 launch);
    // the arrival counter sits at byte ctr_off of the workspace.
    bool fused = false;
    int64_t ctr_off = 0;
#endif
};

// Device pointers of one launch; r/h (forward) and dres (backward) are null
// unless the residual add is fused.
// Row pitches (elements; 0 = N, contiguous) of x and y (forward) or x, dy
// and dx (backward) for the strided entry points.
struct FwdPtrs {
    const void* x;
    const void* r;
    const void* alpha;
    const void* gamma;
    const void* beta;
    void* y;
    void* h;
    int64_t ldx, ldy;
};
struct BwdPtrs {
    const void* x;
    const void* dy;
    const void* dres;
    const void* alpha;
    const void* gamma;
    void* dx;
    float* ws;
    int64_t ldx, lddy, lddx;
};

// Enqueue the forward (or backward pass 1) kernel instance the plan selects,
// for x storage type XT and parameter dtype code pdt; res: residual add
// fused; strided: row pitches in g. False if no instance exists (not
// reachable from the entry points).
template <typename XT>
bool launch_forward(int pdt, bool res, bool strided, const Plan& p, const Geo& g,
                    const FwdPtrs& a, hipStream_t s);
template <typename XT>
bool launch_backward(int pdt, bool res, bool strided, const Plan& p, const Geo& g,
                     const BwdPtrs& a, hipStream_t s);
// The flat forward (contiguous; res: the residual add fused) for a plan with
// p.flat set.
template <typename XT>
bool launch_forward_flat(int pdt, bool res, const Plan& p, const FlatGeo& f, const FwdPtrs& a,
                         hipStream_t s);

}  // namespace host
}  // namespace dyt
