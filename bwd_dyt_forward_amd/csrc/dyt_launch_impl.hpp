// dyt_launch_impl.hpp - kernel instance selection, included by the
// per-dtype translation units dyt_launch_{fwd,bwd}_<dtype>.hip only.
#pragma once

#include <type_traits>

#include "dyt_launch.hpp"

// Tiles per pipeline buffer (loads in flight per wave = U * K per input):
// the forward has one input stream and needs two tiles in flight, the
// backward's two input streams already keep enough bytes in flight.
#ifndef DYT_FWD_U
#define DYT_FWD_U 2
#endif
#ifndef DYT_BWD_U
#define DYT_BWD_U 1
#endif
// The residual forward (two inputs, two outputs) uses the forward's U as
// well: on 32768 x 4096 and 4194304 x 32 bf16 U = 2 measured 0.2-0.8%
// faster than U = 1.
// The plain forward of 2-byte x with 16-byte vectors takes DYT_FWD_U_2B
// tiles per buffer: four measured 2.0% faster than two on 32,768 x 4,096
// bf16 (81.2 -> 79.6 us), while four lost 0.9-4.5% on the float32
// 100,003-row forwards and 4% on the residual forward (bench.py --variants
// fwd_four_units), and the element-wise kernels (V = 1, K = 32) spill
// registers with four.
#ifndef DYT_FWD_U_2B
#define DYT_FWD_U_2B 4
#endif

namespace dyt {
namespace host {

template <typename XT, int V, bool RES>
constexpr int fwd_units() {
    return (!RES && sizeof(XT) == 2 && V > 1) ? DYT_FWD_U_2B : DYT_FWD_U;
}

// The element-wise variant (V = 1) exists only for row-strided packed tiles.
template <typename XT, typename PT, int V, int K, bool RES, bool STRIDED>
bool launch_fwd_vk(const Plan& p, const Geo& g, const FwdPtrs& a, hipStream_t s) {
    constexpr int U = fwd_units<XT, V, RES>();
    const dim3 grid((unsigned)p.grid), block(kBlock);
    if constexpr (V == 1) {
        if constexpr (!STRIDED || RES) return false;
        if (!p.packed) return false;
    }
    if (p.packed) {
        hipLaunchKernelGGL((dyt::dyt_fwd_kernel<XT, PT, V, K, U, true, RES, STRIDED, false>), grid,
                           block, 0, s, (const XT*)a.x, (const XT*)a.r, (const PT*)a.alpha,
                           (const PT*)a.gamma, (const PT*)a.beta, (XT*)a.y, (XT*)a.h, g);
    } else if constexpr (V > 1) {
        if (g.N % V != 0)
            hipLaunchKernelGGL((dyt::dyt_fwd_kernel<XT, PT, V, K, U, false, RES, STRIDED, true>), grid,
                               block, 0, s, (const XT*)a.x, (const XT*)a.r, (const PT*)a.alpha,
                               (const PT*)a.gamma, (const PT*)a.beta, (XT*)a.y, (XT*)a.h, g);
        else
            hipLaunchKernelGGL((dyt::dyt_fwd_kernel<XT, PT, V, K, U, false, RES, STRIDED, false>), grid,
                               block, 0, s, (const XT*)a.x, (const XT*)a.r, (const PT*)a.alpha,
                               (const PT*)a.gamma, (const PT*)a.beta, (XT*)a.y, (XT*)a.h, g);
    }
    return true;
}

template <typename XT, typename PT, int V, int K, bool RES, bool STRIDED, bool PACKED, bool RAG>
void launch_bwd_kernel(const Plan& p, const Geo& g, const BwdPtrs& a, hipStream_t s) {
    hipLaunchKernelGGL((dyt::dyt_bwd_partial_kernel<XT, PT, V, K, DYT_BWD_U, PACKED, RES, STRIDED, RAG>),
                       dim3((unsigned)p.grid), dim3(kBlock), 0, s, (const XT*)a.x, (const XT*)a.dy,
                       (const XT*)a.dres, (const PT*)a.alpha, (const PT*)a.gamma, (XT*)a.dx, a.ws, g);
}

template <typename XT, typename PT, int V, int K, bool RES, bool STRIDED>
bool launch_bwd_vk(const Plan& p, const Geo& g, const BwdPtrs& a, hipStream_t s) {
    if constexpr (V == 1) {
        if constexpr (!STRIDED || RES) return false;
        if (!p.packed) return false;
    }
    if (p.packed) {
        launch_bwd_kernel<XT, PT, V, K, RES, STRIDED, true, false>(p, g, a, s);
    } else if constexpr (V > 1) {
        if (g.N % V != 0) launch_bwd_kernel<XT, PT, V, K, RES, STRIDED, false, true>(p, g, a, s);
        else launch_bwd_kernel<XT, PT, V, K, RES, STRIDED, false, false>(p, g, a, s);
    }
    return true;
}

// Kernel instances: vector access at K = 1 .. 4, and the element-wise
// variant (V = 1) at K = 16 or 32 (packed, row-strided only). dispatch_vk
// calls launch(V, K), both as integral constants, for the instance the plan
// selects.
template <typename XT, typename L>
bool dispatch_vk(const Plan& p, L&& launch) {
    constexpr int VV = 16 / sizeof(XT);
    using I = std::integral_constant<int, VV>;
    if (p.vec == 1) {
        if (p.slots == 16) return launch(std::integral_constant<int, 1>{}, std::integral_constant<int, 16>{});
        if (p.slots == 32) return launch(std::integral_constant<int, 1>{}, std::integral_constant<int, 32>{});
        return false;
    }
    if (p.vec != VV) return false;
    switch (p.slots) {
        case 1: return launch(I{}, std::integral_constant<int, 1>{});
        case 2: return launch(I{}, std::integral_constant<int, 2>{});
        case 3: return launch(I{}, std::integral_constant<int, 3>{});
        case 4: return launch(I{}, std::integral_constant<int, 4>{});
        default: return false;
    }
}

template <typename XT, typename PT, bool RES, bool STRIDED>
bool launch_fwd(const Plan& p, const Geo& g, const FwdPtrs& a, hipStream_t s) {
    return dispatch_vk<XT>(p, [&](auto v, auto k) {
        return launch_fwd_vk<XT, PT, decltype(v)::value, decltype(k)::value, RES, STRIDED>(p, g, a, s);
    });
}

template <typename XT, typename PT, bool RES, bool STRIDED>
bool launch_bwd(const Plan& p, const Geo& g, const BwdPtrs& a, hipStream_t s) {
    return dispatch_vk<XT>(p, [&](auto v, auto k) {
        return launch_bwd_vk<XT, PT, decltype(v)::value, decltype(k)::value, RES, STRIDED>(p, g, a, s);
    });
}

template <typename XT, typename PT>
bool forward_pt(bool res, bool strided, const Plan& p, const Geo& g, const FwdPtrs& a,
                hipStream_t s) {
    if (res) return launch_fwd<XT, PT, true, false>(p, g, a, s);
    return strided ? launch_fwd<XT, PT, false, true>(p, g, a, s)
                   : launch_fwd<XT, PT, false, false>(p, g, a, s);
}

template <typename XT, typename PT>
bool backward_pt(bool res, bool strided, const Plan& p, const Geo& g, const BwdPtrs& a,
                 hipStream_t s) {
    if (res) return launch_bwd<XT, PT, true, false>(p, g, a, s);
    return strided ? launch_bwd<XT, PT, false, true>(p, g, a, s)
                   : launch_bwd<XT, PT, false, false>(p, g, a, s);
}

template <typename XT>
bool launch_forward(int pdt, bool res, bool strided, const Plan& p, const Geo& g,
                    const FwdPtrs& a, hipStream_t s) {
    switch (pdt) {
        case DYT_F32: return forward_pt<XT, float>(res, strided, p, g, a, s);
        case DYT_BF16: return forward_pt<XT, bf16_t>(res, strided, p, g, a, s);
        case DYT_F16: return forward_pt<XT, f16_t>(res, strided, p, g, a, s);
        default: return false;
    }
}

template <typename XT, typename PT, bool RES>
bool launch_flat_pt(const Plan& p, const FlatGeo& f, const FwdPtrs& a, hipStream_t s) {
    constexpr int V = 16 / sizeof(XT);
    const bool rag = f.N % V != 0 || f.head > 0;
    // gamma and beta as float32; rows that are not whole vectors carry V more of each
    const size_t lds = 2 * (size_t)(rag ? 4 * dyt::flat_rag_len(f.N, V) : f.N) * sizeof(float);
    if (rag) {
        hipLaunchKernelGGL((dyt::dyt_fwd_flat_kernel<XT, PT, DYT_FLAT_U, RES, true>),
                           dim3((unsigned)p.flat_grid), dim3(kBlock), lds, s, (const XT*)a.x,
                           (const XT*)a.r, (const PT*)a.alpha, (const PT*)a.gamma,
                           (const PT*)a.beta, (XT*)a.y, (XT*)a.h, f);
    } else {
        hipLaunchKernelGGL((dyt::dyt_fwd_flat_kernel<XT, PT, DYT_FLAT_U, RES, false>),
                           dim3((unsigned)p.flat_grid), dim3(kBlock), lds, s, (const XT*)a.x,
                           (const XT*)a.r, (const PT*)a.alpha, (const PT*)a.gamma,
                           (const PT*)a.beta, (XT*)a.y, (XT*)a.h, f);
    }
    return true;
}

template <typename XT, typename PT>
bool launch_flat_res(bool res, const Plan& p, const FlatGeo& f, const FwdPtrs& a, hipStream_t s) {
    return res ? launch_flat_pt<XT, PT, true>(p, f, a, s) : launch_flat_pt<XT, PT, false>(p, f, a, s);
}

template <typename XT>
bool launch_forward_flat(int pdt, bool res, const Plan& p, const FlatGeo& f, const FwdPtrs& a,
                         hipStream_t s) {
    if (!p.flat || p.flat_grid < 1) return false;
    switch (pdt) {
        case DYT_F32: return launch_flat_res<XT, float>(res, p, f, a, s);
        case DYT_BF16: return launch_flat_res<XT, bf16_t>(res, p, f, a, s);
        case DYT_F16: return launch_flat_res<XT, f16_t>(res, p, f, a, s);
        default: return false;
    }
}

template <typename XT>
bool launch_backward(int pdt, bool res, bool strided, const Plan& p, const Geo& g,
                     const BwdPtrs& a, hipStream_t s) {
    switch (pdt) {
        case DYT_F32: return backward_pt<XT, float>(res, strided, p, g, a, s);
        case DYT_BF16: return backward_pt<XT, bf16_t>(res, strided, p, g, a, s);
        case DYT_F16: return backward_pt<XT, f16_t>(res, strided, p, g, a, s);
        default: return false;
    }
}

}  // namespace host
}  // namespace dyt
