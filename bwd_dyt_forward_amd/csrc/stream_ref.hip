// stream_ref.hip - reference streaming kernels for measurement only (loaded
// by bench.py, not part of the DyT C ABI): the plain memory streams the DyT
// kernels are compared against on the same GPU.
//
//   stream_ref_copy      out = a               (1 read + 1 write stream,
//                                               the forward's traffic)
//   stream_ref_2in1out   out = a xor b         (2 read + 1 write streams,
//                                               backward pass 1's traffic)
//   stream_ref_2in2out   out = a xor b,        (2 read + 2 write streams, the
//                        out2 = a + b           residual-fused forward's)
//   stream_ref_3in1out   out = a xor b xor c   (3 read + 1 write streams, the
//                                               residual-fused pass 1's)
//
// 16-byte nontemporal loads, each workgroup streaming contiguous chunks of
// U x (block x 16 B) in a grid-stride loop. The launch shapes and store
// kinds of the first two are the fastest of steady-state sweeps on MI355X
// (copy: 256 workgroups of 256 threads, U = 4, ordinary write-back stores,
// which ran a 256 MiB copy in 76.5 us against 85.0 us with nontemporal
// ones; 2-in-1-out: 256 workgroups of 512 threads, U = 2, nontemporal
// stores); the last two take the 2-in-1-out shape and the store kind the
// caller names.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

template <int NIN, int NOUT, int U, int BS, bool NTST>
__global__ void __launch_bounds__(BS) stream_kernel(const v4u* __restrict__ a,
                                                    const v4u* __restrict__ b,
                                                    const v4u* __restrict__ c,
                                                    v4u* __restrict__ out, v4u* __restrict__ out2,
                                                    int64_t n) {
    int64_t i = (int64_t)blockIdx.x * BS * U + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * BS * U;
    for (; i + (int64_t)(U - 1) * BS < n; i += stride) {
        v4u va[U], vb[U], vc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            va[u] = __builtin_nontemporal_load(a + i + u * BS);
            if constexpr (NIN >= 2) vb[u] = __builtin_nontemporal_load(b + i + u * BS);
            if constexpr (NIN >= 3) vc[u] = __builtin_nontemporal_load(c + i + u * BS);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            v4u r = va[u];
            if constexpr (NIN >= 2) r ^= vb[u];
            if constexpr (NIN >= 3) r ^= vc[u];
            if constexpr (NTST) __builtin_nontemporal_store(r, out + i + u * BS);
            else out[i + u * BS] = r;
            if constexpr (NOUT == 2) {
                const v4u r2 = va[u] + vb[u];
                if constexpr (NTST) __builtin_nontemporal_store(r2, out2 + i + u * BS);
                else out2[i + u * BS] = r2;
            }
        }
    }
    // the last partial chunk, one vector per thread and step
    for (; i < n; i += BS) {
        v4u r = a[i];
        if constexpr (NIN >= 2) r ^= b[i];
        if constexpr (NIN >= 3) r ^= c[i];
        out[i] = r;
        if constexpr (NOUT == 2) out2[i] = a[i] + b[i];
    }
}

bool ok_args(const void* a, const void* out, int64_t bytes) {
    return a && out && bytes > 0 && bytes % 16 == 0 && (uintptr_t)a % 16 == 0 &&
           (uintptr_t)out % 16 == 0;
}

}  // namespace

extern "C" {

// out[0 .. bytes) = a[0 .. bytes). Returns 0, 1 (bad arguments: null, size
// not a positive multiple of 16, pointers not 16-byte aligned) or 2 (launch
// failure).
int stream_ref_copy(const void* a, void* out, int64_t bytes, void* stream) {
    if (!ok_args(a, out, bytes)) return 1;
    hipLaunchKernelGGL((stream_kernel<1, 1, 4, 256, false>), dim3(256), dim3(256), 0,
                       static_cast<hipStream_t>(stream), (const v4u*)a, (const v4u*)a, (const v4u*)a,
                       (v4u*)out, (v4u*)out, bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// out = a xor b over bytes bytes (b as a, 16-byte aligned). Returns as above.
int stream_ref_2in1out(const void* a, const void* b, void* out, int64_t bytes, void* stream) {
    if (!ok_args(a, out, bytes) || !b || (uintptr_t)b % 16 != 0) return 1;
    hipLaunchKernelGGL((stream_kernel<2, 1, 2, 512, true>), dim3(256), dim3(512), 0,
                       static_cast<hipStream_t>(stream), (const v4u*)a, (const v4u*)b, (const v4u*)b,
                       (v4u*)out, (v4u*)out, bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// out = a xor b, out2 = a + b (lane-wise) over bytes bytes each, with
// nontemporal stores if nt != 0, else write-back ones. Returns as above.
int stream_ref_2in2out(const void* a, const void* b, void* out, void* out2, int64_t bytes, int nt,
                       void* stream) {
    if (!ok_args(a, out, bytes) || !b || (uintptr_t)b % 16 != 0 || !out2 || (uintptr_t)out2 % 16 != 0)
        return 1;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (nt)
        hipLaunchKernelGGL((stream_kernel<2, 2, 2, 512, true>), dim3(256), dim3(512), 0, s, (const v4u*)a,
                           (const v4u*)b, (const v4u*)b, (v4u*)out, (v4u*)out2, bytes / 16);
    else
        hipLaunchKernelGGL((stream_kernel<2, 2, 2, 512, false>), dim3(256), dim3(512), 0, s, (const v4u*)a,
                           (const v4u*)b, (const v4u*)b, (v4u*)out, (v4u*)out2, bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// out = a xor b xor c over bytes bytes, with nontemporal stores if nt != 0.
// Returns as above.
int stream_ref_3in1out(const void* a, const void* b, const void* c, void* out, int64_t bytes, int nt,
                       void* stream) {
    if (!ok_args(a, out, bytes) || !b || (uintptr_t)b % 16 != 0 || !c || (uintptr_t)c % 16 != 0)
        return 1;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (nt)
        hipLaunchKernelGGL((stream_kernel<3, 1, 2, 512, true>), dim3(256), dim3(512), 0, s, (const v4u*)a,
                           (const v4u*)b, (const v4u*)c, (v4u*)out, (v4u*)out, bytes / 16);
    else
        hipLaunchKernelGGL((stream_kernel<3, 1, 2, 512, false>), dim3(256), dim3(512), 0, s, (const v4u*)a,
                           (const v4u*)b, (const v4u*)c, (v4u*)out, (v4u*)out, bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
