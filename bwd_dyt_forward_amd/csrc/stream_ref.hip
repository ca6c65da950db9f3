// stream_ref.hip - reference streaming kernels for measurement only (loaded
// by bench.py, not part of the DyT C ABI): the plain memory streams the DyT
// kernels are compared against on the same GPU.
//
//   stream_ref_copy     out = a                    (1 read + 1 write stream,
//                                                   the forward's traffic)
//   stream_ref_2in1out  out = a xor b              (2 read + 1 write streams,
//                                                   backward pass 1's traffic)
//
// 16-byte nontemporal loads, each workgroup streaming contiguous chunks of
// U x (block x 16 B) in a grid-stride loop. The launch shapes and store
// kinds are the fastest of steady-state sweeps on MI355X (copy: 256
// workgroups of 256 threads, U = 4, ordinary write-back stores, which ran a
// 256 MiB copy in 76.5 us against 85.0 us with nontemporal ones;
// 2-in-1-out: 256 workgroups of 512 threads, U = 2, nontemporal stores).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

template <int NIN, int U, int BS, bool NTST>
__global__ void __launch_bounds__(BS) stream_kernel(const v4u* __restrict__ a,
                                                    const v4u* __restrict__ b,
                                                    v4u* __restrict__ out, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * BS * U + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * BS * U;
    for (; i + (int64_t)(U - 1) * BS < n; i += stride) {
        v4u va[U], vb[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            va[u] = __builtin_nontemporal_load(a + i + u * BS);
            if constexpr (NIN == 2) vb[u] = __builtin_nontemporal_load(b + i + u * BS);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            v4u r = va[u];
            if constexpr (NIN == 2) r ^= vb[u];
            if constexpr (NTST) __builtin_nontemporal_store(r, out + i + u * BS);
            else out[i + u * BS] = r;
        }
    }
    // the last partial chunk, one vector per thread and step
    for (; i < n; i += BS) {
        v4u r = a[i];
        if constexpr (NIN == 2) r ^= b[i];
        out[i] = r;
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
    hipLaunchKernelGGL((stream_kernel<1, 4, 256, false>), dim3(256), dim3(256), 0,
                       static_cast<hipStream_t>(stream), (const v4u*)a, (const v4u*)a, (v4u*)out,
                       bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// out = a xor b over bytes bytes (b as a, 16-byte aligned). Returns as above.
int stream_ref_2in1out(const void* a, const void* b, void* out, int64_t bytes, void* stream) {
    if (!ok_args(a, out, bytes) || !b || (uintptr_t)b % 16 != 0) return 1;
    hipLaunchKernelGGL((stream_kernel<2, 2, 512, true>), dim3(256), dim3(512), 0,
                       static_cast<hipStream_t>(stream), (const v4u*)a, (const v4u*)b, (v4u*)out,
                       bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
