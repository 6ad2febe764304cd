// probe.hip -- calibration kernels for the measurements reported beside the conv and
// GEMM kernels: the int8 MFMA rate a register-only loop reaches on this GPU (the
// practical ceiling of the contraction, below the spec-sheet peak when the clock
// drops under load) and the duration of an empty launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "iqnn_internal.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__global__ void empty_kernel() {}

// Eight independent 32x32x32 int8 MFMA accumulators per wave; the operands differ per
// lane and hold all byte values, so the multipliers see ordinary data.  Each wave
// writes a sum of its accumulators so the loop cannot be removed.
__global__ __launch_bounds__(256, 2) void mfma_rate_kernel(int32_t* sink, int32_t iters) {
    const uint32_t l = threadIdx.x;
    const v4i a = {(int)(l * 2654435761u), (int)(l * 40503u + 977u), (int)((l ^ 0x5bd1e995u) * 2246822519u),
                   (int)(l * 3266489917u)};
    const v4i b = {(int)(l * 668265263u), (int)(l * 374761393u + 1u), (int)(l * 2654435761u + 7u),
                   (int)((l + 3) * 2246822519u)};
    v16i acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = v16i{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[j], 0, 0, 0);
    }
    int32_t s = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    sink[(int64_t)blockIdx.x * 256 + l] = s;
}

}  // namespace

namespace iqnn {

hipError_t launch_probe_empty(hipStream_t stream) {
    hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, stream);
    return hipGetLastError();
}

hipError_t launch_probe_mfma_rate(int32_t iters, int32_t blocks, int32_t* sink, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_rate_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, sink, iters);
    return hipGetLastError();
}

}  // namespace iqnn
