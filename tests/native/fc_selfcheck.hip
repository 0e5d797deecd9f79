// Test support (not part of libfc.so): exhaustive checks of the quantizer's exact-quotient helpers in
// fc_device.h against the GPU's own IEEE division.
//   div_by_qmax<15>, div_by_qmax<255>: every non-negative finite float x (bit patterns 0 .. 0x7f7fffff);
//   recip_fp16: every positive finite fp16 value s (bit patterns 0x0001 .. 0x7bff).
// Each lane walks its share of the inputs with a grid stride and writes its own mismatch count; the host
// adds them up.  No atomics, no out-of-bounds index: counts[] holds one word per lane of the grid.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fc_device.h"

namespace {

constexpr int kBlocks = 2048, kThreads = 256;

template <int QMAX>
__global__ __launch_bounds__(kThreads) void k_check_div(uint32_t* counts) {
    const uint32_t gid = blockIdx.x * kThreads + threadIdx.x, stride = kBlocks * kThreads;
    uint32_t bad = 0;
    for (uint32_t u = gid; u <= 0x7f7fffffu; u += stride) {
        const float x = __builtin_bit_cast(float, u);
        const float ieee = x / (float)QMAX;
        bad += __builtin_bit_cast(uint32_t, fc::div_by_qmax<QMAX>(x)) != __builtin_bit_cast(uint32_t, ieee);
    }
    counts[gid] = bad;
}

__global__ __launch_bounds__(kThreads) void k_check_recip(uint32_t* counts) {
    const uint32_t gid = blockIdx.x * kThreads + threadIdx.x;
    uint32_t bad = 0;
    if (gid >= 1 && gid < 0x7c00u) {
        const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)gid);
        const float ieee = 1.0f / s;
        bad = __builtin_bit_cast(uint32_t, fc::recip_fp16(s)) != __builtin_bit_cast(uint32_t, ieee);
    }
    counts[gid] = bad;
}

uint64_t total(const uint32_t* d, int n, int* err) {
    static uint32_t h[kBlocks * kThreads];
    if (hipMemcpy(h, d, sizeof(uint32_t) * n, hipMemcpyDeviceToHost) != hipSuccess) *err = 1;
    uint64_t t = 0;
    for (int i = 0; i < n; ++i) t += h[i];
    return t;
}

}  // namespace

// out[0], out[1]: mismatches of div_by_qmax<15> and <255>; out[2]: of recip_fp16.  Returns 0, or -1 on a
// HIP error.
extern "C" int fc_selfcheck_quotients(uint64_t* out) {
    uint32_t* d = nullptr;
    const int n = kBlocks * kThreads;
    if (hipMalloc(&d, sizeof(uint32_t) * n) != hipSuccess) return -1;
    int err = 0;
    k_check_div<15><<<kBlocks, kThreads>>>(d);
    out[0] = total(d, n, &err);
    k_check_div<255><<<kBlocks, kThreads>>>(d);
    out[1] = total(d, n, &err);
    k_check_recip<<<(0x8000 + kThreads - 1) / kThreads, kThreads>>>(d);
    out[2] = total(d, 0x8000, &err);
    if (hipGetLastError() != hipSuccess) err = 1;
    hipFree(d);
    return err ? -1 : 0;
}
