// debug.hip — the BQA_DEBUG=1 input scan of the C ABI.
//
// With the environment variable BQA_DEBUG set to 1, every call scans its
// floating-point inputs (bf16 / fp16 tensors, fp32 arrays) for NaN and
// infinity before it launches anything, waits for the scan on its stream and
// returns BQA_E_NONFINITE when one is found.  The count lives in a static
// device word (one per device); the scan is for debugging only: it
// synchronises the stream, so it must not run under graph capture, and calls
// that overlap on one device share the word.
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "internal.hpp"

namespace bqa {

namespace {

__device__ __attribute__((aligned(256))) uint32_t nonfinite_count[64];

// 16-bit values of a [B, H, N, d] view; exp_mask 0x7F80 (bf16) or 0x7C00 (fp16)
__global__ __launch_bounds__(256) void scan16_kernel(Dense x, int H, int N, int d, int64_t total, uint32_t exp_mask,
                                                     uint32_t* __restrict__ count) {
    uint32_t bad = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t c = i % d, r = i / d, n = r % N, bh = r / N, b = bh / H, h = bh % H;
        const uint32_t v = ((const uint16_t*)x.p)[b * x.sB + h * x.sH + n * x.sN + c];
        bad |= (v & exp_mask) == exp_mask;
    }
    if (__any(bad) && (threadIdx.x & 63) == 0) atomicAdd(count, 1u);
}

__global__ __launch_bounds__(256) void scan32_kernel(const uint32_t* __restrict__ x, int64_t n,
                                                     uint32_t* __restrict__ count) {
    uint32_t bad = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        bad |= (x[i] & 0x7F800000u) == 0x7F800000u;
    if (__any(bad) && (threadIdx.x & 63) == 0) atomicAdd(count, 1u);
}

__global__ void zero_kernel(uint32_t* p) { *p = 0u; }

std::mutex g_mu;
uint32_t* g_ptr[64] = {};

hipError_t counter(uint32_t** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(nonfinite_count));
        if (e != hipSuccess) return e;
        g_ptr[dev] = (uint32_t*)p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

unsigned grid_for(int64_t n) {
    const int64_t g = (n + 255) / 256;
    return (unsigned)(g < 4096 ? (g < 1 ? 1 : g) : 4096);
}

}  // namespace

bool debug_enabled() {
    const char* v = std::getenv("BQA_DEBUG");
    return v && std::strcmp(v, "1") == 0;
}

// 1: a non-finite value was found, 0: none, -1: a HIP call failed
int debug_scan(hipStream_t st, const DebugInput* in, int n_in) {
    uint32_t* cnt = nullptr;
    if (counter(&cnt) != hipSuccess) return -1;
    zero_kernel<<<1, 1, 0, st>>>(cnt);
    for (int i = 0; i < n_in; ++i) {
        const DebugInput& x = in[i];
        if (!x.p) continue;
        if (x.kind == DebugInput::F32) {
            scan32_kernel<<<grid_for(x.n), 256, 0, st>>>((const uint32_t*)x.p, x.n, cnt);
        } else {
            const int64_t total = (int64_t)x.B * x.H * x.N * x.d;
            scan16_kernel<<<grid_for(total), 256, 0, st>>>(Dense{(void*)x.p, x.sB, x.sH, x.sN}, x.H, x.N, x.d, total,
                                                          x.kind == DebugInput::F16 ? 0x7C00u : 0x7F80u, cnt);
        }
    }
    uint32_t host = 0;
    if (hipGetLastError() != hipSuccess) return -1;
    if (hipMemcpyAsync(&host, cnt, sizeof(host), hipMemcpyDeviceToHost, st) != hipSuccess) return -1;
    if (hipStreamSynchronize(st) != hipSuccess) return -1;
    return host ? 1 : 0;
}

}  // namespace bqa
