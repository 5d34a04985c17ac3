// Device twin of workloads/gen.py: the same counter-based draws, so large
// synthetic inputs (8B-shaped weights, long KV pre-fills) are generated in
// place on the GPU.  Input generation only; it holds none of the decode
// step's arithmetic and is not part of libubd.
//
// Element i of a stream with 64-bit key k takes h = mix64(k + (i+1)*G) (the
// SplitMix64 output function, Steele, Lea and Flood, OOPSLA 2014); normal
// values are table[h >> 48] from a host-built quantile table.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t hash_at(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * kGolden); }

__global__ void table16_kernel(uint16_t *out, int64_t n, uint64_t key, int64_t start, const uint16_t *table) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        out[i] = table[hash_at(key, (uint64_t)(start + i)) >> 48];
}

__global__ void table32_kernel(float *out, int64_t n, uint64_t key, int64_t start, const float *table) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        out[i] = table[hash_at(key, (uint64_t)(start + i)) >> 48];
}

__global__ void q8_codes_kernel(int8_t *out, int64_t n, uint64_t key, int64_t start) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        out[i] = (int8_t)((int)((hash_at(key, (uint64_t)(start + i)) >> 32) % 255u) - 127);
}

__global__ void q8_scales_kernel(uint16_t *out, int64_t n, uint64_t key, int64_t start) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t m = 263u + (uint32_t)((hash_at(key, (uint64_t)(start + i)) >> 32) % 786u);
        _Float16 v = (_Float16)((float)m * 0x1p-19f);   // exact: m * 2^-19 fits f16
        uint16_t b;
        __builtin_memcpy(&b, &v, 2);
        out[i] = b;
    }
}

dim3 grid_for(int64_t n) {
    int64_t b = (n + 255) / 256;
    if (b > 65536) b = 65536;
    if (b < 1) b = 1;
    return dim3((unsigned)b);
}

}  // namespace

extern "C" int ubd_synth_table16(uint16_t *out, int64_t n, uint64_t key, int64_t start, const uint16_t *table,
                                 void *stream) {
    if (n <= 0) return 0;
    hipLaunchKernelGGL(table16_kernel, grid_for(n), dim3(256), 0, (hipStream_t)stream, out, n, key, start, table);
    return (int)hipGetLastError();
}

extern "C" int ubd_synth_table32(float *out, int64_t n, uint64_t key, int64_t start, const float *table,
                                 void *stream) {
    if (n <= 0) return 0;
    hipLaunchKernelGGL(table32_kernel, grid_for(n), dim3(256), 0, (hipStream_t)stream, out, n, key, start, table);
    return (int)hipGetLastError();
}

extern "C" int ubd_synth_q8_codes(int8_t *out, int64_t n, uint64_t key, int64_t start, void *stream) {
    if (n <= 0) return 0;
    hipLaunchKernelGGL(q8_codes_kernel, grid_for(n), dim3(256), 0, (hipStream_t)stream, out, n, key, start);
    return (int)hipGetLastError();
}

extern "C" int ubd_synth_q8_scales(uint16_t *out, int64_t n, uint64_t key, int64_t start, void *stream) {
    if (n <= 0) return 0;
    hipLaunchKernelGGL(q8_scales_kernel, grid_for(n), dim3(256), 0, (hipStream_t)stream, out, n, key, start);
    return (int)hipGetLastError();
}
