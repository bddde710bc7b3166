// Microbenchmarks of the three hardware rates the correlation path is bound
// by, for reporting measured peaks beside the published ones: streaming HBM
// writes, v_dot4_u32_u8 issue, and int8 matrix-core issue.  Built into a
// library of its own (libncc_peaks.so) that only the benchmark loads.
#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace {

// The buffer as rows of `row16` 16-byte words (a 4096-column int64 table:
// 2048); workgroup b writes a tile of 64 words (1 KB) x 32 rows, wavefront
// w rows 8w .. 8w+7 of it, one 1 KB store instruction per row: the store
// pattern of the table build.
__global__ __launch_bounds__(256) void peak_write(uint4 *__restrict__ p, int row16, int tiles_x,
                                                  uint32_t v) {
    // workgroups go to the 8 XCDs round-robin: give each XCD one contiguous
    // run of tiles (the grid is a multiple of 8)
    const int per = gridDim.x / 8;
    const int k = (blockIdx.x % 8) * per + blockIdx.x / 8;
    const int tx = k % tiles_x, ty = k / tiles_x;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    uint4 *q = p + ((size_t)ty * 32 + 8 * w) * row16 + (size_t)tx * 64 + l;
#pragma unroll
    for (int r = 0; r < 8; r++) q[(size_t)r * row16] = make_uint4(v, v + 1, v + 2, v + r);
}

// 8 independent dot4 chains per lane, `iters` rounds of 8 dot4 each.
__global__ __launch_bounds__(256) void peak_dot4(uint32_t *__restrict__ out, int iters, uint32_t seed) {
    uint32_t a = seed ^ threadIdx.x, b = seed * 2654435761u + blockIdx.x;
    uint32_t c[8];
#pragma unroll
    for (int k = 0; k < 8; k++) c[k] = a + k;
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int k = 0; k < 8; k++) c[k] = __builtin_amdgcn_udot4(a, b + k, c[k], false);
    }
    uint32_t s = 0;
#pragma unroll
    for (int k = 0; k < 8; k++) s += c[k];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

typedef int v4i __attribute__((ext_vector_type(4)));

// 8 independent 16x16x64 int8 accumulations per wavefront, `iters` rounds.
__global__ __launch_bounds__(256) void peak_mfma_i8(int32_t *__restrict__ out, int iters, int seed) {
    const v4i a = {seed, seed + 1, seed + 2, (int)threadIdx.x};
    const v4i b = {seed ^ 5, seed ^ 7, (int)blockIdx.x, seed ^ 11};
    v4i acc[8];
#pragma unroll
    for (int k = 0; k < 8; k++) acc[k] = (v4i){k, 0, 0, 0};
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int k = 0; k < 8; k++) acc[k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[k], 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int k = 0; k < 8; k++) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Compute units and peak engine clock (kHz) of the current device.
int ncc_peak_props(int *cus, int *clock_khz) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    if (hipDeviceGetAttribute(clock_khz, hipDeviceAttributeClockRate, dev) != hipSuccess) return -1;
    return 0;
}

// Writes `bytes` at dst as rows of `row_bytes` in tiles of 1 KB x 32 rows;
// row_bytes must be a multiple of 1 KB, bytes of 32 * row_bytes, and the
// tile count of 8.
int ncc_peak_write(void *dst, size_t bytes, int row_bytes, void *stream) {
    if (!dst || row_bytes < 1024 || row_bytes % 1024 || bytes % (32 * (size_t)row_bytes)) return -1;
    const size_t tiles = bytes / (32 * (size_t)row_bytes) * (row_bytes / 1024);
    if (tiles > 0x7fffffff || tiles % 8) return -1;
    hipLaunchKernelGGL(peak_write, dim3((unsigned)tiles), dim3(256), 0, (hipStream_t)stream,
                       (uint4 *)dst, row_bytes / 16, row_bytes / 1024, 7u);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// `blocks` workgroups of 256 lanes, each lane 8 * iters dot4; out holds
// blocks * 256 uint32.
int ncc_peak_dot4(uint32_t *out, int blocks, int iters, void *stream) {
    if (!out || blocks < 1 || iters < 1) return -1;
    hipLaunchKernelGGL(peak_dot4, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters, 12345u);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// `blocks` workgroups of 4 wavefronts, each wavefront 8 * iters MFMAs of
// 16x16x64 int8; out holds blocks * 256 int32.
int ncc_peak_mfma_i8(int32_t *out, int blocks, int iters, void *stream) {
    if (!out || blocks < 1 || iters < 1) return -1;
    hipLaunchKernelGGL(peak_mfma_i8, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters, 3);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
