// bench_readbw.hip -- read-bandwidth calibration for the decode's roofline.
//
// A standalone program (not part of libdiffattn): it streams a 4 GiB device
// buffer with 16-byte loads (U loads in flight per thread, XOR-folded into
// one word per thread so the loads are not dead) and prints the achieved read
// bandwidth for several grid sizes and three access patterns: grid-stride,
// grid-stride with non-temporal loads, and one contiguous chunk per
// work-group (as the decode reads whole pages). It gives the read rate a
// plain streaming kernel reaches on the device, the practical ceiling the
// memory-bound decode is compared with beside the published HBM peak.
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//       bench_readbw.hip -o gpurun_out/bench_readbw && ./gpurun_out/bench_readbw
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#define CHECK(x)                                                              \
    do {                                                                      \
        hipError_t e_ = (x);                                                  \
        if (e_ != hipSuccess) {                                               \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));           \
            return 1;                                                         \
        }                                                                     \
    } while (0)

template <int U>
__global__ __launch_bounds__(256) void read_kernel(const uint4 *__restrict__ p, int64_t n, uint32_t *out) {
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    int64_t i = tid;
    for (; i + (U - 1) * stride < n; i += U * stride) {  // every load below is < n
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = p[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n; i += stride) {
        const uint4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    out[tid] = acc;  // one word per thread: out holds grid * 256 words
}

// grid-stride, non-temporal loads (no reuse expected: do not keep the lines)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt(const uint4 *q) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4 *)q);
    return make_uint4(v.x, v.y, v.z, v.w);
}
template <int U>
__global__ __launch_bounds__(256) void read_nt_kernel(const uint4 *__restrict__ p, int64_t n, uint32_t *out) {
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    int64_t i = tid;
    for (; i + (U - 1) * stride < n; i += U * stride) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = ld_nt(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n; i += stride) {
        const uint4 v = ld_nt(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    out[tid] = acc;
}

// one contiguous chunk of n / gridDim.x elements per work-group, block-stride inside it
template <int U>
__global__ __launch_bounds__(256) void read_chunk_kernel(const uint4 *__restrict__ p, int64_t n, uint32_t *out) {
    const int64_t chunk = n / gridDim.x;
    const int64_t beg = (int64_t)blockIdx.x * chunk, end = beg + chunk;
    uint32_t acc = 0;
    int64_t i = beg + threadIdx.x;
    for (; i + (U - 1) * 256 < end; i += U * 256) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = p[i + u * 256];
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < end; i += 256) {
        const uint4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

int main() {
    const int64_t bytes = 4LL << 30, n = bytes / 16;
    const int max_grid = 256 * 256;
    uint4 *p = nullptr;
    uint32_t *out = nullptr;
    CHECK(hipMalloc(&p, bytes));
    CHECK(hipMemset(p, 1, bytes));
    CHECK(hipMalloc(&out, (size_t)max_grid * 256 * sizeof(uint32_t)));
    hipEvent_t a, b;
    CHECK(hipEventCreate(&a));
    CHECK(hipEventCreate(&b));
    double best = 0.0;
    const char *names[3] = {"grid-stride", "grid-stride, non-temporal", "chunk per work-group"};
    for (int kind = 0; kind < 3; ++kind)
    for (int grid : {256 * 4, 256 * 8, 256 * 16, 256 * 32, 256 * 64, 256 * 128, 256 * 256}) {
        for (int u : {4, 8}) {
            auto launch = [&]() {
                if (kind == 0 && u == 4) hipLaunchKernelGGL(read_kernel<4>, dim3(grid), dim3(256), 0, 0, p, n, out);
                if (kind == 0 && u == 8) hipLaunchKernelGGL(read_kernel<8>, dim3(grid), dim3(256), 0, 0, p, n, out);
                if (kind == 1 && u == 4) hipLaunchKernelGGL(read_nt_kernel<4>, dim3(grid), dim3(256), 0, 0, p, n, out);
                if (kind == 1 && u == 8) hipLaunchKernelGGL(read_nt_kernel<8>, dim3(grid), dim3(256), 0, 0, p, n, out);
                if (kind == 2 && u == 4)
                    hipLaunchKernelGGL(read_chunk_kernel<4>, dim3(grid), dim3(256), 0, 0, p, n, out);
                if (kind == 2 && u == 8)
                    hipLaunchKernelGGL(read_chunk_kernel<8>, dim3(grid), dim3(256), 0, 0, p, n, out);
            };
            for (int w = 0; w < 3; ++w) launch();
            CHECK(hipGetLastError());
            CHECK(hipEventRecord(a));
            for (int r = 0; r < 10; ++r) launch();
            CHECK(hipEventRecord(b));
            CHECK(hipEventSynchronize(b));
            float ms = 0.0f;
            CHECK(hipEventElapsedTime(&ms, a, b));
            ms /= 10;
            const double gbs = bytes / (ms * 1e-3) / 1e9;
            best = gbs > best ? gbs : best;
            printf("%s, grid %5d x 256 threads, %d loads in flight per thread: %.3f ms, %.0f GB/s\n", names[kind],
                   grid, u, ms, gbs);
        }
    }
    printf("best read bandwidth: %.0f GB/s (%.1f %% of 8000 GB/s)\n", best, best / 80.0);
    CHECK(hipFree(out));
    CHECK(hipFree(p));
    return 0;
}
