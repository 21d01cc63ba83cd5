// bench_ldsbw.hip -- LDS read-rate calibration for the attention kernels.
//
// A standalone program (not part of libdiffattn). Each work-group of 256
// threads fills a 64 KB LDS buffer, then every thread issues 32768 reads:
//   * ds_read_b128 (16 bytes per lane, consecutive lanes on consecutive
//     16-byte slots: the conflict-free row-read pattern), or
//   * ds_read_b64_tr_b16 at the addresses the prefill uses for its value
//     tile (64 rows x 256 bytes, 16-byte chunk XOR 4 (row & 3)),
// XOR-folding the data into one word per thread so no read is dead. It prints
// the bytes per second per compute unit and per clock (2.1 GHz, the engine
// clock under load, and the 2.4 GHz rating): the cost of one LDS read
// instruction per compute unit, whatever its width.
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//       bench_ldsbw.hip -o gpurun_out/bench_ldsbw && ./gpurun_out/bench_ldsbw
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

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kIter = 2048;  // x 16 reads per iteration

__global__ __launch_bounds__(256) void read_b128(uint32_t *out) {
    __shared__ uint4 buf[4096];  // 64 KB
    const int t = threadIdx.x;
    for (int i = t; i < 4096; i += 256) buf[i] = uint4{(uint32_t)i, (uint32_t)i * 3u, 7u, (uint32_t)t};
    __syncthreads();
    uint32_t acc = 0;
    for (int it = 0; it < kIter; ++it) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {  // 16 distinct 4 KB rows of slots per iteration
            const uint4 v = buf[(t + u * 256 + it * 64) & 4095];
            acc ^= v.x ^ v.y ^ v.z ^ v.w;
        }
    }
    out[blockIdx.x * 256 + t] = acc;
}

// transposing-read address of one lane in a 64 x 256-byte value tile
// (sub-block sb, k step t, value block dc, half), as the prefill reads it
__device__ __forceinline__ int tr_addr(int lane, int sb, int t, int dc, int half) {
    const int vi = lane & 15, hh = lane >> 5;
    const int row = 32 * sb + 16 * t + 8 * hh + 4 * half + (vi >> 2);
    const int col = 32 * dc + 16 * ((lane >> 4) & 1) + 4 * (vi & 3);
    const int c = (col >> 3) ^ ((row & 3) << 2);
    return row * 256 + 16 * c + 2 * (col & 7);  // < 16384, 8-byte aligned
}

__global__ __launch_bounds__(256) void read_tr(uint32_t *out) {
    __shared__ __attribute__((aligned(16))) unsigned char buf[65536];
    const int t = threadIdx.x, lane = t & 63;
    for (int i = t; i < 4096; i += 256) ((uint4 *)buf)[i] = uint4{(uint32_t)i, 1u, 2u, 3u};
    __syncthreads();
    const unsigned char *tile = buf + (t >> 6) * 16384;  // each wave reads its own 16 KB tile
    uint32_t acc = 0;
    for (int it = 0; it < kIter; ++it) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int sb = (u >> 3) & 1, tt = (u >> 2) & 1, dc = u & 3, half = it & 1;
            const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(tile + tr_addr(lane, sb, tt, dc, half)));
            acc ^= (uint32_t)v[0] ^ ((uint32_t)v[1] << 8) ^ ((uint32_t)v[2] << 16) ^ (uint32_t)v[3];
        }
    }
    out[blockIdx.x * 256 + t] = acc;
}

int main() {
    int cus = 0;
    CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
    const int max_per_cu = 8;
    uint32_t *out = nullptr;
    CHECK(hipMalloc(&out, (size_t)cus * max_per_cu * 256 * sizeof(uint32_t)));
    hipEvent_t a, b;
    CHECK(hipEventCreate(&a));
    CHECK(hipEventCreate(&b));
    for (int kind = 0; kind < 2; ++kind) {
        for (int per_cu : {2, 4, 8}) {
            const int grid = cus * per_cu;
            auto launch = [&]() {
                if (kind == 0)
                    hipLaunchKernelGGL(read_b128, dim3(grid), dim3(256), 0, 0, out);
                else
                    hipLaunchKernelGGL(read_tr, dim3(grid), dim3(256), 0, 0, out);
            };
            launch();
            CHECK(hipGetLastError());
            CHECK(hipDeviceSynchronize());
            CHECK(hipEventRecord(a));
            for (int r = 0; r < 5; ++r) launch();
            CHECK(hipEventRecord(b));
            CHECK(hipEventSynchronize(b));
            float ms = 0.0f;
            CHECK(hipEventElapsedTime(&ms, a, b));
            ms /= 5;
            const double bytes = (double)grid * 256 * kIter * 16 * (kind == 0 ? 16 : 8);
            const double per_cu_s = bytes / (ms * 1e-3) / cus;
            printf("%-20s %d work-groups per CU: %.3f ms, %.1f GB/s per CU = %.1f B/clk at 2.1 GHz, %.1f at 2.4 GHz\n",
                   kind == 0 ? "ds_read_b128" : "ds_read_b64_tr_b16", per_cu, ms, per_cu_s / 1e9, per_cu_s / 2.1e9,
                   per_cu_s / 2.4e9);
        }
    }
    CHECK(hipFree(out));
    return 0;
}
