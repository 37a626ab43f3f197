// Streaming-read probe: the practical HBM read rate of this GPU, as a
// reference beside the published peak for HBM-bound kernels.  It reads a
// device buffer of the given size once per launch with 16-byte loads, in two
// patterns:
//   linear  each workgroup streams a contiguous chunk;
//   pages   the buffer is cut into 4 KiB pages (the size of one 16-token page
//           of one KV head at d = 128, bf16) visited in a seeded random order,
//           each wave reading a whole page per step,
// sweeping the grid, the loads in flight per lane and the load kind
// (ordinary or non-temporal), and prints one JSON line with each pattern's
// best median rate.  A standalone program: it takes no part in attention and
// links nothing of the library.
//
//   hbm_read_probe [bytes]        (default 4 GiB)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <numeric>
#include <random>
#include <vector>

using u32x4 = unsigned __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

template <int U, bool NT>
__global__ __launch_bounds__(256) void read_linear(const u32x4* __restrict__ src, size_t n16, size_t per_wg,
                                                   unsigned* sink) {
    const size_t base = (size_t)blockIdx.x * per_wg;
    const size_t end = base + per_wg < n16 ? base + per_wg : n16;
    unsigned acc = 0;
    for (size_t i = base + threadIdx.x; i < end; i += 256 * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t j = i + (size_t)u * 256;
            v[u] = j < end ? load16<NT>(src + j) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    // The buffer holds 0x01 bytes, so acc is 0 and nothing is written; the
    // branch keeps the loads from being removed.
    if (acc == 0x12345678u) sink[blockIdx.x] = acc;
}

// One 4 KiB page is 256 16-byte pieces: lane l of a wave reads pieces
// l, l + 64, l + 128, l + 192.  Page perm[c] is visited at step c.
template <int U, bool NT>
__global__ __launch_bounds__(256) void read_pages(const u32x4* __restrict__ src, const int* __restrict__ perm,
                                                  int npages, unsigned* sink) {
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nw = gridDim.x * 4;
    unsigned acc = 0;
    for (int c0 = gw; c0 < npages; c0 += nw * U) {
        u32x4 v[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * nw;
            const size_t base = c < npages ? (size_t)perm[c] * 256 : 0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[u][i] = c < npages ? load16<NT>(src + base + i * 64 + lane) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc ^= v[u][i][0] ^ v[u][i][1] ^ v[u][i][2] ^ v[u][i][3];
    }
    if (acc == 0x12345678u) sink[blockIdx.x] = acc;
}

#define CHECK(x)                                                                                \
    do {                                                                                        \
        hipError_t e_ = (x);                                                                    \
        if (e_ != hipSuccess) {                                                                 \
            fprintf(stderr, "hbm_read_probe: %s (line %d)\n", hipGetErrorString(e_), __LINE__); \
            return 1;                                                                           \
        }                                                                                       \
    } while (0)

struct Result {
    double median_gbs = 0.0;
    int u = 0, grid = 0;
    bool nt = false;
};

// Median over 21 timed launches (after 3 warm-ups) of launch(), as GB/s.
template <class F>
int time_launches(F launch, double bytes, double& gbs) {
    hipEvent_t a, b;
    CHECK(hipEventCreate(&a));
    CHECK(hipEventCreate(&b));
    for (int w = 0; w < 3; ++w) launch();
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    std::vector<float> ms;
    for (int r = 0; r < 21; ++r) {
        CHECK(hipEventRecord(a, 0));
        launch();
        CHECK(hipEventRecord(b, 0));
        CHECK(hipEventSynchronize(b));
        float t = 0.f;
        CHECK(hipEventElapsedTime(&t, a, b));
        ms.push_back(t);
    }
    CHECK(hipGetLastError());
    CHECK(hipEventDestroy(a));
    CHECK(hipEventDestroy(b));
    std::sort(ms.begin(), ms.end());
    gbs = bytes / (ms[ms.size() / 2] * 1e-3) / 1e9;
    return 0;
}

template <int U, bool NT>
int sweep_linear(const u32x4* d, size_t n16, unsigned* sink, int grid, Result& best) {
    const size_t per_wg = (n16 + grid - 1) / grid;
    double gbs = 0.0;
    if (time_launches([&] { hipLaunchKernelGGL((read_linear<U, NT>), dim3(grid), dim3(256), 0, 0, d, n16, per_wg, sink); },
                      (double)n16 * 16.0, gbs))
        return 1;
    if (gbs > best.median_gbs) best = Result{gbs, U, grid, NT};
    return 0;
}

template <int U, bool NT>
int sweep_pages(const u32x4* d, const int* perm, int npages, unsigned* sink, int grid, Result& best) {
    double gbs = 0.0;
    if (time_launches([&] { hipLaunchKernelGGL((read_pages<U, NT>), dim3(grid), dim3(256), 0, 0, d, perm, npages, sink); },
                      (double)npages * 4096.0, gbs))
        return 1;
    if (gbs > best.median_gbs) best = Result{gbs, U, grid, NT};
    return 0;
}

int main(int argc, char** argv) {
    size_t bytes = argc > 1 ? strtoull(argv[1], nullptr, 10) : ((size_t)4 << 30);
    bytes &= ~(size_t)4095;
    if (bytes < ((size_t)1 << 20) || bytes / 4096 > (size_t)0x7fffffff) {
        fprintf(stderr, "hbm_read_probe: size out of range\n");
        return 2;
    }
    const size_t n16 = bytes / 16;
    const int npages = (int)(bytes / 4096);
    const int grids[] = {2048, 4096, 16384};
    u32x4* d = nullptr;
    unsigned* sink = nullptr;
    int* perm_d = nullptr;
    std::vector<int> perm(npages);
    std::iota(perm.begin(), perm.end(), 0);
    std::shuffle(perm.begin(), perm.end(), std::mt19937(12345));
    CHECK(hipMalloc(&d, bytes));
    CHECK(hipMalloc(&sink, 16384 * sizeof(unsigned)));
    CHECK(hipMalloc(&perm_d, (size_t)npages * sizeof(int)));
    CHECK(hipMemcpy(perm_d, perm.data(), (size_t)npages * sizeof(int), hipMemcpyHostToDevice));
    CHECK(hipMemset(d, 1, bytes));
    CHECK(hipDeviceSynchronize());
    Result lin, pg;
    for (int grid : grids) {
        if (sweep_linear<4, false>(d, n16, sink, grid, lin) || sweep_linear<8, false>(d, n16, sink, grid, lin) ||
            sweep_linear<4, true>(d, n16, sink, grid, lin) || sweep_linear<8, true>(d, n16, sink, grid, lin))
            return 1;
        if (sweep_pages<2, false>(d, perm_d, npages, sink, grid, pg) || sweep_pages<4, false>(d, perm_d, npages, sink, grid, pg) ||
            sweep_pages<2, true>(d, perm_d, npages, sink, grid, pg) || sweep_pages<4, true>(d, perm_d, npages, sink, grid, pg))
            return 1;
    }
    CHECK(hipFree(d));
    CHECK(hipFree(sink));
    CHECK(hipFree(perm_d));
    printf("{\"bytes\": %zu, \"linear\": {\"median_gbs\": %.1f, \"loads_in_flight_per_lane\": %d, \"grid\": %d, "
           "\"nontemporal\": %s}, \"pages\": {\"median_gbs\": %.1f, \"pages_in_flight_per_wave\": %d, \"grid\": %d, "
           "\"nontemporal\": %s}}\n",
           bytes, lin.median_gbs, lin.u, lin.grid, lin.nt ? "true" : "false", pg.median_gbs, pg.u, pg.grid,
           pg.nt ? "true" : "false");
    return 0;
}
