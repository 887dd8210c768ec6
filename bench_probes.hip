// Microbenchmarks behind two design decisions of the library (standalone; not
// part of libnectar):
//
//  1. MFMA / VALU co-issue on one SIMD: cycles per step of a wave that issues
//     32x32x16 bf16 MFMAs (dependent chains or independent ones), plain fp32
//     VALU work (FMAs), transcendental work (exp2), and mixes of them, in the
//     same wave or in the two waves of a SIMD.  This bounds the batched MLP
//     (an activation of ~10 VALU operations per hidden value against 16 MFMA
//     cycles per value) and the batched attention (softmax against products).
//  2. A grid-wide barrier between the blocks of one launch (the alternative to
//     a second launch for the finishing pass of a decode step): one counter,
//     or eight group counters with sense-reversing flags, 64-256 blocks of 256
//     threads at one block per compute unit, device-scope atomics, with and
//     without the release/acquire fences the data exchange needs.
//
// Build and run (on the GPU host, from the repository root):
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         -o gpurun_out/bench_probes bench_probes.hip && gpurun_out/bench_probes
//
// Every access is in bounds (one store per thread into `out`, counters in an
// 8 KB buffer); every wait is bounded (1 << 22 polls, then an error word).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <vector>

#define CHECK(x)                                                                      \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            std::exit(1);                                                             \
        }                                                                             \
    } while (0)

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// 1. co-issue
__device__ __forceinline__ f32x16 mf(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

enum Mode { CHAIN1, CHAIN4, FMA8, EXP8, CHAIN_FMA2, CHAIN_FMA4, CHAIN_FMA8, CHAIN_EXP8, PAIR_FMA, PAIR_EXP };

// One "step" per wave: MODE's unit of work (one MFMA and/or 8 VALU operations);
// PAIR_*: waves 0-3 of a block do the VALU work, waves 4-7 (the other wave of
// each SIMD) the MFMAs.
template <int MODE>
__global__ __launch_bounds__(512) void coissue(float *out, long long *cyc, int iters) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const u32x4 a = {(unsigned)lane * 0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    const u32x4 b = {0x3c003c00u, 0x3c003c00u, (unsigned)w, 0x3c003c00u};
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    float v[8];
    for (int j = 0; j < 8; ++j) v[j] = 1.0f + lane * 1e-3f + j;
    const bool mwave = (w >> 2) & 1;
    const long long t0 = clock64();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const bool do_mfma = MODE == CHAIN1 || MODE == CHAIN4 || (MODE >= CHAIN_FMA2 && MODE <= CHAIN_EXP8) ||
                                 ((MODE == PAIR_FMA || MODE == PAIR_EXP) && mwave);
            const bool do_fma = MODE == FMA8 || MODE == CHAIN_FMA8 || (MODE == PAIR_FMA && !mwave);
            const bool do_exp = MODE == EXP8 || MODE == CHAIN_EXP8 || (MODE == PAIR_EXP && !mwave);
            if (do_mfma) {
                if (MODE == CHAIN4 || MODE == PAIR_FMA || MODE == PAIR_EXP) {
                    if ((k & 3) == 0) c0 = mf(a, b, c0);
                    else if ((k & 3) == 1) c1 = mf(a, b, c1);
                    else if ((k & 3) == 2) c2 = mf(a, b, c2);
                    else c3 = mf(a, b, c3);
                } else {
                    c0 = mf(a, b, c0);
                }
            }
            if (do_fma)
                for (int j = 0; j < 8; ++j) v[j] = __builtin_fmaf(v[j], 0.999f, 0.5f);
            if (do_exp)
                for (int j = 0; j < 8; ++j) v[j] = __builtin_amdgcn_exp2f(v[j]);
            if (MODE == CHAIN_FMA2)
                for (int j = 0; j < 2; ++j) v[j] = __builtin_fmaf(v[j], 0.999f, 0.5f);
            if (MODE == CHAIN_FMA4)
                for (int j = 0; j < 4; ++j) v[j] = __builtin_fmaf(v[j], 0.999f, 0.5f);
        }
    }
    const long long t1 = clock64();
    float s = 0.f;
    for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
    for (int j = 0; j < 8; ++j) s += v[j];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
    if (threadIdx.x == 0) cyc[blockIdx.x] = t1 - t0;
}

template <int MODE>
static void run_coissue(const char *what, int threads, float *out, long long *cyc) {
    const int blocks = 256, iters = 2000;
    hipLaunchKernelGGL(coissue<MODE>, dim3(blocks), dim3(threads), 0, 0, out, cyc, 10);
    CHECK(hipDeviceSynchronize());
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(coissue<MODE>, dim3(blocks), dim3(threads), 0, 0, out, cyc, iters);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    std::vector<long long> h(blocks);
    CHECK(hipMemcpy(h.data(), cyc, blocks * sizeof(long long), hipMemcpyDeviceToHost));
    double avg = 0;
    for (long long x : h) avg += (double)x;
    avg /= blocks;
    std::printf("| %s | %d | %.3f | %.1f |\n", what, threads / 64 / 4, ms, avg / (iters * 8.0));
}

// ---------------------------------------------------------------------------
// 2. grid barrier
constexpr unsigned kPolls = 1u << 22;

// one counter: arrive (release add), poll, depart (the last resets)
template <int FENCE>
__global__ __launch_bounds__(256, 1) void barrier_one(unsigned *sync, long long *t, int nb) {
    __shared__ float pad[150 * 1024 / 4];    // one block per compute unit
    pad[threadIdx.x] = (float)threadIdx.x;
    const long long t0 = wall_clock64();
    __syncthreads();
    if (threadIdx.x == 0) {
        if (FENCE) __threadfence();
        __hip_atomic_fetch_add(sync, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        unsigned polls = 0;
        while (__hip_atomic_load(sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (unsigned)nb) {
            __builtin_amdgcn_s_sleep(1);
            if (++polls >= kPolls) {
                __hip_atomic_store(sync + 1152, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
        if (FENCE) __threadfence();
        const long long t1 = wall_clock64();
        const unsigned done = __hip_atomic_fetch_add(sync + 64, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (done == (unsigned)nb - 1) {
            __hip_atomic_store(sync, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(sync + 64, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        t[3 * blockIdx.x] = t0;
        t[3 * blockIdx.x + 1] = t1;
        t[3 * blockIdx.x + 2] = wall_clock64();
    }
    if (pad[(threadIdx.x + 1) & 255] < -1.f) t[0] = 0;
}

// eight group counters (blockIdx % 8), a top counter and per-group
// sense-reversing flags: no departure phase
template <int FENCE>
__global__ __launch_bounds__(256, 1) void barrier_tree(unsigned *sync, long long *t, int nb) {
    __shared__ float pad[150 * 1024 / 4];
    pad[threadIdx.x] = (float)threadIdx.x;
    const long long t0 = wall_clock64();
    __syncthreads();
    if (threadIdx.x == 0) {
        constexpr int kGroups = 8;
        const int g = blockIdx.x % kGroups;
        const unsigned ng = (unsigned)((nb - g + kGroups - 1) / kGroups);
        unsigned *flag = sync + 576 + 64 * g;
        const unsigned sense = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (FENCE) __threadfence();
        const unsigned old = __hip_atomic_fetch_add(sync + 64 * g, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (old == ng - 1) {
            __hip_atomic_store(sync + 64 * g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const unsigned o2 = __hip_atomic_fetch_add(sync + 512, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            if (o2 == (unsigned)std::min(nb, kGroups) - 1) {
                __hip_atomic_store(sync + 512, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                for (int k = 0; k < kGroups; ++k)
                    __hip_atomic_store(sync + 576 + 64 * k, sense ^ 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        unsigned polls = 0;
        while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == sense) {
            __builtin_amdgcn_s_sleep(1);
            if (++polls >= kPolls) {
                __hip_atomic_store(sync + 1152, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
        if (FENCE) __threadfence();
        t[3 * blockIdx.x] = t0;
        t[3 * blockIdx.x + 1] = wall_clock64();
        t[3 * blockIdx.x + 2] = t[3 * blockIdx.x + 1];
    }
    if (pad[(threadIdx.x + 1) & 255] < -1.f) t[0] = 0;
}

template <typename K>
static void run_barrier(const char *what, K kernel, int nb, unsigned *sync, long long *t, int rate) {
    float ms = 0.f;
    std::vector<long long> h(3 * nb);
    for (int rep = 0; rep < 4; ++rep) {
        hipEvent_t e0, e1;
        CHECK(hipEventCreate(&e0));
        CHECK(hipEventCreate(&e1));
        CHECK(hipEventRecord(e0));
        hipLaunchKernelGGL(kernel, dim3(nb), dim3(256), 0, 0, sync, t, nb);
        CHECK(hipGetLastError());
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        CHECK(hipEventElapsedTime(&ms, e0, e1));
    }
    CHECK(hipMemcpy(h.data(), t, h.size() * sizeof(long long), hipMemcpyDeviceToHost));
    unsigned err = 0;
    CHECK(hipMemcpy(&err, sync + 1152, 4, hipMemcpyDeviceToHost));
    long long st = h[0], wait = 0, dep = 0;
    for (int b = 0; b < nb; ++b) st = std::min(st, h[3 * b]);
    for (int b = 0; b < nb; ++b) {
        wait = std::max(wait, h[3 * b + 1] - st);
        dep = std::max(dep, h[3 * b + 2] - st);
    }
    const double us = 1e3 / rate;
    std::printf("| %s | %d | %.2f | %.2f | %.2f | %s |\n", what, nb, ms * 1e3, wait * us, dep * us,
                err ? "gave up" : "ok");
}

int main() {
    int rate = 0, cus = 0;
    CHECK(hipDeviceGetAttribute(&rate, hipDeviceAttributeWallClockRate, 0));
    CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
    std::printf("compute units %d, wall clock %d kHz\n\n", cus, rate);
    float *out;
    long long *cyc;
    unsigned *sync;
    CHECK(hipMalloc(&out, 256 * 512 * sizeof(float)));
    CHECK(hipMalloc(&cyc, 3 * 256 * sizeof(long long)));
    CHECK(hipMalloc(&sync, 8192));
    CHECK(hipMemset(sync, 0, 8192));

    std::printf("MFMA / VALU co-issue, 256 blocks (one per compute unit); a step = one 32x32x16 bf16 MFMA and/or 8 VALU "
                "operations; shader cycles per step per wave\n\n");
    std::printf("| work per step | waves per SIMD | kernel ms | cycles per step |\n|---|---|---|---|\n");
    run_coissue<CHAIN1>("1 MFMA, one dependent chain", 256, out, cyc);
    run_coissue<CHAIN4>("1 MFMA, four independent chains", 256, out, cyc);
    run_coissue<FMA8>("8 FMA", 256, out, cyc);
    run_coissue<EXP8>("8 exp2", 256, out, cyc);
    run_coissue<CHAIN_FMA2>("1 MFMA + 2 FMA, same wave", 256, out, cyc);
    run_coissue<CHAIN_FMA4>("1 MFMA + 4 FMA, same wave", 256, out, cyc);
    run_coissue<CHAIN_FMA8>("1 MFMA + 8 FMA, same wave", 256, out, cyc);
    run_coissue<CHAIN_EXP8>("1 MFMA + 8 exp2, same wave", 256, out, cyc);
    run_coissue<CHAIN4>("1 MFMA (four chains), two waves", 512, out, cyc);
    run_coissue<FMA8>("8 FMA, two waves", 512, out, cyc);
    run_coissue<PAIR_FMA>("one wave 8 FMA, the other 1 MFMA", 512, out, cyc);
    run_coissue<PAIR_EXP>("one wave 8 exp2, the other 1 MFMA", 512, out, cyc);

    std::printf("\nGrid barrier, 256-thread blocks at one per compute unit; times from the first block's start "
                "(wall clock), the kernel by events\n\n");
    std::printf("| barrier | blocks | kernel us | last wait ends us | last departure us | waits |\n"
                "|---|---|---|---|---|---|\n");
    for (int nb : {64, 128, 212, 256}) {
        if (nb > cus) continue;
        run_barrier("one counter, fences", barrier_one<1>, nb, sync, cyc, rate);
        run_barrier("one counter, no fences", barrier_one<0>, nb, sync, cyc, rate);
        run_barrier("8 groups + flags, fences", barrier_tree<1>, nb, sync, cyc, rate);
        run_barrier("8 groups + flags, no fences", barrier_tree<0>, nb, sync, cyc, rate);
    }
    return 0;
}
