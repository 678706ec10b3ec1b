// Device helpers shared by the gfx950 kernels: wave64 / workgroup reductions, bf16
// unpacking, order-preserving keys. Wavefronts are 64 lanes wide on CDNA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define SD_DEV __device__ __forceinline__

namespace sd {

// The tree walk's clamp on a residual mass (its residual chain is formed from fp32
// exponentials): at or below 2^-20 the replacement is drawn from the distribution the
// child was tested against, flagged. Target and draft rows that agree leave only rounding
// noise in p - q, about 2^-22 of p per token there, so a smaller mass is not resolved.
constexpr double kResidFloor = 0x1p-20;

constexpr int kWave = 64;

SD_DEV float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
SD_DEV float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
SD_DEV float bf16_at(const uint16_t* p, long i) { return __uint_as_float(uint32_t(p[i]) << 16); }

SD_DEV float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}
SD_DEV double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
SD_DEV unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
SD_DEV int wave_sum_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
SD_DEV int wave_min_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
    return v;
}
SD_DEV int wave_max_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
    return v;
}

// Workgroup reductions through LDS; every thread gets the result. `red` must hold
// NT / 64 entries; all threads of the workgroup must call.
template <int NT>
SD_DEV float block_max(float v, float* red) {
    v = wave_max(v);
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    if (l == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < NT / kWave; ++i) r = fmaxf(r, red[i]);
    __syncthreads();
    return r;
}
// Sum in a fixed order (lane tree, then waves in index order): deterministic.
template <int NT>
SD_DEV double block_sum(double v, double* red) {
    v = wave_sum(v);
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    if (l == 0) red[w] = v;
    __syncthreads();
    double r = red[0];
#pragma unroll
    for (int i = 1; i < NT / kWave; ++i) r += red[i];
    __syncthreads();
    return r;
}
template <int NT>
SD_DEV int block_sum_i(int v, int* red) {
    v = wave_sum_i(v);
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    if (l == 0) red[w] = v;
    __syncthreads();
    int r = 0;
#pragma unroll
    for (int i = 0; i < NT / kWave; ++i) r += red[i];
    __syncthreads();
    return r;
}
template <int NT>
SD_DEV int block_min_i(int v, int* red) {
    v = wave_min_i(v);
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    if (l == 0) red[w] = v;
    __syncthreads();
    int r = red[0];
#pragma unroll
    for (int i = 1; i < NT / kWave; ++i) r = min(r, red[i]);
    __syncthreads();
    return r;
}
template <int NT>
SD_DEV int block_max_i(int v, int* red) {
    v = wave_max_i(v);
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    if (l == 0) red[w] = v;
    __syncthreads();
    int r = red[0];
#pragma unroll
    for (int i = 1; i < NT / kWave; ++i) r = max(r, red[i]);
    __syncthreads();
    return r;
}

// Exclusive prefix sum over the workgroup (integers). `red` holds NT / 64 + 1 ints.
// Returns this thread's exclusive prefix; *total receives the sum.
template <int NT>
SD_DEV int block_excl_scan_i(int v, int* red, int* total) {
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    int x = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int y = __shfl_up(x, o, kWave);
        if (l >= o) x += y;
    }
    if (l == kWave - 1) red[w] = x;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / kWave; ++i) {
        if (i < w) base += red[i];
        tot += red[i];
    }
    __syncthreads();
    *total = tot;
    return base + x - v;
}
// Exclusive prefix sum of doubles in a fixed association order: lane-inclusive scan in
// the wave, exclusive value taken from the lane below, wave totals added in index order.
// `red` holds NT / 64 doubles. *total receives the workgroup sum.
template <int NT>
SD_DEV double block_excl_scan_d(double v, double* red, double* total) {
    const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
    double x = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        double y = __shfl_up(x, o, kWave);
        if (l >= o) x += y;
    }
    double ex = __shfl_up(x, 1, kWave);
    if (l == 0) ex = 0.0;
    if (l == kWave - 1) red[w] = x;
    __syncthreads();
    double base = 0.0, tot = 0.0;
#pragma unroll
    for (int i = 0; i < NT / kWave; ++i) {
        if (i < w) base += red[i];
        tot += red[i];
    }
    __syncthreads();
    *total = tot;
    return base + ex;
}

}  // namespace sd
