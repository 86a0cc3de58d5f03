// probes.hip -- bandwidth probes that measure the practical HBM ceilings the
// step kernels are compared with (libprobes.so, loaded by the benchmark only;
// not part of the lattice library).
//
//   probe_copy_f4     dst[i] = src[i] over n 16-byte elements: the plainest
//                     fully coalesced streaming pattern (one 16-byte load and
//                     one 16-byte store per lane and element).
//   probe_swap19      for every cell i < n: the 19 values at q * stride + i
//                     are read and written back at (18 - q) * stride + i, the
//                     access pattern of the in-place (AA) even step without
//                     its arithmetic (19 coalesced 4-byte planes read and
//                     written per cell, in place).
// Both move 2 bytes per byte of payload (one read, one write).  `nt` selects
// nontemporal loads and stores (streaming data that is not reused).
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

constexpr int kBlock = 256;
constexpr int kPerThread = 4;

template <bool NT>
__global__ __launch_bounds__(kBlock) void copy_f4_kernel(const float4* __restrict__ src, float4* __restrict__ dst,
                                                          size_t n) {
    const size_t base = (size_t)blockIdx.x * kBlock * kPerThread + threadIdx.x;
    float4 v[kPerThread];
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const size_t i = base + (size_t)k * kBlock;
        if (i < n) {
            if (NT) {
                v[k].x = __builtin_nontemporal_load(&src[i].x);
                v[k].y = __builtin_nontemporal_load(&src[i].y);
                v[k].z = __builtin_nontemporal_load(&src[i].z);
                v[k].w = __builtin_nontemporal_load(&src[i].w);
            } else {
                v[k] = src[i];
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const size_t i = base + (size_t)k * kBlock;
        if (i < n) {
            if (NT) {
                __builtin_nontemporal_store(v[k].x, &dst[i].x);
                __builtin_nontemporal_store(v[k].y, &dst[i].y);
                __builtin_nontemporal_store(v[k].z, &dst[i].z);
                __builtin_nontemporal_store(v[k].w, &dst[i].w);
            } else {
                dst[i] = v[k];
            }
        }
    }
}

template <bool NT>
__global__ __launch_bounds__(kBlock) void swap19_kernel(float* __restrict__ buf, size_t stride, size_t n) {
    const size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= n) return;
    float v[19];
#pragma unroll
    for (int q = 0; q < 19; ++q) v[q] = NT ? __builtin_nontemporal_load(&buf[q * stride + i]) : buf[q * stride + i];
#pragma unroll
    for (int q = 0; q < 19; ++q) {
        if (NT)
            __builtin_nontemporal_store(v[q], &buf[(18 - q) * stride + i]);
        else
            buf[(18 - q) * stride + i] = v[q];
    }
}

}  // namespace

extern "C" {

// 0 on success, else the hipError_t of the launch.  n = 16-byte elements;
// src and dst device pointers, 16-byte aligned, not overlapping.
int probe_copy_f4(const void* src, void* dst, size_t n, int nontemporal, void* stream) {
    if (n == 0) return 0;
    const size_t per = (size_t)kBlock * kPerThread;
    const dim3 grid((unsigned)((n + per - 1) / per));
    if (nontemporal)
        copy_f4_kernel<true><<<grid, kBlock, 0, (hipStream_t)stream>>>((const float4*)src, (float4*)dst, n);
    else
        copy_f4_kernel<false><<<grid, kBlock, 0, (hipStream_t)stream>>>((const float4*)src, (float4*)dst, n);
    return (int)hipGetLastError();
}

// buf: device float[19 * stride], stride >= n.
int probe_swap19(void* buf, size_t stride, size_t n, int nontemporal, void* stream) {
    if (n == 0) return 0;
    if (stride < n) return (int)hipErrorInvalidValue;
    const dim3 grid((unsigned)((n + kBlock - 1) / kBlock));
    if (nontemporal)
        swap19_kernel<true><<<grid, kBlock, 0, (hipStream_t)stream>>>((float*)buf, stride, n);
    else
        swap19_kernel<false><<<grid, kBlock, 0, (hipStream_t)stream>>>((float*)buf, stride, n);
    return (int)hipGetLastError();
}

}  // extern "C"
