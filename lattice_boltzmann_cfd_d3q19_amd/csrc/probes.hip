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
//                     its arithmetic (19 coalesced planes read and written
//                     per cell, in place), with 1, 2 or 4 cells per work-item.
//   probe_swap19_blocked  the same swap in the compact layout's store: cells in
//                     blocks of 64, each block holding its 19 planes side by
//                     side (value q of cell i at (i / 64) * 19 * 64 + q * 64 +
//                     i % 64), one cell per work-item.
// Both move 2 bytes per byte of payload (one read, one write).  `nt` selects
// nontemporal loads and stores (streaming data that is not reused).
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

constexpr int kBlock = 256;

// PER 16-byte elements per work-item, the workgroup's elements contiguous
// per round (work-item t takes elements base + t + k * kBlock).
template <bool NT, int PER>
__global__ __launch_bounds__(kBlock) void copy_f4_kernel(const float4* __restrict__ src, float4* __restrict__ dst,
                                                          size_t n) {
    const size_t base = (size_t)blockIdx.x * kBlock * PER + threadIdx.x;
    float4 v[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
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
    for (int k = 0; k < PER; ++k) {
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

template <bool NT, int PER>
int launch_copy(const void* src, void* dst, size_t n, size_t lds, void* stream) {
    const size_t per = (size_t)kBlock * PER;
    const dim3 grid((unsigned)((n + per - 1) / per));
    copy_f4_kernel<NT, PER><<<grid, kBlock, lds, (hipStream_t)stream>>>((const float4*)src, (float4*)dst, n);
    return (int)hipGetLastError();
}

// PER consecutive cells per work-item, each plane's PER values in one
// PER * 4-byte access (PER = 1, 2, 4).
template <bool NT, int PER>
__global__ __launch_bounds__(kBlock) void swap19_kernel(float* __restrict__ buf, size_t stride, size_t n) {
    typedef float vec __attribute__((ext_vector_type(PER == 1 ? 2 : PER), aligned(4 * PER)));
    const size_t i = ((size_t)blockIdx.x * kBlock + threadIdx.x) * PER;
    if (i >= n) return;
    if constexpr (PER == 1) {
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
    } else {
        vec v[19];
#pragma unroll
        for (int q = 0; q < 19; ++q) {
            const vec* p = (const vec*)&buf[q * stride + i];
            v[q] = NT ? __builtin_nontemporal_load(p) : *p;
        }
#pragma unroll
        for (int q = 0; q < 19; ++q) {
            vec* p = (vec*)&buf[(18 - q) * stride + i];
            if (NT)
                __builtin_nontemporal_store(v[q], p);
            else
                *p = v[q];
        }
    }
}

template <bool NT, int PER>
int launch_swap(void* buf, size_t stride, size_t n, size_t lds, void* stream) {
    const size_t cells = (size_t)kBlock * PER;
    const dim3 grid((unsigned)((n + cells - 1) / cells));
    swap19_kernel<NT, PER><<<grid, kBlock, lds, (hipStream_t)stream>>>((float*)buf, stride, n);
    return (int)hipGetLastError();
}

template <bool NT>
__global__ __launch_bounds__(kBlock) void swap19_blocked_kernel(float* __restrict__ buf, size_t n) {
    const size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= n) return;
    const size_t base = (i / 64) * (19 * 64) + i % 64;
    float v[19];
#pragma unroll
    for (int q = 0; q < 19; ++q) v[q] = NT ? __builtin_nontemporal_load(&buf[base + q * 64]) : buf[base + q * 64];
#pragma unroll
    for (int q = 0; q < 19; ++q) {
        if (NT)
            __builtin_nontemporal_store(v[q], &buf[base + (18 - q) * 64]);
        else
            buf[base + (18 - q) * 64] = v[q];
    }
}

}  // namespace

extern "C" {

// 0 on success, else the hipError_t of the launch.  n = 16-byte elements;
// src and dst device pointers, 16-byte aligned, not overlapping.  per: 16-byte
// elements per work-item, 1, 2, 4 or 8 (other values: hipErrorInvalidValue).
// lds: bytes of LDS reserved per workgroup and not used (caps the workgroups
// a CU holds at once; at most 160 KiB).
int probe_copy_f4(const void* src, void* dst, size_t n, int nontemporal, int per, size_t lds, void* stream) {
    if (n == 0) return 0;
    if (lds > 160 * 1024) return (int)hipErrorInvalidValue;
    switch (per * 2 + (nontemporal ? 1 : 0)) {
    case 2: return launch_copy<false, 1>(src, dst, n, lds, stream);
    case 3: return launch_copy<true, 1>(src, dst, n, lds, stream);
    case 4: return launch_copy<false, 2>(src, dst, n, lds, stream);
    case 5: return launch_copy<true, 2>(src, dst, n, lds, stream);
    case 8: return launch_copy<false, 4>(src, dst, n, lds, stream);
    case 9: return launch_copy<true, 4>(src, dst, n, lds, stream);
    case 16: return launch_copy<false, 8>(src, dst, n, lds, stream);
    case 17: return launch_copy<true, 8>(src, dst, n, lds, stream);
    default: return (int)hipErrorInvalidValue;
    }
}

// buf: device float[19 * stride], stride >= n.  per: cells per work-item,
// 1, 2 or 4; for 2 and 4, n and stride must be multiples of per (else
// hipErrorInvalidValue) and buf 4 * per-byte aligned.  lds as for the copy.
int probe_swap19(void* buf, size_t stride, size_t n, int nontemporal, int per, size_t lds, void* stream) {
    if (n == 0) return 0;
    if (stride < n || per < 1 || n % per || stride % per || lds > 160 * 1024) return (int)hipErrorInvalidValue;
    switch (per * 2 + (nontemporal ? 1 : 0)) {
    case 2: return launch_swap<false, 1>(buf, stride, n, lds, stream);
    case 3: return launch_swap<true, 1>(buf, stride, n, lds, stream);
    case 4: return launch_swap<false, 2>(buf, stride, n, lds, stream);
    case 5: return launch_swap<true, 2>(buf, stride, n, lds, stream);
    case 8: return launch_swap<false, 4>(buf, stride, n, lds, stream);
    case 9: return launch_swap<true, 4>(buf, stride, n, lds, stream);
    default: return (int)hipErrorInvalidValue;
    }
}

// buf: device float[19 * roundup(n, 64)].  lds as for the copy.
int probe_swap19_blocked(void* buf, size_t n, int nontemporal, size_t lds, void* stream) {
    if (n == 0) return 0;
    if (lds > 160 * 1024) return (int)hipErrorInvalidValue;
    const dim3 grid((unsigned)((n + kBlock - 1) / kBlock));
    if (nontemporal)
        swap19_blocked_kernel<true><<<grid, kBlock, lds, (hipStream_t)stream>>>((float*)buf, n);
    else
        swap19_blocked_kernel<false><<<grid, kBlock, lds, (hipStream_t)stream>>>((float*)buf, n);
    return (int)hipGetLastError();
}

}  // extern "C"
