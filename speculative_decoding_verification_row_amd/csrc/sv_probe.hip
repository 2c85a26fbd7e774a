// sv_probe.hip -- plain streaming-read kernels for MI355X (gfx950): the
// empirical ceiling of a single read pass over the same bytes the
// verification kernels read, reported beside their roofline as context (the
// target stays the published 8 TB/s).  No arithmetic beyond a sum that keeps
// the loads alive.
//
// Two launch shapes over one logical range made of two buffers (the target
// and the draft operands of a call):
//   one-shot    one block per 32 KB chunk (the shape of the verification
//               grid's blocks), 256 threads, eight 16-byte loads per thread
//               in flight together;
//   persistent  a fixed grid (blocks_per_cu x 256 CUs) in which block j reads
//               chunks j, j + G, j + 2G, ..., the next chunk's loads issued
//               before the current one is summed.
// Loads use the non-temporal cache policy of the verification kernels.  Each
// block writes one float (its sum) to `out`, which must hold one float per
// block of the launch.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "sv_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kVec = 8;                               // 16-byte loads per thread per chunk
constexpr int64_t kChunkBytes = kThreads * kVec * 16;  // 32 KB
constexpr int kNonTemporal = 2;
constexpr int kRsrcWord3 = 0x00020000;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct Range {
    const unsigned char* b0;
    const unsigned char* b1;
    int64_t n0, n1;        // chunks in each buffer (the last may be partial)
    int64_t bytes0, bytes1;
};

__device__ __forceinline__ float sum4(u32x4 v)
{
    return (__uint_as_float(v.x) + __uint_as_float(v.y)) + (__uint_as_float(v.z) + __uint_as_float(v.w));
}

// Loads of logical chunk k (buffer 0, then buffer 1); bytes past a buffer's
// end read as 0 through the buffer resource's range check.
__device__ __forceinline__ void load_chunk(const Range& r, int64_t k, u32x4 (&v)[kVec])
{
    const bool first = k < r.n0;
    const unsigned char* base = first ? r.b0 + k * kChunkBytes : r.b1 + (k - r.n0) * kChunkBytes;
    const int64_t left = (first ? r.bytes0 - k * kChunkBytes : r.bytes1 - (k - r.n0) * kChunkBytes);
    const int range = left < kChunkBytes ? (int)left : (int)kChunkBytes;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(base), (short)0, range, kRsrcWord3);
#pragma unroll
    for (int j = 0; j < kVec; ++j)
        v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (j * kThreads + (int)threadIdx.x) * 16, 0, kNonTemporal);
}

__device__ __forceinline__ void write_sum(float s, float* out)
{
    __shared__ float part[kThreads / 64];
    for (int d = 32; d > 0; d >>= 1) s += __shfl_xor(s, d);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = (part[0] + part[1]) + (part[2] + part[3]);
}

__global__ __launch_bounds__(kThreads) void probe_oneshot(Range r, float* out)
{
    u32x4 v[kVec];
    load_chunk(r, blockIdx.x, v);
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kVec; ++j) s += sum4(v[j]);
    write_sum(s, out);
}

__global__ __launch_bounds__(kThreads) void probe_persistent(Range r, float* out)
{
    const int64_t n = r.n0 + r.n1, G = gridDim.x;
    float s = 0.0f;
    int64_t k = blockIdx.x;
    u32x4 v[kVec], w[kVec];
    if (k < n) load_chunk(r, k, v);
    while (k < n) {
        const int64_t nx = k + G;
        if (nx < n) load_chunk(r, nx, w);
#pragma unroll
        for (int j = 0; j < kVec; ++j) s += sum4(v[j]);
#pragma unroll
        for (int j = 0; j < kVec; ++j) v[j] = w[j];
        k = nx;
    }
    write_sum(s, out);
}

}  // namespace

extern "C" {

int64_t sv_probe_blocks(size_t bytes0, size_t bytes1, int32_t mode, int32_t blocks_per_cu)
{
    const int64_t n = (int64_t)((bytes0 + kChunkBytes - 1) / kChunkBytes + (bytes1 + kChunkBytes - 1) / kChunkBytes);
    if (mode == SV_PROBE_ONESHOT) return n;
    if (mode != SV_PROBE_PERSISTENT || blocks_per_cu < 1 || blocks_per_cu > 8) return -1;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return -1;
    const int64_t g = (int64_t)cus * blocks_per_cu;
    return g < n ? g : n;
}

int32_t sv_probe_read(const void* buf0, size_t bytes0, const void* buf1, size_t bytes1, int32_t mode,
                      int32_t blocks_per_cu, float* out, void* stream)
{
    if (!buf0 || !out || (bytes1 && !buf1) || bytes0 == 0) return -1;
    if (((uintptr_t)buf0 | (uintptr_t)buf1) % 16 || bytes0 % 16 || bytes1 % 16) return -1;
    if (bytes0 > (size_t)1 << 40 || bytes1 > (size_t)1 << 40) return -1;
    const int64_t blocks = sv_probe_blocks(bytes0, bytes1, mode, blocks_per_cu);
    if (blocks < 1 || blocks > INT32_MAX) return -1;
    Range r{static_cast<const unsigned char*>(buf0), static_cast<const unsigned char*>(buf1),
            (int64_t)((bytes0 + kChunkBytes - 1) / kChunkBytes), (int64_t)((bytes1 + kChunkBytes - 1) / kChunkBytes),
            (int64_t)bytes0, (int64_t)bytes1};
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (mode == SV_PROBE_ONESHOT)
        hipLaunchKernelGGL(probe_oneshot, dim3((unsigned)blocks), dim3(kThreads), 0, s, r, out);
    else
        hipLaunchKernelGGL(probe_persistent, dim3((unsigned)blocks), dim3(kThreads), 0, s, r, out);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
