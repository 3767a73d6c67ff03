// Measurement probes, kept out of the indexer's C ABI (their own library,
// loaded by the benchmark only): what this GPU sustains on a plain read of
// device memory, on a gather of scattered rows and on back-to-back
// matrix-core instructions, as measured ceilings beside the datasheet peaks
// the kernels' roofline fractions use.
#include <hip/hip_runtime.h>

#include "device_common.h"

#include <cstdint>

namespace {

using namespace ds4idx;

// Every 16-byte word of p read once, grid-stride, four loads in flight per
// lane; each thread XOR-folds what it read into sink[thread], so no load can
// be dropped and the caller can check that every word was read once.
__global__ __launch_bounds__(512) void read_kernel(const uint4 *__restrict__ p, long long n16,
                                                   uint32_t *__restrict__ sink)
{
    const long long stride = (long long)gridDim.x * blockDim.x;
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    long long i = t;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
    }
    for (; i < n16; i += stride) {
        const uint4 a = p[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    sink[t] = acc;
}

// rows[idx[i]] (row16 16-byte pieces, at most 128) for every i < n with
// 0 <= idx[i] < nrows, gathered the way the sparse attention gathers its
// rows: straight into LDS (global_load_lds_dwordx4), one instruction per
// 1 KB of a row, from a wavefront-uniform row base. Block b takes the
// indices [b n / grid, (b + 1) n / grid); each wavefront loads 64 of them at
// once (one per lane) and gathers their rows eight at a time into its own
// LDS slots, then reads its pieces back and XOR-folds them into
// sink[thread], so every gathered word is counted once.
constexpr int GROWS = 8;  // rows in flight per wavefront
__global__ __launch_bounds__(512) void gather_kernel(const uint4 *__restrict__ rows, int row16, long long nrows,
                                                     const int *__restrict__ idx, long long n,
                                                     uint32_t *__restrict__ sink)
{
    __shared__ uint4 slot[8][GROWS][128];
    const long long lo = (long long)blockIdx.x * n / gridDim.x, hi = (long long)(blockIdx.x + 1) * n / gridDim.x;
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    uint32_t acc = 0;
    for (long long g0 = lo + 64 * wid; g0 < hi; g0 += 64 * 8) {
        const int mine = g0 + lane < hi ? idx[g0 + lane] : -1;
        const int cnt = hi - g0 < 64 ? (int)(hi - g0) : 64;
        for (int u = 0; u < cnt; u += GROWS) {
            bool okj[GROWS];
#pragma unroll
            for (int j = 0; j < GROWS; ++j) {
                const int r = u + j < cnt ? __builtin_amdgcn_readlane(mine, u + j) : -1;
                okj[j] = r >= 0 && r < nrows;
                if (okj[j]) {
                    const uint4 *rb = uniform_ptr(rows + (long long)r * row16);
                    const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_addr(&slot[wid][j][0]));
                    if (lane < row16) gather16_at(rb, (uint32_t)lane * 16, l0);
                    if (64 + lane < row16) gather16_at(rb, (uint32_t)(64 + lane) * 16, l0 + 1024);
                }
            }
            wait_vm<0>();
#pragma unroll
            for (int j = 0; j < GROWS; ++j) {
                if (okj[j]) {
                    uint4 a = lane < row16 ? slot[wid][j][lane] : make_uint4(0, 0, 0, 0);
                    uint4 c = 64 + lane < row16 ? slot[wid][j][64 + lane] : make_uint4(0, 0, 0, 0);
                    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ c.x ^ c.y ^ c.z ^ c.w;
                }
            }
            // the slots are refilled only after these reads
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        }
    }
    sink[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

// Four independent accumulator chains of v_mfma_f32_32x32x16_bf16 per
// wavefront on register operands: 4 x 32768 flop per iteration.
__global__ __launch_bounds__(256) void mfma_kernel(int iters, float *__restrict__ sink)
{
    const int tid = threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (short)(0x3f80 + ((tid + j) & 7));  // bf16 values near 1, not known to the compiler
        b[j] = (short)(0x3f80 + ((tid * 3 + j) & 7));
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
    sink[blockIdx.x * blockDim.x + tid] = s;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16, 16-byte aligned) at `buf` with `blocks`
// workgroups of 512 threads; sink holds blocks * 512 words. Returns a
// hipError_t value (0 = launched).
int ds4probe_hbm_read(const void *buf, long long bytes, uint32_t *sink, int blocks, void *stream)
{
    if (!buf || !sink || bytes <= 0 || (bytes & 15) || ((uintptr_t)buf & 15) || blocks < 1)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(512), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4 *>(buf), bytes / 16, sink);
    return (int)hipGetLastError();
}

// Gathers rows[idx[i]] (row_bytes each: a multiple of 16, at most 2048;
// rows 16-byte aligned) for the n indices at idx, skipping those outside
// [0, nrows), with `blocks` workgroups of 512 threads; sink holds
// blocks * 512 words. Returns a hipError_t value (0 = launched).
int ds4probe_gather(const void *rows, int row_bytes, long long nrows, const int *idx, long long n, uint32_t *sink,
                    int blocks, void *stream)
{
    if (!rows || !idx || !sink || row_bytes < 16 || row_bytes > 2048 || (row_bytes & 15) || ((uintptr_t)rows & 15) ||
        nrows < 1 || n < 1 || blocks < 1)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(gather_kernel, dim3(blocks), dim3(512), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4 *>(rows), row_bytes / 16, nrows, idx, n, sink);
    return (int)hipGetLastError();
}

// `blocks` workgroups of 256 threads, each wavefront issuing 4 * iters
// 32x32x16 bf16 MFMAs (32768 flop each); sink holds blocks * 256 floats.
int ds4probe_mfma(int iters, int blocks, float *sink, void *stream)
{
    if (!sink || iters < 1 || blocks < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters, sink);
    return (int)hipGetLastError();
}

}  // extern "C"
