// The attainable HBM read bandwidth of this device: the streaming pattern of the GEMM
// kernels (persistent blocks, one per CU; each wave reads its contiguous share of a
// 160 KiB chunk, the size of one FC13 item, with five 1 KiB loads in flight, buffer
// loads with the weight stream's non-temporal policy) without their arithmetic.  It
// gives the measured ceiling the kernels are compared with, beside the data-sheet peak.
#pragma once

#include <stdint.h>

#include "layout.hpp"

namespace moe {

constexpr int kReadThreads = 512;
constexpr uint32_t kReadChunk = 160 * 1024;
constexpr int kReadUnroll = 5;
constexpr uint32_t kReadPerWave = kReadChunk / (kReadThreads / 64);
static_assert(kReadPerWave % (kReadUnroll * 1024) == 0, "whole rounds of loads per wave");

// Reads bytes (a multiple of 16) from p; a thread writes sink[0] only if the XOR of the
// words it read equals a fixed value, so the loads cannot be dropped.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint8_t* __restrict__ p, uint64_t bytes,
                                                                   uint32_t* sink) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint64_t nchunks = bytes / kReadChunk;
    uint32_t acc = 0;
    for (uint64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const BufRes r = make_res(p + c * kReadChunk, kReadChunk);
        const uint32_t base = (uint32_t)wave * kReadPerWave + lane * 16;
        for (uint32_t off = 0; off < kReadPerWave; off += kReadUnroll * 1024) {
            uint4 v[kReadUnroll];
#pragma unroll
            for (int u = 0; u < kReadUnroll; ++u) v[u] = buf_ld16_stream(r, base + off + u * 1024);
#pragma unroll
            for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        }
    }
    // the bytes past the last whole chunk, 16 at a time
    const uint64_t tail0 = nchunks * kReadChunk;
    for (uint64_t i = tail0 + ((uint64_t)blockIdx.x * kReadThreads + threadIdx.x) * 16; i < bytes;
         i += (uint64_t)gridDim.x * kReadThreads * 16) {
        const uint4 v = *reinterpret_cast<const uint4*>(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace moe
