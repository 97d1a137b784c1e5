// Offline weight prepack: a pure permutation of the e4m3 codes of one expert into
// the operand-block order of layout.hpp.  The pages reorder GEMM weights into a
// swizzled format ahead of time so that the matrix unit's data is laid out well
// (Blackwell 1,000 TPS/user blog, zh translation, section "CUDA kernel optimisation
// and fusion", item "GEMM weight swizzle"); on gfx950 the aim is that each lane's
// operand bytes are one contiguous 16-byte load and each wave instruction reads
// 1 KiB of consecutive memory.
//
// One thread per 16-byte chunk of the packed array: it gathers 16 codes that are
// consecutive in the reduction index (a strided column walk in the row-major input).
// The unpack kernels apply the inverse map, for round-trip tests.
#pragma once

#include "codec.hpp"
#include "layout.hpp"

namespace moe {

// packed chunk c (16 bytes) -> (row-major [R][C] source row of byte 0, column)
// FC13: source w13 [K][2I]; FC2: source w2 [I][K].
struct ChunkCoord {
    uint64_t row;  // reduction index of byte 0 (bytes j = 0..15 are rows row + j)
    uint64_t col;  // output channel
};

__device__ __forceinline__ ChunkCoord fc13_chunk(uint64_t c, int K, int I) {
    const uint64_t ksteps = (uint64_t)(K >> 7);
    const uint64_t blk = c >> 7, within = c & 127u;
    const uint32_t half = (uint32_t)(within >> 6), lane = (uint32_t)(within & 63u);
    const uint64_t u = blk & 1u, t = blk >> 1;
    const uint64_t kstep = t % ksteps, pair = t / ksteps;
    ChunkCoord cc;
    cc.col = u * (uint64_t)I + pair * 16u + (lane & 15u);
    cc.row = kstep * kKStep + 32u * (lane >> 4) + 16u * half;
    return cc;
}

__device__ __forceinline__ ChunkCoord fc2_chunk(uint64_t c, int K, int I) {
    const uint64_t ksteps = (uint64_t)(I >> 7);
    const uint64_t blk = c >> 7, within = c & 127u;
    const uint32_t half = (uint32_t)(within >> 6), lane = (uint32_t)(within & 63u);
    const uint64_t sub = blk % kFc2Sub, t = blk / kFc2Sub;
    const uint64_t kstep = t % ksteps, ctile = t / ksteps;
    ChunkCoord cc;
    cc.col = ctile * kFc2Cols + sub * 16u + (lane & 15u);
    cc.row = kstep * kKStep + 32u * (lane >> 4) + 16u * half;
    return cc;
}

template <bool FC13>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ src,
                                                   uint8_t* __restrict__ dst, int K, int I) {
    const uint64_t nchunks = (uint64_t)K * I * (FC13 ? 2u : 1u) / 16u;
    const uint64_t ncols = FC13 ? 2u * (uint64_t)I : (uint64_t)K;
    for (uint64_t c = (uint64_t)blockIdx.x * 256 + threadIdx.x; c < nchunks;
         c += (uint64_t)gridDim.x * 256) {
        const ChunkCoord cc = FC13 ? fc13_chunk(c, K, I) : fc2_chunk(c, K, I);
        uint32_t v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t word = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                word |= (uint32_t)src[(cc.row + q * 4 + j) * ncols + cc.col] << (8 * j);
            v[q] = word;
        }
        *reinterpret_cast<uint4*>(dst + c * 16) = make_uint4(v[0], v[1], v[2], v[3]);
    }
}

template <bool FC13>
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t* __restrict__ src,
                                                     uint8_t* __restrict__ dst, int K, int I) {
    const uint64_t nchunks = (uint64_t)K * I * (FC13 ? 2u : 1u) / 16u;
    const uint64_t ncols = FC13 ? 2u * (uint64_t)I : (uint64_t)K;
    for (uint64_t c = (uint64_t)blockIdx.x * 256 + threadIdx.x; c < nchunks;
         c += (uint64_t)gridDim.x * 256) {
        const ChunkCoord cc = FC13 ? fc13_chunk(c, K, I) : fc2_chunk(c, K, I);
        const uint4 v = *reinterpret_cast<const uint4*>(src + c * 16);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                dst[(cc.row + q * 4 + j) * ncols + cc.col] = (uint8_t)(w[q] >> (8 * j));
    }
}

__global__ __launch_bounds__(256) void encode_kernel(const float* in, uint8_t* out, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        out[i] = (uint8_t)e4m3_encode(in[i], 0);
}

// Pairs (2i, 2i + 1); an odd tail pairs the last element with itself.
__global__ __launch_bounds__(256) void quantize_kernel(const float* in, float s, uint8_t* out, int64_t n) {
    const float r = s < kTinyScale ? 0.0f : 1.0f / s;  // unused below kTinyScale
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; 2 * i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t j = min(2 * i + 1, n - 1);
        const uint32_t c = e4m3_quant2(in[2 * i], in[j], s, r);
        out[2 * i] = (uint8_t)c;
        if (j != 2 * i) out[j] = (uint8_t)(c >> 8);
    }
}

__global__ __launch_bounds__(256) void decode_kernel(const uint8_t* in, float* out, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        out[i] = e4m3_decode(in[i]);
}

}  // namespace moe
