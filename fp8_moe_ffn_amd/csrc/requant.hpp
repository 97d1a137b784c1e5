// Stage 3 of the forward: per-row FP8 re-quantisation of the SwiGLU intermediate.
//
// The pages quantise a kernel's result to FP8 before it feeds the next GEMM (Blackwell
// 1,000 TPS/user blog, zh translation, section "CUDA kernel optimisation and fusion",
// item "operator fusion").  The scale s_a = fp32(amax / 448) of a row needs the amax
// over the whole intermediate row; each FC13 block left its own per-row maxima, so a
// block here first takes the max over them, and the encoding runs once, after FC13;
// FC2 reads finished codes.  Rows: shared
// rows [0, M), routed rows [M, 2M) (none when E == 0).  Codes come from the float32
// intermediate (never a bf16 copy): aq = e4m3(a / s_a), 0 when amax == 0.
#pragma once

#include "codec.hpp"
#include "params.hpp"

namespace moe {

constexpr int kRequantThreads = 256;
constexpr int kRequantCols = kRequantThreads * 4;  // intermediate columns per block

// Grid: (active rows) x ceil(I / 1024) blocks; thread t encodes 4 consecutive columns.
__host__ __device__ inline int requant_blocks_per_row(int I) {
    return (I + kRequantCols - 1) / kRequantCols;
}

__global__ __launch_bounds__(kRequantThreads) void requant_kernel(const FwdParams p) {
    const int per_row = requant_blocks_per_row(p.I);
    const int row = blockIdx.x / per_row;
    const int col = (blockIdx.x - row * per_row) * kRequantCols + threadIdx.x * 4;
    const RouteLayout rl{p.T, p.S};
    // the row's values first (in bounds: columns of the last block clamp to the row end),
    // so that their latency overlaps the reduction below
    const float4 v = *reinterpret_cast<const float4*>(p.ws.a + (size_t)row * p.I + min(col, p.I - 4));
    // max |a| of the row over the FC13 blocks' maxima (non-negative floats: compare bits)
    __shared__ uint32_t red[kRequantThreads / 64];
    uint32_t m = 0;
    for (int b = threadIdx.x; b < p.grid13; b += kRequantThreads)
        m = max(m, p.ws.amax[(size_t)b * 2 * p.T + row]);
    for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    if (col >= p.I) return;  // I is a multiple of 128, so a thread's 4 columns are all in
    const float s = __uint_as_float(m) / kE4M3Max;  // IEEE division: fp32(amax / 448)
    uint32_t packed = 0;
    if (s > 0.0f) {
        const float r = 1.0f / s;
        packed = e4m3_quant2(v.x, v.y, s, r) | (e4m3_quant2(v.z, v.w, s, r) << 16);
    }
    *reinterpret_cast<uint32_t*>(p.ws.aq + (size_t)row * p.I + col) = packed;
    if (col == 0) p.ws.sa[row] = s;

    // debug copies, indexed by token: shared rows [0, M), routed rows by their token
    uint8_t* qd = row < p.M ? p.dbg.aq_shared : p.dbg.aq_routed;
    float* sd = row < p.M ? p.dbg.sa_shared : p.dbg.sa_routed;
    if (qd || sd) {
        const int tok = row < p.M ? row : p.ws.route[rl.row_token() + row];
        if (qd) *reinterpret_cast<uint32_t*>(qd + (size_t)tok * p.I + col) = packed;
        if (sd && col == 0) sd[tok] = s;
    }
}

}  // namespace moe
