// Stage 2 of the forward: the FC13 GEMM (gate and up projections side by side)
// with SwiGLU applied in its epilogue, for the shared expert and every distinct
// routed expert.  The pages fuse SwiGLU into the GEMM in front of it (Blackwell
// 1,000 TPS/user blog, zh translation, section "CUDA kernel optimisation and
// fusion", item "operator fusion") and build low-latency GEMMs that load weights so
// as to use the whole HBM bandwidth (same section, item on spatial partitioning and
// efficient memory loads).
//
// gfx950 design: at M <= 16 tokens the GEMM is a weight stream, so each block owns
// one "pair" (16 gate + 16 up channels of one expert) over the whole hidden size
// K.  Its WAVES waves split K; each wave issues all 16-byte loads of its NSTEP
// k-steps at once (4 KiB per step, coalesced 1 KiB per instruction) and keeps them
// in registers, so occupancy rather than a software pipeline hides HBM latency.
// The tokens' codes are staged once per block in LDS; weights and tokens are widened
// exactly to f16 in registers and contracted with v_mfma_f32_16x16x32_f16 (tokens
// padded to 16 with zeros; layout.hpp says why not an e4m3-input instruction).  Partial sums are
// reduced over the waves in LDS; then the scales, SwiGLU and the mask of routed
// tokens are applied and the float32 intermediate plus its per-token amax are
// written.  The amax feeds the re-quantisation done by stage 3.
#pragma once

#include "codec.hpp"
#include "layout.hpp"
#include "params.hpp"

namespace moe {

__device__ __forceinline__ uint4 ld16(const uint8_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}

// B operand (tokens) of one k-step from a row-major [tokens][row_stride] LDS copy of
// the e4m3 codes, widened to f16; tokens M..15 are zero.
__device__ __forceinline__ Operand token_operand(const uint8_t* lds, int row_stride, int kstep,
                                                 int lane, int M) {
    const int tok = lane & 15;
    uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
    if (tok < M) {
        const uint8_t* src = lds + tok * row_stride + kstep * kKStep + (lane >> 4) * 32;
        lo = *reinterpret_cast<const uint4*>(src);
        hi = *reinterpret_cast<const uint4*>(src + 16);
    }
    return widen(lo, hi);
}

// LDS bytes needed by fc13_swiglu_kernel.
__host__ __device__ inline int fc13_lds_bytes(int waves, int M, int K) {
    const int xq = M * (K + 16);
    const int red = waves * 8 * 64 * 4;
    return xq > red ? xq : red;
}

template <int WAVES, int NSTEP>
__global__ __launch_bounds__(WAVES * 64) void fc13_swiglu_kernel(const FwdParams p) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int npairs = p.I >> 4;
    const int slot = blockIdx.x / npairs;
    const int pair = blockIdx.x - slot * npairs;
    const int* route = p.ws.route;
    if (slot > route[0]) return;  // slot not active in this step
    const int expert = route[1 + slot];
    const int KS = p.K >> 7;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint8_t* wp = p.w13p + (uint64_t)expert * p.w13_bytes +
                        fc13_block(pair, 0, 0, KS) + lane * 16;

    // issue this wave's first weight loads before anything else
    uint4 w[NSTEP][4];
    int base = wave * NSTEP;
    auto load_round = [&](int b) {
        if (b + NSTEP <= KS) {
#pragma unroll
            for (int i = 0; i < NSTEP; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) w[i][q] = ld16(wp + (size_t)(b + i) * 4096 + q * 1024);
        } else {
#pragma unroll
            for (int i = 0; i < NSTEP; ++i)
                if (b + i < KS)
#pragma unroll
                    for (int q = 0; q < 4; ++q) w[i][q] = ld16(wp + (size_t)(b + i) * 4096 + q * 1024);
        }
    };
    if (base < KS) load_round(base);

    // stage the token codes [M][K] into LDS (row stride K + 16 avoids bank conflicts);
    // loads go out in batches of 4 per thread so their latencies overlap
    const int row_stride = p.K + 16;
    {
        const int chunks_per_row = p.K >> 4;
        const int total = p.M * chunks_per_row;
        for (int c0 = threadIdx.x; c0 < total; c0 += 4 * WAVES * 64) {
            uint4 v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = min(c0 + i * WAVES * 64, total - 1);  // clamped: always in bounds
                const int t = c / chunks_per_row, j = c - t * chunks_per_row;
                v[i] = ld16(p.ws.xq + (size_t)t * p.K + j * 16);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = c0 + i * WAVES * 64;
                if (c < total) {
                    const int t = c / chunks_per_row, j = c - t * chunks_per_row;
                    *reinterpret_cast<uint4*>(lds + t * row_stride + j * 16) = v[i];
                }
            }
        }
    }
    __syncthreads();

    v4f accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
    while (base < KS) {
        if (base + NSTEP <= KS) {
#pragma unroll
            for (int i = 0; i < NSTEP; ++i) {
                const Operand b = token_operand(lds, row_stride, base + i, lane, p.M);
                accg = mma_kstep(widen(w[i][0], w[i][1]), b, accg);
                accu = mma_kstep(widen(w[i][2], w[i][3]), b, accu);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NSTEP; ++i) {
                if (base + i < KS) {
                    const Operand b = token_operand(lds, row_stride, base + i, lane, p.M);
                    accg = mma_kstep(widen(w[i][0], w[i][1]), b, accg);
                    accu = mma_kstep(widen(w[i][2], w[i][3]), b, accu);
                }
            }
        }
        base += WAVES * NSTEP;
        if (base < KS) load_round(base);
    }

    // reduce the WAVES partial tiles in LDS (reusing the token buffer)
    __syncthreads();
    float* red = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        red[(wave * 8 + r) * 64 + lane] = accg[r];
        red[(wave * 8 + 4 + r) * 64 + lane] = accu[r];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int wv = 1; wv < WAVES; ++wv)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            accg[r] += red[(wv * 8 + r) * 64 + lane];
            accu[r] += red[(wv * 8 + 4 + r) * 64 + lane];
        }

    // epilogue: lane holds channels n0 + r (r = 0..3) of token tok
    const int tok = lane & 15;
    const int n0 = pair * 16 + 4 * (lane >> 4);
    float amax = 0.0f;
    if (tok < p.M) {
        const bool keep = (slot == 0) || (route[1 + p.S + tok] == slot);
        const float sx = p.ws.sx[tok];
        const float* s13 = p.s13 + (size_t)expert * 2 * p.I;
        const float4 sg = *reinterpret_cast<const float4*>(s13 + n0);
        const float4 su = *reinterpret_cast<const float4*>(s13 + p.I + n0);
        const float sgv[4] = {sg.x, sg.y, sg.z, sg.w};
        const float suv[4] = {su.x, su.y, su.z, su.w};
        float a[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float g = accg[r] * sx * sgv[r];
            const float u = accu[r] * sx * suv[r];
            a[r] = keep ? g / (1.0f + expf(-g)) * u : 0.0f;
            amax = fmaxf(amax, fabsf(a[r]));
        }
        *reinterpret_cast<float4*>(p.ws.a + ((size_t)slot * p.T + tok) * p.I + n0) =
            make_float4(a[0], a[1], a[2], a[3]);
    }
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    if (lane < 16 && tok < p.M && amax > 0.0f)
        atomicMax(p.ws.amax + slot * p.T + tok, __float_as_uint(amax));
}

}  // namespace moe
