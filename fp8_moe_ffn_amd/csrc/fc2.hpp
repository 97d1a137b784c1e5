// Stages 3 and 4 of the forward: re-quantisation of the intermediate to FP8, the
// FC2 (down projection) GEMM split over the intermediate dimension, and the combine
// of the shared and routed experts into the bf16 output.
//
// The pages quantise the result of one kernel in the kernel that feeds the next
// GEMM (Blackwell 1,000 TPS/user blog, zh translation, section "CUDA kernel
// optimisation and fusion", item "operator fusion").  Here the per-token scale
// s_a = fp32(amax / 448) needs the amax over the whole intermediate row, which
// stage 2 accumulated with atomics; each FC2 block therefore starts by encoding the
// slice of the float32 intermediate it contracts (after it has issued its weight
// loads, so the two latencies overlap) and needs no grid-wide synchronisation.
//
// gfx950 design: a block owns (slot, 64 output columns, one split of I); its four
// waves each stream NSTEP k-steps of four 16 x 128 operand blocks with 16-byte
// loads issued up front, widen them exactly to f16 and contract them with
// v_mfma_f32_16x16x32_f16 against the re-quantised tokens in LDS, and reduce over
// the waves in LDS.  Partial sums
// go to [slot][split][token][column]; stage 4 adds the splits in a fixed order
// (no atomics, so results are bitwise reproducible), applies s_a * s2, the gate,
// and rounds to bf16.
#pragma once

#include "codec.hpp"
#include "fc13.hpp"
#include "layout.hpp"
#include "params.hpp"

namespace moe {

constexpr int kFc2Waves = kFc2Sub;  // wave w reduces sub-tile w

__host__ __device__ inline int fc2_lds_bytes(int M, int split_steps) {
    const int aq = M * (split_steps * kKStep + 16);
    const int aq_aligned = (aq + 15) & ~15;
    return aq_aligned + kFc2Waves * kFc2Sub * 4 * 64 * 4;
}

template <int NSTEP>
__global__ __launch_bounds__(kFc2Waves * 64) void fc2_kernel(const FwdParams p) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int nct = p.K / kFc2Cols;
    const int per_slot = nct * p.nsplit;
    const int slot = blockIdx.x / per_slot;
    const int rem = blockIdx.x - slot * per_slot;
    const int ctile = rem / p.nsplit;
    const int split = rem - ctile * p.nsplit;
    const int* route = p.ws.route;
    if (slot > route[0]) return;
    const int expert = route[1 + slot];
    const int IS = p.I >> 7;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int step0 = split * p.split_steps;            // first k-step of the split
    const int nsteps = min(p.split_steps, IS - step0);  // k-steps in this split
    const int my0 = wave * NSTEP;                        // local first step of this wave

    // 1. weight loads of this wave's k-steps, all issued before anything else
    const uint8_t* wp = p.w2p + (uint64_t)expert * p.w2_bytes +
                        fc2_block(ctile, step0 + my0, 0, IS) + lane * 16;
    uint4 w[NSTEP][kFc2Sub][2];
    const bool full = my0 + NSTEP <= nsteps;
    if (full) {
#pragma unroll
        for (int i = 0; i < NSTEP; ++i)
#pragma unroll
            for (int s = 0; s < kFc2Sub; ++s)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    w[i][s][h] = ld16(wp + (size_t)(i * kFc2Sub + s) * kBlockBytes + h * 1024);
    } else {
#pragma unroll
        for (int i = 0; i < NSTEP; ++i)
            if (my0 + i < nsteps)
#pragma unroll
                for (int s = 0; s < kFc2Sub; ++s)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        w[i][s][h] = ld16(wp + (size_t)(i * kFc2Sub + s) * kBlockBytes + h * 1024);
    }

    // 2. re-quantise this split of the float32 intermediate into LDS:
    //    s_a = fp32(amax / 448), aq = e4m3(a / s_a) (codes 0 when amax == 0).
    //    Thread t owns columns 4t..4t+3 of the split; tokens go in batches of 4 so
    //    the loads of a batch are in flight together.
    const int len = nsteps * kKStep;
    const int row_stride = p.split_steps * kKStep + 16;
    const int j0 = step0 * kKStep;
    const float* arow = p.ws.a + (size_t)slot * p.T * p.I + j0;
    uint8_t* dbg_aq = nullptr;
    if (ctile == 0) dbg_aq = slot == 0 ? p.dbg.aq_shared : p.dbg.aq_routed;
    const int j = threadIdx.x * 4;
    if (j < len) {
        for (int t0 = 0; t0 < p.M; t0 += 4) {
            float4 v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = min(t0 + i, p.M - 1);  // clamped: always in bounds
                v[i] = *reinterpret_cast<const float4*>(arow + (size_t)tok * p.I + j);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = t0 + i;
                if (tok < p.M) {
                    const float s = __uint_as_float(p.ws.amax[slot * p.T + tok]) / kE4M3Max;
                    uint32_t packed = 0;
                    if (s > 0.0f)
                        packed = e4m3_encode_div(v[i].x, s) | (e4m3_encode_div(v[i].y, s) << 8) |
                                 (e4m3_encode_div(v[i].z, s) << 16) | (e4m3_encode_div(v[i].w, s) << 24);
                    *reinterpret_cast<uint32_t*>(lds + tok * row_stride + j) = packed;
                    if (dbg_aq && (slot == 0 || route[1 + p.S + tok] == slot))
                        *reinterpret_cast<uint32_t*>(dbg_aq + (size_t)tok * p.I + j0 + j) = packed;
                }
            }
        }
    }
    if (ctile == 0 && split == 0 && threadIdx.x < p.M) {
        const int tok = threadIdx.x;
        const float s = __uint_as_float(p.ws.amax[slot * p.T + tok]) / kE4M3Max;
        if (slot == 0 && p.dbg.sa_shared) p.dbg.sa_shared[tok] = s;
        if (slot != 0 && p.dbg.sa_routed && route[1 + p.S + tok] == slot) p.dbg.sa_routed[tok] = s;
    }
    __syncthreads();

    // 3. contraction
    v4f acc[kFc2Sub];
#pragma unroll
    for (int s = 0; s < kFc2Sub; ++s) acc[s] = (v4f){0.f, 0.f, 0.f, 0.f};
    if (full) {
#pragma unroll
        for (int i = 0; i < NSTEP; ++i) {
            const Operand b = token_operand(lds, row_stride, my0 + i, lane, p.M);
#pragma unroll
            for (int s = 0; s < kFc2Sub; ++s) acc[s] = mma_kstep(widen(w[i][s][0], w[i][s][1]), b, acc[s]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < NSTEP; ++i) {
            if (my0 + i < nsteps) {
                const Operand b = token_operand(lds, row_stride, my0 + i, lane, p.M);
#pragma unroll
                for (int s = 0; s < kFc2Sub; ++s) acc[s] = mma_kstep(widen(w[i][s][0], w[i][s][1]), b, acc[s]);
            }
        }
    }

    // 4. reduce over the waves: wave w sums sub-tile w
    const int aq_bytes = (p.M * row_stride + 15) & ~15;
    float* red = reinterpret_cast<float*>(lds + aq_bytes);  // [wave][sub][r][lane]
#pragma unroll
    for (int s = 0; s < kFc2Sub; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[((wave * kFc2Sub + s) * 4 + r) * 64 + lane] = acc[s][r];
    __syncthreads();
    float out[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int wv = 0; wv < kFc2Waves; ++wv)
#pragma unroll
        for (int r = 0; r < 4; ++r) out[r] += red[((wv * kFc2Sub + wave) * 4 + r) * 64 + lane];
    const int tok = lane & 15;
    if (tok < p.M) {
        const int col = ctile * kFc2Cols + wave * kTile + 4 * (lane >> 4);
        float* dst = p.ws.part + (((size_t)slot * p.nsplit + split) * p.T + tok) * p.K + col;
        *reinterpret_cast<float4*>(dst) = make_float4(out[0], out[1], out[2], out[3]);
    }
}

// out[m, k] = bf16(y_shared + gate[m] * y_routed), y = (sum over splits) * s_a * s2.
__global__ __launch_bounds__(256) void combine_kernel(const FwdParams p) {
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= p.M * p.K) return;
    const int tok = idx / p.K, col = idx - tok * p.K;
    const int* route = p.ws.route;
    const size_t split_stride = (size_t)p.T * p.K;
    const float* ps = p.ws.part + (size_t)tok * p.K + col;
    float sum = 0.0f;
    for (int s = 0; s < p.nsplit; ++s) sum += ps[s * split_stride];
    const float sa = __uint_as_float(p.ws.amax[tok]) / kE4M3Max;
    float y = sum * sa * p.s2[(size_t)p.E * p.K + col];
    if (p.E > 0) {
        const int slot = route[1 + p.S + tok];
        const int expert = route[1 + slot];
        const float* pr = ps + (size_t)slot * p.nsplit * split_stride;
        float sr = 0.0f;
        for (int s = 0; s < p.nsplit; ++s) sr += pr[s * split_stride];
        const float sar = __uint_as_float(p.ws.amax[slot * p.T + tok]) / kE4M3Max;
        const float yr = sr * sar * p.s2[(size_t)expert * p.K + col];
        y = y + p.ws.gate[tok] * yr;
    }
    p.out[idx] = float_to_bf16(y);
}

}  // namespace moe
