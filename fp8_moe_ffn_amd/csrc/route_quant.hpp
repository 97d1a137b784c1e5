// Stage 1 of the forward: top-1 routing with de-duplication of the active experts,
// and per-token dynamic FP8 quantisation of the activations.
//
// Block 0 routes: e[m] = lowest index of the largest logit, gate = sigmoid of it
// (the pages only name MoE; top-1 with a sigmoid gate is the reading taken), then
// the distinct experts in ascending order become slots 1..d (slot 0 is the shared
// expert), and the per-(slot, token) amax words used by the next stages are reset.
// Doing this on the device keeps the step free of host round trips, as the pages
// do for their verification logic (Blackwell 1,000 TPS/user blog, zh translation,
// section on CUDA Graphs and the overlap scheduler).
// Blocks 1..M each quantise one token: s = fp32(amax / 448), q = e4m3(x / s),
// which is the quantize step placed in front of a GEMM (same page, section "CUDA
// kernel optimisation and fusion", item "operator fusion").
#pragma once

#include "codec.hpp"
#include "params.hpp"

namespace moe {

constexpr int kRouteThreads = 256;

__device__ __forceinline__ float block_max_256(float v, float* red) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    return v;
}

__global__ __launch_bounds__(kRouteThreads) void route_quant_kernel(const FwdParams p) {
    const int tid = threadIdx.x;
    const Workspace& ws = p.ws;
    if (blockIdx.x == 0) {
        __shared__ int s_expert[16];
        __shared__ int s_list[17];
        for (int i = tid; i < p.S * p.T; i += kRouteThreads) ws.amax[i] = 0u;
        int32_t* slot_expert = ws.route + 1;
        int32_t* tok_slot = ws.route + 1 + p.S;
        int32_t* tok_expert = ws.route + 1 + p.S + p.T;
        if (p.E == 0) {
            if (tid == 0) { ws.route[0] = 0; slot_expert[0] = 0; }
            if (tid < p.M) {
                tok_slot[tid] = 0;
                tok_expert[tid] = -1;
                ws.gate[tid] = 0.0f;
                if (p.dbg.expert) p.dbg.expert[tid] = -1;
                if (p.dbg.gate) p.dbg.gate[tid] = 0.0f;
            }
            if (tid == 0 && p.dbg.num_active) p.dbg.num_active[0] = 0;
            return;
        }
        if (tid < p.M) {  // M <= 16: one thread per token scans its logits
            const uint16_t* row = p.logits + (size_t)tid * p.E;
            int best = 0;
            float bv = bf16_to_float(row[0]);
            for (int e = 1; e < p.E; ++e) {
                const float v = bf16_to_float(row[e]);
                if (v > bv) { bv = v; best = e; }  // strict: the lowest index wins ties
            }
            s_expert[tid] = best;
            const float g = 1.0f / (1.0f + expf(-bv));
            ws.gate[tid] = g;
            tok_expert[tid] = best;
            if (p.dbg.expert) p.dbg.expert[tid] = best;
            if (p.dbg.gate) p.dbg.gate[tid] = g;
        }
        __syncthreads();
        if (tid == 0) {  // sorted distinct experts, at most M <= 16 of them
            int n = 0;
            for (int m = 0; m < p.M; ++m) {
                const int e = s_expert[m];
                int pos = 0;
                while (pos < n && s_list[pos] < e) ++pos;
                if (pos < n && s_list[pos] == e) continue;
                for (int j = n; j > pos; --j) s_list[j] = s_list[j - 1];
                s_list[pos] = e;
                ++n;
            }
            ws.route[0] = n;
            slot_expert[0] = p.E;  // the shared expert's packed index
            for (int j = 0; j < n; ++j) slot_expert[1 + j] = s_list[j];
            if (p.dbg.num_active) p.dbg.num_active[0] = n;
        }
        __syncthreads();
        if (tid < p.M) {
            const int e = s_expert[tid];
            int j = 0;
            while (s_list[j] != e) ++j;
            tok_slot[tid] = 1 + j;
        }
        return;
    }

    // ---- blocks 1..M: per-token quantisation -------------------------------
    __shared__ float red[4];
    const int m = blockIdx.x - 1;
    const uint16_t* row = p.x + (size_t)m * p.K;
    float amax = 0.0f;
    for (int k = tid; k < p.K; k += kRouteThreads) amax = fmaxf(amax, fabsf(bf16_to_float(row[k])));
    amax = block_max_256(amax, red);
    const float s = amax / kE4M3Max;  // IEEE division: fp32(amax / 448)
    uint8_t* q = ws.xq + (size_t)m * p.K;
    for (int k4 = tid * 4; k4 < p.K; k4 += kRouteThreads * 4) {
        uint32_t packed = 0;
        if (s > 0.0f) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                packed |= e4m3_encode_div(bf16_to_float(row[k4 + j]), s) << (8 * j);
        }
        *reinterpret_cast<uint32_t*>(q + k4) = packed;
        if (p.dbg.xq) *reinterpret_cast<uint32_t*>(p.dbg.xq + (size_t)m * p.K + k4) = packed;
    }
    if (tid == 0) {
        ws.sx[m] = s;
        if (p.dbg.sx) p.dbg.sx[m] = s;
    }
}

}  // namespace moe
