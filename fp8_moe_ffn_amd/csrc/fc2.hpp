// Stages 4 and 5 of the forward: the FC2 (down projection) GEMM split over the
// intermediate dimension, and the combine of the shared and routed experts into the
// bf16 output.
//
// gfx950 design of FC2 (the streaming scheme of FC13, fc13.hpp): a work item is
// (expert slot, 64 output columns, one split of I of 1024), numbered slot-major.
// Blocks are persistent; block b takes items b, b + G, b + 2G, ...  Each of the 4 waves owns NSTEP k-steps of
// the split for all four 16-column sub-tiles.  Per k-step a wave loads its four
// 16 x 128 weight operands (8 x 16 B per lane) and the re-quantised intermediate codes
// of the slot's rows (2 x 16 B per lane, L2-resident), and after feeding k-step s of
// item i to the matrix unit it issues the loads of k-step s of item i + 1 into the
// same registers.  All of them are unconditional buffer loads; k-steps past the end of
// I fall outside the tile's resource and read as zeros, and after the last item the
// resources have 0 bytes.  Partial tiles are reduced over the waves in LDS (two
// buffers, one barrier per item); wave w writes sub-tile w as float32 partial sums
// [split][row][column].  The combine adds the splits in a fixed order (no atomics, so
// results are bitwise reproducible), applies s_a * s2 and the gate, and rounds once to
// bf16.
#pragma once

#include "codec.hpp"
#include "fc13.hpp"
#include "layout.hpp"
#include "params.hpp"

namespace moe {

constexpr int kFc2Waves = kFc2Sub;  // wave w finishes sub-tile w
constexpr int kFc2Threads = kFc2Waves * 64;
constexpr int kFc2Steps = 2;                                // k-steps per wave
constexpr int kFc2SplitSteps = kFc2Waves * kFc2Steps;       // k-steps per split of I

struct Fc2Lds {
    int red;    // [2][WAVES][4 sub][4][64] float partial tiles
    int route;  // RouteLayout copy
    int total;
};

__host__ __device__ inline Fc2Lds fc2_lds(int T, int S) {
    Fc2Lds l{};
    l.red = 0;
    l.route = 2 * kFc2Waves * kFc2Sub * 4 * 64 * 4;
    l.total = align16(l.route + RouteLayout{T, S}.count() * 4);
    return l;
}

__global__ __launch_bounds__(kFc2Threads) void fc2_kernel(const FwdParams p) {
    extern __shared__ __align__(16) uint8_t lds[];
    const RouteLayout rl{p.T, p.S};
    const int per_slot = (p.K / kFc2Cols) * p.nsplit;
    const int G = (int)gridDim.x;
    const int d = p.ws.route[rl.d()];
    const int total = (1 + d) * per_slot;  // work items
    const int IS = p.I >> 7;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int j = lane & 15, grp = lane >> 4;
    const Fc2Lds L = fc2_lds(p.T, p.S);
    const uint32_t ctile_bytes = (uint32_t)IS * kFc2Sub * kBlockBytes;
    // item -> (slot, column tile, split); a wave's first k-step of the item's split
    auto tile_of = [&](int it) { return it >= 0 ? it % per_slot : 0; };
    auto step_of = [&](int it) { return (tile_of(it) % p.nsplit) * kFc2SplitSteps + wave * kFc2Steps; };
    auto wres = [&](int expert, int it) {
        return make_res(p.w2p + (uint64_t)expert * p.w2_bytes + (uint64_t)(tile_of(it) / p.nsplit) * ctile_bytes,
                        it >= 0 ? ctile_bytes : 0u);
    };
    const BufRes aall = make_res(p.ws.aq, (uint32_t)(2 * p.T) * p.I);
    const BufRes anone = make_res(p.ws.aq, 0u);

    int cur = blockIdx.x;                      // G <= per_slot <= total: the shared expert's
    int nxt = cur + G < total ? cur + G : -1;  // next item, -1 if none

    // 1. operand loads of the first item (the shared expert: rows [0, M))
    uint4 w[kFc2Steps][kFc2Sub][2];
    uint4 b[kFc2Steps][2];
    {
        const BufRes rw = wres(p.ws.route[rl.slot_expert()], cur);
        const int st = step_of(cur);
        const uint32_t wo = (uint32_t)st * kFc2Sub * kBlockBytes + lane * 16;
        const uint32_t ao = (uint32_t)min(j, p.M - 1) * p.I + st * kKStep + grp * 32;
#pragma unroll
        for (int s = 0; s < kFc2Steps; ++s) {
#pragma unroll
            for (int u = 0; u < kFc2Sub; ++u)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    w[s][u][h] = buf_ld16(rw, wo + (s * kFc2Sub + u) * kBlockBytes + h * 1024);
            b[s][0] = buf_ld16(aall, ao + s * kKStep);
            b[s][1] = buf_ld16(aall, ao + s * kKStep + 16);
        }
    }
    // 2. routing table into LDS
    for (int i = threadIdx.x; i < rl.count(); i += kFc2Threads)
        reinterpret_cast<int*>(lds + L.route)[i] = p.ws.route[i];
    lds_barrier();

    const int* rt = reinterpret_cast<const int*>(lds + L.route);
    float* red = reinterpret_cast<float*>(lds + L.red);
    int par = 0;
    for (;;) {
        const int nslot = nxt >= 0 ? nxt / per_slot : 0;
        const int nexpert = __builtin_amdgcn_readfirstlane(rt[rl.slot_expert() + nslot]);
        const BufRes rn = wres(nexpert, nxt);
        const BufRes an = nxt >= 0 ? aall : anone;
        const int nst = step_of(nxt);
        const uint32_t wo = (uint32_t)nst * kFc2Sub * kBlockBytes + lane * 16;
        const int nr0 = rt[rl.slot_row0() + nslot], nnr = rt[rl.slot_rows() + nslot];
        const uint32_t ao = (uint32_t)(nr0 + min(j, nnr - 1)) * p.I + nst * kKStep + grp * 32;

        v4f acc[kFc2Sub];
#pragma unroll
        for (int u = 0; u < kFc2Sub; ++u) acc[u] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kFc2Steps; ++s) {
            const Operand bo = widen(b[s][0], b[s][1]);
#pragma unroll
            for (int u = 0; u < kFc2Sub; ++u) acc[u] = mma_kstep(widen(w[s][u][0], w[s][u][1]), bo, acc[u]);
#pragma unroll
            for (int u = 0; u < kFc2Sub; ++u)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    w[s][u][h] = buf_ld16(rn, wo + (s * kFc2Sub + u) * kBlockBytes + h * 1024);
            b[s][0] = buf_ld16(an, ao + s * kKStep);
            b[s][1] = buf_ld16(an, ao + s * kKStep + 16);
            // keep k-steps in order, so the wave waits for one k-step's loads at a time
            __builtin_amdgcn_sched_barrier(0);
        }

        // reduce over the waves: wave w sums sub-tile w
        float* rb = red + par * (kFc2Waves * kFc2Sub * 4 * 64);
#pragma unroll
        for (int u = 0; u < kFc2Sub; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q) rb[((wave * kFc2Sub + u) * 4 + q) * 64 + lane] = acc[u][q];
        lds_barrier();
        float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int wv = 0; wv < kFc2Waves; ++wv)
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] += rb[((wv * kFc2Sub + wave) * 4 + q) * 64 + lane];
        const int slot = cur / per_slot, tile = cur - slot * per_slot;
        const int r0 = rt[rl.slot_row0() + slot], nr = rt[rl.slot_rows() + slot];
        if (j < nr) {
            const int split = tile % p.nsplit;
            const int col = (tile / p.nsplit) * kFc2Cols + wave * kTile + 4 * grp;
            float* dst = p.ws.part + ((size_t)split * 2 * p.T + r0 + j) * p.K + col;
            *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
        }
        if (nxt < 0) break;
        cur = nxt;
        nxt = nxt + G < total ? nxt + G : -1;
        par ^= 1;
    }
}

// out[m, k] = bf16(y_shared + gate[m] * y_routed), y = (sum over splits) * s_a * s2.
// One thread per token and 4 consecutive columns; the partial sums of 8 splits are
// loaded together, then added in split order.
constexpr int kCombineBatch = 8;

__device__ __forceinline__ float4 add4(float4 a, float4 b) {
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

__device__ __forceinline__ float4 sum_splits(const float* p, size_t stride, int nsplit) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < nsplit; s0 += kCombineBatch) {
        float4 v[kCombineBatch];
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u)
            v[u] = s0 + u < nsplit ? *reinterpret_cast<const float4*>(p + (s0 + u) * stride)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u)
            if (s0 + u < nsplit) acc = add4(acc, v[u]);
    }
    return acc;
}

__global__ __launch_bounds__(256) void combine_kernel(const FwdParams p) {
    const int idx = blockIdx.x * 256 + threadIdx.x;
    const int k4 = p.K >> 2;
    if (idx >= p.M * k4) return;
    const RouteLayout rl{p.T, p.S};
    const int tok = idx / k4, col = (idx - tok * k4) * 4;
    const size_t split_stride = (size_t)2 * p.T * p.K;
    const bool routed = p.E > 0;
    const int rrow = routed ? p.ws.route[rl.token_row() + tok] : 0;
    const int rexp = routed ? p.ws.route[rl.token_expert() + tok] : 0;
    const float4 sh = sum_splits(p.ws.part + (size_t)tok * p.K + col, split_stride, p.nsplit);
    const float sa = p.ws.sa[tok];
    const float4 s2 = *reinterpret_cast<const float4*>(p.s2 + (size_t)p.E * p.K + col);
    float y[4] = {sh.x * sa * s2.x, sh.y * sa * s2.y, sh.z * sa * s2.z, sh.w * sa * s2.w};
    if (routed) {
        const float4 ro = sum_splits(p.ws.part + (size_t)rrow * p.K + col, split_stride, p.nsplit);
        const float sar = p.ws.sa[rrow];
        const float g = p.ws.gate[tok];
        const float4 s2r = *reinterpret_cast<const float4*>(p.s2 + (size_t)rexp * p.K + col);
        y[0] = y[0] + g * (ro.x * sar * s2r.x);
        y[1] = y[1] + g * (ro.y * sar * s2r.y);
        y[2] = y[2] + g * (ro.z * sar * s2r.z);
        y[3] = y[3] + g * (ro.w * sar * s2r.w);
    }
    uint2 packed;
    packed.x = (uint32_t)float_to_bf16(y[0]) | ((uint32_t)float_to_bf16(y[1]) << 16);
    packed.y = (uint32_t)float_to_bf16(y[2]) | ((uint32_t)float_to_bf16(y[3]) << 16);
    *reinterpret_cast<uint2*>(p.out + (size_t)tok * p.K + col) = packed;
}

}  // namespace moe
