// Stage 1 of the forward: top-1 routing with de-duplication of the active experts,
// and per-token dynamic FP8 quantisation of the activations.
//
// Block 0 routes.  One wave per token finds e[m] = the lowest index of the largest
// logit (each lane scans a strided subset of the experts, then a butterfly of
// shuffles combines (value, index) pairs), and gate[m] = sigmoid of that logit.  The
// pages only name MoE; top-1 with a sigmoid gate is the reading taken.  Counts per
// expert go to LDS; one block scan over the experts in ascending id numbers the
// active ones 1..d (slot 0 is the shared expert) and gives each its range of routed
// rows; a token's row inside its expert's range is the number of earlier tokens routed
// to the same expert.  Nothing depends on arrival order, so the table is
// deterministic.  Doing this on the device keeps the step free of host round trips, as
// the pages do for their verification logic (Blackwell 1,000 TPS/user blog, zh
// translation, section on CUDA Graphs and the overlap scheduler).  Block 0 also clears
// the work counters the later stages use.
//
// Blocks 1..M quantise one token each: s = fp32(amax / 448), q = e4m3(x / s), the
// quantize step placed in front of a GEMM (same page, section "CUDA kernel
// optimisation and fusion", item "operator fusion").
#pragma once

#include "codec.hpp"
#include "params.hpp"

namespace moe {

constexpr int kRouteThreads = 256;
constexpr int kMaxRouteExperts = 1024;
constexpr int kQuantChunks = 4;  // 16-byte chunks of x per thread: K <= 4 * 256 * 8 = 8192

__device__ __forceinline__ float block_max_256(float v, float* red) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Exclusive prefix sums over the 256 threads of two counters at once; *total gets
// the block sums.  `tmp` holds 8 ints of LDS.
__device__ __forceinline__ int2 block_exclusive_scan2(int a, int b, int* tmp, int2* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int ia = a, ib = b;  // inclusive scan inside the wave
    for (int o = 1; o < 64; o <<= 1) {
        const int ta = __shfl_up(ia, o), tb = __shfl_up(ib, o);
        if (lane >= o) { ia += ta; ib += tb; }
    }
    if (lane == 63) { tmp[wave] = ia; tmp[4 + wave] = ib; }
    __syncthreads();
    int pa = 0, pb = 0;
    for (int w = 0; w < wave; ++w) { pa += tmp[w]; pb += tmp[4 + w]; }
    *total = make_int2(tmp[0] + tmp[1] + tmp[2] + tmp[3], tmp[4] + tmp[5] + tmp[6] + tmp[7]);
    return make_int2(pa + ia - a, pb + ib - b);
}

__device__ void route_block(const FwdParams& p) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const RouteLayout rl{p.T, p.S};
    int32_t* rt = p.ws.route;
    if (tid < kWorkKernels * kWorkParts) p.ws.work[tid * kWorkStride] = 0u;
    if (p.E == 0) {  // dense: the shared expert alone
        if (tid == 0) {
            rt[rl.d()] = 0;
            rt[rl.slot_expert()] = 0;
            rt[rl.slot_row0()] = 0;
            rt[rl.slot_rows()] = p.M;
            if (p.dbg.num_active) p.dbg.num_active[0] = 0;
        }
        if (tid < p.M) {
            rt[rl.token_row() + tid] = -1;
            rt[rl.token_expert() + tid] = -1;
            rt[rl.row_token() + tid] = tid;
            p.ws.gate[tid] = 0.0f;
            if (p.dbg.expert) p.dbg.expert[tid] = -1;
            if (p.dbg.gate) p.dbg.gate[tid] = 0.0f;
        }
        return;
    }

    __shared__ int s_cnt[kMaxRouteExperts];
    __shared__ int s_off[kMaxRouteExperts];
    __shared__ int s_exp[256];
    __shared__ int s_tmp[8];
    for (int e = tid; e < p.E; e += kRouteThreads) s_cnt[e] = 0;

    // arg-max per token: lanes scan experts lane, lane + 64, ... in ascending order,
    // keeping the first maximum; the butterfly keeps the lower index on equal values
    for (int m = wave; m < p.M; m += kRouteThreads / 64) {
        const uint16_t* row = p.logits + (size_t)m * p.E;
        uint16_t lv[kMaxRouteExperts / 64];  // all of the lane's logits, loaded together
#pragma unroll
        for (int i = 0; i < kMaxRouteExperts / 64; ++i) lv[i] = row[min(lane + 64 * i, p.E - 1)];
        float bv = -INFINITY;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int i = 0; i < kMaxRouteExperts / 64; ++i) {
            const int e = lane + 64 * i;
            const float v = bf16_to_float(lv[i]);
            if (e < p.E && (v > bv || bi == 0x7FFFFFFF)) { bv = v; bi = e; }
        }
        for (int o = 32; o > 0; o >>= 1) {
            const float ov = __shfl_xor(bv, o);
            const int oi = __shfl_xor(bi, o);
            if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
        }
        if (lane == 0) {
            s_exp[m] = bi;
            const float g = 1.0f / (1.0f + expf(-bv));
            p.ws.gate[m] = g;
            rt[rl.token_expert() + m] = bi;
            if (p.dbg.expert) p.dbg.expert[m] = bi;
            if (p.dbg.gate) p.dbg.gate[m] = g;
        }
    }
    __syncthreads();
    for (int m = tid; m < p.M; m += kRouteThreads) atomicAdd(&s_cnt[s_exp[m]], 1);
    __syncthreads();

    // thread t owns experts [4t, 4t + 4): number the active ones and their rows
    constexpr int kPer = kMaxRouteExperts / kRouteThreads;
    int act = 0, rows = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = tid * kPer + i;
        const int c = e < p.E ? s_cnt[e] : 0;
        act += c > 0;
        rows += c;
    }
    int2 tot;
    const int2 pre = block_exclusive_scan2(act, rows, s_tmp, &tot);
    int slot = 1 + pre.x, row = p.M + pre.y;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = tid * kPer + i;
        const int c = e < p.E ? s_cnt[e] : 0;
        if (c > 0) {
            rt[rl.slot_expert() + slot] = e;
            rt[rl.slot_row0() + slot] = row;
            rt[rl.slot_rows() + slot] = c;
            s_off[e] = row;
            ++slot;
            row += c;
        }
    }
    if (tid == 0) {
        rt[rl.d()] = tot.x;
        rt[rl.slot_expert()] = p.E;  // the shared expert's packed index
        rt[rl.slot_row0()] = 0;
        rt[rl.slot_rows()] = p.M;
        if (p.dbg.num_active) p.dbg.num_active[0] = tot.x;
    }
    __syncthreads();
    for (int m = tid; m < p.M; m += kRouteThreads) {
        const int e = s_exp[m];
        int before = 0;
        for (int k = 0; k < m; ++k) before += s_exp[k] == e;
        const int r = s_off[e] + before;
        rt[rl.token_row() + m] = r;
        rt[rl.row_token() + r] = m;
        rt[rl.row_token() + m] = m;
    }
}

// One token: amax over the row, then the codes, with the row held in registers.
__device__ void quant_block(const FwdParams& p, int m) {
    __shared__ float red[4];
    const int tid = threadIdx.x;
    const uint4* row = reinterpret_cast<const uint4*>(p.x + (size_t)m * p.K);  // 8 bf16 each
    const int nchunks = p.K >> 3;
    uint4 v[kQuantChunks];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kQuantChunks; ++i) {
        const int c = tid + i * kRouteThreads;
        v[i] = c < nchunks ? row[c] : make_uint4(0, 0, 0, 0);
        const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int h = 0; h < 4; ++h)
            amax = fmaxf(amax, fmaxf(fabsf(u2f(w[h] << 16)), fabsf(u2f(w[h] & 0xFFFF0000u))));
    }
    amax = block_max_256(amax, red);
    const float s = amax / kE4M3Max;  // IEEE division: fp32(amax / 448)
    uint2* q = reinterpret_cast<uint2*>(p.ws.xq + (size_t)m * p.K);
    uint2* qd = p.dbg.xq ? reinterpret_cast<uint2*>(p.dbg.xq + (size_t)m * p.K) : nullptr;
#pragma unroll
    for (int i = 0; i < kQuantChunks; ++i) {
        const int c = tid + i * kRouteThreads;
        if (c < nchunks) {
            const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
            uint32_t lo = 0, hi = 0;
            if (s > 0.0f) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    lo |= e4m3_encode_div(u2f(w[h] << 16), s) << (16 * h);
                    lo |= e4m3_encode_div(u2f(w[h] & 0xFFFF0000u), s) << (16 * h + 8);
                    hi |= e4m3_encode_div(u2f(w[2 + h] << 16), s) << (16 * h);
                    hi |= e4m3_encode_div(u2f(w[2 + h] & 0xFFFF0000u), s) << (16 * h + 8);
                }
            }
            q[c] = make_uint2(lo, hi);
            if (qd) qd[c] = make_uint2(lo, hi);
        }
    }
    if (tid == 0) {
        p.ws.sx[m] = s;
        if (p.dbg.sx) p.dbg.sx[m] = s;
    }
}

__global__ __launch_bounds__(kRouteThreads) void route_quant_kernel(const FwdParams p) {
    if (blockIdx.x == 0) route_block(p);
    else quant_block(p, blockIdx.x - 1);
}

}  // namespace moe
