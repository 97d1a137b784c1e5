// Stage 2 of the forward: the FC13 GEMM (gate and up projections side by side)
// with SwiGLU applied in its epilogue, for the shared expert and every distinct
// routed expert.  The pages fuse SwiGLU into the GEMM in front of it (Blackwell
// 1,000 TPS/user blog, zh translation, section "CUDA kernel optimisation and
// fusion", item "operator fusion") and build low-latency GEMMs that load weights so
// as to use the whole HBM bandwidth (same section, item on spatial partitioning and
// efficient memory loads).
//
// gfx950 design.  At M <= 16 tokens the GEMM is a weight stream.  A work item is one
// "pair" (16 gate + 16 up channels) of one active expert over the whole hidden size K;
// items are numbered slot-major, (1 + d) * I/16 of them.  Blocks are persistent (as
// many as are resident at once).  Block b's first two items are b and b + G; after
// that it takes items from a work counter of its partition (WorkPlan: one counter per
// XCD, as blocks are dealt to the XCDs in turn), so blocks whose share of the HBM
// bandwidth is larger simply do more items and the blocks finish together.  A ticket
// is taken two items ahead (its latency hides under one item) and passed to the
// block's waves through LDS.
//
// Each of the WAVES waves owns NSTEP consecutive 128-deep k-steps of every item and
// keeps them in registers as 16-byte loads (4 KiB per k-step and wave, 1 KiB coalesced
// per instruction).  As soon as a wave has fed k-step s of item i to the matrix unit
// it issues the loads of k-step s of item i + 1 into the same registers, so every wave
// always has one item's worth of weight bytes in flight.
//
// Memory counters retire in order, so a per-lane global load issued after that
// prefetch would make the wave wait for all of it.  Inside the loop every global load
// is therefore an unconditional buffer load (after the last item the resource has 0
// bytes: zeros, no memory access); the routing table, activation codes and scales are
// staged into LDS once per block.
//
// Tokens of the item's slot form the B operand (16 columns; columns past the slot's
// row count repeat its last row and are discarded).  Weights and tokens are widened
// exactly to f16 in registers and contracted with v_mfma_f32_16x16x32_f16
// (layout.hpp says why not an e4m3-input instruction).  Partial tiles are reduced
// over the waves in LDS (two buffers, one barrier per item).  Wave w finishes
// channel r = w mod 4 of every lane: scales, SwiGLU, the float32 intermediate row and
// the block's running max |a| per row (an LDS atomic max on the float bit pattern).
// Waves 4..7 repeat waves 0..3's arithmetic without storing, so that the scale loads
// of every wave have a use and stay where they are issued.  At the end the block
// writes its per-row maxima to its own row of ws.amax; the re-quantisation kernel
// takes the max over the blocks.  No global atomics sit on the streaming path.
#pragma once

#include "codec.hpp"
#include "layout.hpp"
#include "params.hpp"

namespace moe {

constexpr int kFc13Waves = 8;
constexpr int kFc13Threads = kFc13Waves * 64;

__device__ __forceinline__ uint4 ld16(const uint8_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}

__host__ __device__ constexpr int align16(int v) { return (v + 15) & ~15; }

// LDS layout of fc13_swiglu_kernel, in bytes.
struct Fc13Lds {
    int red;    // [2][WAVES][8][64] float partial tiles
    int next;   // [2] int: the item after next, passed from wave 0 to all waves
    int rowmax; // [2T] uint32: the block's max |a| per row (float bits)
    int route;  // RouteLayout copy
    int sx;     // [M] float
    int xq;     // [M][K + 16] token codes (row stride padded against bank conflicts)
    int total;
};

__host__ __device__ inline Fc13Lds fc13_lds(int T, int S, int M, int K) {
    Fc13Lds l{};
    int off = 0;
    l.red = off;
    off += 2 * kFc13Waves * 8 * 64 * 4;
    l.next = off;
    off += 16;
    l.rowmax = off;
    off = align16(off + 2 * T * 4);
    l.route = off;
    off = align16(off + RouteLayout{T, S}.count() * 4);
    l.sx = off;
    off = align16(off + M * 4);
    l.xq = off;
    off += M * (K + 16);
    l.total = off;
    return l;
}

// Block barrier that orders LDS only: waits for this wave's LDS operations, then
// s_barrier.  Outstanding global loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int NSTEP, bool FULL>
__global__ __launch_bounds__(kFc13Threads) void fc13_swiglu_kernel(const FwdParams p) {
    extern __shared__ __align__(16) uint8_t lds[];
    const RouteLayout rl{p.T, p.S};
    const int npairs = p.I >> 4;
    const int G = (int)gridDim.x;
    const int d = p.ws.route[rl.d()];
    const int total = (1 + d) * npairs;  // work items
    const int KS = p.K >> 7;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int s0 = wave * NSTEP;  // first k-step of this wave
    const int ns = FULL ? NSTEP : max(0, min(NSTEP, KS - s0));
    const Fc13Lds L = fc13_lds(p.T, p.S, p.M, p.K);
    const int xstride = p.K + 16;
    const uint32_t pair_bytes = (uint32_t)KS * 2 * kBlockBytes;
    const uint32_t woff = (uint32_t)s0 * 2 * kBlockBytes + lane * 16;  // lane's bytes in a pair
    const int j = lane & 15;    // B column (row of the slot) / C column
    const int grp = lane >> 4;  // 32-deep reduction group of the lane; C rows 4*grp..4*grp+3
    const int r = wave & 3;     // C row (channel) of the lane this wave finishes
    // weight resource of item `it` (0 bytes when there is none, it < 0)
    auto wres = [&](int expert, int it) {
        return make_res(p.w13p + (uint64_t)expert * p.w13_bytes + (uint64_t)(it >= 0 ? it % npairs : 0) * pair_bytes,
                        it >= 0 ? pair_bytes : 0u);
    };
    // scales of an expert ([2I] floats; 0 bytes when there is no item) and the byte
    // offset of this lane's gate scale in item `it` (the up scale is 4I bytes further)
    auto sres = [&](int expert, int it) {
        return make_res(p.s13 + (size_t)expert * 2 * p.I, it >= 0 ? (uint32_t)p.I * 8 : 0u);
    };
    auto soff = [&](int it) { return (uint32_t)((it >= 0 ? it % npairs : 0) * 16 + 4 * grp + r) * 4; };

    const WorkPlan plan(G, blockIdx.x, total);
    uint32_t* counter = p.ws.work + work_index(kWorkFc13, plan.x);
    int cur = plan.first();   // = blockIdx.x (G <= npairs <= total): the shared expert's
    int nxt = plan.second();  // next item, -1 if none
    const int expert0 = p.ws.route[rl.slot_expert()];  // items < npairs are the shared expert's

    // 1. weight and scale loads of the first item
    uint4 w[NSTEP][4];
    float sg, su;
    {
        const BufRes rw = wres(expert0, cur);
        const BufRes rs = sres(expert0, cur);
        sg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, soff(cur), 0, 0));
        su = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, soff(cur) + p.I * 4, 0, 0));
#pragma unroll
        for (int s = 0; s < NSTEP; ++s)
            if (FULL || s < ns)
#pragma unroll
                for (int q = 0; q < 4; ++q) w[s][q] = buf_ld16(rw, woff + s * 2 * kBlockBytes + q * 1024);
    }

    // 2. stage the routing table, activation scales and token codes into LDS
    {
        const int nroute = rl.count();
        for (int i = threadIdx.x; i < nroute; i += kFc13Threads)
            reinterpret_cast<int*>(lds + L.route)[i] = p.ws.route[i];
        for (int i = threadIdx.x; i < p.M; i += kFc13Threads)
            reinterpret_cast<float*>(lds + L.sx)[i] = p.ws.sx[i];
        for (int i = threadIdx.x; i < 2 * p.T; i += kFc13Threads)
            reinterpret_cast<uint32_t*>(lds + L.rowmax)[i] = 0u;
        const int cpr = p.K >> 4;  // 16-byte chunks per token row
        const int nch = p.M * cpr;
        for (int c0 = threadIdx.x; c0 < nch; c0 += 4 * kFc13Threads) {
            uint4 v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = min(c0 + i * kFc13Threads, nch - 1);  // clamped: in bounds
                const int t = c / cpr, jj = c - t * cpr;
                v[i] = ld16(p.ws.xq + (size_t)t * p.K + jj * 16);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = c0 + i * kFc13Threads;
                if (c < nch) {
                    const int t = c / cpr, jj = c - t * cpr;
                    *reinterpret_cast<uint4*>(lds + L.xq + t * xstride + jj * 16) = v[i];
                }
            }
        }
    }
    lds_barrier();

    const int* rt = reinterpret_cast<const int*>(lds + L.route);
    const float* sxl = reinterpret_cast<const float*>(lds + L.sx);
    int* next_slot = reinterpret_cast<int*>(lds + L.next);
    uint32_t* rowmax = reinterpret_cast<uint32_t*>(lds + L.rowmax);
    float* red = reinterpret_cast<float*>(lds + L.red);
    int par = 0;
    for (;;) {
        // ticket for the item after next (wave 0, lane 0; written to LDS before the barrier)
        uint32_t ticket = 0;
        if (threadIdx.x == 0 && nxt >= 0) ticket = atomicAdd(counter, 1u);

        const int slot = cur / npairs, pair = cur - slot * npairs;
        const int nexpert = __builtin_amdgcn_readfirstlane(rt[rl.slot_expert() + (nxt >= 0 ? nxt / npairs : 0)]);
        const BufRes rn = wres(nexpert, nxt);
        const BufRes rsn = sres(nexpert, nxt);

        const int r0 = rt[rl.slot_row0() + slot], nr = rt[rl.slot_rows() + slot];
        const int tok = rt[rl.row_token() + r0 + min(j, nr - 1)];
        const uint8_t* brow = lds + L.xq + tok * xstride + grp * 32;

        // scales of the next item (consumed one item later)
        const float nsg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsn, soff(nxt), 0, 0));
        const float nsu =
            __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsn, soff(nxt) + p.I * 4, 0, 0));
        v4f accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NSTEP; ++s) {
            if (FULL || s < ns) {
                const uint8_t* bp = brow + (s0 + s) * kKStep;
                const Operand b = widen(*reinterpret_cast<const uint4*>(bp),
                                        *reinterpret_cast<const uint4*>(bp + 16));
                accg = mma_kstep(widen(w[s][0], w[s][1]), b, accg);
                accu = mma_kstep(widen(w[s][2], w[s][3]), b, accu);
#pragma unroll
                for (int q = 0; q < 4; ++q) w[s][q] = buf_ld16(rn, woff + s * 2 * kBlockBytes + q * 1024);
            }
            // keep k-steps in order, so the wave waits for one k-step's loads at a time
            __builtin_amdgcn_sched_barrier(0);
        }

        // reduce the WAVES partial tiles
        float* rb = red + par * (kFc13Waves * 8 * 64);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            rb[(wave * 8 + q) * 64 + lane] = accg[q];
            rb[(wave * 8 + 4 + q) * 64 + lane] = accu[q];
        }
        if (threadIdx.x == 0) next_slot[par] = nxt >= 0 ? plan.from_ticket(ticket) : -1;
        lds_barrier();
        float g = 0.0f, u = 0.0f;
#pragma unroll
        for (int wv = 0; wv < kFc13Waves; ++wv) {
            g += rb[(wv * 8 + r) * 64 + lane];
            u += rb[(wv * 8 + 4 + r) * 64 + lane];
        }
        // channel 16 * pair + 4 * grp + r of row r0 + j
        const float sx = sxl[tok];
        g = g * sx * sg;
        u = u * sx * su;
        const float a = g / (1.0f + expf(-g)) * u;
        float amax = j < nr ? fabsf(a) : 0.0f;
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        if (wave < 4) {
            if (j < nr) p.ws.a[(size_t)(r0 + j) * p.I + pair * 16 + 4 * grp + r] = a;
            if (lane < 16 && j < nr && amax > 0.0f) atomicMax(rowmax + r0 + j, __float_as_uint(amax));
        }
        if (nxt < 0) break;
        cur = nxt;
        nxt = __builtin_amdgcn_readfirstlane(next_slot[par]);
        sg = nsg;
        su = nsu;
        par ^= 1;
    }
    lds_barrier();
    for (int i = threadIdx.x; i < 2 * p.T; i += kFc13Threads)
        p.ws.amax[(size_t)blockIdx.x * 2 * p.T + i] = rowmax[i];
}

}  // namespace moe
