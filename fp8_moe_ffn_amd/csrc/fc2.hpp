// Second and third kernels of the forward: re-quantisation of the intermediate and
// the FC2 (down projection) GEMM split over the intermediate dimension; then the
// combine of the shared and routed experts into the bf16 output.  The pages quantise
// a kernel's result to FP8 before it feeds the next GEMM (Blackwell 1,000 TPS/user
// blog, zh translation, section "CUDA kernel optimisation and fusion", item "operator
// fusion"); the scale s_a = fp32(amax / 448) of a row needs the amax over the whole
// row, so the quantisation runs after FC13, inside this kernel.
//
// gfx950 design of FC2 (the streaming scheme of FC13, fc13.hpp): a work item is
// (expert slot, 64 output columns, one split of I of 2048), numbered slot-major.
// Blocks are persistent, one per CU (two resident blocks measured slower: their
// prologues and item boundaries cost more than the bytes they add in flight), at most
// the items the largest step has, and half of them when that is between one and two
// items per CU (so that every block takes two); block b takes item b (the shared expert's unless the
// grid outnumbers one slot's items, at small I), then a fixed share of the rest dealt so
// that the blocks that continue all end within one item (EvenPlan).  An item (about 5 us) is about as long as a work
// counter's round trip under the weight stream, and a pool measured slower.  Each of
// the 8 waves (128 KiB of weights in flight per CU; 4 waves and splits of 1024 measured
// slower with the non-temporal weight loads)
// owns kFc2Steps k-steps of the split for all four 16-column sub-tiles.  Per
// k-step a wave loads its four 16 x 128 weight operands (8 x 16 B per lane), and after
// feeding k-step s of item i to the matrix unit it issues the loads of k-step s of
// item i + 1 into the same registers.  All of them are unconditional buffer loads;
// k-steps past the end of I fall outside the tile's resource and read as zeros, and
// after the last item the resources have 0 bytes.
//
// The B operand (the item's rows of the re-quantised intermediate, its split of I) is
// made by the block itself in LDS: the float32 slice of item i + 1 (one float4 per
// thread and row) is requested at the top of item i, ahead of that item's weight
// reloads, and encoded to e4m3 at its end with the row scales, which the block's
// prologue computes from the FC13 blocks' per-row maxima.  Several blocks encode the
// same slice (one per column tile): a few instructions per value, in exchange for no
// separate kernel and no grid-wide dependency.  Partial tiles are reduced over the
// waves in LDS (two buffers, one barrier per item); wave w < 4 writes sub-tile w as float32
// partial sums [split][row][column], already multiplied by s_a of the row and s2 of the
// column (requested with the slice, one item ahead).  A routed row is written at row
// M + token, so the combine finds every operand of a token without the routing table:
// it adds the splits in a fixed order (no atomics, so results are bitwise
// reproducible), applies the gate, and rounds once to bf16.
#pragma once

#include "codec.hpp"
#include "fc13.hpp"
#include "layout.hpp"
#include "params.hpp"

namespace moe {

constexpr int kFc2Waves = 8;  // wave w finishes sub-tile w mod 4 (waves 4..7 without storing)
constexpr int kFc2Threads = kFc2Waves * 64;
constexpr int kFc2Steps = 2;                                // k-steps per wave
constexpr int kFc2SplitSteps = kFc2Waves * kFc2Steps;       // k-steps per split of I
constexpr int kFc2Split = kFc2SplitSteps * kKStep;          // columns of I per split
constexpr int kFc2BStride = kFc2Split + 16;                 // LDS row stride of the B codes
constexpr int kAmaxLoads = 4;  // FC13 block maxima per lane and row loaded early (<= 256 blocks)
constexpr int kSliceVec = kFc2Split / (4 * kFc2Threads);  // float4s of a row per thread and split
static_assert(kSliceVec * 4 * kFc2Threads == kFc2Split, "whole float4s of each row per thread");

struct Fc2Lds {
    int red;    // [2][WAVES][4 sub][4][64] float partial tiles
    int route;  // RouteLayout table
    int sa;     // [2T] float: s_a per row
    int rcp;    // [2T] float: fp32(1 / s_a)
    int b;      // [2][ROWS][kFc2BStride] e4m3 codes of the B operand
    int total;
};

__host__ __device__ inline Fc2Lds fc2_lds(int T, int S, int rows) {
    Fc2Lds l{};
    l.red = 0;
    l.route = 2 * kFc2Waves * kFc2Sub * 4 * 64 * 4;
    l.sa = align16(l.route + RouteLayout{T, S}.count() * 4);
    l.rcp = align16(l.sa + 2 * T * 4);
    l.b = align16(l.rcp + 2 * T * 4);
    l.total = l.b + 2 * rows * kFc2BStride;
    return l;
}

// ROWS >= max tokens: rows of one slot's B operand.  The leading arguments (Fc2Lead) are
// what the first loads need; they repeat fields of p and are preloaded into SGPRs.
// The kernel's body, for block `bid` of G.  WAIT (the second phase of the single launch):
// the first item's weights (the shared expert's, known without the routing) are requested
// first, then the block waits until `fc13_done` reaches `fc13_target` (every FC13 block of
// the launch has arrived), and only then loads what FC13 wrote (routing table, maxima,
// intermediate).
template <int ROWS, bool WAIT = false>
__device__ __forceinline__ void fc2_body(int bid, const int32_t* lead_route, const uint32_t* lead_amax,
                                         const float* lead_a, const float* lead_s2e, const uint8_t* lead_w2e,
                                         uint32_t lead_mts, uint32_t lead_ki, uint32_t lead_grids,
                                         const FwdParams& p0, uint8_t* lds, uint32_t* fc13_done = nullptr,
                                         uint32_t* timeouts = nullptr, uint32_t fc13_target = 0) {
    static_assert(ROWS * kSliceVec <= 64, "redo flags fit in 64 bits");
    FwdParams p = p0;
    p.ws.route = const_cast<int32_t*>(lead_route);
    p.ws.amax = const_cast<uint32_t*>(lead_amax);
    p.ws.a = const_cast<float*>(lead_a);
    p.M = (int)(lead_mts & 0xFFu);
    p.T = (int)((lead_mts >> 8) & 0xFFu);
    p.S = (int)((lead_mts >> 16) & 0xFFu);
    p.nsplit = (int)(lead_mts >> 24);
    p.K = (int)(lead_ki & 0xFFFFu);
    p.I = (int)(lead_ki >> 16);
    p.grid13 = (int)(lead_grids & 0xFFFFu);
    const RouteLayout rl{p.T, p.S};
    const int per_slot = (p.K / kFc2Cols) * p.nsplit;
    const int G = (int)(lead_grids >> 16);  // gridDim.x
    const int IS = p.I >> 7;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int sub = wave & (kFc2Sub - 1);  // the sub-tile this wave finishes
    const int j = lane & 15, grp = lane >> 4;
    const Fc2Lds L = fc2_lds(p.T, p.S, ROWS);
    const int nrows = p.E > 0 ? 2 * p.M : p.M;  // rows of the intermediate in use
    const uint32_t ctile_bytes = (uint32_t)IS * kFc2Sub * kBlockBytes;
    // item -> (slot, column tile, split); a wave's first k-step of the item's split
    auto tile_of = [&](int it) { return it >= 0 ? it % per_slot : 0; };
    auto split_of = [&](int it) { return tile_of(it) % p.nsplit; };
    auto step_of = [&](int it) { return split_of(it) * kFc2SplitSteps + wave * kFc2Steps; };
    auto wres = [&](int expert, int it) {
        return make_res(p.w2p + (uint64_t)expert * p.w2_bytes + (uint64_t)(tile_of(it) / p.nsplit) * ctile_bytes,
                        it >= 0 ? ctile_bytes : 0u);
    };
    const BufRes ares = make_res(p.ws.a, (uint32_t)(2 * p.T) * p.I * 4);
    const BufRes anone = make_res(p.ws.a, 0u);
    // this thread's float4 of row `row`, split `split`, in bytes (past I: the next row's
    // values or zeros past the buffer; never encoded).  Rows past the slot's row count
    // are placed outside the resource: they read as zeros without a memory access.
    auto aoff = [&](int row, int split, int v) {
        return ((uint32_t)row * p.I + split * kFc2Split + 4 * (tid + v * kFc2Threads)) * 4;
    };
    constexpr uint32_t kOutside = 0x80000000u;

    // block b's first item is item b: the shared expert's for b < per_slot, its weights
    // requested before the routing table is read; a block past those (a grid larger than
    // one slot's items, at small I) starts on a routed expert's item once it has the table
    int cur = bid;
    const bool early = bid < per_slot;
    uint4 w[kFc2Steps][kFc2Sub][2];
    // the expert's packed W2 (no expert: 0 bytes, zeros without a memory access).  A block
    // that starts later issues the shared expert's loads with 0-byte resources, so that
    // both kinds of block have the same loads outstanding in the same order where their
    // paths meet (the waits the compiler places there stay exact).
    auto first_weights = [&](const uint8_t* w2e, bool any, int s0 = 0, int s1 = kFc2Steps) {  // k-steps [s0, s1)
        const BufRes rw = make_res(w2e + (uint64_t)(tile_of(cur) / p.nsplit) * ctile_bytes, any ? ctile_bytes : 0u);
        const uint32_t wo = (uint32_t)step_of(cur) * kFc2Sub * kBlockBytes + lane * 16;
#pragma unroll
        for (int s = s0; s < s1; ++s)
#pragma unroll
            for (int u = 0; u < kFc2Sub; ++u)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    w[s][u][h] = buf_ld16_stream(rw, wo + (s * kFc2Sub + u) * kBlockBytes + h * 1024);
    };
    if constexpr (WAIT) {
        first_weights(lead_w2e, early);
        __builtin_amdgcn_sched_barrier(0);
        block_wait(fc13_done, fc13_target, timeouts);
    }

    // 1. early loads: the routing table, the FC13 blocks' maxima of this wave's rows and
    //    the first item's slice (shared expert: rows [0, M)), ahead of the weights
    const int ncount = rl.count();
    const int rtv = p.ws.route[min(tid, ncount - 1)];
    constexpr int kRowsPerWave = (2 * ROWS + kFc2Waves - 1) / kFc2Waves;
    uint32_t mx[kRowsPerWave][kAmaxLoads];
    {
        const BufRes mres = make_res(p.ws.amax, (uint32_t)p.grid13 * 2 * p.T * 4);
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i)
#pragma unroll
            for (int u = 0; u < kAmaxLoads; ++u) {
                const int row = min(wave + kFc2Waves * i, 2 * p.T - 1);
                const int blk = min(lane + 64 * u, p.grid13 - 1);  // repeats are harmless for a max
                // (a row's maxima are contiguous: 256 bytes per load)
                mx[i][u] = __builtin_amdgcn_raw_buffer_load_b32(mres, ((uint32_t)row * p.grid13 + blk) * 4, 0, 0);
            }
    }
    // output-channel scales s2 of the lane's 4 columns of item `it` (0 bytes: none)
    auto s2res = [&](int expert, int it) { return make_res(p.s2 + (size_t)expert * p.K, it >= 0 ? (uint32_t)p.K * 4 : 0u); };
    auto s2off = [&](int it) {
        return (uint32_t)((tile_of(it) / p.nsplit) * kFc2Cols + sub * kTile + 4 * grp) * 4;
    };
    // the shared expert's s2 (0 bytes for a block that starts later)
    float4 s2c = buf_ldf4(make_res(lead_s2e, early ? (uint32_t)p.K * 4 : 0u), s2off(cur));
    float4 av[ROWS][kSliceVec];
#pragma unroll
    for (int q = 0; q < ROWS; ++q)
#pragma unroll
        for (int v = 0; v < kSliceVec; ++v)
            av[q][v] = buf_ldf4(ares, early && q < p.M ? aoff(q, split_of(cur), v) : kOutside);
    __builtin_amdgcn_sched_barrier(0);

    // 2. weights of the first item (WAIT: requested already): its first k-step here, the
    //    second once the B operand is encoded (a wave whose loads back up in the memory
    //    queues cannot issue its prologue's work; this order measured 0.3-1.3 us faster
    //    per step, the bytes in flight still covering the prologue)
    if constexpr (!WAIT) first_weights(lead_w2e, early, 0, 1);
    __builtin_amdgcn_sched_barrier(0);

    // 3. routing table and row scales into LDS (block 0 writes the debug copies of s_a);
    //    FC13's work counter is cleared for the next forward
    if (bid == 0 && tid == 0) atomicExch(p.ws.work + kWorkFc13, 0u);
    int* rt = reinterpret_cast<int*>(lds + L.route);
    float* sa = reinterpret_cast<float*>(lds + L.sa);
    float* rcp = reinterpret_cast<float*>(lds + L.rcp);
    if (tid < ncount) rt[tid] = rtv;
    for (int i = tid + kFc2Threads; i < ncount; i += kFc2Threads) rt[i] = p.ws.route[i];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
        const int row = wave + kFc2Waves * i;
        uint32_t m = 0;
#pragma unroll
        for (int u = 0; u < kAmaxLoads; ++u) m = max(m, mx[i][u]);
        for (int blk = lane + 64 * kAmaxLoads; blk < p.grid13; blk += 64)  // more FC13 blocks
            m = max(m, p.ws.amax[(size_t)min(row, 2 * p.T - 1) * p.grid13 + blk]);
        m = wave_max_u32(m);  // DPP, no LDS round trips (non-negative floats: bit order)
        if (lane == 0 && row < 2 * p.T) {
            // static scale (a variant reading), else fp32(amax / 448) by IEEE division
            const float s = p.a_scale > 0.0f ? p.a_scale : __uint_as_float(m) / kE4M3Max;
            sa[row] = s;
            rcp[row] = s >= kTinyScale ? 1.0f / s : 0.0f;  // below: unused (the lifted exact path)
        }
    }
    lds_barrier();
    if (bid == 0)
        for (int row = tid; row < nrows; row += kFc2Threads) {
            const int tok = row < p.M ? row : rt[rl.row_token() + row];
            float* sd = row < p.M ? p.dbg.sa_shared : p.dbg.sa_routed;
            if (sd) sd[rt[rl.batch_row() + tok]] = sa[row];
        }

    // B codes of item `it` from av into buf; the block whose column tile is 0 also
    // writes them to the debug copies.  A pair close to a rounding midpoint sends the
    // thread through the exact path afterwards, from the same registers (a reload
    // would wait for the weight stream in flight).
    auto encode_b = [&](int it, uint8_t* buf) {
        const int slot = it / per_slot, split = split_of(it);
        const int r0 = rt[rl.slot_row0() + slot], nr = rt[rl.slot_rows() + slot];
        const bool dbg = (tile_of(it) / p.nsplit) == 0 && (slot == 0 ? p.dbg.aq_shared : p.dbg.aq_routed);
        uint64_t redo = 0;  // bit q * kSliceVec + v
#pragma unroll
        for (int q = 0; q < ROWS; ++q) {
            if (q < nr && sa[r0 + q] > 0.0f && sa[r0 + q] < kTinyScale) {
                // a row whose largest magnitude is below about 448 * 2^-96 (never in
                // practice): exact codes over the lifted scale (codec.hpp)
                const float s = sa[r0 + q];
#pragma unroll
                for (int v = 0; v < kSliceVec; ++v) {
                    const int c4 = tid + v * kFc2Threads;
                    uint32_t c = 0;
                    if (split * kFc2Split + 4 * c4 < p.I)
                        c = e4m3_quant2_tiny(av[q][v].x, av[q][v].y, s) |
                            (e4m3_quant2_tiny(av[q][v].z, av[q][v].w, s) << 16);
                    *reinterpret_cast<uint32_t*>(buf + q * kFc2BStride + 4 * c4) = c;
                }
            } else if (q < nr) {
                const float s = sa[r0 + q], r = rcp[r0 + q];
#pragma unroll
                for (int v = 0; v < kSliceVec; ++v) {
                    const int c4 = tid + v * kFc2Threads;  // float4 index in the split
                    uint32_t c = 0;
                    if (split * kFc2Split + 4 * c4 < p.I && s > 0.0f) {
                        const uint32_t c0 = e4m3_quant2_fast<true>(av[q][v].x, av[q][v].y, r);
                        const uint32_t c1 = e4m3_quant2_fast<true>(av[q][v].z, av[q][v].w, r);
                        if (c0 == kQuantExact || c1 == kQuantExact) redo |= 1ull << (q * kSliceVec + v);
                        c = c0 | (c1 << 16);
                    }
                    *reinterpret_cast<uint32_t*>(buf + q * kFc2BStride + 4 * c4) = c;
                }
            }
        }
        if (redo != 0u) {  // unrolled: the values stay in their registers
#pragma unroll
            for (int q = 0; q < ROWS; ++q)
#pragma unroll
                for (int v = 0; v < kSliceVec; ++v) {
                    if (!((redo >> (q * kSliceVec + v)) & 1ull)) continue;
                    const int c4 = tid + v * kFc2Threads;
                    const float s = sa[r0 + q], rr = rcp[r0 + q];
                    const float4 x = av[q][v];
                    *reinterpret_cast<uint32_t*>(buf + q * kFc2BStride + 4 * c4) =
                        e4m3_quant2_exact(x.x, x.y, s, rr) | (e4m3_quant2_exact(x.z, x.w, s, rr) << 16);
                }
        }
        if (dbg) {
            uint8_t* dst = slot == 0 ? p.dbg.aq_shared : p.dbg.aq_routed;
            for (int q = 0; q < nr; ++q) {
                const int tok = rt[rl.batch_row() + (slot == 0 ? q : rt[rl.row_token() + r0 + q])];
                for (int v = 0; v < kSliceVec; ++v) {
                    const int c4 = tid + v * kFc2Threads, col = split * kFc2Split + 4 * c4;
                    if (col < p.I)
                        *reinterpret_cast<uint32_t*>(dst + (size_t)tok * p.I + col) =
                            *reinterpret_cast<const uint32_t*>(buf + q * kFc2BStride + 4 * c4);
                }
            }
        }
    };
    // items of the 1 + d slots
    const EvenPlan plan(G, bid, (1 + rt[rl.d()]) * per_slot);
    const uint8_t* w2first = lead_w2e;  // the first item's expert (packed W2)
    if (!early) {  // the first item is a routed expert's, or there is none (-1)
        cur = plan.fixed(0);
        if (cur >= 0) {  // the loads in the order of the early ones: s2, slice, weights
            const int slot = cur / per_slot;
            const int e0 = __builtin_amdgcn_readfirstlane(rt[rl.slot_expert() + slot]);
            const int r0 = rt[rl.slot_row0() + slot], nr = rt[rl.slot_rows() + slot];
            w2first = p.w2p + (uint64_t)e0 * p.w2_bytes;
            s2c = buf_ldf4(s2res(e0, cur), s2off(cur));
#pragma unroll
            for (int q = 0; q < ROWS; ++q)
#pragma unroll
                for (int v = 0; v < kSliceVec; ++v)
                    av[q][v] = buf_ldf4(ares, q < nr ? aoff(r0 + q, split_of(cur), v) : kOutside);
            __builtin_amdgcn_sched_barrier(0);
            first_weights(w2first, true, 0, WAIT ? kFc2Steps : 1);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    uint8_t* bbuf = lds + L.b;
    if (cur >= 0) encode_b(cur, bbuf);
    if constexpr (!WAIT) first_weights(w2first, cur >= 0, 1, kFc2Steps);  // both kinds of block
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();

    int nxt = plan.fixed(1);  // next item, -1 if none
    float* red = reinterpret_cast<float*>(lds + L.red);
    int par = 0;
    for (int pos = 0; cur >= 0; ++pos) {
        const int slot = cur / per_slot, tile = cur - slot * per_slot;
        const int r0 = rt[rl.slot_row0() + slot], nr = rt[rl.slot_rows() + slot];
        const int nslot = nxt >= 0 ? nxt / per_slot : 0;
        const int nexpert = __builtin_amdgcn_readfirstlane(rt[rl.slot_expert() + nslot]);
        const BufRes rn = wres(nexpert, nxt);
        const uint32_t wo = (uint32_t)step_of(nxt) * kFc2Sub * kBlockBytes + lane * 16;

        // the next item's slice, ahead of the weight reloads
        {
            const BufRes an = nxt >= 0 ? ares : anone;
            const int nr0 = rt[rl.slot_row0() + nslot], nnr = rt[rl.slot_rows() + nslot];
            const int nsp = split_of(nxt);
#pragma unroll
            for (int q = 0; q < ROWS; ++q)
#pragma unroll
                for (int v = 0; v < kSliceVec; ++v) av[q][v] = buf_ldf4(an, q < nnr ? aoff(nr0 + q, nsp, v) : kOutside);
        }
        const float4 s2n = buf_ldf4(s2res(nexpert, nxt), s2off(nxt));
        __builtin_amdgcn_sched_barrier(0);

        const uint8_t* brow = bbuf + par * ROWS * kFc2BStride + min(j, nr - 1) * kFc2BStride +
                              wave * kFc2Steps * kKStep + grp * 32;
        v4f acc[kFc2Sub];
#pragma unroll
        for (int u = 0; u < kFc2Sub; ++u) acc[u] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kFc2Steps; ++s) {
            const Operand bo = widen(*reinterpret_cast<const uint4*>(brow + s * kKStep),
                                     *reinterpret_cast<const uint4*>(brow + s * kKStep + 16));
#pragma unroll
            for (int u = 0; u < kFc2Sub; ++u) acc[u] = mma_kstep(widen(w[s][u][0], w[s][u][1]), bo, acc[u]);
#pragma unroll
            for (int u = 0; u < kFc2Sub; ++u)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    w[s][u][h] = buf_ld16_stream(rn, wo + (s * kFc2Sub + u) * kBlockBytes + h * 1024);
            // keep k-steps in order, so the wave waits for one k-step's loads at a time
            __builtin_amdgcn_sched_barrier(0);
        }

        // B of the next item into the other buffer (last read one item ago)
        if (nxt >= 0) encode_b(nxt, bbuf + (par ^ 1) * ROWS * kFc2BStride);

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
            for (int q = 0; q < 4; ++q) o[q] += rb[((wv * kFc2Sub + sub) * 4 + q) * 64 + lane];
        if (j < nr && wave < kFc2Sub) {
            const int split = tile % p.nsplit;
            const int col = (tile / p.nsplit) * kFc2Cols + sub * kTile + 4 * grp;
            const int row = slot == 0 ? j : p.M + rt[rl.row_token() + r0 + j];  // shared: token j
            const float f = sa[r0 + j];
            float* dst = p.ws.part + ((size_t)split * 2 * p.T + row) * p.K + col;
            const float4 v = make_float4(o[0] * f * s2c.x, o[1] * f * s2c.y, o[2] * f * s2c.z, o[3] * f * s2c.w);
            if constexpr (WAIT) {  // the single launch's combine phase reads them (device scope)
                xstore<true>(dst, v.x);
                xstore<true>(dst + 1, v.y);
                xstore<true>(dst + 2, v.z);
                xstore<true>(dst + 3, v.w);
            } else {
                *reinterpret_cast<float4*>(dst) = v;
            }
        }
        s2c = s2n;
        if (nxt < 0) break;
        cur = nxt;
        nxt = __builtin_amdgcn_readfirstlane(plan.fixed(pos + 2));
        par ^= 1;
    }
}

template <int ROWS>
__global__ __launch_bounds__(kFc2Threads) void fc2_kernel(const int32_t* lead_route, const uint32_t* lead_amax,
                                                          const float* lead_a, const float* lead_s2e,
                                                          const uint8_t* lead_w2e, uint32_t lead_mts,
                                                          uint32_t lead_ki, uint32_t lead_grids, const FwdParams p0) {
    extern __shared__ __align__(16) uint8_t lds[];
    fc2_body<ROWS>(blockIdx.x, lead_route, lead_amax, lead_a, lead_s2e, lead_w2e, lead_mts, lead_ki, lead_grids, p0, lds);
}

// out[m, k] = bf16(y_shared + gate[m] * y_routed), y = the sum over the splits of the
// scaled partial sums (shared: row m, routed: row M + m).  One thread per token and 4
// consecutive columns; every load is independent of the others (one latency level),
// and the splits are added in split order.
constexpr int kCombineBatch = 8;

__device__ __forceinline__ float4 add4(float4 a, float4 b) {
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// All arguments are scalars (preloaded into SGPRs): route = the routing table (RouteLayout
// with T tokens and S slots), gate [T], part [nsplit][2T][K], out [*][K];
// mtn = M | T << 8 | nsplit << 16 | routed << 24, S, K.
__device__ __forceinline__ void combine_store(uint16_t* out, float4 sh, float4 ro, float g) {
    const float y[4] = {sh.x + g * ro.x, sh.y + g * ro.y, sh.z + g * ro.z, sh.w + g * ro.w};
    uint2 packed;
    packed.x = (uint32_t)float_to_bf16(y[0]) | ((uint32_t)float_to_bf16(y[1]) << 16);
    packed.y = (uint32_t)float_to_bf16(y[2]) | ((uint32_t)float_to_bf16(y[3]) << 16);
    *reinterpret_cast<uint2*>(out) = packed;
}

// Output element group `idx` (token idx / (K/4), 4 columns); also the last phase of the
// single launch.
__device__ __forceinline__ void combine_at(int idx, const int32_t* route, const float* gate, const float* part,
                                           uint16_t* out, uint32_t mtn, int32_t S, int32_t K) {
    const int M = (int)(mtn & 0xFFu), T = (int)((mtn >> 8) & 0xFFu), nsplit = (int)((mtn >> 16) & 0xFFu);
    const bool routed = ((mtn >> 24) & 1u) != 0u;
    const bool gate_in = ((mtn >> 25) & 1u) != 0u;  // the gate scaled the routed input instead
    const int k4 = K >> 2;
    if (idx >= M * k4) return;
    const RouteLayout rl{T, S};
    const int tok = idx / k4, col = (idx - tok * k4) * 4;
    const size_t ss = (size_t)2 * T * K;
    const float* ps = part + (size_t)tok * K + col;
    const float* pr = part + (size_t)(M + tok) * K + col;  // without routed experts: read, not added
    float4 sh = make_float4(0.f, 0.f, 0.f, 0.f), ro = sh;
    if (nsplit <= kCombineBatch) {  // I <= 8192: every load of the thread in flight at once
        float4 a[kCombineBatch], b[kCombineBatch];
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u) {
            const int sp = min(u, nsplit - 1);  // repeats past the end are not added
            a[u] = *reinterpret_cast<const float4*>(ps + sp * ss);
            b[u] = *reinterpret_cast<const float4*>(pr + sp * ss);
        }
        const int brow = route[rl.batch_row() + tok];
        const float g = routed ? (gate_in ? 1.0f : gate[tok]) : 0.0f;
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u)
            if (u < nsplit) {
                sh = add4(sh, a[u]);
                ro = add4(ro, b[u]);
            }
        combine_store(out + (size_t)brow * K + col, sh, routed ? ro : make_float4(0.f, 0.f, 0.f, 0.f), g);
        return;
    }
    const int brow = route[rl.batch_row() + tok];
    const float g = routed ? (gate_in ? 1.0f : gate[tok]) : 0.0f;
    for (int s0 = 0; s0 < nsplit; s0 += kCombineBatch) {
        float4 a[kCombineBatch], b[kCombineBatch];
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u) {
            const int sp = min(s0 + u, nsplit - 1);
            a[u] = *reinterpret_cast<const float4*>(ps + sp * ss);
            b[u] = *reinterpret_cast<const float4*>(pr + sp * ss);
        }
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u)
            if (s0 + u < nsplit) {
                sh = add4(sh, a[u]);
                ro = add4(ro, b[u]);
            }
    }
    combine_store(out + (size_t)brow * K + col, sh, routed ? ro : make_float4(0.f, 0.f, 0.f, 0.f), g);
}

__global__ __launch_bounds__(256) void combine_kernel(const int32_t* route, const float* gate, const float* part,
                                                      uint16_t* out, uint32_t mtn, int32_t S, int32_t K) {
    combine_at(blockIdx.x * 256 + threadIdx.x, route, gate, part, out, mtn, S, K);
}

}  // namespace moe
