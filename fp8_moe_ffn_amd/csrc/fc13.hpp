// First kernel of the forward: routing and activation quantisation (prologue.hpp),
// then the FC13 GEMM (gate and up projections side by side) with SwiGLU applied in
// its epilogue, for the shared expert and every distinct routed expert.  The pages
// fuse SwiGLU into the GEMM in front of it (Blackwell 1,000 TPS/user blog, zh
// translation, section "CUDA kernel optimisation and fusion", item "operator
// fusion") and build low-latency GEMMs that load weights so as to use the whole HBM
// bandwidth (same section, item on spatial partitioning and efficient memory loads).
//
// gfx950 design.  At M <= 16 tokens the GEMM is a weight stream.  A work item is one
// "pair" (16 gate + 16 up channels) of one active expert over the whole hidden size K;
// items are numbered slot-major, (1 + d) * I/16 of them.  Blocks are persistent (as
// many as are resident at once, at most the items the largest step has); block b takes
// items b, b + G, b + 2G, ... for all but its last two or so positions, which come from
// a pool through a work counter (ItemPlan): blocks whose share of the bandwidth is
// smaller take fewer of them.  A ticket is requested two items ahead, before that item's
// weight reloads, so its latency hides under an item.  The first item of block b < I/16
// belongs to the shared expert, so its weights are requested before the routing is
// known; the routing and the token codes are computed in the block's prologue while
// those bytes arrive.  At small I (fewer than G pairs per expert) the other blocks start
// on routed experts' pairs, requested once the prologue has the routing.
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
// bytes: zeros, no memory access); the routing table, activation codes and scales
// live in LDS.
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
// writes its per-row maxima to its own column of ws.amax (row-major by intermediate row,
// so that the re-quantisation reads each row's maxima over the blocks contiguously) and
// the re-quantisation takes the max over the blocks.  No global atomics sit on the streaming path.
#pragma once

#include "codec.hpp"
#include "layout.hpp"
#include "params.hpp"
#include "prologue.hpp"

namespace moe {

constexpr int kFc13Waves = 8;
constexpr int kFc13Threads = kFc13Waves * 64;
static_assert(kFc13Threads == kPrologueThreads, "the prologue runs on the FC13 block");

__host__ __device__ constexpr int align16(int v) { return (v + 15) & ~15; }

// LDS layout of fc13_swiglu_kernel, in bytes.
struct Fc13Lds {
    int red;    // [2][WAVES][8][64] float partial tiles
    int rowmax; // [2T] uint32: the block's max |a| per row (float bits)
    int ring;   // [4] int: items of the next positions drawn from the pool
    int route;  // RouteLayout table
    int sx;     // [M] float
    int pro;    // prologue scratch: exp[T], gate[T], amaxp[T][kMaxParts], ssqp[T][kMaxParts] (f64)
    int nw;     // [K] bf16 norm weight (with the fused RMSNorm only)
    int xq;     // [M][K + 16] token codes (row stride padded against bank conflicts)
    int xs;     // chunks of x loaded early into LDS (x_stage_bytes; -1: none)
    int total;
};

__host__ __device__ inline Fc13Lds fc13_lds(int T, int S, int E, int M, int K, bool rms = false) {
    Fc13Lds l{};
    int off = 0;
    l.red = off;
    off += 2 * kFc13Waves * 8 * 64 * 4;
    l.rowmax = off;
    off = align16(off + 2 * T * 4);
    l.ring = off;
    off += 16;
    l.route = off;
    off = align16(off + RouteLayout{T, S}.count() * 4);
    l.sx = off;
    off = align16(off + M * 4);
    l.pro = off;
    off = align16(off + (2 + kMaxParts) * T * 4);
    off = align16(off + kMaxParts * T * 8);  // ssqp
    l.nw = off;
    if (rms) off = align16(off + K * 2);
    l.xq = off;
    off = align16(off + M * (K + 16));
    const int xsb = x_stage_bytes(M, K);
    l.xs = xsb > 0 ? off : -1;
    off += xsb;
    l.total = off;
    return l;
}

__device__ __forceinline__ PrologueLds prologue_lds(uint8_t* lds, const Fc13Lds& L, int T, bool rms) {
    PrologueLds q;
    int* pro = reinterpret_cast<int*>(lds + L.pro);
    q.exp = pro;
    q.gate = reinterpret_cast<float*>(pro + T);
    q.amaxp = reinterpret_cast<uint32_t*>(pro + 2 * T);
    q.ssqp = reinterpret_cast<double*>(lds + align16(L.pro + (2 + kMaxParts) * T * 4));
    q.nw = rms ? lds + L.nw : nullptr;
    q.xs = L.xs >= 0 ? lds + L.xs : nullptr;
    return q;
}

// The leading arguments repeat what the first loads need from p (x, the token rows, the
// logits, the shared expert's weights, the norm weight, the sizes and mode, the grid);
// they are preloaded into SGPRs, where p is fetched from memory first (about a
// microsecond).  lead_mts = M | T << 8 | S << 16 | (fused RMSNorm) << 24.
// The kernel's body, for block `bid` of G; also the first phase of the single launch
// (XD: what the next phase reads is stored at device scope).  XE: the early chunks of x a
// prologue lane holds (prologue.hpp).
template <int NSTEP, bool FULL, bool RMS, bool XD = false, int XE = kXEarly>
__device__ __forceinline__ void fc13_body(int bid, const uint16_t* lead_x, const int32_t* lead_tok,
                                          const uint16_t* lead_logits, const uint8_t* lead_w13e,
                                          const uint16_t* lead_normw, uint32_t lead_mts, uint32_t lead_ki,
                                          uint32_t lead_eg, const FwdParams& p0, uint8_t* lds) {
    FwdParams p = p0;
    p.x = lead_x;
    p.tok = lead_tok;
    p.logits = lead_logits;
    p.M = (int)(lead_mts & 0xFFu);
    p.T = (int)((lead_mts >> 8) & 0xFFu);
    p.S = (int)((lead_mts >> 16) & 0xFFu);
    p.K = (int)(lead_ki & 0xFFFFu);
    p.I = (int)(lead_ki >> 16);
    p.E = (int)(lead_eg & 0xFFFFu);
    p.norm_w = lead_normw;
    constexpr bool rms = RMS;  // lead_mts bit 24 says the same
    const RouteLayout rl{p.T, p.S};
    const int npairs = p.I >> 4;
    const int G = (int)(lead_eg >> 16);  // gridDim.x
    const int KS = p.K >> 7;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int s0 = wave * NSTEP;  // first k-step of this wave
    const int ns = FULL ? NSTEP : max(0, min(NSTEP, KS - s0));
    const Fc13Lds L = fc13_lds(p.T, p.S, p.E, p.M, p.K, rms);
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

    // 1. early loads of x and the logits, then the first item's weights and scales when
    //    they are the shared expert's (packed index E): block b's first item is item b,
    //    one of the shared expert's pairs for b < I/16.  A block past those (a grid larger
    //    than I/16, at small I) starts on a routed expert's pair, requested after the
    //    routing is known.
    //    The loads are issued by every block, with 0-byte resources (zeros, no memory
    //    access) in a block that starts later, so that both kinds of block reach the
    //    prologue with the same loads outstanding in the same order: the waits the
    //    compiler places where the two meet stay exact.
    PrologueRegs pr;
    prologue_load<RMS, XE>(p, pr, rms ? lds + L.nw : nullptr, L.xs >= 0 ? lds + L.xs : nullptr);
    __builtin_amdgcn_sched_barrier(0);
    //    A wave whose loads back up in the memory queues cannot issue its prologue's work,
    //    and the prologue's block barriers wait for the wave that is last to get its loads
    //    accepted (a CU's loads enter the memory system at its share of the HBM drain
    //    rate).  So the first item's k-steps are requested in three parts: kPreA before
    //    the prologue, the rest but the last at the prologue's first barrier (after the
    //    token maxima and the routing keys), the last after the prologue.  Against all but
    //    the last before it, at hidden 5120: 0.8-2.1 us faster per step.
    constexpr int kPre = NSTEP > 1 ? NSTEP - 1 : NSTEP;  // k-steps requested by the prologue's end
    constexpr int kPreA = kPre < 2 ? kPre : 2;           // ... of them before it
    int cur = bid;
    const bool early = bid < npairs;
    uint4 w[NSTEP][4];
    float sg, su;
    const BufRes rw0 = make_res(lead_w13e + (uint64_t)(early ? cur : 0) * pair_bytes, early ? pair_bytes : 0u);
    {  // the shared expert's pair; its two scales after the weights (their base comes from
       // p, fetched meanwhile; they are used last)
#pragma unroll
        for (int s = 0; s < kPreA; ++s)
            if (FULL || s < ns)
#pragma unroll
                for (int q = 0; q < 4; ++q) w[s][q] = buf_ld16_stream(rw0, woff + s * 2 * kBlockBytes + q * 1024);
        const BufRes rs = sres(p.E, early ? cur : -1);
        sg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, soff(cur), 0, 0));
        su = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, soff(cur) + p.I * 4, 0, 0));
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. routing, token scales and codes into LDS while the weights arrive
    for (int i = threadIdx.x; i < 2 * p.T; i += kFc13Threads)
        reinterpret_cast<uint32_t*>(lds + L.rowmax)[i] = 0u;
    prologue_finish<RMS, XD, XE>(p, pr, prologue_lds(lds, L, p.T, rms), reinterpret_cast<int*>(lds + L.route),
                    reinterpret_cast<float*>(lds + L.sx), lds + L.xq, xstride, bid == 0, [&] {
#pragma unroll
                        for (int s = kPreA; s < kPre; ++s)
                            if (FULL || s < ns)
#pragma unroll
                                for (int q = 0; q < 4; ++q)
                                    w[s][q] = buf_ld16_stream(rw0, woff + s * 2 * kBlockBytes + q * 1024);
                        __builtin_amdgcn_sched_barrier(0);
                    });
#pragma unroll
    for (int s = kPre; s < NSTEP; ++s)  // the first item's last k-step
        if (FULL || s < ns)
#pragma unroll
            for (int q = 0; q < 4; ++q) w[s][q] = buf_ld16_stream(rw0, woff + s * 2 * kBlockBytes + q * 1024);
    __builtin_amdgcn_sched_barrier(0);

    const int* rt = reinterpret_cast<const int*>(lds + L.route);
    const float* sxl = reinterpret_cast<const float*>(lds + L.sx);
    const float* gatel = prologue_lds(lds, L, p.T, rms).gate;
    uint32_t* rowmax = reinterpret_cast<uint32_t*>(lds + L.rowmax);
    float* red = reinterpret_cast<float*>(lds + L.red);
    int* ring = reinterpret_cast<int*>(lds + L.ring);
    const ItemPlan plan(G, bid, (1 + rt[rl.d()]) * npairs, true);  // pairs of the 1 + d slots
    if (!early) {  // the first item is a routed expert's pair, or there is none (-1)
        cur = plan.fixed(0);
        if (cur >= 0) {
            const int e0 = __builtin_amdgcn_readfirstlane(rt[rl.slot_expert() + cur / npairs]);
            const BufRes rw = wres(e0, cur);
#pragma unroll
            for (int s = 0; s < NSTEP; ++s)
                if (FULL || s < ns)
#pragma unroll
                    for (int q = 0; q < 4; ++q) w[s][q] = buf_ld16_stream(rw, woff + s * 2 * kBlockBytes + q * 1024);
            const BufRes rs = sres(e0, cur);
            sg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, soff(cur), 0, 0));
            su = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, soff(cur) + p.I * 4, 0, 0));
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    int nxt = plan.fixed(1);  // next item, -1 if none
    int par = 0;
    for (int pos = 0; cur >= 0; ++pos) {
        // ticket for the item two positions ahead, taken before this item's reloads so
        // that its return does not wait for them; published through LDS at the barrier
        const bool take = plan.pooled(pos + 2);
        uint32_t ticket = 0;
        if (take && threadIdx.x == 0) ticket = atomicAdd(p.ws.work + kWorkFc13, 1u);

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
                for (int q = 0; q < 4; ++q) w[s][q] = buf_ld16_stream(rn, woff + s * 2 * kBlockBytes + q * 1024);
            }
            // keep k-steps in order, so the wave waits for one k-step's loads at a time
            __builtin_amdgcn_sched_barrier(0);
        }

        if (take && threadIdx.x == 0) ring[(pos + 2) & 3] = plan.from_ticket(ticket);

        // reduce the WAVES partial tiles
        float* rb = red + par * (kFc13Waves * 8 * 64);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            rb[(wave * 8 + q) * 64 + lane] = accg[q];
            rb[(wave * 8 + 4 + q) * 64 + lane] = accu[q];
        }
        lds_barrier();
        float g = 0.0f, u = 0.0f;
#pragma unroll
        for (int wv = 0; wv < kFc13Waves; ++wv) {
            g += rb[(wv * 8 + r) * 64 + lane];
            u += rb[(wv * 8 + 4 + r) * 64 + lane];
        }
        // channel 16 * pair + 4 * grp + r of row r0 + j; a routed row's scale takes the
        // gate when it scales the input (a variant reading: then h = gate * s_x * ...)
        const float sx = (p.gate_input && slot > 0) ? sxl[tok] * gatel[tok] : sxl[tok];
        g = g * sx * sg;
        u = u * sx * su;
        const float a = g / (1.0f + expf(-g)) * u;
        float amax = j < nr ? fabsf(a) : 0.0f;
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        if (wave < 4) {
            if (j < nr) xstore<XD>(p.ws.a + (size_t)(r0 + j) * p.I + pair * 16 + 4 * grp + r, a);
            if (lane < 16 && j < nr && amax > 0.0f) atomicMax(rowmax + r0 + j, __float_as_uint(amax));
        }
        if (nxt < 0) break;
        cur = nxt;
        nxt = __builtin_amdgcn_readfirstlane(take ? ring[(pos + 2) & 3] : plan.fixed(pos + 2));
        sg = nsg;
        su = nsu;
        par ^= 1;
    }
    lds_barrier();
    for (int i = threadIdx.x; i < 2 * p.T; i += kFc13Threads)
        xstore<XD>(p.ws.amax + (size_t)i * G + bid, rowmax[i]);
}

template <int NSTEP, bool FULL, bool RMS, int XE = kXEarly>
__global__ __launch_bounds__(kFc13Threads) void fc13_swiglu_kernel(
    const uint16_t* lead_x, const int32_t* lead_tok, const uint16_t* lead_logits, const uint8_t* lead_w13e,
    const uint16_t* lead_normw, uint32_t lead_mts, uint32_t lead_ki, uint32_t lead_eg, const FwdParams p0) {
    extern __shared__ __align__(16) uint8_t lds[];
    fc13_body<NSTEP, FULL, RMS, false, XE>(blockIdx.x, lead_x, lead_tok, lead_logits, lead_w13e, lead_normw, lead_mts,
                                           lead_ki, lead_eg, p0, lds);
}

}  // namespace moe
