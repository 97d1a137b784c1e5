// Prologue of the FC13 kernel: top-1 routing with de-duplication of the active
// experts, and per-token dynamic FP8 quantisation of the activations.  Every FC13
// block computes both for itself, into its LDS, while the weights of its first item
// stream in; block 0 also publishes the routing table for the later kernels and the
// debug copies.  The results are deterministic, so all blocks hold the same table.
//
// Routing.  e[m] = the lowest index of the largest logit and gate[m] = sigmoid of
// that logit (the pages only name MoE; top-1 with a sigmoid gate is the reading
// taken).  Counts per expert go to LDS; one block scan over the experts in ascending
// id numbers the active ones 1..d (slot 0 is the shared expert) and gives each its
// range of routed rows; a token's row inside its expert's range is the number of
// earlier tokens routed to the same expert.  Doing this on the device keeps the step
// free of host round trips, as the pages do for their verification logic (Blackwell
// 1,000 TPS/user blog, zh translation, section on CUDA Graphs and the overlap
// scheduler).
//
// Quantisation: s = fp32(amax / 448), q = e4m3(x / s) per token, the quantize step
// placed in front of a GEMM (same page, section "CUDA kernel optimisation and
// fusion", item "operator fusion").
//
// The loads of x and of the logits are issued before the weight stream (prologue_load)
// and consumed after it has been issued (prologue_finish): memory counters retire in
// order, so a load issued after the weights could only be waited for together with
// them.  Inputs larger than the register budget take further rounds of loads, which
// do wait for the weights.
#pragma once

#include "codec.hpp"
#include "layout.hpp"
#include "params.hpp"

namespace moe {

constexpr int kMaxRouteExperts = 1024;
constexpr int kPrologueThreads = 512;
constexpr int kXChunks = 8;      // 16-byte chunks of x (8 bf16) per thread, loaded early
constexpr int kLogitLoads = 4;   // logits (bf16) per thread, loaded early

struct PrologueRegs {
    uint4 x[kXChunks];
    uint32_t lg[kLogitLoads];
};

// LDS the prologue needs besides the route table, sx and xq of the FC13 layout.
struct PrologueLds {
    int* cnt;        // [E] tokens per expert (later reused)
    int* off;        // [E] first routed row of each expert
    uint16_t* lg;    // [M][E] logits
    int* exp;        // [M] chosen expert
    float* gate;     // [M]
    uint32_t* amax;  // [M] max |x| per token (float bits)
    float* rcp;      // [M] fp32(1 / s_x)
    int* tmp;        // [2 * waves] scan scratch
};

__device__ __forceinline__ uint4 load_x_chunk(const FwdParams& p, int c, int nch) {
    return reinterpret_cast<const uint4*>(p.x)[min(c, nch - 1)];  // clamped: in bounds
}

__device__ __forceinline__ uint32_t load_logit(const FwdParams& p, int i, int n) {
    return p.logits[min(i, n - 1)];
}

// Issue the early loads: x chunks tid + 512 i and logits tid + 512 i.
__device__ __forceinline__ void prologue_load(const FwdParams& p, PrologueRegs& r) {
    const int nch = p.M * (p.K >> 3);
#pragma unroll
    for (int i = 0; i < kXChunks; ++i) r.x[i] = load_x_chunk(p, threadIdx.x + i * kPrologueThreads, nch);
    const int nl = p.M * p.E;
    if (nl > 0) {
#pragma unroll
        for (int i = 0; i < kLogitLoads; ++i) r.lg[i] = load_logit(p, threadIdx.x + i * kPrologueThreads, nl);
    }
}

// Exclusive prefix sums over the block of two counters at once; *total gets the sums.
__device__ __forceinline__ int2 block_exclusive_scan2(int a, int b, int* tmp, int2* total) {
    constexpr int kWaves = kPrologueThreads / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int ia = a, ib = b;  // inclusive scan inside the wave
    for (int o = 1; o < 64; o <<= 1) {
        const int ta = __shfl_up(ia, o), tb = __shfl_up(ib, o);
        if (lane >= o) { ia += ta; ib += tb; }
    }
    if (lane == 63) { tmp[wave] = ia; tmp[kWaves + wave] = ib; }
    lds_barrier();
    int pa = 0, pb = 0, sa = 0, sb = 0;
    for (int w = 0; w < kWaves; ++w) {
        if (w < wave) { pa += tmp[w]; pb += tmp[kWaves + w]; }
        sa += tmp[w];
        sb += tmp[kWaves + w];
    }
    *total = make_int2(sa, sb);
    return make_int2(pa + ia - a, pb + ib - b);
}

__device__ __forceinline__ float chunk_absmax(uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float m = 0.0f;
#pragma unroll
    for (int h = 0; h < 4; ++h) m = fmaxf(m, fmaxf(fabsf(u2f(w[h] << 16)), fabsf(u2f(w[h] & 0xFFFF0000u))));
    return m;
}

// Codes of a chunk's 8 values: e4m3(x / s) with r = fp32(1 / s); zeros when s == 0.
// Returns false when a pair needs the exact path (the caller redoes the chunk).
__device__ __forceinline__ bool chunk_encode_fast(uint4 v, float s, float r, uint2* out) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t c[4] = {0u, 0u, 0u, 0u};
    bool ok = true;
    if (s > 0.0f) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            c[h] = e4m3_quant2_fast(u2f(w[h] << 16), u2f(w[h] & 0xFFFF0000u), r);
            ok = ok && c[h] != kQuantExact;
        }
    }
    *out = make_uint2(c[0] | (c[1] << 16), c[2] | (c[3] << 16));
    return ok;
}

__device__ __forceinline__ uint2 chunk_encode_exact(uint4 v, float s) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t c[4] = {0u, 0u, 0u, 0u};
    if (s > 0.0f)
        for (int h = 0; h < 4; ++h)
            c[h] = e4m3_encode_div(u2f(w[h] << 16), s) | (e4m3_encode_div(u2f(w[h] & 0xFFFF0000u), s) << 8);
    return make_uint2(c[0] | (c[1] << 16), c[2] | (c[3] << 16));
}

// Max |x| of the chunks into amax[token] (LDS, float bits): a wave whose 64 chunks all
// belong to one token reduces across lanes first and issues a single LDS atomic.
__device__ __forceinline__ void chunk_max_to_lds(float m, int c, int nch, int cpr, uint32_t* amax) {
    const int t = min(c, nch - 1) / cpr;
    const int t0 = __builtin_amdgcn_readfirstlane(t);
    if (__ballot(t != t0) == 0) {
        for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
        if ((threadIdx.x & 63) == 0 && m > 0.0f) atomicMax(amax + t0, __float_as_uint(m));
    } else if (c < nch && m > 0.0f) {
        atomicMax(amax + t, __float_as_uint(m));
    }
}

// Routing table into `rt` (LDS, RouteLayout), token scales into `sx`, token codes into
// `xq` (row stride xstride bytes).  Ends with a block barrier.  The barriers here order
// LDS only (lds_barrier), so the weight loads issued before stay in flight.
__device__ void prologue_finish(const FwdParams& p, PrologueRegs& r, const PrologueLds& L, int* rt,
                                float* sx, uint8_t* xq, int xstride) {
    const int tid = threadIdx.x;
    const RouteLayout rl{p.T, p.S};
    const int cpr = p.K >> 3;  // chunks per token row
    const int nch = p.M * cpr;
    const int xrounds = (nch + kXChunks * kPrologueThreads - 1) / (kXChunks * kPrologueThreads);
    const int nl = p.M * p.E;

    // 1. logits into LDS, per-token amax cleared, expert counts cleared
    if (nl > 0) {
#pragma unroll
        for (int i = 0; i < kLogitLoads; ++i) {
            const int k = tid + i * kPrologueThreads;
            if (k < nl) L.lg[k] = (uint16_t)r.lg[i];
        }
        for (int k = tid + kLogitLoads * kPrologueThreads; k < nl; k += kPrologueThreads) L.lg[k] = p.logits[k];
    }
    for (int e = tid; e < p.E; e += kPrologueThreads) L.cnt[e] = 0;
    if (tid < p.M) L.amax[tid] = 0u;
    lds_barrier();

    // 2. per-token max |x| (LDS max on the bit patterns of non-negative floats).  One
    //    round uses the chunks loaded early; larger inputs reload chunk by chunk, each
    //    used where it is loaded, so that no load is left pending where the paths join
    if (xrounds == 1) {
#pragma unroll
        for (int i = 0; i < kXChunks; ++i) {
            const int c = tid + i * kPrologueThreads;
            if (i * kPrologueThreads < nch)  // uniform: whole waves take part in the reduction
                chunk_max_to_lds(c < nch ? chunk_absmax(r.x[i]) : 0.0f, c, nch, cpr, L.amax);
        }
    } else {
        for (int c0 = 0; c0 < nch; c0 += kPrologueThreads) {
            const int c = c0 + tid;
            chunk_max_to_lds(c < nch ? chunk_absmax(load_x_chunk(p, c, nch)) : 0.0f, c, nch, cpr, L.amax);
        }
    }
    // 3. arg-max per token: one wave per token, lanes scan experts lane, lane + 64, ...
    //    keeping the first maximum; the butterfly keeps the lower index on equal values
    const int lane = tid & 63, wave = tid >> 6;
    if (p.E > 0) {
        for (int m = wave; m < p.M; m += kPrologueThreads / 64) {
            float bv = -INFINITY;
            int bi = 0x7FFFFFFF;
            for (int e = lane; e < p.E; e += 64) {
                const float v = bf16_to_float(L.lg[m * p.E + e]);
                if (v > bv || bi == 0x7FFFFFFF) { bv = v; bi = e; }
            }
            for (int o = 32; o > 0; o >>= 1) {
                const float ov = __shfl_xor(bv, o);
                const int oi = __shfl_xor(bi, o);
                if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
            }
            if (lane == 0) {
                L.exp[m] = bi;
                L.gate[m] = 1.0f / (1.0f + expf(-bv));
            }
        }
    }
    lds_barrier();

    // 4. token scales and their reciprocals; tokens per expert
    if (tid < p.M) {
        const float s = __uint_as_float(L.amax[tid]) / kE4M3Max;  // IEEE division: fp32(amax / 448)
        sx[tid] = s;
        L.rcp[tid] = s > 0.0f ? 1.0f / s : 0.0f;
    }
    if (p.E > 0)
        for (int m = tid; m < p.M; m += kPrologueThreads) atomicAdd(&L.cnt[L.exp[m]], 1);
    lds_barrier();

    // 5. token codes.  Chunks with a pair close to a rounding midpoint are redone on the
    //    exact path afterwards, from x reloaded (rare; kept out of the unrolled code)
    uint32_t redo = 0;  // bit i: chunk tid + i * 512 (first round only)
    if (xrounds == 1) {
#pragma unroll
        for (int i = 0; i < kXChunks; ++i) {
            const int c = tid + i * kPrologueThreads;
            if (c < nch) {
                const int t = c / cpr, jj = c - t * cpr;
                uint2 q;
                if (!chunk_encode_fast(r.x[i], sx[t], L.rcp[t], &q)) redo |= 1u << i;
                *reinterpret_cast<uint2*>(xq + t * xstride + jj * 8) = q;
            }
        }
    } else {
        redo = ~0u;  // larger inputs: every chunk on the exact path
    }
    if (redo != 0u) {
#pragma unroll 1
        for (int c = tid; c < nch; c += kPrologueThreads) {
            const int i = (c - tid) / kPrologueThreads;
            if (i < 32 && !((redo >> i) & 1u)) continue;
            const int t = c / cpr, jj = c - t * cpr;
            *reinterpret_cast<uint2*>(xq + t * xstride + jj * 8) = chunk_encode_exact(load_x_chunk(p, c, nch), sx[t]);
        }
    }

    // 6. slots: thread t owns experts [2t, 2t + 2) and numbers the active ones
    if (p.E == 0) {  // dense: the shared expert alone
        if (tid == 0) {
            rt[rl.d()] = 0;
            rt[rl.slot_expert()] = 0;
            rt[rl.slot_row0()] = 0;
            rt[rl.slot_rows()] = p.M;
        }
        for (int m = tid; m < p.M; m += kPrologueThreads) {
            rt[rl.token_row() + m] = -1;
            rt[rl.token_expert() + m] = -1;
            rt[rl.row_token() + m] = m;
            L.gate[m] = 0.0f;
        }
    } else {
        constexpr int kPer = kMaxRouteExperts / kPrologueThreads;
        int act = 0, rows = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = tid * kPer + i;
            const int c = e < p.E ? L.cnt[e] : 0;
            act += c > 0;
            rows += c;
        }
        int2 tot;
        const int2 pre = block_exclusive_scan2(act, rows, L.tmp, &tot);
        int slot = 1 + pre.x, row = p.M + pre.y;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = tid * kPer + i;
            const int c = e < p.E ? L.cnt[e] : 0;
            if (c > 0) {
                rt[rl.slot_expert() + slot] = e;
                rt[rl.slot_row0() + slot] = row;
                rt[rl.slot_rows() + slot] = c;
                L.off[e] = row;
                ++slot;
                row += c;
            }
        }
        if (tid == 0) {
            rt[rl.d()] = tot.x;
            rt[rl.slot_expert()] = p.E;  // the shared expert's packed index
            rt[rl.slot_row0()] = 0;
            rt[rl.slot_rows()] = p.M;
        }
        lds_barrier();
        for (int m = tid; m < p.M; m += kPrologueThreads) {
            const int e = L.exp[m];
            int before = 0;
            for (int k = 0; k < m; ++k) before += L.exp[k] == e;
            const int rr = L.off[e] + before;
            rt[rl.token_row() + m] = rr;
            rt[rl.token_expert() + m] = e;
            rt[rl.row_token() + rr] = m;
            rt[rl.row_token() + m] = m;
        }
    }
    lds_barrier();

    // 7. block 0 publishes the table, the gates and the debug copies
    if (blockIdx.x == 0) {
        for (int i = tid; i < rl.count(); i += kPrologueThreads) p.ws.route[i] = rt[i];
        for (int m = tid; m < p.M; m += kPrologueThreads) {
            p.ws.gate[m] = L.gate[m];
            if (p.dbg.sx) p.dbg.sx[m] = sx[m];
            if (p.dbg.expert) p.dbg.expert[m] = p.E > 0 ? L.exp[m] : -1;
            if (p.dbg.gate) p.dbg.gate[m] = L.gate[m];
        }
        if (tid == 0 && p.dbg.num_active) p.dbg.num_active[0] = rt[rl.d()];
        if (p.dbg.xq)
            for (int c = tid; c < nch; c += kPrologueThreads) {
                const int t = c / cpr, jj = c - t * cpr;
                reinterpret_cast<uint2*>(p.dbg.xq)[c] = *reinterpret_cast<const uint2*>(xq + t * xstride + jj * 8);
            }
    }
}

}  // namespace moe
