// Prologue of the FC13 kernel: top-1 routing with de-duplication of the active
// experts, and per-token dynamic FP8 quantisation of the activations.  Every FC13
// block computes both for itself, into its LDS, while the weights of its first item
// stream in; block 0 also publishes the routing table for the later kernels and the
// debug copies.  The results are deterministic, so all blocks hold the same table.
//
// Routing.  e[m] = the lowest index of the largest logit and gate[m] = sigmoid of
// that logit (the pages only name MoE; top-1 with a sigmoid gate is the reading
// taken).  The distinct experts are numbered 1..d in ascending id (slot 0 is the
// shared expert); each gets the range of routed rows of its tokens, and a token's row
// inside that range is the number of earlier tokens routed to the same expert.
// Nothing depends on arrival order, so the table is deterministic.  Doing this on the
// device keeps the step free of host round trips, as the pages do for their
// verification logic (Blackwell 1,000 TPS/user blog, zh translation, section on CUDA
// Graphs and the overlap scheduler).
//
// Quantisation: s = fp32(amax / 448), q = e4m3(x / s) per token, the quantize step
// placed in front of a GEMM (same page, section "CUDA kernel optimisation and
// fusion", item "operator fusion").
//
// gfx950 layout of the work.  While the weight stream is in flight every global access
// waits in the memory queues, so the prologue is built as short dependency chains:
// each wave works on one token (or one part of it), a lane reduces its own values in
// registers, and a wave finishes a reduction with DPP row shifts and broadcasts (no
// LDS round trips).  The arg-max reduces one 32-bit key per lane, (orderable bf16
// bits << 16) | (0xFFFF - expert), whose maximum is the largest logit with the lowest
// index.  With at most 16 tokens the routing table is built by one wave in O(M)
// lane reads and a ballot, without a scan over the experts.  Two block barriers in all.
//
// The loads of x and of the logits are issued before the weights (prologue_load) and
// consumed after them (prologue_finish): memory counters retire in order, so a load
// issued after the weights could only be waited for together with them.  A lane keeps
// kXChunks chunks of its wave's first unit in registers; up to kXStage more go
// straight from memory into LDS (a direct load, no registers), also ahead of the
// weights, which covers up to 8 tokens at hidden size 5120.  Inputs beyond that are
// loaded later, each where it is used.
#pragma once

#include "codec.hpp"
#include "layout.hpp"
#include "params.hpp"

namespace moe {

constexpr int kMaxRouteExperts = 1024;
constexpr int kPrologueThreads = 512;
constexpr int kPrologueWaves = kPrologueThreads / 64;
constexpr int kXChunks = 8;     // 16-byte chunks of x (8 bf16) per lane, loaded early
constexpr int kXStage = 2;      // further chunks per lane loaded early into LDS
constexpr int kXEarly = kXChunks + kXStage;
constexpr int kLogitLoads = 2;  // logits per lane loaded early (experts lane, lane + 64)
constexpr int kMaxParts = kPrologueWaves;

struct PrologueRegs {
    uint4 x[kXChunks];
    uint32_t lg[kLogitLoads];
    int tok;  // batch row of the launch's token (lane mod 16)
};

// Batch row of the launch's token m (wave-uniform), from the lanes' rows.
__device__ __forceinline__ int batch_row_of(int tok, int m) {
    return __builtin_amdgcn_readlane(tok, __builtin_amdgcn_readfirstlane(m));
}

// LDS the prologue needs besides the route table, sx and xq of the FC13 layout.
struct PrologueLds {
    int* exp;           // [T] chosen expert
    float* gate;        // [T]
    uint32_t* amaxp;    // [T][kMaxParts] max |x| per token and part (float bits)
    double* ssqp;       // [T][kMaxParts] sum of x^2 per token and part (RMSNorm)
    const uint8_t* nw;  // [K] bf16 norm weight, staged by the prologue (RMSNorm), else null
    const uint8_t* xs;  // [waves][kXStage][64] 16-byte chunks of x loaded early, or null
};

// Work split of the x quantisation: P = max(1, 8 / M) waves ("parts") per token.
// Unit u = wave + 8t (t = 0, 1, ...) while u < M * P is token u % M, part u / M; a
// lane of a unit owns chunks j = part * 64 + lane + 64 * P * i of the token's row.
struct XSplit {
    int P, units, cpr;
    __host__ __device__ XSplit(int M, int K) {
        P = M < kPrologueWaves ? kPrologueWaves / M : 1;
        units = M * P;
        cpr = K >> 3;
    }
    __device__ int chunk(int part, int lane, int i) const { return part * 64 + lane + 64 * P * i; }
    __host__ __device__ int per_lane() const { return (cpr + 64 * P - 1) / (64 * P); }
};

// Bytes of LDS for the chunks of x loaded early into LDS: needed when a lane's chunks
// exceed the registers but not the registers and the LDS slots together.
__host__ __device__ inline int x_stage_bytes(int M, int K) {
    const int n = XSplit(M, K).per_lane();
    return n > kXChunks && n <= kXEarly ? kPrologueWaves * kXStage * 64 * 16 : 0;
}

// LDS slot of early chunk i >= kXChunks of a lane
__device__ __forceinline__ int x_stage_off(int wave, int lane, int i) {
    return ((wave * kXStage + (i - kXChunks)) * 64 + lane) * 16;
}

// Early chunk i of the lane's first unit: registers, then the LDS slots.
__device__ __forceinline__ uint4 early_chunk(const PrologueRegs& r, const uint8_t* xs, int wave, int lane, int i) {
    return i < kXChunks ? r.x[i] : *reinterpret_cast<const uint4*>(xs + x_stage_off(wave, lane, i));
}


// Chunk j of batch row `row` of x.
__device__ __forceinline__ uint4 load_x_chunk(const FwdParams& p, int row, int j, int cpr) {
    return reinterpret_cast<const uint4*>(p.x)[(size_t)row * cpr + min(j, cpr - 1)];  // clamped: in bounds
}

// Orderable key of a bf16 logit of expert e (see the header); 0 is below every key.
__device__ __forceinline__ uint32_t logit_key(uint32_t b, int e) {
    b = (b == 0x8000u) ? 0u : b;  // -0 compares equal to +0
    const uint32_t o = (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
    return (o << 16) | (0xFFFFu - (uint32_t)e);
}

__device__ __forceinline__ float key_logit(uint32_t key) {
    const uint32_t o = key >> 16;
    const uint32_t b = (o & 0x8000u) ? (o & 0x7FFFu) : (~o & 0xFFFFu);
    return bf16_to_float((uint16_t)b);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max(uint32_t v) {
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false));
}

// Maximum of v over the wave (unsigned; 0 is the identity): prefix maxima inside each
// row of 16 lanes (row_shr 1, 2, 4, 8), then row 0/2's maximum into rows 1/3
// (row_bcast:15) and row 1's into rows 2 and 3 (row_bcast:31); lane 63 holds the result.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = dpp_max<0x111, 0xF>(v);
    v = dpp_max<0x112, 0xF>(v);
    v = dpp_max<0x114, 0xF>(v);
    v = dpp_max<0x118, 0xF>(v);
    v = dpp_max<0x142, 0xA>(v);
    v = dpp_max<0x143, 0xC>(v);
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Issue the early loads: this wave's first unit's x chunks and its first token's logits.
// A launch over rows of a larger batch first loads the rows of its tokens (at the
// kernel's start, nothing else is in flight yet).  With the norm (nw != null), the norm
// weight is first copied into LDS straight from memory (16 bytes per lane, no
// registers); it is issued before x, so once a wave has its x chunks, its share of the
// copy has landed too (memory counters retire in order).  With xst != null, chunks
// kXChunks.. of the wave's first unit go to LDS at xst the same way, but as buffer
// loads: a flat load into LDS issued after the token-row wait would make the compiler
// wait for every load at the next use of x.
// XE (at most kXEarly): the early chunks a lane holds, as many as its unit needs for the
// launch's tokens (XSplit::per_lane) or more; the kernel is compiled for it, so that no
// instruction is spent on chunks that cannot be there.
template <bool RMS, int XE = kXEarly>
__device__ __forceinline__ void prologue_load(const FwdParams& p, PrologueRegs& r, uint8_t* nw, uint8_t* xst) {
    static_assert(XE >= 1 && XE <= kXEarly, "early chunks");
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const XSplit xs(p.M, p.K);
    if (RMS)
        for (int c = threadIdx.x; c < xs.cpr; c += kPrologueThreads)  // lanes write consecutive 16 B
            __builtin_amdgcn_global_load_lds(p.norm_w + (size_t)c * 8, (lds_u8*)nw + c * 16, 16, 0, 0);
    r.tok = lane & (kTile - 1);  // M <= kTile
    if (p.tok) r.tok = p.tok[min(r.tok, p.M - 1)];
    const int u = min(wave, xs.units - 1);  // waves without a unit repeat the last one's loads
    const int xrow = batch_row_of(r.tok, u % p.M);
#pragma unroll
    for (int i = 0; i < (XE < kXChunks ? XE : kXChunks); ++i)
        r.x[i] = load_x_chunk(p, xrow, xs.chunk(u / p.M, lane, i), xs.cpr);
    if (XE > kXChunks && xst != nullptr) {  // chunks past the row read as zeros, without a memory access
        const BufRes xr = make_res(reinterpret_cast<const uint4*>(p.x) + (size_t)xrow * xs.cpr, (uint32_t)xs.cpr * 16);
#pragma unroll
        for (int i = kXChunks; i < XE; ++i)
            buf_ld16_lds(xr, xst + x_stage_off(wave, lane, i), (uint32_t)xs.chunk(u / p.M, lane, i) * 16);
    }
    if (p.E > 0) {
        const uint16_t* row = p.logits + (size_t)batch_row_of(r.tok, min(wave, p.M - 1)) * p.E;
#pragma unroll
        for (int i = 0; i < kLogitLoads; ++i) r.lg[i] = row[min(lane + 64 * i, p.E - 1)];
    }
}

__device__ __forceinline__ float chunk_absmax(uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float m = 0.0f;
#pragma unroll
    for (int h = 0; h < 4; ++h) m = fmaxf(m, fmaxf(fabsf(u2f(w[h] << 16)), fabsf(u2f(w[h] & 0xFFFF0000u))));
    return m;
}

// Codes of a chunk's 8 values: e4m3(x / s) with r = fp32(1 / s); zeros when s == 0.
// Returns false when a pair needs the exact path (the caller redoes the chunk).  The
// values are used on every path (s == 0 is a select at the end), so a load feeding
// them is never left pending.  lift: the values are multiplied by it first (kTinyLift
// with a lifted scale s, codec.hpp; else 1).
template <bool SAT>
__device__ __forceinline__ bool chunk_encode_fast(uint4 v, float s, float r, uint2* out, float lift = 1.0f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t c[4];
    bool ok = true;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        c[h] = e4m3_quant2_fast<SAT>(u2f(w[h] << 16) * lift, u2f(w[h] & 0xFFFF0000u) * lift, r);
        ok = ok && c[h] != kQuantExact;
    }
    const bool live = s > 0.0f;
    *out = live ? make_uint2(c[0] | (c[1] << 16), c[2] | (c[3] << 16)) : make_uint2(0u, 0u);
    return ok || !live;
}

// The early chunks of a unit (bf16 x over its dynamic scale; dir, rs = fp32(1 / s) and the
// bracket's ends as for e4m3_quant4_bf16_end) into its row of codes; every code resolved,
// nothing to redo.  Zeros when s == 0.  s, rs and dir belong to the unit's token, so the
// choice of end is uniform over the wave.
template <int XE>
__device__ __forceinline__ void encode_early_chunks_bf16(const PrologueRegs& r, const uint8_t* xst, const XSplit& xs,
                                                         int part, int wave, int lane, int npl, float s, float rs,
                                                         float dir, uint8_t* row) {
    const bool live = s > 0.0f;
    const float rlo = rs * kBracketLo, rhi = rs * kBracketHi;
    auto chunk = [&](int i, auto&& quant4) {
        const int j = xs.chunk(part, lane, i);
        if (i < npl && j < xs.cpr) {
            const uint4 v = early_chunk(r, xst, wave, lane, i);
            const uint2 q = make_uint2(quant4(u2f(v.x << 16), u2f(v.x & 0xFFFF0000u), u2f(v.y << 16), u2f(v.y & 0xFFFF0000u)),
                                       quant4(u2f(v.z << 16), u2f(v.z & 0xFFFF0000u), u2f(v.w << 16), u2f(v.w & 0xFFFF0000u)));
            *reinterpret_cast<uint2*>(row + j * 8) = live ? q : make_uint2(0u, 0u);
        }
    };
    if (dir != 0.0f) {  // the end on dir's side
        const float rq = dir > 0.0f ? rhi : rlo;
#pragma unroll
        for (int i = 0; i < XE; ++i)
            chunk(i, [&](float a, float b, float c, float d) { return e4m3_quant4_bf16_end(a, b, c, d, rq); });
    } else {
#pragma unroll
        for (int i = 0; i < XE; ++i)
            chunk(i, [&](float a, float b, float c, float d) { return e4m3_quant4_bf16_even(a, b, c, d, rlo, rhi); });
    }
}

// The early chunks of a unit into its row of codes; returns the chunks to redo exactly.
template <bool SAT, int XE>
__device__ __forceinline__ uint32_t encode_early_chunks(const PrologueRegs& r, const uint8_t* xst, const XSplit& xs,
                                                        int part, int wave, int lane, int npl, float s, float rs,
                                                        float lift, uint8_t* row) {
    uint32_t redo = 0;
#pragma unroll
    for (int i = 0; i < XE; ++i) {
        const int j = xs.chunk(part, lane, i);
        if (i < npl && j < xs.cpr) {
            uint2 q;
            if (!chunk_encode_fast<SAT>(early_chunk(r, xst, wave, lane, i), s, rs, &q, lift)) redo |= 1u << i;
            *reinterpret_cast<uint2*>(row + j * 8) = q;
        }
    }
    return redo;
}

// --- the fused RMSNorm (the pages fuse it with the quantize step; see the oracle) ---

__device__ __forceinline__ void chunk_floats(uint4 v, float f[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        f[2 * h] = u2f(w[h] << 16);
        f[2 * h + 1] = u2f(w[h] & 0xFFFF0000u);
    }
}

// Sum of x^2 over a chunk: each square is exact in float32 (bf16 has 8 significant
// bits), the sum is kept in float64.
__device__ __forceinline__ double chunk_sumsq(uint4 v) {
    float f[8];
    chunk_floats(v, f);
    double s = 0.0;
#pragma unroll
    for (int h = 0; h < 8; ++h) s += (double)(f[h] * f[h]);
    return s;
}

// The normalised values x * r * w of a chunk (float32).
__device__ __forceinline__ void chunk_normed(uint4 xv, uint4 wv, float r, float out[8]) {
    float x[8], w[8];
    chunk_floats(xv, x);
    chunk_floats(wv, w);
#pragma unroll
    for (int h = 0; h < 8; ++h) out[h] = (x[h] * r) * w[h];
}

__device__ __forceinline__ uint4 nw_chunk(const uint8_t* nw, int j) {
    return *reinterpret_cast<const uint4*>(nw + j * 16);
}

__device__ __forceinline__ bool vals_encode_fast(const float v[8], float s, float rs, uint2* out) {
    uint32_t c[4];
    bool ok = true;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        c[h] = e4m3_quant2_fast<true>(v[2 * h], v[2 * h + 1], rs);
        ok = ok && c[h] != kQuantExact;
    }
    const bool live = s > 0.0f;
    *out = live ? make_uint2(c[0] | (c[1] << 16), c[2] | (c[3] << 16)) : make_uint2(0u, 0u);
    return ok || !live;
}

__device__ __forceinline__ uint2 vals_encode_exact(const float v[8], float s, float rs) {
    uint32_t c[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) c[h] = e4m3_quant2_exact(v[2 * h], v[2 * h + 1], s, rs);
    return s > 0.0f ? make_uint2(c[0] | (c[1] << 16), c[2] | (c[3] << 16)) : make_uint2(0u, 0u);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_add_f64(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROW_MASK, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROW_MASK, 0xF, false);
    return v + __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over the wave, the row shifts and broadcasts of wave_max_u32 (an inclusive scan
// whose last lane holds the total).
__device__ __forceinline__ double wave_sum_f64(double v) {
    v = dpp_add_f64<0x111, 0xF>(v);
    v = dpp_add_f64<0x112, 0xF>(v);
    v = dpp_add_f64<0x114, 0xF>(v);
    v = dpp_add_f64<0x118, 0xF>(v);
    v = dpp_add_f64<0x142, 0xA>(v);
    v = dpp_add_f64<0x143, 0xC>(v);
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 63);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// 1 / rms of token m from the parts' sums of squares: float64, rounded once to float32.
__device__ __forceinline__ float token_rinv(const FwdParams& p, const PrologueLds& L, const XSplit& xs, int m) {
    double ss = 0.0;
    for (int q = 0; q < xs.P; ++q) ss += L.ssqp[m * kMaxParts + q];
    return (float)(1.0 / sqrt(ss / (double)p.K + (double)p.norm_eps));
}

__device__ __forceinline__ uint2 chunk_encode_exact(uint4 v, float s, float rs, float lift = 1.0f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t c[4];
#pragma unroll
    for (int h = 0; h < 4; ++h)
        c[h] = e4m3_quant2_exact(u2f(w[h] << 16) * lift, u2f(w[h] & 0xFFFF0000u) * lift, s, rs);
    return s > 0.0f ? make_uint2(c[0] | (c[1] << 16), c[2] | (c[3] << 16)) : make_uint2(0u, 0u);
}

// Routing table into `rt` (LDS, RouteLayout), token scales into `sx`, token codes into
// `xq` (row stride xstride bytes).  Ends with a block barrier.  The barriers order
// LDS only (lds_barrier), so the weight loads issued before stay in flight.  RMS: the
// fused norm (L.nw holds its weight); a compile-time choice, so that the plain step's
// code carries none of it.  mid: the caller's work at the first barrier (once the token
// maxima and the routing keys are in LDS), run by every thread.
template <bool RMS, bool XD = false, int XE = kXEarly, class Mid>
__device__ __forceinline__ void prologue_finish(const FwdParams& p, PrologueRegs& r, const PrologueLds& L, int* rt,
                                float* sx, uint8_t* xq, int xstride, bool publish, Mid&& mid) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const RouteLayout rl{p.T, p.S};
    const XSplit xs(p.M, p.K);
    const int npl = xs.per_lane();
    const int nearly = min(XE, L.xs != nullptr ? kXEarly : kXChunks);  // chunks a lane has early

    // 0. every early load is taken here, on every path, so that no branch below leaves
    //    one pending (where paths join, a pending load could only be waited for together
    //    with the weight stream issued after it)
#pragma unroll
    for (int i = 0; i < (XE < kXChunks ? XE : kXChunks); ++i)
        asm volatile("" ::"v"(r.x[i].x), "v"(r.x[i].y), "v"(r.x[i].z), "v"(r.x[i].w));
    if (p.E > 0) {
#pragma unroll
        for (int i = 0; i < kLogitLoads; ++i) asm volatile("" ::"v"(r.lg[i]));
    }

    constexpr bool rms = RMS;
    // 1. max |x| of each unit (with the norm: the sum of x^2): lanes over their chunks,
    //    then the wave (DPP)
    for (int u = wave; rms && u < xs.units; u += kPrologueWaves) {
        const int m = u % p.M, part = u / p.M;
        double ss = 0.0;
        if (u == wave && npl <= nearly) {
#pragma unroll
            for (int i = 0; i < XE; ++i)
                if (i < npl && xs.chunk(part, lane, i) < xs.cpr) ss += chunk_sumsq(early_chunk(r, L.xs, wave, lane, i));
        } else {
            const int xrow = batch_row_of(r.tok, m);
            for (int i = 0; i < npl; ++i) {
                const int j = xs.chunk(part, lane, i);
                if (j < xs.cpr) ss += chunk_sumsq(load_x_chunk(p, xrow, j, xs.cpr));
            }
        }
        const double t = wave_sum_f64(ss);
        if (lane == 0) L.ssqp[m * kMaxParts + part] = t;
    }
    for (int u = wave; !rms && u < xs.units; u += kPrologueWaves) {
        const int m = u % p.M, part = u / p.M;
        float mx = 0.0f;
        if (u == wave && npl <= nearly) {  // the early chunks
#pragma unroll
            for (int i = 0; i < XE; ++i)
                if (i < npl && xs.chunk(part, lane, i) < xs.cpr)
                    mx = fmaxf(mx, chunk_absmax(early_chunk(r, L.xs, wave, lane, i)));
        } else {
            const int xrow = batch_row_of(r.tok, m);
            for (int i = 0; i < npl; ++i) {
                const int j = xs.chunk(part, lane, i);
                if (j < xs.cpr) mx = fmaxf(mx, chunk_absmax(load_x_chunk(p, xrow, j, xs.cpr)));
            }
        }
        const uint32_t wm = wave_max_u32(__float_as_uint(mx));  // non-negative floats: bit order
        if (lane == 0) L.amaxp[m * kMaxParts + part] = wm;
    }
    // 2. arg-max per token (wave m mod 8), one key per lane
    if (p.E > 0) {
        for (int m = wave; m < p.M; m += kPrologueWaves) {
            uint32_t key = 0;
            if (m == wave && p.E <= 64 * kLogitLoads) {
#pragma unroll
                for (int i = 0; i < kLogitLoads; ++i) {
                    const int e = lane + 64 * i;
                    if (e < p.E) key = max(key, logit_key(r.lg[i], e));
                }
            } else {
                const uint16_t* row = p.logits + (size_t)batch_row_of(r.tok, m) * p.E;
                for (int e = lane; e < p.E; e += 64) key = max(key, logit_key(row[e], e));
            }
            key = wave_max_u32(key);
            if (lane == 0) {
                L.exp[m] = (int)(0xFFFFu - (key & 0xFFFFu));
                L.gate[m] = 1.0f / (1.0f + expf(-key_logit(key)));
            }
        }
    }
    lds_barrier();
    mid();  // the caller's work between the two halves (more weight requests)

    // 1b. with the norm: max |x r w| of each unit, r = 1 / rms of its token (the norm
    //     weight in LDS is complete: every wave has taken its x, issued after its copy)
    if (rms) {
        for (int u = wave; u < xs.units; u += kPrologueWaves) {
            const int m = u % p.M, part = u / p.M;
            const float rn = token_rinv(p, L, xs, m);
            float mx = 0.0f;
            if (u == wave && npl <= nearly) {
#pragma unroll
                for (int i = 0; i < XE; ++i) {
                    const int j = xs.chunk(part, lane, i);
                    if (i < npl && j < xs.cpr) {
                        float v[8];
                        chunk_normed(early_chunk(r, L.xs, wave, lane, i), nw_chunk(L.nw, j), rn, v);
#pragma unroll
                        for (int h = 0; h < 8; ++h) mx = fmaxf(mx, fabsf(v[h]));
                    }
                }
            } else {
                const int xrow = batch_row_of(r.tok, m);
                for (int i = 0; i < npl; ++i) {
                    const int j = xs.chunk(part, lane, i);
                    if (j >= xs.cpr) continue;
                    float v[8];
                    chunk_normed(load_x_chunk(p, xrow, j, xs.cpr), nw_chunk(L.nw, j), rn, v);
                    for (int h = 0; h < 8; ++h) mx = fmaxf(mx, fabsf(v[h]));
                }
            }
            const uint32_t wm = wave_max_u32(__float_as_uint(mx));
            if (lane == 0) L.amaxp[m * kMaxParts + part] = wm;
        }
        lds_barrier();
    }

    // 3. token codes with the token's scale (uniform per wave); chunks with a pair close
    //    to a rounding midpoint are redone on the exact path from the same registers
    //    (bf16 inputs often fall exactly on a midpoint; a reload would wait for the
    //    whole weight stream)
    for (int u = wave; u < xs.units; u += kPrologueWaves) {
        const int m = u % p.M, part = u / p.M;
        uint32_t am = 0;
        for (int q = 0; q < xs.P; ++q) am = max(am, L.amaxp[m * kMaxParts + q]);
        // static scale (a variant reading), else fp32(amax / 448) by IEEE division
        const bool stat = p.x_scale > 0.0f;
        const float s = stat ? p.x_scale : __uint_as_float(am) / kE4M3Max;
        // a scale below kTinyScale (a row whose largest magnitude is below about 448 * 2^-96;
        // never in practice) is lifted with its values (codec.hpp) and takes the path of a
        // static scale: fast codes, the exact path where they are unsure
        const bool tiny = s > 0.0f && s < kTinyScale;
        const float lift = tiny ? kTinyLift : 1.0f;
        const float sl = s * lift;  // exact
        const float rs = s > 0.0f ? 1.0f / sl : 0.0f;
        if (part == 0 && lane == 0) sx[m] = s;
        uint8_t* row = xq + m * xstride;
        uint32_t redo = 0;
        if (rms) {  // codes of the normalised values (the exact path where the fast one is unsure)
            const float rn = token_rinv(p, L, xs, m);
            if (u == wave && npl <= nearly) {
#pragma unroll
                for (int i = 0; i < XE; ++i) {
                    const int j = xs.chunk(part, lane, i);
                    if (i < npl && j < xs.cpr) {
                        float v[8];
                        chunk_normed(early_chunk(r, L.xs, wave, lane, i), nw_chunk(L.nw, j), rn, v);
#pragma unroll
                        for (int h = 0; h < 8; ++h) v[h] *= lift;
                        uint2 q;
                        if (!vals_encode_fast(v, sl, rs, &q)) redo |= 1u << i;
                        *reinterpret_cast<uint2*>(row + j * 8) = q;
                    }
                }
            } else {
                const int xrow = batch_row_of(r.tok, m);
#pragma unroll 1
                for (int i = 0; i < npl; ++i) {
                    const int j = xs.chunk(part, lane, i);
                    if (j >= xs.cpr) continue;
                    float v[8];
                    chunk_normed(load_x_chunk(p, xrow, j, xs.cpr), nw_chunk(L.nw, j), rn, v);
#pragma unroll
                    for (int h = 0; h < 8; ++h) v[h] *= lift;
                    uint2 q;
                    if (!vals_encode_fast(v, sl, rs, &q)) q = vals_encode_exact(v, sl, rs);
                    *reinterpret_cast<uint2*>(row + j * 8) = q;
                }
            }
            if (redo != 0u) {  // unrolled: the chunks stay in their registers
#pragma unroll
                for (int i = 0; i < XE; ++i) {
                    if (!((redo >> i) & 1u)) continue;
                    const int j = xs.chunk(part, lane, i);
                    float v[8];
                    chunk_normed(early_chunk(r, L.xs, wave, lane, i), nw_chunk(L.nw, j), rn, v);
#pragma unroll
                    for (int h = 0; h < 8; ++h) v[h] *= lift;
                    *reinterpret_cast<uint2*>(row + j * 8) = vals_encode_exact(v, sl, rs);
                }
            }
            continue;
        }
        if (u == wave && npl <= nearly) {
            if (stat || tiny) {
                redo = encode_early_chunks<true, XE>(r, L.xs, xs, part, wave, lane, npl, sl, rs, lift, row);
            } else {  // bf16 x over fp32(amax / 448): the row's rounding of s decides the ties
                const float dir = fmaf(-kE4M3Max, s, __uint_as_float(am));
                encode_early_chunks_bf16<XE>(r, L.xs, xs, part, wave, lane, npl, s, rs, dir, row);
            }
        } else {  // larger inputs: chunks loaded here
            const int xrow = batch_row_of(r.tok, m);
#pragma unroll 1
            for (int i = 0; i < npl; ++i) {
                const int j = xs.chunk(part, lane, i);
                if (j >= xs.cpr) continue;
                const uint4 v = load_x_chunk(p, xrow, j, xs.cpr);
                uint2 q;
                if (!chunk_encode_fast<true>(v, sl, rs, &q, lift)) q = chunk_encode_exact(v, sl, rs, lift);
                *reinterpret_cast<uint2*>(row + j * 8) = q;
            }
        }
        if (redo != 0u) {  // unrolled: the chunks stay in their registers
#pragma unroll
            for (int i = 0; i < XE; ++i) {
                if (!((redo >> i) & 1u)) continue;
                const int j = xs.chunk(part, lane, i);
                *reinterpret_cast<uint2*>(row + j * 8) =
                    chunk_encode_exact(early_chunk(r, L.xs, wave, lane, i), sl, rs, lift);
            }
        }
    }

    // 4. routing table, by wave 0: lane m < M compares its expert with every token's
    if (wave == 0) {
        if (lane < p.M) rt[rl.batch_row() + lane] = r.tok;
        if (p.E == 0) {  // dense: the shared expert alone
            if (lane == 0) {
                rt[rl.d()] = 0;
                rt[rl.slot_expert()] = 0;
                rt[rl.slot_row0()] = 0;
                rt[rl.slot_rows()] = p.M;
            }
            for (int m = lane; m < p.M; m += 64) {
                rt[rl.token_row() + m] = -1;
                rt[rl.token_expert() + m] = -1;
                rt[rl.row_token() + m] = m;
                L.gate[m] = 0.0f;
            }
        } else {
            const int em = lane < p.M ? L.exp[lane] : 0x7FFFFFFF;
            bool first = lane < p.M;  // is this token the first with its expert?
            for (int k = 0; k < p.M; ++k) {
                const int ek = __builtin_amdgcn_readlane(em, k);
                first = first && !(k < lane && ek == em);
            }
            const uint64_t firsts = __ballot(first);  // bit k: token k is its expert's first
            int less = 0, same_before = 0, same = 0, first_less = 0;
            for (int k = 0; k < p.M; ++k) {
                const int ek = __builtin_amdgcn_readlane(em, k);
                less += ek < em;
                same += ek == em;
                same_before += (ek == em) && (k < lane);
                first_less += ((firsts >> k) & 1u) && ek < em;
            }
            const int distinct = __popcll(firsts);
            if (lane < p.M) {
                const int slot = 1 + first_less, row0 = p.M + less, row = row0 + same_before;
                if (same_before == 0) {  // the expert's first token writes its slot
                    rt[rl.slot_expert() + slot] = em;
                    rt[rl.slot_row0() + slot] = row0;
                    rt[rl.slot_rows() + slot] = same;
                }
                rt[rl.token_row() + lane] = row;
                rt[rl.token_expert() + lane] = em;
                rt[rl.row_token() + row] = lane;
                rt[rl.row_token() + lane] = lane;
            }
            if (lane == 0) {
                rt[rl.d()] = distinct;
                rt[rl.slot_expert()] = p.E;  // the shared expert's packed index
                rt[rl.slot_row0()] = 0;
                rt[rl.slot_rows()] = p.M;
            }
        }
    }
    lds_barrier();

    // 5. block 0 (`publish`) publishes the table, the gates and the debug copies
    if (publish) {
        for (int i = tid; i < rl.count(); i += kPrologueThreads) xstore<XD>(p.ws.route + i, rt[i]);
        for (int m = tid; m < p.M; m += kPrologueThreads) {
            xstore<XD>(p.ws.gate + m, L.gate[m]);
            const int t = rt[rl.batch_row() + m];
            if (p.dbg.sx) p.dbg.sx[t] = sx[m];
            if (p.dbg.expert) p.dbg.expert[t] = p.E > 0 ? L.exp[m] : -1;
            if (p.dbg.gate) p.dbg.gate[t] = L.gate[m];
        }
        if (tid == 0 && p.dbg.num_active) {  // summed over the chunks of a large forward
            if (p.first_chunk) p.dbg.num_active[0] = rt[rl.d()];
            else atomicAdd(p.dbg.num_active, rt[rl.d()]);
        }
        if (p.dbg.xq)
            for (int c = tid; c < p.M * xs.cpr; c += kPrologueThreads) {
                const int t = c / xs.cpr, j = c - t * xs.cpr;
                reinterpret_cast<uint2*>(p.dbg.xq)[(size_t)rt[rl.batch_row() + t] * xs.cpr + j] =
                    *reinterpret_cast<const uint2*>(xq + t * xstride + j * 8);
            }
    }
}

}  // namespace moe
