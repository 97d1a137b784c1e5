// Grouped forward for batches above one 16-token launch: every active expert's weights
// are streamed once for all of its tokens.
//
// The pages build their MoE GEMMs to run at full HBM bandwidth (Blackwell 1,000
// TPS/user blog, zh translation, section "CUDA kernel optimisation and fusion", item on
// spatial partitioning and efficient memory loads).  With a batch of a few hundred
// tokens and top-1 routing, the shared expert meets every token and a popular expert
// dozens of them.  Running such a batch as consecutive 16-token launches streams the
// shared expert once per launch; here each expert is streamed once per pass of up to
// kGroupMax tokens, and a work item loops over the item's row tiles of 16 tokens while
// its weights sit in registers.
//
// One pass over M tokens (M <= kGroupMax), six kernels on one stream:
//   gprep     one block per token: top-1 routing (lowest index of the largest logit,
//             sigmoid gate) and the per-token e4m3 quantisation of x, into global
//             buffers; clears the pass's row maxima and work counters.
//   gorder    one block: the distinct experts in ascending id as slots 1..d (slot 0 =
//             shared expert, rows [0, M), row m = token m) with their rows [row0,
//             row0 + n) inside [M, 2M), tokens in ascending order inside a slot.
//   gfc13     FC13 + SwiGLU (persistent): item = (slot, 16 gate + 16 up channels) over
//             all of K.  Writes the float32 intermediate a [2M][I] and, at its end, each
//             row's max |a| (device-scope atomic max of the float bits).
//   grequant  one block per row: s_a = fp32(amax / 448), aq = e4m3(a / s_a).
//   gfc2      FC2 split over I (persistent): item = (slot, 64 output columns, 2048 of
//             I); float32 partial sums [split][row][K] times s_a and s2; a routed row
//             is written at row M + token.
//   gcombine  out = bf16(y_shared + gate * y_routed), the splits added in order.
//
// The arithmetic is that of the 16-token kernels, operation for operation (the same
// k-step split over the waves, the same wave order in the reductions, the same
// quantiser and SwiGLU expression), so both give bitwise the same output.
//
// gfx950 streaming.  A wave keeps one item's weight k-steps in registers (16-byte
// buffer loads in the packed operand order), and one row tile's token codes for the
// same k-steps, gathered from the code buffer (L2-resident: M x K bytes).  A position
// is (item, row tile).  As soon as the matrix unit has taken k-step s of a position,
// the wave requests k-step s of the next position's token codes (the next row tile, or
// the next item's first) into the same registers, and, on an item's last row tile,
// k-step s of the next item's weights.  Memory counters retire in order, so a position
// waits for its k-step s only behind loads it needs anyway, and one register set of
// each kind holds one position in flight.
#pragma once

#include "codec.hpp"
#include "fc13.hpp"
#include "fc2.hpp"
#include "group_order.hpp"
#include "layout.hpp"
#include "prologue.hpp"

namespace moe {

constexpr int kGroupMax = 1024;       // tokens per grouped pass
constexpr int kGroupPrepThreads = 256;
constexpr int kGroupOrderThreads = 1024;
constexpr int kGroupTableRegs = 11;   // route-table words per thread loaded early (>= (1 + 3S + 2M) / 512)
static_assert(kGroupTableRegs * kFc13Threads >= 1 + 3 * (1 + kMaxRouteExperts) + 2 * kGroupMax, "table fits");
static_assert(kGroupMax <= kGroupOrderThreads, "one order tile");

// Routing table of a pass (int32), T = tokens of the workspace, S = 1 + min(T, E):
struct GroupRoute {
    int T, S;
    __host__ __device__ int count() const { return 1 + 3 * S + 3 * T; }
    __host__ __device__ int d() const { return 0; }                        // [1]
    __host__ __device__ int slot_expert() const { return 1; }              // [S] packed expert index (E = shared)
    __host__ __device__ int slot_row0() const { return 1 + S; }            // [S]
    __host__ __device__ int slot_rows() const { return 1 + 2 * S; }        // [S]
    __host__ __device__ int row_token() const { return 1 + 3 * S; }        // [2T] token of each row
    __host__ __device__ int token_expert() const { return 1 + 3 * S + 2 * T; }  // [T] -1 when E == 0
    // words the GEMM kernels copy into LDS: the slot arrays and the rows of an M-token pass
    __host__ __device__ int prefix(int M) const { return 1 + 3 * S + 2 * M; }
};

struct GroupParams {
    const uint16_t* x;       // [M][K] bf16, the pass's tokens
    const uint16_t* logits;  // [M][E] bf16, or null when E == 0
    uint16_t* out;           // [M][K] bf16
    const uint8_t* w13p;     // packed FC13 weights of E + 1 experts
    const uint8_t* w2p;      // packed FC2 weights
    const float* s13;        // [E+1][2I]
    const float* s2;         // [E+1][K]
    uint64_t w13_bytes, w2_bytes;  // per expert
    int32_t M, K, I, E, S, T;      // T: token capacity of the workspace
    int32_t nsplit;                // FC2 splits of I (2048 each)
    int32_t first;                 // the forward's first pass (debug counter)
    int32_t* route;   // GroupRoute
    float* gate;      // [T]
    float* sx;        // [T]
    uint8_t* xq;      // [T][K]
    uint32_t* amax;   // [2T] float bits of max |a| per row
    float* a;         // [2T][I]
    uint8_t* aq;      // [2T][I]
    float* sa;        // [2T]
    float* part;      // [nsplit][2T][K]
    uint32_t* work;   // [2] pool counters of gfc13 and gfc2
    int32_t item0_13; // the first item gfc13 takes: I/16 when the wide kernels (wide.hpp) take slot 0, else 0
    int32_t item0_2;  // the same for gfc2: one slot's items (K/64 * nsplit), else 0
    uint8_t* xt;      // the wide kernels' copy of xq in operand order (tile_byte), or null
    uint8_t* at;      // the same of aq's rows [0, M) (the shared expert's), or null
    Debug dbg;        // token-indexed like x
};

// Operand order of a pass's codes for the wide kernels (wide.hpp): k-step s of row tile t
// (rows 16t..16t+15) is one 2048-byte block at (s * ntiles + t) * 2048, laid out as a
// weight block ([half][lane][16 B], lane = 16 * (32-code group) + row mod 16), so that a
// wave reads a k-step of a tile as two fully used 1 KB loads, and a k-step of all tiles
// is one contiguous range.  (A layout with each row's 128 codes of a k-step in one line
// lets the producers write whole lines, 2.3 us less for the two of them at 256 tokens,
// but the wide FC13's reads then touch 16 half-used lines per load: 6 us more.)  Byte of
// code k of row r:
__host__ __device__ inline uint32_t tile_byte(int r, int k, int ntiles) {
    const int c = k & 127;
    return (uint32_t)((k >> 7) * ntiles + (r >> 4)) * 2048u + (uint32_t)(((c >> 4) & 1) * 1024) +
           (uint32_t)((((c >> 5) << 4) | (r & 15)) * 16) + (uint32_t)(c & 15);
}

// Row of block b in a launch of n one-row blocks.  The blocks of a launch go to the 8 XCDs in
// turn (b mod 8), each XCD with its own L2.  A 128-byte line of the operand-order copies
// holds 16 bytes of each of 8 consecutive rows, so with row = b every line would be written
// in 8 different L2s, 16 bytes in each, and reach memory as 8 partial writes.  In each
// aligned run of 64 blocks the 8 blocks of one XCD take 8 consecutive rows instead (an 8 x 8
// transpose), so that each line is completed in one L2; the blocks past the last whole run
// keep row = b.
__device__ __forceinline__ int xcd_row(int b, int n) {
    if (b >= (n & ~63)) return b;
    const int o = b & 63;
    return (b & ~63) + (o & 7) * 8 + (o >> 3);
}

// ---------------------------------------------------------------------------------
// gprep: routing and activation quantisation, one block per token.

// The leading arguments of the grouped kernels repeat the fields of p that their first
// loads need.  They are preloaded into SGPRs; p, an aggregate, is not, and each field of it
// is a scalar load from the argument block where it is first used (about a microsecond
// at a kernel's start, before which nothing else could be issued).
// gprep: lead_me = M | E << 16.
__global__ __launch_bounds__(kGroupPrepThreads) void gprep_kernel(const uint16_t* lead_x, const uint16_t* lead_logits,
                                                                  uint8_t* lead_xq, uint8_t* lead_xt, uint32_t lead_me,
                                                                  uint32_t lead_k, const GroupParams p0) {
    GroupParams p = p0;
    p.x = lead_x;
    p.logits = lead_logits;
    p.xq = lead_xq;
    p.xt = lead_xt;
    p.M = (int32_t)(lead_me & 0xFFFFu);
    p.E = (int32_t)(lead_me >> 16);
    p.K = (int32_t)lead_k;
    __shared__ uint32_t red[2 * (kGroupPrepThreads / 64)];
    const int m = xcd_row(blockIdx.x, gridDim.x), tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const GroupRoute gr{p.T, p.S};
    const int cpr = p.K >> 3;  // 16-byte chunks (8 bf16) of a row, <= 1024
    constexpr int kC = 4;      // chunks per thread
    uint4 xv[kC];
    const uint4* xrow = reinterpret_cast<const uint4*>(p.x) + (size_t)m * cpr;
#pragma unroll
    for (int i = 0; i < kC; ++i) {
        const int j = tid + kGroupPrepThreads * i;
        xv[i] = j < cpr ? xrow[j] : make_uint4(0u, 0u, 0u, 0u);
    }
    uint32_t key = 0;
    if (p.E > 0)
        for (int e = tid; e < p.E; e += kGroupPrepThreads) key = max(key, logit_key(p.logits[(size_t)m * p.E + e], e));
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < kC; ++i) am = fmaxf(am, chunk_absmax(xv[i]));
    const uint32_t wm = wave_max_u32(__float_as_uint(am)), wk = wave_max_u32(key);
    if (lane == 0) {
        red[wave] = wm;
        red[4 + wave] = wk;
    }
    __syncthreads();
    const uint32_t amax = max(max(red[0], red[1]), max(red[2], red[3]));
    key = max(max(red[4], red[5]), max(red[6], red[7]));
    const float s = __uint_as_float(amax) / kE4M3Max;  // fp32(amax / 448), IEEE division
    const float lift = s > 0.0f && s < kTinyScale ? kTinyLift : 1.0f;  // a tiny scale is lifted (codec.hpp)
    const float sl = s * lift;                                          // exact
    const float rs = s > 0.0f ? 1.0f / sl : 0.0f;
    uint8_t* qrow = p.xq + (size_t)m * p.K;
    // bf16 x over fp32(amax / 448), amax a bf16 value: every code from one end of the bracket
    // chosen by the row's rounding direction, or the even one of both ends when the scale is
    // exact (codec.hpp, e4m3_quant4_bf16_end); a tiny scale takes the lifted path below
    const bool bf16_rule = s >= kTinyScale;  // (the row's: uniform over the block)
    const float dir = fmaf(-kE4M3Max, s, __uint_as_float(amax));
    const float rlo = rs * kBracketLo, rhi = rs * kBracketHi, rq = dir > 0.0f ? rhi : rlo;
    auto quant4 = [&](float a, float b, float c, float d) {
        return dir != 0.0f ? e4m3_quant4_bf16_end(a, b, c, d, rq) : e4m3_quant4_bf16_even(a, b, c, d, rlo, rhi);
    };
#pragma unroll
    for (int i = 0; i < kC; ++i) {
        const int j = tid + kGroupPrepThreads * i;
        if (j < cpr) {
            uint2 q;
            if (bf16_rule) {
                const uint4 v = xv[i];
                q = make_uint2(quant4(u2f(v.x << 16), u2f(v.x & 0xFFFF0000u), u2f(v.y << 16), u2f(v.y & 0xFFFF0000u)),
                               quant4(u2f(v.z << 16), u2f(v.z & 0xFFFF0000u), u2f(v.w << 16), u2f(v.w & 0xFFFF0000u)));
            } else if (!chunk_encode_fast<false>(xv[i], sl, rs, &q, lift)) {
                q = chunk_encode_exact(xv[i], sl, rs, lift);
            }
            *reinterpret_cast<uint2*>(qrow + 8 * j) = q;
            if (p.xt) *reinterpret_cast<uint2*>(p.xt + tile_byte(m, 8 * j, (p.M + 15) >> 4)) = q;
            if (p.dbg.xq) *reinterpret_cast<uint2*>(p.dbg.xq + (size_t)m * p.K + 8 * j) = q;
        }
    }
    if (tid == 0) {
        const int e = p.E > 0 ? (int)(0xFFFFu - (key & 0xFFFFu)) : -1;
        const float g = p.E > 0 ? 1.0f / (1.0f + expf(-key_logit(key))) : 0.0f;
        p.sx[m] = s;
        p.gate[m] = g;
        p.route[gr.token_expert() + m] = e;
        p.amax[m] = 0u;
        p.amax[p.M + m] = 0u;
        if (p.dbg.sx) p.dbg.sx[m] = s;
        if (p.dbg.expert) p.dbg.expert[m] = e;
        if (p.dbg.gate) p.dbg.gate[m] = g;
        // without routed experts a pass that runs wide launches no ordering kernel, whose
        // count of active experts would add 0
        if (m == 0 && p.E == 0 && p.first && p.dbg.num_active) p.dbg.num_active[0] = 0;
        if (m == 0) {
            p.work[0] = 0u;
            p.work[1] = 0u;
        }
    }
}

// ---------------------------------------------------------------------------------
// gorder: the slot table of the pass.  One block of 1024 threads.

// Inclusive sum of v over the block (every thread calls it); wt: 16 ints of LDS.
__device__ __forceinline__ int block_incl_sum(int v, int* wt) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int n = __shfl_up(v, o);
        if (lane >= o) v += n;
    }
    if (lane == 63) wt[wave] = v;
    __syncthreads();
    if (wave == 0) {
        int t = lane < kGroupOrderThreads / 64 ? wt[lane] : 0;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            const int n = __shfl_up(t, o);
            if (lane >= o) t += n;
        }
        if (lane < kGroupOrderThreads / 64) wt[lane] = t;
    }
    __syncthreads();
    if (wave > 0) v += wt[wave - 1];
    __syncthreads();  // wt is free again
    return v;
}

__host__ __device__ inline int gorder_lds_bytes(int M, int E) { return ((2 * M + 15) & ~15) + 4 * max(E, 1) + 64; }

__global__ __launch_bounds__(kGroupOrderThreads) void gorder_kernel(const GroupParams p) {
    extern __shared__ __align__(16) uint8_t lds[];
    uint16_t* texp = reinterpret_cast<uint16_t*>(lds);                       // [M]
    int* next = reinterpret_cast<int*>(lds + ((2 * p.M + 15) & ~15));        // [E] count, then row
    int* wt = next + max(p.E, 1);                                           // [16]
    const int tid = threadIdx.x;
    const GroupRoute gr{p.T, p.S};
    int* rt = p.route;
    for (int e = tid; e < p.E; e += kGroupOrderThreads) next[e] = 0;
    __syncthreads();
    if (p.E > 0)
        for (int m = tid; m < p.M; m += kGroupOrderThreads) {
            const int e = rt[gr.token_expert() + m];
            texp[m] = (uint16_t)e;
            atomicAdd(&next[e], 1);
        }
    for (int m = tid; m < p.M; m += kGroupOrderThreads) rt[gr.row_token() + m] = m;  // shared rows
    __syncthreads();
    // slots in ascending expert id; rows of expert e start at M + (tokens of experts < e)
    const int cnt = tid < p.E ? next[tid] : 0;
    const int has = cnt > 0 ? 1 : 0;
    const int rows_incl = block_incl_sum(cnt, wt);
    const int slots_incl = block_incl_sum(has, wt);
    if (has) {
        const int slot = slots_incl;  // 1 + (earlier active experts)
        rt[gr.slot_expert() + slot] = tid;
        rt[gr.slot_row0() + slot] = p.M + rows_incl - cnt;
        rt[gr.slot_rows() + slot] = cnt;
    }
    if (tid == kGroupOrderThreads - 1) {
        rt[gr.d()] = slots_incl;  // the total
        rt[gr.slot_expert()] = p.E;
        rt[gr.slot_row0()] = 0;
        rt[gr.slot_rows()] = p.M;
        if (p.dbg.num_active) p.dbg.num_active[0] = (p.first ? 0 : p.dbg.num_active[0]) + slots_incl;
    }
    if (tid < p.E) next[tid] = p.M + rows_incl - cnt;
    __syncthreads();
    // stable placement: a token's row is its expert's first row plus the number of earlier
    // tokens with the same expert (M <= kGroupOrderThreads: one tile)
    if (p.E > 0 && tid < p.M) {
        const int e = texp[tid];
        int rank = 0;
        for (int j = 0; j < tid; ++j) rank += texp[j] == e;
        rt[gr.row_token() + next[e] + rank] = tid;
    }
}

// ---------------------------------------------------------------------------------
// gfc13: FC13 + SwiGLU over all row tiles of each item.

struct GroupLds13 {
    int red;     // [2][WAVES][8][64] float partial tiles
    int rowmax;  // [2M] uint32
    int ring;    // [kGroupRing] int
    int sx;      // [M] float
    int route;   // GroupRoute prefix
    int total;
};

__host__ __device__ inline GroupLds13 gfc13_lds(int T, int S) {
    GroupLds13 l{};
    l.red = 0;
    l.rowmax = 2 * kFc13Waves * 8 * 64 * 4;
    l.ring = l.rowmax + 2 * T * 4;
    l.sx = l.ring + kGroupRing * 4;
    l.route = align16(l.sx + T * 4);
    l.total = align16(l.route + GroupRoute{T, S}.prefix(T) * 4);
    return l;
}

template <int NSTEP, bool FULL>
__global__ __launch_bounds__(kFc13Threads) void gfc13_kernel(const GroupParams p) {
    extern __shared__ __align__(16) uint8_t lds[];
    const GroupLds13 L = gfc13_lds(p.T, p.S);
    const GroupRoute gr{p.T, p.S};
    const int npairs = p.I >> 4, KS = p.K >> 7, G = gridDim.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int s0 = wave * NSTEP;
    const int ns = FULL ? NSTEP : max(0, min(NSTEP, KS - s0));
    const int j = lane & 15, grp = lane >> 4, r = wave & 3;
    const uint32_t pair_bytes = (uint32_t)KS * 2 * kBlockBytes;
    const uint32_t woff = (uint32_t)s0 * 2 * kBlockBytes + lane * 16;
    int* rt = reinterpret_cast<int*>(lds + L.route);
    float* sxl = reinterpret_cast<float*>(lds + L.sx);
    uint32_t* rowmax = reinterpret_cast<uint32_t*>(lds + L.rowmax);
    int* ring = reinterpret_cast<int*>(lds + L.ring);
    float* red = reinterpret_cast<float*>(lds + L.red);
    const int ntab = gr.prefix(p.M);
    auto wres = [&](int expert, int it) {
        return make_res(p.w13p + (uint64_t)expert * p.w13_bytes + (uint64_t)(it >= 0 ? it % npairs : 0) * pair_bytes,
                        it >= 0 ? pair_bytes : 0u);
    };
    auto sres = [&](int expert, int it) {
        return make_res(p.s13 + (size_t)expert * 2 * p.I, it >= 0 ? (uint32_t)p.I * 8 : 0u);
    };
    auto soff = [&](int it) { return (uint32_t)((it >= 0 ? it % npairs : 0) * 16 + 4 * grp + r) * 4; };
    const BufRes xres = make_res(p.xq, (uint32_t)p.M * p.K), xnone = make_res(p.xq, 0u);
    const uint32_t xlane = (uint32_t)s0 * kKStep + grp * 32;  // lane's bytes of a token row
    auto load_b = [&](uint4 (&b)[NSTEP][2], BufRes res, uint32_t base) {
#pragma unroll
        for (int s = 0; s < NSTEP; ++s)
            if (FULL || s < ns) {
                b[s][0] = buf_ld16(res, base + s * kKStep);
                b[s][1] = buf_ld16(res, base + s * kKStep + 16);
            }
    };  // the first position's; later ones roll k-step by k-step

    // 1. the table prefix and the token scales into LDS (the first item, which can be a
    //    routed expert's, comes from the table)
    {
        int tv[kGroupTableRegs];
        const BufRes tres = make_res(p.route, (uint32_t)ntab * 4);
#pragma unroll
        for (int i = 0; i < kGroupTableRegs; ++i)
            tv[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(tres, (uint32_t)(tid + kFc13Threads * i) * 4, 0, 0);
        const BufRes sxres = make_res(p.sx, (uint32_t)p.M * 4);
        const float sxv0 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sxres, tid * 4, 0, 0));
        const float sxv1 =
            __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sxres, (tid + kFc13Threads) * 4, 0, 0));
#pragma unroll
        for (int i = 0; i < kGroupTableRegs; ++i) {
            const int k = tid + kFc13Threads * i;
            if (k < ntab) rt[k] = tv[i];
        }
        if (tid < p.M) sxl[tid] = sxv0;
        if (tid + kFc13Threads < p.M) sxl[tid + kFc13Threads] = sxv1;
        for (int i = tid; i < 2 * p.M; i += kFc13Threads) rowmax[i] = 0u;
    }
    lds_barrier();

    // items [item0, (1 + d) I/16): without slot 0's when the wide kernel takes it
    const int item0 = p.item0_13;
    const GroupPlan<2> plan(G, blockIdx.x, (1 + rt[gr.d()]) * npairs - item0);
    const GroupOrder ord(item0 ? 0 : npairs, plan.pool0);
    auto imap = [&](int q) { const int v = ord.map(q); return v < 0 ? v : v + item0; };
    int cur = imap(plan.fixed(0));
    if (cur < 0) return;  // no item (only when the wide kernel takes slot 0): nothing to flush
    int nxt = imap(plan.fixed(1));
    int pos = 0, par = 0;
    float nsg = 0.0f, nsu = 0.0f;

    // lane's token-code offset of row tile `tile` of item `it` (any slot row if none)
    auto boff = [&](int it, int tile) {
        const int ps = it >= 0 ? it / npairs : 0;
        const int pr0 = rt[gr.slot_row0() + ps], pnr = rt[gr.slot_rows() + ps];
        return (uint32_t)rt[gr.row_token() + pr0 + min(16 * tile + j, pnr - 1)] * p.K + xlane;
    };

    // 2. the first position's token codes, then its weights and scales
    uint4 bx[NSTEP][2];
    load_b(bx, xres, boff(cur, 0));
    uint4 w[NSTEP][4];
    float sg, su;
    {
        const int e0 = __builtin_amdgcn_readfirstlane(rt[gr.slot_expert() + cur / npairs]);
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

    // k-step s of one position: the matrix work on the registers, then (after it, so that
    // the loads write the registers just read) the next position's token codes
    auto kstep = [&](int s, v4f& accg, v4f& accu, BufRes bres, uint32_t bbase) {
        const Operand b = widen(bx[s][0], bx[s][1]);
        accg = mma_kstep(widen(w[s][0], w[s][1]), b, accg);
        accu = mma_kstep(widen(w[s][2], w[s][3]), b, accu);
        __builtin_amdgcn_sched_barrier(0);
        bx[s][0] = buf_ld16(bres, bbase + s * kKStep);
        bx[s][1] = buf_ld16(bres, bbase + s * kKStep + 16);
    };
    // reduce the WAVES partial tiles of row tile t; wave w finishes channel w mod 4 of every lane
    auto epilogue = [&](const v4f& accg, const v4f& accu, int pair, int r0, int nr, int t) {
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
        const int nrow = min(16, nr - 16 * t);  // rows of this tile
        const int row = r0 + 16 * t + min(j, nrow - 1);
        const float sx = sxl[rt[gr.row_token() + row]];
        g = g * sx * sg;
        u = u * sx * su;
        const float a = g / (1.0f + expf(-g)) * u;
        float amax = j < nrow ? fabsf(a) : 0.0f;
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        if (wave < 4) {
            if (j < nrow) p.a[(size_t)row * p.I + pair * 16 + 4 * grp + r] = a;
            if (lane < 16 && j < nrow && amax > 0.0f) atomicMax(rowmax + row, __float_as_uint(amax));
        }
        par ^= 1;
    };

    // the last row tile of an item: the next item's first codes and its weights roll in; a
    // pool ticket for the item two positions ahead is taken before those loads
    auto last_tile = [&](int pair, int r0, int nr, int nt) {
        const bool take = plan.pooled(pos + 2);
        uint32_t ticket = 0;
        if (take && tid == 0) ticket = atomicAdd(p.work + 0, 1u);
        const uint32_t bbase = boff(nxt, 0);
        const BufRes bres = nxt >= 0 ? xres : xnone;
        const int nexpert = __builtin_amdgcn_readfirstlane(rt[gr.slot_expert() + (nxt >= 0 ? nxt / npairs : 0)]);
        const BufRes rn = wres(nexpert, nxt);
        const BufRes rsn = sres(nexpert, nxt);
        nsg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsn, soff(nxt), 0, 0));
        nsu = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsn, soff(nxt) + p.I * 4, 0, 0));
        v4f accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NSTEP; ++s) {
            if (FULL || s < ns) {
                kstep(s, accg, accu, bres, bbase);
#pragma unroll
                for (int q = 0; q < 4; ++q) w[s][q] = buf_ld16_stream(rn, woff + s * 2 * kBlockBytes + q * 1024);
            }
            // keep k-steps in order, so the wave waits for one k-step's loads at a time
            __builtin_amdgcn_sched_barrier(0);
        }
        if (take && tid == 0) ring[(pos + 2) % kGroupRing] = plan.from_ticket(ticket);
        epilogue(accg, accu, pair, r0, nr, nt - 1);
    };

    for (;;) {  // items
        const int slot = cur / npairs, pair = cur - slot * npairs;
        const int r0 = rt[gr.slot_row0() + slot], nr = rt[gr.slot_rows() + slot];
        const int nt = (nr + 15) >> 4;
        // row tiles before the last: the weights stay, the next tile's codes roll in
        for (int t = 0; t < nt - 1; ++t) {
            const uint32_t bbase = boff(cur, t + 1);
            v4f accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NSTEP; ++s) {
                if (FULL || s < ns) kstep(s, accg, accu, xres, bbase);
                __builtin_amdgcn_sched_barrier(0);
            }
            epilogue(accg, accu, pair, r0, nr, t);
        }
        last_tile(pair, r0, nr, nt);
        if (nxt < 0) break;
        cur = nxt;
        nxt = __builtin_amdgcn_readfirstlane(imap(plan.at(pos + 2, ring)));
        ++pos;
        sg = nsg;
        su = nsu;
    }
    lds_barrier();
    for (int i = tid; i < 2 * p.M; i += kFc13Threads) {
        const uint32_t v = rowmax[i];
        if (v != 0u && i < (p.E > 0 ? 2 * p.M : p.M)) atomicMax(p.amax + i, v);
    }
}

// ---------------------------------------------------------------------------------
// grequant: one block per row of the intermediate.

constexpr int kGroupRequantThreads = 256;

// lead_mi = M | I << 16.
__global__ __launch_bounds__(kGroupRequantThreads) void grequant_kernel(const float* lead_a, const uint32_t* lead_amax,
                                                                        uint8_t* lead_aq, uint8_t* lead_at,
                                                                        uint32_t lead_mi, const GroupParams p0) {
    GroupParams p = p0;
    p.a = const_cast<float*>(lead_a);
    p.amax = const_cast<uint32_t*>(lead_amax);
    p.aq = lead_aq;
    p.at = lead_at;
    p.M = (int32_t)(lead_mi & 0xFFFFu);
    p.I = (int32_t)(lead_mi >> 16);
    const int row = xcd_row(blockIdx.x, gridDim.x), tid = threadIdx.x;
    const float4* arow = reinterpret_cast<const float4*>(p.a + (size_t)row * p.I);
    const int i4 = p.I >> 2;
    constexpr int kRB = 8;  // float4 loads of a thread in flight at once
    // the row's first values are requested first: nothing they need waits for a scalar load
    float4 va[kRB];
#pragma unroll
    for (int u = 0; u < kRB; ++u) {
        const int c4 = tid + u * kGroupRequantThreads;
        va[u] = c4 < i4 ? arow[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const float s = __uint_as_float(p.amax[row]) / kE4M3Max;  // fp32(amax / 448), IEEE division
    const bool tiny = s > 0.0f && s < kTinyScale;              // the lifted exact path (codec.hpp)
    const float rs = s > 0.0f && !tiny ? 1.0f / s : 0.0f;
    uint8_t* qrow = p.aq + (size_t)row * p.I;
    // the debug copies (token-indexed) need the row's token: the slot table is read only then
    uint8_t* drow = row < p.M ? p.dbg.aq_shared : p.dbg.aq_routed;
    float* sd = row < p.M ? p.dbg.sa_shared : p.dbg.sa_routed;
    int tok = row;
    if (drow != nullptr || sd != nullptr) tok = row < p.M ? row : p.route[GroupRoute{p.T, p.S}.row_token() + row];
    if (drow) drow += (size_t)tok * p.I;
    uint8_t* trow = row < p.M ? p.at : nullptr;  // the shared expert's rows, for the wide FC2
    auto encode4 = [&](const float4 v) -> uint32_t {
        if (tiny) return e4m3_quant2_tiny(v.x, v.y, s) | (e4m3_quant2_tiny(v.z, v.w, s) << 16);
        if (!(s > 0.0f)) return 0u;
        const uint32_t lo = e4m3_quant2_fast<true>(v.x, v.y, rs);
        const uint32_t hi = e4m3_quant2_fast<true>(v.z, v.w, rs);
        return (lo != kQuantExact && hi != kQuantExact)
                   ? lo | (hi << 16)
                   : e4m3_quant2_exact(v.x, v.y, s, rs) | (e4m3_quant2_exact(v.z, v.w, s, rs) << 16);
    };
    for (int base = tid; base < i4; base += kRB * kGroupRequantThreads) {
        if (base != tid) {  // later rows' values (I above kRB * 1024)
#pragma unroll
            for (int u = 0; u < kRB; ++u) {
                const int c4 = base + u * kGroupRequantThreads;
                va[u] = c4 < i4 ? arow[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
#pragma unroll
        for (int u = 0; u < kRB; ++u) {
            const int c4 = base + u * kGroupRequantThreads;
            if (c4 >= i4) break;
            const uint32_t c = encode4(va[u]);
            *reinterpret_cast<uint32_t*>(qrow + 4 * c4) = c;
            if (trow) *reinterpret_cast<uint32_t*>(trow + tile_byte(row, 4 * c4, (p.M + 15) >> 4)) = c;
            if (drow) *reinterpret_cast<uint32_t*>(drow + 4 * c4) = c;
        }
    }
    if (tid == 0) {
        p.sa[row] = s;
        if (sd) sd[tok] = s;
    }
}

// ---------------------------------------------------------------------------------
// gfc2: FC2 split over I, over all row tiles of each item.

struct GroupLds2 {
    int red;    // [2][WAVES][4 sub][4][64] float partial tiles
    int ring;   // [kGroupRing] int
    int sa;     // [2M] float
    int route;  // GroupRoute prefix
    int total;
};

__host__ __device__ inline GroupLds2 gfc2_lds(int T, int S) {
    GroupLds2 l{};
    l.red = 0;
    l.ring = 2 * kFc2Waves * kFc2Sub * 4 * 64 * 4;
    l.sa = l.ring + kGroupRing * 4;
    l.route = align16(l.sa + 2 * T * 4);
    l.total = align16(l.route + GroupRoute{T, S}.prefix(T) * 4);
    return l;
}

constexpr int kGroupSaRegs = 2 * kGroupMax / kFc2Threads;

__global__ __launch_bounds__(kFc2Threads) void gfc2_kernel(const GroupParams p) {
    extern __shared__ __align__(16) uint8_t lds[];
    const GroupLds2 L = gfc2_lds(p.T, p.S);
    const GroupRoute gr{p.T, p.S};
    const int per_slot = (p.K / kFc2Cols) * p.nsplit, G = gridDim.x;
    const int IS = p.I >> 7;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int sub = wave & (kFc2Sub - 1);  // the sub-tile this wave finishes
    const int j = lane & 15, grp = lane >> 4;
    const uint32_t ctile_bytes = (uint32_t)IS * kFc2Sub * kBlockBytes;
    int* rt = reinterpret_cast<int*>(lds + L.route);
    float* sal = reinterpret_cast<float*>(lds + L.sa);
    int* ring = reinterpret_cast<int*>(lds + L.ring);
    float* red = reinterpret_cast<float*>(lds + L.red);
    const int ntab = gr.prefix(p.M);
    const int nrows = p.E > 0 ? 2 * p.M : p.M;
    auto tile_of = [&](int it) { return it >= 0 ? it % per_slot : 0; };
    auto split_of = [&](int it) { return tile_of(it) % p.nsplit; };
    auto step_of = [&](int it) { return split_of(it) * kFc2SplitSteps + wave * kFc2Steps; };
    auto wres = [&](int expert, int it) {
        return make_res(p.w2p + (uint64_t)expert * p.w2_bytes + (uint64_t)(tile_of(it) / p.nsplit) * ctile_bytes,
                        it >= 0 ? ctile_bytes : 0u);
    };
    auto s2res = [&](int expert, int it) {
        return make_res(p.s2 + (size_t)expert * p.K, it >= 0 ? (uint32_t)p.K * 4 : 0u);
    };
    auto s2off = [&](int it) {
        return (uint32_t)((tile_of(it) / p.nsplit) * kFc2Cols + sub * kTile + 4 * grp) * 4;
    };
    const BufRes qres = make_res(p.aq, (uint32_t)nrows * p.I), qnone = make_res(p.aq, 0u);
    auto load_b = [&](uint4 (&b)[kFc2Steps][2], BufRes res, uint32_t base) {
#pragma unroll
        for (int s = 0; s < kFc2Steps; ++s) {
            b[s][0] = buf_ld16(res, base + s * kKStep);
            b[s][1] = buf_ld16(res, base + s * kKStep + 16);
        }
    };
    // lane's bytes of intermediate row `row` in item `it`'s k-steps
    auto boff = [&](int row, int it) { return (uint32_t)row * p.I + (uint32_t)step_of(it) * kKStep + grp * 32; };

    // 1. the table prefix and the row scales into LDS (the first item, which can be a
    //    routed expert's, comes from the table)
    {
        int tv[2 * kGroupTableRegs];
        const BufRes tres = make_res(p.route, (uint32_t)ntab * 4);
#pragma unroll
        for (int i = 0; i < 2 * kGroupTableRegs; ++i)
            tv[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(tres, (uint32_t)(tid + kFc2Threads * i) * 4, 0, 0);
        float sv[kGroupSaRegs];
        const BufRes sres = make_res(p.sa, (uint32_t)nrows * 4);
#pragma unroll
        for (int i = 0; i < kGroupSaRegs; ++i)
            sv[i] = __builtin_bit_cast(float,
                                       __builtin_amdgcn_raw_buffer_load_b32(sres, (uint32_t)(tid + kFc2Threads * i) * 4, 0, 0));
#pragma unroll
        for (int i = 0; i < 2 * kGroupTableRegs; ++i) {
            const int k = tid + kFc2Threads * i;
            if (k < ntab) rt[k] = tv[i];
        }
#pragma unroll
        for (int i = 0; i < kGroupSaRegs; ++i) {
            const int k = tid + kFc2Threads * i;
            if (k < nrows) sal[k] = sv[i];
        }
    }
    lds_barrier();

    const int item0 = p.item0_2;  // without slot 0's items when the wide kernel takes it
    const GroupPlan<2> plan(G, blockIdx.x, (1 + rt[gr.d()]) * per_slot - item0);
    const GroupOrder ord(item0 ? 0 : per_slot, plan.pool0);
    auto imap = [&](int q) { const int v = ord.map(q); return v < 0 ? v : v + item0; };
    int cur = imap(plan.fixed(0));  // -1: no item (only when the wide kernel takes slot 0)
    int nxt = imap(plan.fixed(1));
    int pos = 0, par = 0;
    auto boff_tile = [&](int it, int tile) {
        const int ps = it >= 0 ? it / per_slot : 0;
        const int pr0 = rt[gr.slot_row0() + ps], pnr = rt[gr.slot_rows() + ps];
        return boff(pr0 + min(16 * tile + j, pnr - 1), it);
    };

    // 2. the first position's codes, then its weights and output-channel scales
    uint4 bx[kFc2Steps][2];
    load_b(bx, qres, boff_tile(cur, 0));
    uint4 w[kFc2Steps][kFc2Sub][2];
    float4 s2c;
    {
        const int e0 = __builtin_amdgcn_readfirstlane(rt[gr.slot_expert() + cur / per_slot]);
        const BufRes rw = wres(e0, cur);
        const uint32_t wo = (uint32_t)step_of(cur) * kFc2Sub * kBlockBytes + lane * 16;
#pragma unroll
        for (int s = 0; s < kFc2Steps; ++s)
#pragma unroll
            for (int u = 0; u < kFc2Sub; ++u)
#pragma unroll
                for (int h = 0; h < 2; ++h) w[s][u][h] = buf_ld16_stream(rw, wo + (s * kFc2Sub + u) * kBlockBytes + h * 1024);
        s2c = buf_ldf4(s2res(e0, cur), s2off(cur));
    }
    __builtin_amdgcn_sched_barrier(0);

    auto kstep = [&](int s, v4f (&acc)[kFc2Sub], BufRes bres, uint32_t bbase) {
        const Operand bo = widen(bx[s][0], bx[s][1]);
#pragma unroll
        for (int u = 0; u < kFc2Sub; ++u) acc[u] = mma_kstep(widen(w[s][u][0], w[s][u][1]), bo, acc[u]);
        __builtin_amdgcn_sched_barrier(0);  // the loads write the registers just read
        bx[s][0] = buf_ld16(bres, bbase + s * kKStep);
        bx[s][1] = buf_ld16(bres, bbase + s * kKStep + 16);
    };
    // reduce over the waves (wave w sums sub-tile w) and write row tile t's partial sums
    auto epilogue = [&](v4f (&acc)[kFc2Sub], int slot, int tile, int r0, int nr, int t) {
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
        const int nrow = min(16, nr - 16 * t);
        if (j < nrow && wave < kFc2Sub) {
            const int split = tile % p.nsplit;
            const int col = (tile / p.nsplit) * kFc2Cols + sub * kTile + 4 * grp;
            const int row = r0 + 16 * t + j;
            const int orow = slot == 0 ? row : p.M + rt[gr.row_token() + row];
            const float f = sal[row];
            float* dst = p.part + ((size_t)split * 2 * p.T + orow) * p.K + col;
            *reinterpret_cast<float4*>(dst) =
                make_float4(o[0] * f * s2c.x, o[1] * f * s2c.y, o[2] * f * s2c.z, o[3] * f * s2c.w);
        }
        par ^= 1;
    };

    float4 s2n = s2c;
    auto last_tile = [&](int slot, int tile, int r0, int nr, int nt) {
        const bool take = plan.pooled(pos + 2);
        uint32_t ticket = 0;
        if (take && tid == 0) ticket = atomicAdd(p.work + 1, 1u);
        const uint32_t bbase = boff_tile(nxt, 0);
        const BufRes bres = nxt >= 0 ? qres : qnone;
        const int nexpert = __builtin_amdgcn_readfirstlane(rt[gr.slot_expert() + (nxt >= 0 ? nxt / per_slot : 0)]);
        const BufRes rn = wres(nexpert, nxt);
        const uint32_t wo = (uint32_t)step_of(nxt) * kFc2Sub * kBlockBytes + lane * 16;
        s2n = buf_ldf4(s2res(nexpert, nxt), s2off(nxt));
        v4f acc[kFc2Sub];
#pragma unroll
        for (int u = 0; u < kFc2Sub; ++u) acc[u] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kFc2Steps; ++s) {
            kstep(s, acc, bres, bbase);
#pragma unroll
            for (int u = 0; u < kFc2Sub; ++u)
#pragma unroll
                for (int h = 0; h < 2; ++h) w[s][u][h] = buf_ld16_stream(rn, wo + (s * kFc2Sub + u) * kBlockBytes + h * 1024);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (take && tid == 0) ring[(pos + 2) % kGroupRing] = plan.from_ticket(ticket);
        epilogue(acc, slot, tile, r0, nr, nt - 1);
    };

    while (cur >= 0) {  // items
        const int slot = cur / per_slot, tile = cur - slot * per_slot;
        const int r0 = rt[gr.slot_row0() + slot], nr = rt[gr.slot_rows() + slot];
        const int nt = (nr + 15) >> 4;
        for (int t = 0; t < nt - 1; ++t) {
            const uint32_t bbase = boff_tile(cur, t + 1);
            v4f acc[kFc2Sub];
#pragma unroll
            for (int u = 0; u < kFc2Sub; ++u) acc[u] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < kFc2Steps; ++s) {
                kstep(s, acc, qres, bbase);
                __builtin_amdgcn_sched_barrier(0);
            }
            epilogue(acc, slot, tile, r0, nr, t);
        }
        last_tile(slot, tile, r0, nr, nt);
        s2c = s2n;
        if (nxt < 0) break;
        cur = nxt;
        nxt = __builtin_amdgcn_readfirstlane(imap(plan.at(pos + 2, ring)));
        ++pos;
    }
}

// ---------------------------------------------------------------------------------
// gcombine: out[m] = bf16(sum of the shared splits + gate[m] * sum of the routed ones).

// lead_mk = M | K << 16, lead_tn = T | nsplit << 16 | (E > 0) << 31.
__global__ __launch_bounds__(256) void gcombine_kernel(const float* lead_part, uint16_t* lead_out,
                                                       const float* lead_gate, uint32_t lead_mk, uint32_t lead_tn,
                                                       const GroupParams p0) {
    GroupParams p = p0;
    p.part = const_cast<float*>(lead_part);
    p.out = lead_out;
    p.gate = const_cast<float*>(lead_gate);
    p.M = (int32_t)(lead_mk & 0xFFFFu);
    p.K = (int32_t)(lead_mk >> 16);
    p.T = (int32_t)(lead_tn & 0xFFFFu);
    p.nsplit = (int32_t)((lead_tn >> 16) & 0x7FFFu);
    const bool routed = (lead_tn >> 31) != 0u;
    const int idx = blockIdx.x * 256 + threadIdx.x;
    const int k4 = p.K >> 2;
    if (idx >= p.M * k4) return;
    const int tok = idx / k4, col = (idx - tok * k4) * 4;
    const size_t ss = (size_t)2 * p.T * p.K;
    const float* ps = p.part + (size_t)tok * p.K + col;
    const float* pr = p.part + (size_t)(p.M + tok) * p.K + col;
    float4 sh = make_float4(0.f, 0.f, 0.f, 0.f), ro = sh;
    // kCombineBatch splits' loads in flight at once, added in split order
    for (int s0 = 0; s0 < p.nsplit; s0 += kCombineBatch) {
        float4 a[kCombineBatch], b[kCombineBatch];
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u) {
            const int sp = min(s0 + u, p.nsplit - 1);  // repeats past the end are not added
            a[u] = *reinterpret_cast<const float4*>(ps + sp * ss);
            if (routed) b[u] = *reinterpret_cast<const float4*>(pr + sp * ss);
        }
#pragma unroll
        for (int u = 0; u < kCombineBatch; ++u)
            if (s0 + u < p.nsplit) {
                sh = add4(sh, a[u]);
                if (routed) ro = add4(ro, b[u]);
            }
    }
    combine_store(p.out + (size_t)tok * p.K + col, sh, ro, routed ? p.gate[tok] : 0.0f);
}

}  // namespace moe
