// The shared expert's GEMMs in a grouped pass with many tokens: FC13 + SwiGLU and FC2 with
// the tokens split over the waves instead of the reduction.
//
// At a few hundred tokens the shared expert's GEMMs are no longer a weight stream: 256
// tokens make 512 flop per weight byte, near the matrix unit's ridge.  The grouped
// kernels (group.hpp) keep an item's weights in registers, split its reduction over the
// 8 waves and loop over 16-token row tiles; per row tile each wave re-widens its weights,
// reads its tokens' codes from L2 one tile ahead and the block reduces the 8 waves'
// partial tiles through LDS behind a barrier.  A per-tile timeline of that loop at 256
// tokens (MI355X) measured 1.8 us of k-steps and 1.6 us of reduction per tile against
// 0.53 us of matrix work.
//
// Here a block owns an item for all tokens of the pass: FC13 two pairs (32 gate + 32 up
// channels of the shared expert) over all of K, FC2 SUB 16-column sub-tiles of one
// 2048-split of I.  The weights of each 128-deep k-step pass through LDS, read by all 8
// waves: FC13 widens them to f16 once per block (each thread keeps its 16-byte piece of
// the next R k-steps in registers and stages it one k-step ahead), FC2 loads them as codes
// straight into a ring of k-steps in LDS.  Each wave owns kWideTiles row tiles of 16
// tokens over the whole reduction, their codes loaded in operand order (tile_byte) a few
// k-steps ahead, so the reduction needs no cross-wave pass.  Groups of 256 tokens repeat
// the item's weight stream.
//
// What bounds them (MI355X, 256 tokens, K = 5120, I = 8192): per k-step a block reads 32 KB
// of token codes and 8-10 KB of weights, its 8 waves read 128 KB of f16 weight operands from
// LDS, and its matrix unit needs ~1,024 cycles per SIMD.  FC13's k-step takes ~0.94 us, 0.44-
// 0.48 us of it matrix work; the rest is load issue, staging and the barrier of each group of
// k-steps.  Timing copies with the codes or the weights held in the caches take as long, so
// memory latency is not what bounds them: the CU's LDS, matrix unit and vector-memory path
// are each near their limits and overlap only in part.
//
// The sums are those of the decode kernels bit for bit: the reduction is cut into the
// same 8 ranges of k-steps that the decode kernels give their 8 waves, each range is
// accumulated by the same matrix instructions in the same order from zero, and the
// ranges' sums are added in order starting from 0.0f, as the decode kernels' LDS
// reductions add the waves' partial tiles; scales, SwiGLU and the partial sums' scaling
// are the same expressions.  So grouped passes give the same bits with or without these
// kernels, and the same as launches of the decode kernels.
#pragma once

#include <type_traits>

#include "codec.hpp"
#include "fc13.hpp"
#include "fc2.hpp"
#include "group.hpp"
#include "layout.hpp"

namespace moe {

constexpr int kWideTiles = 2;                                   // row tiles per wave in a group
constexpr int kWideGroup = kFc13Waves * kWideTiles * kTile;     // 256 tokens per group
constexpr int kWideB = 4;                                       // k-steps of codes in flight (FC2; FC13 at short ranges)
// k-steps per loop body: ring slots (r of them) and range ends (every nr) by the body's index
__host__ __device__ constexpr int wide_body(int nr, int r) {
    int p = r;
    while (p % nr != 0) p += r;
    return p;
}
constexpr int kWideStage = 8192;                                // bytes of one k-step's weight codes
constexpr int kWideStage16 = 2 * kWideStage;                    // the same widened to f16 in LDS
constexpr int kWideMin = 128;                                   // tokens of a pass from which it runs wide
static_assert(kFc13Threads * 16 == kWideStage && kFc2Threads == kFc13Threads, "one 16-byte piece per thread");

struct WideLds {
    int stage;   // the weights' stage (FC13: [2][kWideStage16] f16; FC2: its ring of codes)
    int rowmax;  // [T] uint32: the block's max |a| per row (FC13)
    int total;
};

__host__ __device__ inline WideLds wide_lds(int T, int stage_bytes) {
    WideLds l{};
    l.stage = 0;
    l.rowmax = align16(stage_bytes);
    l.total = align16(l.rowmax + T * 4);
    return l;
}

// The wide FC13 stages a group of kWideSG k-steps of weights between two block barriers,
// into one of two groups of stages; the group's last k-step was requested kWideSG k-steps
// later than with one k-step per barrier (R - kWideSG k-steps ahead).  Its LDS before the
// row maxima: 2 kWideSG f16 stages, then 1 KB for the item's gate and up scales.
constexpr int kWideSG = 2;
__host__ __device__ inline int wide13_stage_bytes() { return 2 * kWideSG * kWideStage16 + 1024; }


// The wide path takes slot 0 (the shared expert, rows = the pass's tokens) when the pass has
// at least kWideMin tokens, K is a multiple of 1024 up to 5120 and I a multiple of 2048.
__host__ __device__ inline bool wide_shape(int K, int I) {
    return K % 1024 == 0 && K <= 5120 && I % 2048 == 0;
}

// A thread's 16 codes of a k-step (bytes 16 tid of its 8 KB: block tid / 128, half
// (tid / 64) mod 2, lane tid mod 64) into the stage, widened there once for all 8 waves.
__device__ __forceinline__ void stage_piece(uint8_t* stage16, int tid, uint4 c) {
    stage_store(stage16 + (tid >> 7) * 4096 + ((tid >> 6) & 1) * 2048 + (tid & 63) * 16, c);
}

// Lane's operand of a block of codes in LDS ([half][lane][16 B], 2048 bytes), widened.
__device__ __forceinline__ Operand lds_code_operand(const uint8_t* blk, int lane) {
    return widen(*reinterpret_cast<const uint4*>(blk + lane * 16), *reinterpret_cast<const uint4*>(blk + 1024 + lane * 16));
}

// Lane's operand of block b of the stage.
__device__ __forceinline__ Operand lds_operand(const uint8_t* stage16, int b, int lane) {
    return stage_operand(stage16 + b * 4096 + lane * 16);
}

// ---------------------------------------------------------------------------------
// FC13 + SwiGLU of the shared expert: item i = pairs 2i and 2i + 1, all tokens of the pass.
// KS = K / 128 k-steps, cut into kFc13Waves ranges of KS / kFc13Waves.

template <int KS>
// The leading arguments repeat the fields of p that the kernel uses (group.hpp says why):
// lead_w13e / lead_s13e = the shared expert's packed W13 and scales, lead_mk = M | K << 16,
// lead_ig = I | gridDim.x << 16.
__global__ __launch_bounds__(kFc13Threads) void gwide13_kernel(const uint8_t* lead_w13e, const uint8_t* lead_xt,
                                                               const float* lead_sx, const float* lead_s13e,
                                                               float* lead_a, uint32_t* lead_amax, uint32_t lead_mk,
                                                               uint32_t lead_ig, const GroupParams p0) {
    GroupParams p = p0;
    p.xt = const_cast<uint8_t*>(lead_xt);
    p.sx = const_cast<float*>(lead_sx);
    p.a = lead_a;
    p.amax = lead_amax;
    p.M = (int32_t)(lead_mk & 0xFFFFu);
    p.K = (int32_t)(lead_mk >> 16);
    p.I = (int32_t)(lead_ig & 0xFFFFu);
    extern __shared__ __align__(16) uint8_t lds[];
    constexpr int NR = KS / kFc13Waves;  // k-steps per range
    constexpr int R = NR >= 3 ? NR : kWideB;  // k-steps of weights and codes in flight (ring slots by index)
    constexpr int P = wide_body(NR, R);
    constexpr int SG = kWideSG;  // k-steps per stage group
    static_assert(NR * kFc13Waves == KS && KS % P == 0 && KS % SG == 0, "whole ranges, bodies and groups");
    static_assert(R > SG, "a group's weights are staged from registers not yet reloaded");
    const WideLds L = wide_lds(0, wide13_stage_bytes());  // (the offsets do not depend on T)
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, grp = lane >> 4;
    const int M = p.M, npairs = p.I >> 4, nitems = npairs / 2, G = (int)(lead_ig >> 16);
    const uint32_t pair_bytes = (uint32_t)KS * 2 * kBlockBytes;
    const uint8_t* w13e = lead_w13e;
    const float* s13e = lead_s13e;
    uint8_t* stage = lds + L.stage;
    uint8_t* scl = stage + 2 * kWideSG * kWideStage16;  // the item's scales: gate [32] | up [32] floats
    // k-step s's stage: group (s / SG) mod 2, member s mod SG
    auto stage_of = [&](int s) { return stage + (((s / SG) & 1) * SG + s % SG) * kWideStage16; };
    uint32_t* rowmax = reinterpret_cast<uint32_t*>(lds + L.rowmax);
    for (int i = tid; i < M; i += kFc13Threads) rowmax[i] = 0u;  // before the first barrier below
    const BufRes sres = make_res(s13e, (uint32_t)p.I * 8);
    const int ntiles = (M + 15) >> 4;
    const uint32_t kstride = (uint32_t)ntiles * 2048;  // one k-step of every tile's codes (tile_byte)
    const BufRes xres = make_res(p.xt, (uint32_t)ntiles * 16 * p.K);
    // this thread's 16 bytes of a k-step's 8 KB: pair (tid >> 8) of the item (waves 0-3 and
    // 4-7), byte (tid & 255) * 16 of the pair's [gate 2048 | up 2048] k-step
    const int half = tid >> 8;
    const uint32_t wpiece = (uint32_t)(tid & 255) * 16;

    for (int it = blockIdx.x; it < nitems; it += G) {
        const int pair0 = 2 * it;
        // the wave's pair alone: loads past its last k-step read nothing
        const BufRes wres = make_res(w13e + (uint64_t)(pair0 + half) * pair_bytes, pair_bytes);
        for (int g0 = 0; g0 < M; g0 += kWideGroup) {
            // lane's bytes of its tiles' k-step 0 (tiles past the pass read other codes or
            // nothing: their rows are not stored)
            uint32_t brow[kWideTiles];
#pragma unroll
            for (int t = 0; t < kWideTiles; ++t) brow[t] = (uint32_t)((g0 >> 4) + wave * kWideTiles + t) * 2048 + lane * 16;
            // the item's channel scales into LDS (a direct load, no registers; lanes 0-7 the
            // gate's 32, lanes 8-15 the up's, the rest read nothing) and the scales of the
            // lane's rows, both requested ahead of the pipeline and used in the epilogue
            buf_ld16_lds(sres, scl,
                         lane < 16 ? (uint32_t)((lane >> 3) * p.I + pair0 * 16 + (lane & 7) * 4) * 4 : 0x80000000u);
            float sxr[kWideTiles];
#pragma unroll
            for (int t = 0; t < kWideTiles; ++t) sxr[t] = p.sx[min(g0 + (wave * kWideTiles + t) * kTile + j, M - 1)];
            uint4 wr[R];
            uint4 bx[R][kWideTiles][2];
            // pipeline start: the first R k-steps of weights and of codes
#pragma unroll
            for (int s = 0; s < R; ++s) wr[s] = buf_ld16_stream(wres, wpiece, s * 2 * kBlockBytes);
#pragma unroll
            for (int s = 0; s < R; ++s)
#pragma unroll
                for (int t = 0; t < kWideTiles; ++t) {
                    bx[s][t][0] = buf_ld16(xres, brow[t], s * kstride);
                    bx[s][t][1] = buf_ld16(xres, brow[t] + 1024, s * kstride);
                }
#pragma unroll
            for (int s = 0; s < SG; ++s) stage_piece(stage_of(s), tid, wr[s]);
            lds_barrier();

            v4f tg[2][kWideTiles], tu[2][kWideTiles];  // the ranges' sums, added in order from 0
            v4f ag[2][kWideTiles], au[2][kWideTiles];  // the current range
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int t = 0; t < kWideTiles; ++t) {
                    tg[c][t] = (v4f){0.f, 0.f, 0.f, 0.f};
                    tu[c][t] = tg[c][t];
                    ag[c][t] = tg[c][t];
                    au[c][t] = tg[c][t];
                }
            // P k-steps from s0 (a multiple of P: ring slots and range ends by i); the last P
            // issue no loads, so that nothing is left in flight behind the epilogue's reads
            auto body = [&](const int s0, auto loads) {
#pragma unroll
                for (int i = 0; i < P; ++i) {
                    const int s = s0 + i;
                    const uint8_t* st = stage_of(s);
                    Operand b[kWideTiles];
#pragma unroll
                    for (int t = 0; t < kWideTiles; ++t) b[t] = widen(bx[i % R][t][0], bx[i % R][t][1]);
                    // blocks 2c (gate) and 2c + 1 (up), each read while the previous one's
                    // instructions run: two operands live at a time
                    Operand w = lds_operand(st, 0, lane);
#pragma unroll
                    for (int o = 0; o < 4; ++o) {
                        const Operand wn = lds_operand(st, (o + 1) & 3, lane);  // o = 3: unused
                        v4f* acc = (o & 1) ? au[o >> 1] : ag[o >> 1];
#pragma unroll
                        for (int t = 0; t < kWideTiles; ++t) acc[t] = mma_kstep(w, b[t], acc[t]);
                        __builtin_amdgcn_sched_barrier(0);
                        w = wn;
                    }
                    if (i % NR == NR - 1) {  // a range ends: add its sums, start the next from 0
#pragma unroll
                        for (int c = 0; c < 2; ++c)
#pragma unroll
                            for (int t = 0; t < kWideTiles; ++t) {
                                tg[c][t] += ag[c][t];
                                tu[c][t] += au[c][t];
                                ag[c][t] = (v4f){0.f, 0.f, 0.f, 0.f};
                                au[c][t] = ag[c][t];
                            }
                    }
                    if constexpr (decltype(loads)::value) {  // codes and weights R k-steps ahead
#pragma unroll
                        for (int t = 0; t < kWideTiles; ++t) {
                            bx[i % R][t][0] = buf_ld16(xres, brow[t], (s + R) * kstride);
                            bx[i % R][t][1] = buf_ld16(xres, brow[t] + 1024, (s + R) * kstride);
                        }
                        wr[i % R] = buf_ld16_stream(wres, wpiece, (s + R) * 2 * kBlockBytes);
                    }
                    // at a group's last k-step: the next group into the other group of stages
                    // (its last reads were the previous group's)
                    if (!decltype(loads)::value && i == P - 1) break;
                    if (s % SG == SG - 1) {  // (wave-uniform)
#pragma unroll
                        for (int u = 1; u <= SG; ++u) stage_piece(stage_of(s + u), tid, wr[(i + u) % R]);
                        lds_barrier();
                    }
                    __builtin_amdgcn_sched_barrier(0);  // one k-step at a time
                }
            };
            const int ks_run = (p.K >> 7) - P;  // = KS - P, read at run time: the loop stays a loop
#pragma unroll 1
            for (int s0 = 0; s0 < ks_run; s0 += P) body(s0, std::true_type{});
            body(KS - P, std::false_type{});

            // epilogue: scales, SwiGLU, the float32 intermediate and the rows' maxima
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                // scales of the lane's channels (pair0 + c) * 16 + 4 grp + r, r = 0..3
                const int ch = (pair0 + c) * 16 + 4 * grp;
                const float4 sg = *reinterpret_cast<const float4*>(scl + (c * 16 + 4 * grp) * 4);
                const float4 su = *reinterpret_cast<const float4*>(scl + 128 + (c * 16 + 4 * grp) * 4);
                const float sgv[4] = {sg.x, sg.y, sg.z, sg.w};
                const float suv[4] = {su.x, su.y, su.z, su.w};
#pragma unroll
                for (int t = 0; t < kWideTiles; ++t) {
                    const int tok = g0 + (wave * kWideTiles + t) * kTile + j;
                    const float sx = sxr[t];
                    float a4[4], mx = 0.0f;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float g = tg[c][t][r] * sx * sgv[r];
                        const float u = tu[c][t][r] * sx * suv[r];
                        a4[r] = g / (1.0f + expf(-g)) * u;
                        mx = fmaxf(mx, fabsf(a4[r]));
                    }
                    if (tok < M) *reinterpret_cast<float4*>(p.a + (size_t)tok * p.I + ch) = make_float4(a4[0], a4[1], a4[2], a4[3]);
                    mx = fmaxf(mx, __shfl_xor(mx, 16));
                    mx = fmaxf(mx, __shfl_xor(mx, 32));
                    if (lane < 16 && tok < M && mx > 0.0f) atomicMax(rowmax + tok, __float_as_uint(mx));
                }
            }
        }
    }
    lds_barrier();
    for (int i = tid; i < M; i += kFc13Threads) {
        const uint32_t v = rowmax[i];
        if (v != 0u) atomicMax(p.amax + i, v);
    }
}

// ---------------------------------------------------------------------------------
// FC2 of the shared expert: item = (SUB 16-column sub-tiles, one 2048-split of I), all
// tokens.  SUB is chosen per shape so that the items fill the grid in whole rounds (K =
// 5120: 5 sub-tiles, 256 items).  A k-step's weights (SUB blocks of 2 KB) go from memory
// straight into a ring of kW2Slots k-steps in LDS, as codes, without registers: a wave
// issues its 1 KB pieces of k-step s + kWideB just before its token codes of that k-step,
// so a wait for those codes also covers its pieces, memory counters retiring in order; the
// barrier of each pair of k-steps then makes every wave's pieces of the pair visible.  Each
// wave widens the operands it reads.

constexpr int kW2Slots = kWideB + 2;  // the pair of k-steps in use and kWideB ahead

// s_waitcnt immediate that waits for all but the last n vector memory accesses (gfx9: vmcnt in
// bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima, i.e. not waited for)
__host__ __device__ constexpr int vm_wait_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// the ring, then 1 KB that the loads of a wave without a piece write (zeros, no memory read),
// then 1 KB for the item's output-channel scales s2
__host__ __device__ inline int wide2_stage_bytes(int sub) { return kW2Slots * sub * kBlockBytes + 2048; }

// The sub-tiles per FC2 item for K (K / 16 a multiple of it): the fewest rounds of sub-tile
// work over a grid of G blocks; 0 if none fits.
__host__ __device__ inline int wide2_sub(int K, int nsplit, int G) {
    int best = 0, cost = 0;
    for (int sub = 3; sub <= 5; ++sub) {
        const int nsub = K / kTile;
        if (nsub % sub != 0) continue;
        const int items = nsub / sub * nsplit, c = (items + G - 1) / G * sub;
        if (best == 0 || c < cost) best = sub, cost = c;
    }
    return best;
}

template <int SUB>
// lead_w2e / lead_s2e = the shared expert's packed W2 and scales, lead_mk = M | K << 16,
// lead_in = I | nsplit << 16, lead_tg = T | gridDim.x << 16.
__global__ __launch_bounds__(kFc2Threads) void gwide2_kernel(const uint8_t* lead_w2e, const uint8_t* lead_at,
                                                             const float* lead_sa, const float* lead_s2e,
                                                             float* lead_part, uint32_t lead_mk, uint32_t lead_in,
                                                             uint32_t lead_tg, const GroupParams p0) {
    GroupParams p = p0;
    p.at = const_cast<uint8_t*>(lead_at);
    p.sa = const_cast<float*>(lead_sa);
    p.part = lead_part;
    p.M = (int32_t)(lead_mk & 0xFFFFu);
    p.K = (int32_t)(lead_mk >> 16);
    p.I = (int32_t)(lead_in & 0xFFFFu);
    p.nsplit = (int32_t)(lead_in >> 16);
    p.T = (int32_t)(lead_tg & 0xFFFFu);
    extern __shared__ __align__(16) uint8_t lds[];
    constexpr int KS = kFc2SplitSteps;  // k-steps per split
    constexpr int NR = kFc2Steps;       // k-steps per range (the decode kernel's per-wave share)
    constexpr int P = wide_body(NR, kWideB);
    constexpr int kPieces = 2 * SUB;                                 // 1 KB pieces of a k-step
    constexpr int kPerWave = (kPieces + kFc2Waves - 1) / kFc2Waves;  // pieces a wave loads
    constexpr int kStepLoads = kPerWave + 2 * kWideTiles;            // a wave's accesses per k-step
    constexpr uint32_t kStep = SUB * kBlockBytes;                    // LDS bytes of a k-step
    static_assert(KS % P == 0 && P % kWideB == 0 && P % 2 == 0, "whole loop bodies of whole pairs");
    const WideLds L = wide_lds(0, wide2_stage_bytes(SUB));  // (the offsets do not depend on T)
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, grp = lane >> 4;
    const int M = p.M, IS = p.I >> 7, ncg = (p.K / kTile) / SUB, nitems = ncg * p.nsplit, G = (int)(lead_tg >> 16);
    const uint8_t* w2e = lead_w2e;
    const float* s2e = lead_s2e;
    uint8_t* stage = lds + L.stage;
    uint8_t* sink = stage + kW2Slots * kStep;  // where a wave without a piece loads to
    uint8_t* s2l = sink + 1024;                // the item's SUB * 16 scales s2
    const BufRes s2res = make_res(s2e, (uint32_t)p.K * 4);
    const int ntiles = (M + 15) >> 4;
    const uint32_t kstride = (uint32_t)ntiles * 2048;
    const BufRes qres = make_res(p.at, (uint32_t)ntiles * 16 * p.I);  // slot 0's rows: the pass's tokens

    for (int it = blockIdx.x; it < nitems; it += G) {
        const int cg = it / p.nsplit, sp = it - cg * p.nsplit;
        const int ks0 = sp * KS;  // the split's first k-step of I
        // the wave's pieces: piece q = wave + 8 r is half q mod 2 of sub-tile q / 2 of the
        // item, read from its packed W2 tile ([col tile][k-step][sub][2048]); loads past the
        // split's last k-step read nothing, and so does a wave without an r-th piece
        BufRes wres[kPerWave];
#pragma unroll
        for (int r = 0; r < kPerWave; ++r) {
            const int q = wave + kFc2Waves * r;
            const int g = cg * SUB + (q >> 1);
            const uint64_t off = ((uint64_t)(g >> 2) * IS * kFc2Sub + (g & 3) + (uint64_t)ks0 * kFc2Sub) * kBlockBytes +
                                 (q & 1) * 1024;
            wres[r] = make_res(w2e + (q < kPieces ? off : 0),
                               q < kPieces ? (uint32_t)(KS - 1) * kFc2Sub * kBlockBytes + 1024 : 0u);
        }
        auto load_weights = [&](int s) {  // k-step s of the split into its ring slot
            uint8_t* dst = stage + (uint32_t)(s % kW2Slots) * kStep;
#pragma unroll
            for (int r = 0; r < kPerWave; ++r) {
                const int q = wave + kFc2Waves * r;
                buf_ld16_lds(wres[r], q < kPieces ? dst + q * 1024 : sink, lane * 16, (uint32_t)s * kFc2Sub * kBlockBytes);
            }
        };
        for (int g0 = 0; g0 < M; g0 += kWideGroup) {
            uint32_t brow[kWideTiles];  // lane's bytes of its tiles' k-step 0 (of I: plus the split's)
#pragma unroll
            for (int t = 0; t < kWideTiles; ++t)
                brow[t] = (uint32_t)((g0 >> 4) + wave * kWideTiles + t) * 2048 + lane * 16;
            uint4 bx[kWideB][kWideTiles][2];
            // the first kWideB k-steps: each k-step's weight pieces, then its codes
            lds_barrier();  // the ring's last reads (the previous group or item) are done
            // the item's s2 into LDS (a direct load; every wave the same bytes, lanes past the
            // item's columns read nothing) and s_a of the lane's rows, both requested ahead of
            // the pipeline and used in the epilogue
            buf_ld16_lds(s2res, s2l, lane < SUB * 4 ? (uint32_t)(cg * SUB * kTile + lane * 4) * 4 : 0x80000000u);
            float saf[kWideTiles];
#pragma unroll
            for (int t = 0; t < kWideTiles; ++t) saf[t] = p.sa[min(g0 + (wave * kWideTiles + t) * kTile + j, M - 1)];
#pragma unroll
            for (int s = 0; s < kWideB; ++s) {
                load_weights(s);
#pragma unroll
                for (int t = 0; t < kWideTiles; ++t) {
                    bx[s][t][0] = buf_ld16(qres, brow[t], (ks0 + s) * kstride);
                    bx[s][t][1] = buf_ld16(qres, brow[t] + 1024, (ks0 + s) * kstride);
                }
            }

            v4f to[SUB][kWideTiles], ao[SUB][kWideTiles];
#pragma unroll
            for (int u = 0; u < SUB; ++u)
#pragma unroll
                for (int t = 0; t < kWideTiles; ++t) {
                    to[u][t] = (v4f){0.f, 0.f, 0.f, 0.f};
                    ao[u][t] = to[u][t];
                }
            // P k-steps from s0 (a multiple of P); the last P issue no loads, so that nothing is
            // left in flight behind the epilogue's reads
            auto steps = [&](const int s0, auto loads) {
#pragma unroll
                for (int i = 0; i < P; ++i) {
                    const int s = s0 + i;
                    // the codes of k-step s (and so this wave's weight pieces of it) have landed
                    Operand b[kWideTiles];
#pragma unroll
                    for (int t = 0; t < kWideTiles; ++t) b[t] = widen(bx[i % kWideB][t][0], bx[i % kWideB][t][1]);
                    // one barrier per pair of k-steps: every wave's pieces of k-steps s and s + 1
                    // have landed and its reads of the previous pair's slots are done.  A wave's
                    // own pieces of s + 1 are behind the wait for its codes of s + 1 (issued
                    // after them; memory counters retire in order): all its accesses but those
                    // of the next two k-steps, fewer at the end.  The barrier carries no fence,
                    // which would wait for every direct load in flight, as for any LDS write.
                    if (i % 2 == 0) {
                        const int later = decltype(loads)::value ? 2 : min(2, P - 2 - i);  // k-steps issued after s + 1
                        if (later == 2)
                            __builtin_amdgcn_s_waitcnt(vm_wait_imm(2 * kStepLoads));
                        else if (later == 1)
                            __builtin_amdgcn_s_waitcnt(vm_wait_imm(kStepLoads));
                        else
                            __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
                        __builtin_amdgcn_sched_barrier(0);  // the waits stay before the barrier
                        asm volatile("s_barrier" ::: "memory");
                    }
                    // the slot written (k-step s + kWideB, free since the pair's barrier) and the
                    // slot read (k-step s) differ:
                    // said to the compiler, so that its reads of one need not wait for the other
                    auto body = [&](const uint8_t* __restrict__ st, uint8_t* __restrict__ nx) {
                        if constexpr (decltype(loads)::value) {
#pragma unroll
                            for (int r = 0; r < kPerWave; ++r) {
                                const int q = wave + kFc2Waves * r;
                                buf_ld16_lds(wres[r], q < kPieces ? nx + q * 1024 : sink, lane * 16,
                                             (uint32_t)(s + kWideB) * kFc2Sub * kBlockBytes);
                            }
#pragma unroll
                            for (int t = 0; t < kWideTiles; ++t) {
                                bx[i % kWideB][t][0] = buf_ld16(qres, brow[t], (ks0 + s + kWideB) * kstride);
                                bx[i % kWideB][t][1] = buf_ld16(qres, brow[t] + 1024, (ks0 + s + kWideB) * kstride);
                            }
                        }
                        Operand w = lds_code_operand(st, lane);  // two operands live at a time
#pragma unroll
                        for (int u = 0; u < SUB; ++u) {
                            const Operand wn = lds_code_operand(st + ((u + 1) % SUB) * kBlockBytes, lane);
#pragma unroll
                            for (int t = 0; t < kWideTiles; ++t) ao[u][t] = mma_kstep(w, b[t], ao[u][t]);
                            __builtin_amdgcn_sched_barrier(0);
                            w = wn;
                        }
                    };
                    body(stage + (uint32_t)(s % kW2Slots) * kStep, stage + (uint32_t)((s + kWideB) % kW2Slots) * kStep);
                    if (i % NR == NR - 1) {
#pragma unroll
                        for (int u = 0; u < SUB; ++u)
#pragma unroll
                            for (int t = 0; t < kWideTiles; ++t) {
                                to[u][t] += ao[u][t];
                                ao[u][t] = (v4f){0.f, 0.f, 0.f, 0.f};
                            }
                    }
                    __builtin_amdgcn_sched_barrier(0);  // one k-step at a time
                }
            };
            const int ks_run = (int)(__builtin_amdgcn_readfirstlane(p.nsplit) > 0 ? KS - P : 0);  // a loop at run time
#pragma unroll 1
            for (int s0 = 0; s0 < ks_run; s0 += P) steps(s0, std::true_type{});
            steps(KS - P, std::false_type{});

            // partial sums times s_a of the row and s2 of the column, [split][row][K]
#pragma unroll
            for (int t = 0; t < kWideTiles; ++t) {
                const int tok = g0 + (wave * kWideTiles + t) * kTile + j;
                if (tok < M) {
                    const float f = saf[t];
#pragma unroll
                    for (int u = 0; u < SUB; ++u) {
                        const int col = (cg * SUB + u) * kTile + 4 * grp;
                        const float4 s2c = *reinterpret_cast<const float4*>(s2l + (u * kTile + 4 * grp) * 4);
                        *reinterpret_cast<float4*>(p.part + ((size_t)sp * 2 * p.T + tok) * p.K + col) =
                            make_float4(to[u][t][0] * f * s2c.x, to[u][t][1] * f * s2c.y, to[u][t][2] * f * s2c.z,
                                        to[u][t][3] * f * s2c.w);
                    }
                }
            }
        }
    }
}

}  // namespace moe
