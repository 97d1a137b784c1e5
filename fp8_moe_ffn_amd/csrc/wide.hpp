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
// channels of the shared expert) over all of K, FC2 one item of the decode kernel (64
// output columns, a 2048-split of I).  The weights of each 128-deep k-step (8 KB) pass
// through a double-buffered LDS stage that all 8 waves read; each thread keeps its
// 16-byte piece of the next kWideRing k-steps in flight in registers and writes it into
// the stage one k-step ahead (one barrier per k-step).  Each wave owns kWideTiles row
// tiles of 16 tokens over the whole reduction, its token codes loaded from L2 kWideB
// k-steps ahead, so the reduction needs no cross-wave pass.  Groups of 256 tokens repeat
// the item's weight stream.
//
// The sums are those of the decode kernels bit for bit: the reduction is cut into the
// same 8 ranges of k-steps that the decode kernels give their 8 waves, each range is
// accumulated by the same matrix instructions in the same order from zero, and the
// ranges' sums are added in order starting from 0.0f, as the decode kernels' LDS
// reductions add the waves' partial tiles; scales, SwiGLU and the partial sums' scaling
// are the same expressions.  So grouped passes give the same bits with or without these
// kernels, and the same as launches of the decode kernels.
#pragma once

#include "codec.hpp"
#include "fc13.hpp"
#include "fc2.hpp"
#include "group.hpp"
#include "layout.hpp"

namespace moe {

constexpr int kWideTiles = 2;                                   // row tiles per wave in a group
constexpr int kWideGroup = kFc13Waves * kWideTiles * kTile;     // 256 tokens per group
constexpr int kWideRing = 4;                                    // k-steps of weights in flight per thread
constexpr int kWideB = 4;                                       // k-steps of token codes in flight per wave
// k-steps per loop body: ring slots, stages and range ends by the body's index
__host__ __device__ constexpr int wide_body(int nr) {
    int p = 4;  // kWideRing, kWideB and the 2 stages divide it
    while (p % nr != 0) p += 4;
    return p;
}
constexpr int kWideStage = 8192;                                // bytes of one k-step's weight codes
constexpr int kWideStage16 = 2 * kWideStage;                    // the same widened to f16 in LDS
constexpr int kWideMin = 128;                                   // tokens of a pass from which it runs wide
static_assert(kFc13Threads * 16 == kWideStage && kFc2Threads == kFc13Threads, "one 16-byte piece per thread");
static_assert(4 % kWideRing == 0 && 4 % kWideB == 0, "a body ends where the rings wrap");

struct WideLds {
    int stage;   // [2][kWideStage16] one k-step's weights widened to f16, [block][j][lane][8 halves]
    int rowv;    // [T] float: the row's scale (FC13: s_x of the token; FC2: s_a of the row)
    int rowmax;  // [T] uint32: the block's max |a| per row (FC13)
    int total;
};

__host__ __device__ inline WideLds wide_lds(int T) {
    WideLds l{};
    l.stage = 0;
    l.rowv = 2 * kWideStage16;
    l.rowmax = align16(l.rowv + T * 4);
    l.total = align16(l.rowmax + T * 4);
    return l;
}

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

// Lane's operand of block b of the stage.
__device__ __forceinline__ Operand lds_operand(const uint8_t* stage16, int b, int lane) {
    return stage_operand(stage16 + b * 4096 + lane * 16);
}

// ---------------------------------------------------------------------------------
// FC13 + SwiGLU of the shared expert: item i = pairs 2i and 2i + 1, all tokens of the pass.
// KS = K / 128 k-steps, cut into kFc13Waves ranges of KS / kFc13Waves.

template <int KS>
__global__ __launch_bounds__(kFc13Threads) void gwide13_kernel(const GroupParams p) {
    extern __shared__ __align__(16) uint8_t lds[];
    constexpr int NR = KS / kFc13Waves;  // k-steps per range
    constexpr int P = wide_body(NR);
    static_assert(NR * kFc13Waves == KS && KS % P == 0, "whole ranges and loop bodies");
    const WideLds L = wide_lds(p.T);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, grp = lane >> 4;
    const int M = p.M, npairs = p.I >> 4, nitems = npairs / 2, G = gridDim.x;
    const uint32_t pair_bytes = (uint32_t)KS * 2 * kBlockBytes;
    const uint8_t* w13e = p.w13p + (uint64_t)p.E * p.w13_bytes;
    const float* s13e = p.s13 + (size_t)p.E * 2 * p.I;
    uint8_t* stage = lds + L.stage;
    float* sxl = reinterpret_cast<float*>(lds + L.rowv);
    uint32_t* rowmax = reinterpret_cast<uint32_t*>(lds + L.rowmax);
    for (int i = tid; i < M; i += kFc13Threads) {
        sxl[i] = p.sx[i];
        rowmax[i] = 0u;
    }
    const int ntiles = (M + 15) >> 4;
    const uint32_t kstride = (uint32_t)ntiles * 2048;  // one k-step of every tile's codes (tile_byte)
    const BufRes xres = make_res(p.xt, (uint32_t)ntiles * 16 * p.K);
    // this thread's 16 bytes of a k-step's 8 KB: pair (tid >> 8) of the item (waves 0-3 and
    // 4-7), byte (tid & 255) * 16 of the pair's [gate 2048 | up 2048] k-step
    const int half = tid >> 8;
    const uint32_t wpiece = (uint32_t)(tid & 255) * 16;
    lds_barrier();

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
            uint4 wr[kWideRing];
            uint4 bx[kWideB][kWideTiles][2];
            // pipeline start: the first kWideRing k-steps of weights, the first kWideB of codes
#pragma unroll
            for (int s = 0; s < kWideRing; ++s) wr[s] = buf_ld16_stream(wres, wpiece, s * 2 * kBlockBytes);
#pragma unroll
            for (int s = 0; s < kWideB; ++s)
#pragma unroll
                for (int t = 0; t < kWideTiles; ++t) {
                    bx[s][t][0] = buf_ld16(xres, brow[t], s * kstride);
                    bx[s][t][1] = buf_ld16(xres, brow[t] + 1024, s * kstride);
                }
            stage_piece(stage, tid, wr[0]);
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
#pragma unroll 1
            for (int s0 = 0; s0 < KS; s0 += P) {
#pragma unroll
                for (int i = 0; i < P; ++i) {
                    const int s = s0 + i;  // s0 is a multiple of P: ring slots, stages and ranges by i
                    const uint8_t* st = stage + (i & 1) * kWideStage16;
                    Operand b[kWideTiles];
#pragma unroll
                    for (int t = 0; t < kWideTiles; ++t) b[t] = widen(bx[i % kWideB][t][0], bx[i % kWideB][t][1]);
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
                    // the next loads, codes kWideB k-steps ahead and weights kWideRing ahead,
                    // issued on every k-step (past the end: unused, and the weights' read nothing)
#pragma unroll
                    for (int t = 0; t < kWideTiles; ++t) {
                        bx[i % kWideB][t][0] = buf_ld16(xres, brow[t], (s + kWideB) * kstride);
                        bx[i % kWideB][t][1] = buf_ld16(xres, brow[t] + 1024, (s + kWideB) * kstride);
                    }
                    wr[i % kWideRing] = buf_ld16_stream(wres, wpiece, (s + kWideRing) * 2 * kBlockBytes);
                    // k-step s + 1 into the other stage (its last reads were k-step s - 1's)
                    stage_piece(stage + ((i + 1) & 1) * kWideStage16, tid, wr[(i + 1) % kWideRing]);
                    lds_barrier();
                }
            }

            // epilogue: scales, SwiGLU, the float32 intermediate and the rows' maxima
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                // scales of the lane's channels (pair0 + c) * 16 + 4 grp + r, r = 0..3
                const int ch = (pair0 + c) * 16 + 4 * grp;
                const float4 sg = *reinterpret_cast<const float4*>(s13e + ch);
                const float4 su = *reinterpret_cast<const float4*>(s13e + p.I + ch);
                const float sgv[4] = {sg.x, sg.y, sg.z, sg.w};
                const float suv[4] = {su.x, su.y, su.z, su.w};
#pragma unroll
                for (int t = 0; t < kWideTiles; ++t) {
                    const int tok = g0 + (wave * kWideTiles + t) * kTile + j;
                    const float sx = sxl[min(tok, M - 1)];
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
// FC2 of the shared expert: item = (64 output columns, one 2048-split of I), all tokens.

__global__ __launch_bounds__(kFc2Threads) void gwide2_kernel(const GroupParams p) {
    extern __shared__ __align__(16) uint8_t lds[];
    constexpr int KS = kFc2SplitSteps;  // k-steps per split
    constexpr int NR = kFc2Steps;       // k-steps per range (the decode kernel's per-wave share)
    constexpr int P = wide_body(NR);
    static_assert(KS % P == 0, "whole loop bodies");
    const WideLds L = wide_lds(p.T);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, grp = lane >> 4;
    const int M = p.M, IS = p.I >> 7, ncol = p.K / kFc2Cols, nitems = ncol * p.nsplit, G = gridDim.x;
    const uint8_t* w2e = p.w2p + (uint64_t)p.E * p.w2_bytes;
    const float* s2e = p.s2 + (size_t)p.E * p.K;
    uint8_t* stage = lds + L.stage;
    float* sal = reinterpret_cast<float*>(lds + L.rowv);
    for (int i = tid; i < M; i += kFc2Threads) sal[i] = p.sa[i];
    const int ntiles = (M + 15) >> 4;
    const uint32_t kstride = (uint32_t)ntiles * 2048;
    const BufRes qres = make_res(p.at, (uint32_t)ntiles * 16 * p.I);  // slot 0's rows: the pass's tokens
    lds_barrier();

    for (int it = blockIdx.x; it < nitems; it += G) {
        const int ct = it / p.nsplit, sp = it - ct * p.nsplit;
        const int ks0 = sp * KS;  // the split's first k-step of I
        // the item's weights alone: loads past its last k-step read nothing
        const BufRes wres = make_res(w2e + (uint64_t)(ct * IS + ks0) * kFc2Sub * kBlockBytes, KS * kWideStage);
        for (int g0 = 0; g0 < M; g0 += kWideGroup) {
            uint32_t brow[kWideTiles];  // lane's bytes of its tiles' k-step 0 (of I: plus the split's)
#pragma unroll
            for (int t = 0; t < kWideTiles; ++t)
                brow[t] = (uint32_t)((g0 >> 4) + wave * kWideTiles + t) * 2048 + lane * 16;
            uint4 wr[kWideRing];
            uint4 bx[kWideB][kWideTiles][2];
#pragma unroll
            for (int s = 0; s < kWideRing; ++s) wr[s] = buf_ld16_stream(wres, tid * 16, s * kWideStage);
#pragma unroll
            for (int s = 0; s < kWideB; ++s)
#pragma unroll
                for (int t = 0; t < kWideTiles; ++t) {
                    bx[s][t][0] = buf_ld16(qres, brow[t], (ks0 + s) * kstride);
                    bx[s][t][1] = buf_ld16(qres, brow[t] + 1024, (ks0 + s) * kstride);
                }
            stage_piece(stage, tid, wr[0]);
            lds_barrier();

            v4f to[kFc2Sub][kWideTiles], ao[kFc2Sub][kWideTiles];
#pragma unroll
            for (int u = 0; u < kFc2Sub; ++u)
#pragma unroll
                for (int t = 0; t < kWideTiles; ++t) {
                    to[u][t] = (v4f){0.f, 0.f, 0.f, 0.f};
                    ao[u][t] = to[u][t];
                }
#pragma unroll 1
            for (int s0 = 0; s0 < KS; s0 += P) {
#pragma unroll
                for (int i = 0; i < P; ++i) {
                    const int s = s0 + i;
                    const uint8_t* st = stage + (i & 1) * kWideStage16;
                    Operand b[kWideTiles];
#pragma unroll
                    for (int t = 0; t < kWideTiles; ++t) b[t] = widen(bx[i % kWideB][t][0], bx[i % kWideB][t][1]);
                    Operand w = lds_operand(st, 0, lane);  // as in FC13: two operands live
#pragma unroll
                    for (int u = 0; u < kFc2Sub; ++u) {
                        const Operand wn = lds_operand(st, (u + 1) % kFc2Sub, lane);
#pragma unroll
                        for (int t = 0; t < kWideTiles; ++t) ao[u][t] = mma_kstep(w, b[t], ao[u][t]);
                        __builtin_amdgcn_sched_barrier(0);
                        w = wn;
                    }
                    if (i % NR == NR - 1) {
#pragma unroll
                        for (int u = 0; u < kFc2Sub; ++u)
#pragma unroll
                            for (int t = 0; t < kWideTiles; ++t) {
                                to[u][t] += ao[u][t];
                                ao[u][t] = (v4f){0.f, 0.f, 0.f, 0.f};
                            }
                    }
#pragma unroll
                    for (int t = 0; t < kWideTiles; ++t) {
                        bx[i % kWideB][t][0] = buf_ld16(qres, brow[t], (ks0 + s + kWideB) * kstride);
                        bx[i % kWideB][t][1] = buf_ld16(qres, brow[t] + 1024, (ks0 + s + kWideB) * kstride);
                    }
                    wr[i % kWideRing] = buf_ld16_stream(wres, tid * 16, (s + kWideRing) * kWideStage);
                    stage_piece(stage + ((i + 1) & 1) * kWideStage16, tid, wr[(i + 1) % kWideRing]);
                    lds_barrier();
                }
            }

            // partial sums times s_a of the row and s2 of the column, [split][row][K]
#pragma unroll
            for (int t = 0; t < kWideTiles; ++t) {
                const int tok = g0 + (wave * kWideTiles + t) * kTile + j;
                if (tok < M) {
                    const float f = sal[tok];
#pragma unroll
                    for (int u = 0; u < kFc2Sub; ++u) {
                        const int col = ct * kFc2Cols + u * kTile + 4 * grp;
                        const float4 s2c = *reinterpret_cast<const float4*>(s2e + col);
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
