// Token order of a batch larger than one launch.
//
// A launch takes up to 16 tokens and streams the shared expert and the distinct routed
// experts of its tokens.  Launches over the batch in its own order would stream a
// popular expert once per launch that holds one of its tokens.  The tokens are
// therefore first put in routed-expert order (the same top-1 choice as the forward:
// the lowest index of the largest logit), so that consecutive launches of 16 tokens
// hold each expert's tokens together and every routed expert is streamed by about one
// launch; an expert's tokens span two launches at most at a boundary.  Each token's
// result depends on its own row only, so the order changes no output.
//
// One block.  The expert of each token (a wave per token and pass, several tokens per
// wave with their loads issued together) goes to LDS as 16 bits, with a count per
// expert; an exclusive scan gives each expert's first position; tokens are placed
// stably, in tiles of one token per thread, at their expert's next position plus the
// number of earlier tokens of the tile with the same expert.
#pragma once

#include "prologue.hpp"

namespace moe {

constexpr int kOrderThreads = 1024;
constexpr int kOrderWaves = kOrderThreads / 64;
constexpr int kOrderTokens = 8;  // tokens per wave and pass

__host__ __device__ inline int order_lds_bytes(int M, int E) { return ((2 * M + 15) & ~15) + 2 * 4 * E; }

// order[i] (i < M) = the token at position i; M <= 65536, 1 <= E <= kMaxRouteExperts.
__global__ __launch_bounds__(kOrderThreads) void order_kernel(const uint16_t* logits, int M, int E,
                                                              int32_t* order) {
    extern __shared__ __align__(16) uint8_t lds[];
    uint16_t* texp = reinterpret_cast<uint16_t*>(lds);                   // [M]
    int* next = reinterpret_cast<int*>(lds + ((2 * M + 15) & ~15));      // [E] count, then position
    int* tail = next + E;                                                // [E] scan scratch
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    for (int e = tid; e < E; e += kOrderThreads) next[e] = 0;
    __syncthreads();

    // 1. expert of each token, and the count per expert
    for (int m0 = wave * kOrderTokens; m0 < M; m0 += kOrderWaves * kOrderTokens) {
        uint32_t key[kOrderTokens];
#pragma unroll
        for (int i = 0; i < kOrderTokens; ++i) key[i] = 0;
        for (int e0 = 0; e0 < E; e0 += 64) {
            const int e = e0 + lane;
            uint32_t v[kOrderTokens];
#pragma unroll
            for (int i = 0; i < kOrderTokens; ++i)
                v[i] = logits[(size_t)min(m0 + i, M - 1) * E + min(e, E - 1)];
#pragma unroll
            for (int i = 0; i < kOrderTokens; ++i)
                if (e < E) key[i] = max(key[i], logit_key(v[i], e));
        }
#pragma unroll
        for (int i = 0; i < kOrderTokens; ++i) {
            const uint32_t k = wave_max_u32(key[i]);
            if (lane == 0 && m0 + i < M) {
                const int e = (int)(0xFFFFu - (k & 0xFFFFu));
                texp[m0 + i] = (uint16_t)e;
                atomicAdd(&next[e], 1);
            }
        }
    }
    __syncthreads();

    // 2. exclusive scan of the counts (E <= kOrderThreads): Hillis-Steele on the inclusive sums
    const int cnt = tid < E ? next[tid] : 0;
    int incl = cnt;
    for (int o = 1; o < E; o <<= 1) {
        if (tid < E) tail[tid] = incl;
        __syncthreads();
        if (tid < E && tid >= o) incl += tail[tid - o];
        __syncthreads();
    }
    if (tid < E) next[tid] = incl - cnt;
    __syncthreads();

    // 3. stable placement, one tile of kOrderThreads tokens at a time
    for (int t0 = 0; t0 < M; t0 += kOrderThreads) {
        const int m = t0 + tid;
        int e = -1, rank = 0;
        if (m < M) {
            e = texp[m];
            for (int j = t0; j < m; ++j) rank += texp[j] == e;
            order[next[e] + rank] = m;
        }
        __syncthreads();  // every position of the tile is taken from the old `next`
        if (m < M) atomicAdd(&next[e], 1);
        __syncthreads();
    }
}

}  // namespace moe
