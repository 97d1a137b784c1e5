// Arguments shared by the forward kernels (passed by value), and the layout of the
// routing table the first kernel computes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Rows of the intermediate.  A forward over M tokens works on at most 2M rows:
//   rows [0, M)      the shared expert, row m = token m;
//   rows [M, 2M)     the routed experts, grouped by expert slot in ascending expert
//                    id and, inside a slot, in ascending token order.
// Expert slot 0 is the shared expert (rows [0, M)); slots 1..d are the distinct routed
// experts of the step.  Slot f owns rows [row0[f], row0[f] + nrows[f]).
//
// Routing table (int32), T = max tokens, S = 1 + min(T, E) slots:
struct RouteLayout {
    int T, S;
    __host__ __device__ int count() const { return 1 + 3 * S + 5 * T; }
    __host__ __device__ int d() const { return 0; }                         // [1]: distinct routed experts
    __host__ __device__ int slot_expert() const { return 1; }               // [S]: packed expert index
    __host__ __device__ int slot_row0() const { return 1 + S; }             // [S]
    __host__ __device__ int slot_rows() const { return 1 + 2 * S; }         // [S]
    __host__ __device__ int token_row() const { return 1 + 3 * S; }         // [T]: routed row of token m
    __host__ __device__ int token_expert() const { return 1 + 3 * S + T; }  // [T]: -1 when E == 0
    __host__ __device__ int row_token() const { return 1 + 3 * S + 2 * T; } // [2T]
    __host__ __device__ int batch_row() const { return 1 + 3 * S + 4 * T; } // [T]: token m's row of x and out
};

// Item order of a persistent streaming kernel with G blocks over `total` items.  Block
// b works through positions 0, 1, 2, ...: a position below nstatic is item b + G * pos
// (a fixed share, at least the first two); with a pool, later positions draw from the
// remaining items through a work counter, one ticket per position.  The pool evens out
// the blocks' finishing times, which differ with their share of the memory bandwidth;
// it pays when an item lasts longer than a ticket's round trip under load.
struct ItemPlan {
    int G, b, total, nstatic, pool0;
    __device__ ItemPlan(int G_, int b_, int total_, bool pool) : G(G_), b(b_), total(total_) {
        nstatic = pool ? max(2, total / G - 2) : (total + G - 1) / G;
        pool0 = pool ? nstatic * G : total;
    }
    __device__ int fixed(int pos) const {
        const int it = b + G * pos;
        return it < total ? it : -1;
    }
    __device__ bool pooled(int pos) const { return pos >= nstatic && pool0 < total; }
    __device__ int from_ticket(uint32_t t) const { return t < (uint32_t)(total - pool0) ? pool0 + (int)t : -1; }
};

// Item order of a persistent streaming kernel without a pool: block b takes item b, then
// the items from G on are dealt round-robin over the first Ge <= G blocks, Ge being
// the fewest blocks that still need no more rounds than G would.  Every block that
// continues then ends within one item of the others: with G = 256 and 3200 items, 246
// blocks take 13 or 12 items and 10 stop after one, instead of 128 blocks taking a
// 13th item while the other 128 wait.
struct EvenPlan {
    int G, b, total, Ge;
    __device__ EvenPlan(int G_, int b_, int total_) : G(G_), b(b_), total(total_) {
        const int rest = max(total - G, 0), rounds = (rest + G - 1) / G;
        Ge = rounds > 0 ? (rest + rounds - 1) / rounds : G;
    }
    __device__ int fixed(int pos) const {
        if (pos == 0) return b < total ? b : -1;
        if (b >= Ge) return -1;
        const int it = G + b + Ge * (pos - 1);
        return it < total ? it : -1;
    }
};

// Work counter of FC13's pool (uint32).  FC2 resets it at its start: it is not in use
// then, and is zero again before the next FC13 launch.  The handle clears it once.
// The single launch counts the blocks that have finished each phase (words of their own
// cache line).  The counts are never reset: they grow by each phase's (fixed) block count
// per launch, and kSyncEpoch counts the launches completed, advanced by the last combine
// block once every block of the launch is past its wait.  A block waits for its phase's
// count to reach (epoch + 1) times the previous phase's block count, the epoch read at
// its start; so a block of an earlier launch that arrives late still counts where it
// belongs.  kSyncTimeouts counts waits given up (never expected; see block_wait).
enum WorkCounter {
    kWorkFc13 = 0,
    kSyncFc13 = 32,
    kSyncFc2 = 33,
    kSyncCombine = 34,
    kSyncTimeouts = 35,
    kSyncEpoch = 36,
    kWorkWords = 64
};

// A store that blocks on other XCDs read in the same launch (DEV): device scope, written
// through the XCD's L2 (the XCDs' L2 caches are not coherent with one another).  A plain
// store otherwise.
template <bool DEV, class T>
__device__ __forceinline__ void xstore(T* p, T v) {
    if constexpr (DEV) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *p = v;
}

// Block-level arrival at a phase counter: every wave waits until its stores have
// completed, and after the barrier thread 0 adds one.  The stores that the next phase
// reads are device-scope stores (xstore<true>), complete when other XCDs can see them, so
// no L2 write-back is needed (a write-back per block, 32 per XCD and phase, measured
// about 13 us per phase).  Returns the count before the addition (thread 0; 0 elsewhere).
__device__ __forceinline__ uint32_t block_arrive(uint32_t* count) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    uint32_t before = 0;
    if (threadIdx.x == 0) before = __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return before;
}

// Waits until *count has reached n (modulo 2^32: the counts only grow, and a wait starts
// at most one launch's arrivals short of its target), then orders the block's later loads
// after the arrivals.  Only
// thread 0 polls (device-scope atomic loads, a short sleep between them) and then fences
// (acquire: the CU's L1 and the XCD's L2 drop their stale lines; once per block, so the
// block's other waves load after the barrier).  Device-scope loads of the handed-on data
// instead of the invalidation measured slower: several blocks read each slice of the
// intermediate, and such loads bypass the L2 every time.  The wait is
// bounded by the 100 MHz constant clock: after 0.2 s it gives up and counts the timeout,
// so that every wave ends even if a phase never completes.  The single launch relies on
// in-order dispatch: the blocks of an earlier phase have lower indices, so they all hold
// a CU (or have finished) before any block that waits for them is placed.
constexpr uint64_t kSyncSpinTicks = 20000000ull;
__device__ __forceinline__ void block_wait(uint32_t* count, uint32_t n, uint32_t* timeouts) {
    if (threadIdx.x == 0) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while ((int32_t)(__hip_atomic_load(count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - n) < 0) {
            __builtin_amdgcn_s_sleep(2);
            if (__builtin_amdgcn_s_memrealtime() - t0 > kSyncSpinTicks) {
                __hip_atomic_fetch_add(timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();  // the block's later loads follow the fence (earlier ones: immutable weights)
}

// Forward workspace, device memory owned by the handle.
struct Workspace {
    int32_t* route;  // RouteLayout
    float* gate;     // [T]
    uint32_t* amax;  // [2T][G13]   float bit patterns of max |a| per row, one column per FC13 block
    float* a;        // [2T][I]     SwiGLU output, float32
    float* part;     // [nsplit][2T][K]  FC2 partial sums per split of I, times s_a * s2;
                     //             row m: token m's shared expert, row M + m: its routed one
    uint32_t* work;  // [kWorkWords] work counters
    int32_t* order;  // [max tokens] a batch above one launch, in expert order (or null)
};

// Device buffers for the intermediate results a debug forward exports (all optional).
struct Debug {
    uint8_t* xq;         // [M][K]
    float* sx;           // [M]
    int32_t* expert;     // [M]
    float* gate;         // [M]
    uint8_t* aq_shared;  // [M][I]
    float* sa_shared;    // [M]
    uint8_t* aq_routed;  // [M][I], row m = token m's routed expert
    float* sa_routed;    // [M]
    int32_t* num_active; // [1]
};

struct FwdParams {
    const uint16_t* x;       // [*][K] bf16, row tok[m] for the launch's token m
    const uint16_t* logits;  // [*][E] bf16 or null, the same rows
    uint16_t* out;           // [*][K] bf16, the same rows
    const int32_t* tok;      // [M] batch rows of the launch's tokens, or null (row m); the
                             // first kernel reads it and publishes it in the routing table
    const uint8_t* w13p;     // packed FC13 weights, (E+1) experts
    const uint8_t* w2p;      // packed FC2 weights
    const float* s13;        // [E+1][2I]
    const float* s2;         // [E+1][K]
    uint64_t w13_bytes;      // bytes per expert = K * 2I
    uint64_t w2_bytes;       // bytes per expert = I * K
    int32_t M, K, I, E;
    int32_t S;               // expert slots = 1 + min(T, E)
    int32_t T;               // max tokens (row stride of the workspace)
    int32_t nsplit;          // FC2 splits of the I dimension
    int32_t grid13;          // FC13 blocks (rows of ws.amax)
    int32_t first_chunk;     // the forward's first launch of M tokens (debug counters start)
    int32_t gate_input;      // variant: the gate scales the routed expert's input, not its output
    float x_scale;           // variant: static scale of x (> 0), else per-token dynamic
    float a_scale;           // variant: static scale of the intermediate (> 0), else dynamic
    const uint16_t* norm_w;  // [K] bf16: RMSNorm of x fused in front (x is then the hidden state), or null
    float norm_eps;          // its epsilon
    Workspace ws;
    Debug dbg;              // token-indexed like x
};

}  // namespace moe
