// Arguments shared by the forward kernels (passed by value), and the layout of the
// routing table the first kernel writes.
#pragma once

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
    __host__ __device__ int count() const { return 1 + 3 * S + 4 * T; }
    __host__ __device__ int d() const { return 0; }                         // [1]: distinct routed experts
    __host__ __device__ int slot_expert() const { return 1; }               // [S]: packed expert index
    __host__ __device__ int slot_row0() const { return 1 + S; }             // [S]
    __host__ __device__ int slot_rows() const { return 1 + 2 * S; }         // [S]
    __host__ __device__ int token_row() const { return 1 + 3 * S; }         // [T]: routed row of token m
    __host__ __device__ int token_expert() const { return 1 + 3 * S + T; }  // [T]: -1 when E == 0
    __host__ __device__ int row_token() const { return 1 + 3 * S + 2 * T; } // [2T]
};

// Work counters of the streaming kernels (work-item tickets), reset by the first kernel.
// Each kernel's items are split into kWorkParts partitions with a counter each (block b
// works on partition b mod kWorkParts); counters sit kWorkStride words apart so that
// they do not share a cache line.
constexpr int kWorkParts = 8;
constexpr int kWorkStride = 32;
enum WorkCounter { kWorkFc13 = 0, kWorkFc2 = 1, kWorkKernels = 2 };
constexpr int kWorkWords = kWorkKernels * kWorkParts * kWorkStride;
__host__ __device__ constexpr int work_index(int kernel, int part) {
    return (kernel * kWorkParts + part) * kWorkStride;
}

// Item bookkeeping of a persistent streaming kernel with G blocks over `total` items.
// With P partitions (P = kWorkParts when it divides G, else 1), partition x holds items
// x, x + P, x + 2P, ... and its G / P blocks; a block's first two items are fixed
// (partition positions l and l + G / P, l = b / P), later ones come from the
// partition's counter.  All positions are partition-local; item() maps them back.
struct WorkPlan {
    int P, x, l, gp, total;
    __device__ WorkPlan(int G, int b, int total_items) {
        P = (G % kWorkParts == 0) ? kWorkParts : 1;
        x = b % P;
        l = b / P;
        gp = G / P;
        total = total_items;
    }
    __device__ int count() const { return total > x ? (total - x + P - 1) / P : 0; }  // items of the partition
    __device__ int item(int pos) const { return pos < count() ? pos * P + x : -1; }
    __device__ int first() const { return item(l); }
    __device__ int second() const { return item(l + gp); }
    __device__ int from_ticket(uint32_t t) const { return item(2 * gp + (int)t); }
};

// Forward workspace, device memory owned by the handle.
struct Workspace {
    uint8_t* xq;     // [T][K]      activation codes
    float* sx;       // [T]         activation scales
    int32_t* route;  // RouteLayout
    float* gate;     // [T]
    uint32_t* amax;  // [G13][2T]   float bit patterns of max |a| per row, one row per FC13 block
    float* a;        // [2T][I]     SwiGLU output, float32
    uint8_t* aq;     // [2T][I]     re-quantised intermediate
    float* sa;       // [2T]        its scales
    float* part;     // [nsplit][2T][K]  FC2 partial sums per split of I
    uint32_t* work;  // [kWorkWords] work counters
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
    const uint16_t* x;       // [M][K] bf16
    const uint16_t* logits;  // [M][E] bf16 or null
    uint16_t* out;           // [M][K] bf16
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
    Workspace ws;
    Debug dbg;
};

}  // namespace moe
