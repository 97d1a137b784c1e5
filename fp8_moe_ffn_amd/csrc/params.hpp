// Arguments shared by the forward kernels (passed by value).
#pragma once

#include <stdint.h>

namespace moe {

// Forward workspace, all device memory owned by the handle.
//   route: [0] = d (distinct routed experts), [1 + f] = expert index of slot f
//          (slot 0 = shared expert = packed index E, slots 1..d ascending expert ids),
//          [1 + S + m] = slot of token m's routed expert, [1 + S + T + m] = expert of m
//   amax:  float32 bit patterns of max |a| per (slot, token), reset by the router
struct Workspace {
    uint8_t* xq;     // [T][K]
    float* sx;       // [T]
    int32_t* route;  // [1 + S + 2T]
    float* gate;     // [T]
    uint32_t* amax;  // [S][T]
    float* a;        // [S][T][I]    SwiGLU output, float32
    float* part;     // [S][nsplit][T][K]  FC2 partial sums per I split
};

struct Debug {
    uint8_t* xq;
    float* sx;
    int32_t* expert;
    float* gate;
    uint8_t* aq_shared;
    float* sa_shared;
    uint8_t* aq_routed;
    float* sa_routed;
    int32_t* num_active;
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
    int32_t S;               // expert slots in the workspace = 1 + min(T, E)
    int32_t T;               // max tokens (row stride of the workspace)
    int32_t nsplit;          // FC2 splits of the I dimension
    int32_t split_steps;     // 128-wide k-steps per FC2 split
    Workspace ws;
    Debug dbg;
};

}  // namespace moe
