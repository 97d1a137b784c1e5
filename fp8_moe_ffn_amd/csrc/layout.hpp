// Packed weight layout read by the FC13 and FC2 kernels, and the gfx950 matrix
// instruction they use.
//
// Matrix instruction: v_mfma_f32_16x16x128_f8f6f4 with both operands in OCP fp8
// e4m3.  A is 16 x 128 (output channel x reduction), B is 128 x 16 (reduction x
// token), C is 16 x 16 float32.  Each lane holds 32 bytes of A and 32 of B:
//     lane l: row/column (l & 15), reduction offsets 32*(l >> 4) + [0, 32)
// and four accumulators: C[4*(l >> 4) + r][l & 15], r = 0..3.
// The reduction offsets within a lane only have to be the same for A and B, which
// they are since both are packed with the function below.
//
// One "operand block" = the A operand of one instruction = 16 output channels x
// 128 reduction indices = 2048 bytes, stored as [half h][lane l][16 bytes]:
// byte j of (h, l) is reduction offset 32*(l >> 4) + 16*h + j of channel (l & 15).
// A wave reads a block with two fully coalesced 1 KiB loads (16 bytes per lane).
//
// FC13, per expert, blocks in the order [pair p][kstep s][u]:
//   channel n = u*I + 16*p + (row), reduction index k = 128*s + offset;
//   u = 0 gate, u = 1 up.  The gate and up channels of one pair sit next to each
//   other so that SwiGLU is applied in registers.  A pair holds K/128 * 4 KiB.
// FC2, per expert, blocks in the order [column tile c][kstep s][sub]:
//   output column = 64*c + 16*sub + (row), reduction index j = 128*s + offset.
//   A column tile of 64 columns holds I/128 * 8 KiB, k-steps contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kBlockBytes = 2048;  // one 16 x 128 fp8 operand
constexpr int kKStep = 128;        // reduction length of one instruction
constexpr int kTile = 16;          // output channels per instruction (and max tokens)
constexpr int kFc2Sub = 4;         // 16-column sub-tiles per FC2 column tile
constexpr int kFc2Cols = kTile * kFc2Sub;

// Byte offset, inside an operand block, of (row r, reduction offset kk).
__host__ __device__ __forceinline__ uint32_t block_offset(uint32_t r, uint32_t kk) {
    const uint32_t lane = r + 16u * (kk >> 5);
    const uint32_t half = (kk >> 4) & 1u;
    return half * 1024u + lane * 16u + (kk & 15u);
}

__host__ __device__ __forceinline__ uint64_t fc13_block(uint64_t pair, uint64_t kstep,
                                                       uint64_t u, uint64_t ksteps) {
    return ((pair * ksteps + kstep) * 2u + u) * kBlockBytes;
}

__host__ __device__ __forceinline__ uint64_t fc2_block(uint64_t ctile, uint64_t kstep,
                                                      uint64_t sub, uint64_t ksteps) {
    return ((ctile * ksteps + kstep) * kFc2Sub + sub) * kBlockBytes;
}

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v8i make_operand(uint4 lo, uint4 hi) {
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

// acc += A(16x128 e4m3) * B(128x16 e4m3).  Format selectors 0/0 = e4m3/e4m3; the
// zero scale operands select the unscaled form of the instruction.
__device__ __forceinline__ v4f mfma_e4m3(v8i a, v8i b, v4f acc) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 0, 0, 0);
}

}  // namespace moe
