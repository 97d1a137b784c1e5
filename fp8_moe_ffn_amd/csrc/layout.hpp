// Packed weight layout read by the FC13 and FC2 kernels, and the gfx950 matrix
// instruction they use.
//
// Matrix instruction: v_mfma_f32_16x16x32_f16.  The e4m3 codes travel from HBM as
// bytes and are widened in registers with v_cvt_scalef32_pk_f16_fp8 (scale 1): every
// finite e4m3 value is exactly representable in f16, and the f16 instruction's
// float32 accumulation matches sequential float32 sums.  The e4m3-input matrix
// instructions were measured to carry about 1.3e-5 relative error even for a single
// 128-deep instruction, enough to flip far more than 0.1% of the re-quantised
// intermediate codes, so they are not used.
//
// One 128-deep k-step of one 16-row tile: A is 16 x 128 (output channel x
// reduction), B is 128 x 16 (reduction x token), C is 16 x 16 float32.  Lane l holds
// 32 codes of A and 32 of B:
//     lane l: row/column (l & 15), reduction offsets 32*(l >> 4) + [0, 32)
// Codes [8j, 8j+8) of the lane feed instruction j (j = 0..3); the mapping of
// reduction offsets to lanes only has to be the same for A and B, which it is since
// both are packed with the function below.  C: lane l holds C[4*(l >> 4) + r][l & 15],
// r = 0..3.
//
// One "operand block" = A of one k-step = 16 output channels x 128 reduction indices
// = 2048 bytes, stored as [half h][lane l][16 bytes]: byte j of (h, l) is reduction
// offset 32*(l >> 4) + 16*h + j of channel (l & 15).  A wave reads a block with two
// fully coalesced 1 KiB loads (16 bytes per lane).
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

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

#ifndef MOE_FFN_FP8_MMA_E4M3
// One lane's 32 codes of a k-step, widened to f16: q[j] feeds instruction j.
struct Operand {
    v8h q[4];
};

__device__ __forceinline__ v8h widen8(uint32_t w0, uint32_t w1) {
    union {
        v8h v;
        v2h p[4];
    } u;
    u.p[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
    u.p[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
    u.p[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
    u.p[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
    return u.v;
}

__device__ __forceinline__ Operand widen(uint4 lo, uint4 hi) {
    Operand o;
    o.q[0] = widen8(lo.x, lo.y);
    o.q[1] = widen8(lo.z, lo.w);
    o.q[2] = widen8(hi.x, hi.y);
    o.q[3] = widen8(hi.z, hi.w);
    return o;
}

__device__ __forceinline__ Operand zero_operand() {
    Operand o;
    const v8h z = {0, 0, 0, 0, 0, 0, 0, 0};
    o.q[0] = z; o.q[1] = z; o.q[2] = z; o.q[3] = z;
    return o;
}

// An operand block staged in LDS once for all waves of a block.  The 16 codes of
// half h, lane l of the block are stored at 2048 h + 16 l (4096 bytes a block): widened,
// as instruction 2h's and 2h + 1's 8 halves, the second 1024 bytes on.  A lane reads its
// operand as 4 x 16 bytes at 16 l + 1024 j.
__device__ __forceinline__ void stage_store(uint8_t* d, uint4 c) {
    *reinterpret_cast<v8h*>(d) = widen8(c.x, c.y);
    *reinterpret_cast<v8h*>(d + 1024) = widen8(c.z, c.w);
}
__device__ __forceinline__ Operand stage_operand(const uint8_t* s) {
    Operand o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o.q[j] = *reinterpret_cast<const v8h*>(s + j * 1024);
    return o;
}
#else
// A build with the e4m3-input instruction (v_mfma_f32_16x16x128_f8f6f4 on the raw codes, one
// per k-step), kept to measure the choice above: it misses the parity bar of the re-quantised
// codes at every size (0.14-0.24% of them one step off, 0.1% allowed) and is no faster.
struct Operand {
    uint4 lo, hi;
};
__device__ __forceinline__ Operand widen(uint4 lo, uint4 hi) { return Operand{lo, hi}; }
typedef int v8i __attribute__((ext_vector_type(8)));
// the staged block holds the codes: half h at 2048 h + 16 l
__device__ __forceinline__ void stage_store(uint8_t* d, uint4 c) { *reinterpret_cast<uint4*>(d) = c; }
__device__ __forceinline__ Operand stage_operand(const uint8_t* s) {
    return Operand{*reinterpret_cast<const uint4*>(s), *reinterpret_cast<const uint4*>(s + 2048)};
}
#endif

// Raw buffer loads.  A buffer resource covers [base, base + bytes); a load at an
// offset past the end returns zeros without touching memory.  The streaming kernels
// use a resource with 0 bytes when there is nothing left to prefetch, so that every
// pass of their loops issues the same loads and the memory counters stay in step.
typedef __amdgpu_buffer_rsrc_t BufRes;

__device__ __forceinline__ BufRes make_res(const void* base, uint32_t bytes) {
    // the resource lives in scalar registers: make the wave-uniform inputs provably so.
    // readfirstlane returns a signed int: widen through uint32_t, or an address with
    // bit 31 set would sign-extend into the high word.
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    // last word: raw (unformatted) 32-bit data, as gfx9-family buffer loads expect
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(hi << 32 | lo), (short)0,
                                             (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

__device__ __forceinline__ uint4 buf_ld16(BufRes r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// The same at a per-lane offset plus a wave-uniform one (held in a scalar register).
__device__ __forceinline__ uint4 buf_ld16(BufRes r, uint32_t off, uint32_t uniform) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, (int)uniform, 0));
}

// The weight stream: 16 bytes with the non-temporal cache policy.  Every weight byte is
// read once per step, so keeping it in the caches buys nothing; measured on MI355X, a
// streaming read of 4 GiB in the GEMMs' pattern reaches 7.07-7.13 TB/s with the policy
// and 6.31-6.37 TB/s without it.
constexpr int kStreamPolicy = 2;  // nt
__device__ __forceinline__ uint4 buf_ld16_stream(BufRes r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStreamPolicy));
}
__device__ __forceinline__ uint4 buf_ld16_stream(BufRes r, uint32_t off, uint32_t uniform) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, (int)uniform, kStreamPolicy));
}

__device__ __forceinline__ float4 buf_ldf4(BufRes r, uint32_t off) {
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// 16 bytes per lane from a buffer straight into LDS, without registers.  Lane l writes
// dst + 16 l, dst being the address the wave's first active lane passes, so lanes pass
// consecutive 16-byte slots.  A buffer load is not a flat access: the compiler's wait
// analysis keeps counting the loads issued around it exactly.
__device__ __forceinline__ void buf_ld16_lds(BufRes r, uint8_t* dst, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_u8*)dst, 16, off, 0, 0, 0);
}
// The same at a per-lane offset plus a wave-uniform one, with the weight stream's policy.
__device__ __forceinline__ void buf_ld16_lds(BufRes r, uint8_t* dst, uint32_t off, uint32_t uniform) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_u8*)dst, 16, off, (int)uniform, 0, kStreamPolicy);
}

#ifndef MOE_FFN_FP8_MMA_E4M3
// acc += A(16x128) * B(128x16) for one k-step.
__device__ __forceinline__ v4f mma_kstep(const Operand& a, const Operand& b, v4f acc) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.q[j], b.q[j], acc, 0, 0, 0);
    return acc;
}
#else
__device__ __forceinline__ v4f mma_kstep(const Operand& a, const Operand& b, v4f acc) {
    const v8i av = {(int)a.lo.x, (int)a.lo.y, (int)a.lo.z, (int)a.lo.w, (int)a.hi.x, (int)a.hi.y, (int)a.hi.z, (int)a.hi.w};
    const v8i bv = {(int)b.lo.x, (int)b.lo.y, (int)b.lo.z, (int)b.lo.w, (int)b.hi.x, (int)b.hi.y, (int)b.hi.z, (int)b.hi.w};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, 0, 0, 0);  // unscaled form
}
#endif

// Block barrier that orders LDS only: waits for this wave's LDS operations, then
// s_barrier.  Outstanding global loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace moe
