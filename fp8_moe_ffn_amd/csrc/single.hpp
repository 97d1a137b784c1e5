// The forward as one launch: FC13 + SwiGLU, then re-quantisation + FC2, then the combine,
// as three phases of one grid.  It stands in for programmatic dependent launch (Blackwell
// 1,000 TPS/user blog, zh translation, section "Programmatic dependent launch"), which
// lets a kernel's preamble run while the previous kernel's tail finishes; HIP has no such
// launch attribute.
//
// Blocks [0, G13) run the FC13 body, blocks [G13, G13 + G2) the FC2 body and the rest the
// combine, each with its phase-local block index.  One block fills a CU, so the FC2
// blocks are placed as FC13 blocks finish: each requests its first item's weights (the
// shared expert's W2, which needs no routing) while FC13's tail still runs, then waits
// for the FC13 count before it loads FC13's results.  The combine blocks wait for the FC2
// count (the counters only grow; params.hpp says how a wait finds its target).  What a
// phase hands on (the intermediate, row maxima, routing table and gates;
// the partial sums) is stored at device scope, so that a block counts itself once its
// stores are complete (block_arrive); a waiting block's thread 0 fences (acquire) before
// the block reads them, and the waits are bounded (block_wait).  The arithmetic is the
// three kernels', so the results are identical to theirs bit for bit.
#pragma once

#include "fc13.hpp"
#include "fc2.hpp"
#include "params.hpp"

namespace moe {

static_assert(kFc13Threads == kFc2Threads, "the phases share the block size");

// grids = G13 | G2 << 16; the combine takes the blocks past G13 + G2 (a fixed number per
// handle, those past the launch's tokens idle), so that every phase adds the same count
// to its counter in every launch.
template <int NSTEP, bool FULL, int ROWS>
__global__ __launch_bounds__(kFc13Threads) void single_kernel(const FwdParams p, uint32_t grids) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int g13 = (int)(grids & 0xFFFFu), g2 = (int)(grids >> 16);
    const uint32_t gc = gridDim.x - (uint32_t)(g13 + g2);
    const int b = blockIdx.x;
    uint32_t* sync = p.ws.work;
    const uint32_t ki = (uint32_t)p.K | ((uint32_t)p.I << 16);
    // launches completed before this one (advanced only after every block of the previous
    // launch has passed its waits, and read before this block arrives anywhere)
    const uint32_t ep = b < g13 ? 0u : __hip_atomic_load(sync + kSyncEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (b < g13) {
        const uint32_t mts = (uint32_t)p.M | ((uint32_t)p.T << 8) | ((uint32_t)p.S << 16);
        const uint32_t eg = (uint32_t)p.E | ((uint32_t)g13 << 16);
        fc13_body<NSTEP, FULL, false, true>(b, p.x, p.tok, p.logits, p.w13p + (uint64_t)p.E * p.w13_bytes, p.norm_w, mts,
                                      ki, eg, p, lds);
        block_arrive(sync + kSyncFc13);
    } else if (b < g13 + g2) {
        const uint32_t mts = (uint32_t)p.M | ((uint32_t)p.T << 8) | ((uint32_t)p.S << 16) | ((uint32_t)p.nsplit << 24);
        fc2_body<ROWS, true>(b - g13, p.ws.route, p.ws.amax, p.ws.a, p.s2 + (size_t)p.E * p.K,
                             p.w2p + (uint64_t)p.E * p.w2_bytes, mts, ki, grids, p, lds, sync + kSyncFc13,
                             sync + kSyncTimeouts, (ep + 1u) * (uint32_t)g13);
        block_arrive(sync + kSyncFc2);
    } else {
        block_wait(sync + kSyncFc2, (ep + 1u) * (uint32_t)g2, sync + kSyncTimeouts);
        const uint32_t mtn = (uint32_t)p.M | ((uint32_t)p.T << 8) | ((uint32_t)p.nsplit << 16) |
                             ((uint32_t)(p.E > 0) << 24) | ((uint32_t)(p.gate_input != 0) << 25);
        combine_at((b - g13 - g2) * kFc13Threads + (int)threadIdx.x, p.ws.route, p.ws.gate, p.ws.part, p.out, mtn, p.S,
                   p.K);
        // the last combine block of the launch: every block of every phase is past its
        // wait (and has read the epoch), so the launch is counted complete
        const uint32_t before = block_arrive(sync + kSyncCombine);
        if (threadIdx.x == 0 && before == (ep + 1u) * gc - 1u)
            __hip_atomic_store(sync + kSyncEpoch, ep + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace moe
