// Item order of the grouped pass's persistent GEMM kernels (group.hpp).  No device
// builtins: the host tests build it too.
//
// Items are numbered slot-major: the shared expert's Ns items first (slot 0), then the
// routed slots'.  Blocks take a fixed share of the item sequence and the rest from a
// pool (GroupPlan).  At a few hundred tokens the shared expert's items loop over many
// row tiles of tokens and spend most of their time in the matrix unit, not streaming;
// if they all came first, every block would compute at once while the weight stream
// stood idle.  GroupOrder spreads them evenly over the fixed share, so that at any
// moment a few blocks compute shared tiles while the others stream, and keeps them out
// of the pool, so that none is drawn at the end.
#pragma once

#include <stdint.h>

namespace moe {

constexpr int kGroupRing = 8;  // pool tickets in flight (LDS ring)

// Block b takes items b, b + G, ... for its first nstatic positions, the rest from a pool
// through a work counter (a ticket taken LA positions ahead).  Blocks stream at
// different rates (their share of the bandwidth depends on where they sit), and over a
// pass of a millisecond a fixed share would leave tens of microseconds of tail; the pool
// holds about a quarter of the items.
template <int LA>
struct GroupPlan {
    int G, b, total, nstatic, pool0;
    __host__ __device__ GroupPlan(int G_, int b_, int total_) : G(G_), b(b_), total(total_) {
        nstatic = (3 * total) / (4 * G);
        nstatic = nstatic > LA ? nstatic : LA;
        pool0 = nstatic * G < total ? nstatic * G : total;
    }
    __host__ __device__ int fixed(int pos) const {
        const int it = b + G * pos;
        return pos < nstatic && it < total ? it : -1;
    }
    __host__ __device__ bool pooled(int pos) const { return pos >= nstatic && pool0 < total; }
    __host__ __device__ int from_ticket(uint32_t t) const {
        return t < (uint32_t)(total - pool0) ? pool0 + (int)t : -1;
    }
    __host__ __device__ int at(int pos, const int* ring) const {
        return pooled(pos) ? ring[pos % kGroupRing] : fixed(pos);
    }
};

// Sequence index -> slot-major item index.  The Ns shared items sit at indices
// floor(q F / Ns), q = 0..Ns-1, F = max(the fixed share, Ns); the routed items fill the
// other indices in slot-major order.  A bijection on [0, total); -1 stays -1.
struct GroupOrder {
    int Ns, F;
    __host__ __device__ GroupOrder(int Ns_, int fixed_share) : Ns(Ns_), F(fixed_share > Ns_ ? fixed_share : Ns_) {}
    __host__ __device__ int map(int it) const {
        if (it < 0 || it >= F) return it;  // past F: every shared index lies before
        // the smallest q with q F / Ns >= it; index it is shared iff floor(q F / Ns) == it
        const int q = (int)(((int64_t)it * Ns + F - 1) / F);
        if (q < Ns && (int)((int64_t)q * F / Ns) == it) return q;
        // shared indices below it: the q with q F / Ns < it + 1
        int before = (int)(((int64_t)(it + 1) * Ns + F - 1) / F);
        before = before < Ns ? before : Ns;
        return Ns + (it - before);
    }
};

}  // namespace moe
