// The grouped pass's item order (group_order.hpp) built for the host.
#include <stdint.h>

#include "group_order.hpp"

extern "C" {

// out[it] = the slot-major item at sequence index it, for a pass of `total` items of which
// the first ns (slot-major) belong to the shared expert, G blocks.
void host_group_order(int ns, int total, int G, int32_t* out) {
    const moe::GroupPlan<2> plan(G, 0, total);
    const moe::GroupOrder ord(ns, plan.pool0);
    for (int it = 0; it < total; ++it) out[it] = ord.map(it);
}

// The fixed share (sequence indices below it are dealt round-robin) of the same pass.
int host_group_fixed_share(int total, int G) { return moe::GroupPlan<2>(G, 0, total).pool0; }
}
