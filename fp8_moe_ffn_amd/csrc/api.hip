// C ABI of the FP8 MoE feed-forward step: handle lifecycle, argument checks and
// kernel launches.  The operation and every entry point are specified in
// include/moe_ffn_fp8.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <mutex>
#include <new>
#include <vector>

#include "moe_ffn_fp8.h"

#include "codec.hpp"
#include "fc13.hpp"
#include "fc2.hpp"
#include "group.hpp"
#include "single.hpp"
#include "wide.hpp"
#include "layout.hpp"
#include "order.hpp"
#include "params.hpp"
#include "prepack.hpp"
#include "probe.hpp"
#include "prologue.hpp"

#define MOE_API extern "C" __attribute__((visibility("default")))

// Scratch of the allocation-free forward (moe_ffn_fp8_forward_scratch): its workspace in
// one file-scope array, which every device the library runs on holds (zero when the
// library loads) until the process ends, shared by every such call on that device.  In
// host code `scratch` only names the array; its device address is taken per device with
// hipGetSymbolAddress (scratch_address) and only that address is ever passed on.
constexpr size_t kScratchBytes = MOE_FFN_FP8_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

// Clears n words (the allocation-free forward's work counters, before its FC13 kernel: a
// kernel rather than a memset node, so that the clear can be captured into a HIP graph).
__global__ __launch_bounds__(64) void clear_words_kernel(uint32_t* w, int n) {
    for (int i = threadIdx.x; i < n; i += 64) w[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
bool g_scratch_done[kMaxDevices] = {};

// Device address of device `dev`'s copy of `scratch`, or null if HIP could not give it.
// Called with `dev` current (moe_ffn_fp8_create), once per device.
void* scratch_address(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_done[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();
            ptr = nullptr;
        }
        g_scratch_ptr[dev] = ptr;
        g_scratch_done[dev] = true;
    }
    return g_scratch_ptr[dev];
}

// The decode launch's workspace carved out of a scratch area at `base` (T tokens per
// launch, S slots, G13 FC13 blocks); returns the bytes it needs (256-byte aligned parts).
size_t carve_workspace(uint8_t* base, int T, int S, int G13, int K, int I, int nsplit, moe::Workspace* ws) {
    size_t off = 0;
    auto take = [&](size_t bytes) {
        uint8_t* p = base ? base + off : nullptr;
        off += (bytes + 255) & ~size_t(255);
        return p;
    };
    moe::Workspace w{};
    w.route = reinterpret_cast<int32_t*>(take((size_t)moe::RouteLayout{T, S}.count() * 4));
    w.gate = reinterpret_cast<float*>(take((size_t)T * 4));
    w.amax = reinterpret_cast<uint32_t*>(take((size_t)G13 * 2 * T * 4));
    w.a = reinterpret_cast<float*>(take((size_t)2 * T * I * 4));
    w.part = reinterpret_cast<float*>(take((size_t)nsplit * 2 * T * K * 4));
    w.work = reinterpret_cast<uint32_t*>(take((size_t)moe::kWorkWords * 4));
    w.order = nullptr;
    if (ws) *ws = w;
    return off;
}

constexpr int kProfSlots = 1024;
constexpr int kChunk = MOE_FFN_FP8_CHUNK;  // tokens per kernel launch (one B-operand tile)
static_assert(kChunk == moe::kTile, "a chunk is one 16-column operand tile");
constexpr int kMaxBatch = 1 << 16;
constexpr int kMaxExperts = moe::kMaxRouteExperts;
constexpr int kMaxHidden = 8192;
constexpr int kMaxInter = 32768;
constexpr int kLdsBytes = 160 * 1024;
static_assert(kMaxHidden < 65536 && kMaxInter < 65536 && kMaxExperts < 65536, "16-bit kernel argument fields");
static_assert(kChunk < 256, "8-bit kernel argument fields (M, T, S = 1 + min(T, E), nsplit <= I / 1024)");

typedef void (*KernelFn)(const uint16_t*, const int32_t*, const uint16_t*, const uint8_t*, const uint16_t*,
                         uint32_t, uint32_t, uint32_t, moe::FwdParams);
typedef void (*Fc2Fn)(const int32_t*, const uint32_t*, const float*, const float*, const uint8_t*, uint32_t,
                      uint32_t, uint32_t, moe::FwdParams);
typedef void (*GroupFn)(moe::GroupParams);
typedef void (*Wide13Fn)(const uint8_t*, const uint8_t*, const float*, const float*, float*, uint32_t*, uint32_t,
                         uint32_t, moe::GroupParams);
typedef void (*Wide2Fn)(const uint8_t*, const uint8_t*, const float*, const float*, float*, uint32_t, uint32_t,
                        uint32_t, moe::GroupParams);
typedef void (*SingleFn)(moe::FwdParams, uint32_t);

// FC13 variant for K/128 k-steps: NSTEP = ceil(k-steps / 8) per wave, FULL when every
// wave owns exactly NSTEP of them.
template <int N, bool RMS>
KernelFn fc13_variant(bool full) {
    return full ? moe::fc13_swiglu_kernel<N, true, RMS> : moe::fc13_swiglu_kernel<N, false, RMS>;
}

// FC13 for hidden 5120 (5 full k-steps per wave) whose prologue holds exactly the early
// chunks of x that a launch of m tokens needs (prologue.hpp: XSplit::per_lane); null
// otherwise (the general kernel then serves).
template <bool RMS>
KernelFn pick_fc13_m(int ksteps, int m) {
    if (ksteps != 5 * moe::kFc13Waves) return nullptr;
    switch (moe::XSplit(m, ksteps * moe::kKStep).per_lane()) {
        case 1:
        case 2: return moe::fc13_swiglu_kernel<5, true, RMS, 2>;
        case 3: return moe::fc13_swiglu_kernel<5, true, RMS, 3>;
        case 4:
        case 5: return moe::fc13_swiglu_kernel<5, true, RMS, 5>;
        default: return nullptr;
    }
}

template <bool RMS>
KernelFn pick_fc13(int ksteps) {
    const int n = (ksteps + moe::kFc13Waves - 1) / moe::kFc13Waves;
    const bool full = ksteps == n * moe::kFc13Waves;
    switch (n) {
        case 1: return fc13_variant<1, RMS>(full);
        case 2: return fc13_variant<2, RMS>(full);
        case 3: return fc13_variant<3, RMS>(full);
        case 4: return fc13_variant<4, RMS>(full);
        case 5: return fc13_variant<5, RMS>(full);
        case 6: return fc13_variant<6, RMS>(full);
        case 7: return fc13_variant<7, RMS>(full);
        case 8: return fc13_variant<8, RMS>(full);
        default: return nullptr;
    }
}

// Grouped FC13 variant for K/128 k-steps (the same split of k-steps over the waves).
template <int N>
GroupFn gfc13_variant(bool full) {
    return full ? moe::gfc13_kernel<N, true> : moe::gfc13_kernel<N, false>;
}

// Only the variants that fit their registers without spilling: every wave owning the
// same k-steps (K a multiple of 1024) up to 5 each (K <= 5120), or up to 3 otherwise.
// Other sizes run larger batches as chunked launches.
GroupFn pick_gfc13(int ksteps) {
    const int n = (ksteps + moe::kFc13Waves - 1) / moe::kFc13Waves;
    const bool full = ksteps == n * moe::kFc13Waves;
    if (n > (full ? 5 : 3)) return nullptr;
    switch (n) {
        case 1: return gfc13_variant<1>(full);
        case 2: return gfc13_variant<2>(full);
        case 3: return gfc13_variant<3>(full);
        case 4: return gfc13_variant<4>(full);
        case 5: return gfc13_variant<5>(full);
        case 6: return gfc13_variant<6>(full);
        case 7: return gfc13_variant<7>(full);
        case 8: return gfc13_variant<8>(full);
        default: return nullptr;
    }
}

// The wide FC13 kernel for K/128 k-steps (K a multiple of 1024 up to 5120), or null.
Wide13Fn pick_gwide13(int ksteps) {
    switch (ksteps) {
        case 8: return moe::gwide13_kernel<8>;
        case 16: return moe::gwide13_kernel<16>;
        case 24: return moe::gwide13_kernel<24>;
        case 32: return moe::gwide13_kernel<32>;
        case 40: return moe::gwide13_kernel<40>;
        default: return nullptr;
    }
}

// The wide FC2 kernel for SUB 16-column sub-tiles per item (wide.hpp), or null.
Wide2Fn pick_gwide2(int sub) {
    switch (sub) {
        case 3: return moe::gwide2_kernel<3>;
        case 4: return moe::gwide2_kernel<4>;
        case 5: return moe::gwide2_kernel<5>;
        default: return nullptr;
    }
}

// Blocks of a persistent streaming kernel: as many as are resident at once, at most
// `units` (its first items are then one per block).
int persistent_grid(const void* fn, int threads, int lds, int units, int cus) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return std::min(std::max(per_cu, 0) * cus, units);
}

}  // namespace

struct moe_ffn_fp8_handle {
    moe_ffn_fp8_dims dims{};
    int device = 0;
    int S = 0;        // expert slots of the workspace
    int nsplit = 0;   // FC2 splits of I
    int grid13 = 0;   // persistent FC13 grid
    int grid2 = 0;    // persistent FC2 grid
    uint64_t w13_bytes = 0, w2_bytes = 0;
    uint8_t* w13p = nullptr;
    uint8_t* w2p = nullptr;
    float* s13 = nullptr;
    float* s2 = nullptr;
    KernelFn fc13 = nullptr;      // variant for this hidden size
    KernelFn fc13_rms = nullptr;  // the same with the fused RMSNorm
    KernelFn fc13_m[2][moe::kTile + 1] = {};  // [RMS][tokens of a launch]: the kernel launched
    Fc2Fn fc2 = nullptr;      // variant for this token count
    int fc2_rows = 0;         // its B rows per slot
    int chunk = 0;            // tokens per launch, min(max_tokens, MOE_FFN_FP8_CHUNK)
    bool rms_ok = false;      // the fused RMSNorm's LDS fits beside the rest
    moe::Workspace ws{};
    // grouped passes (max_tokens above one launch): up to gT tokens per pass
    int gT = 0, gS = 0;
    GroupFn gfc13 = nullptr;
    int ggrid13 = 0, ggrid2 = 0, glds13 = 0, glds2 = 0;
    // the shared expert's GEMMs of a grouped pass of at least moe::kWideMin tokens (wide.hpp)
    Wide13Fn gwide13 = nullptr;
    Wide2Fn gwide2 = nullptr;
    int gwgrid13 = 0, gwgrid2 = 0, gwlds = 0, gwlds2 = 0;
    int32_t* g_route = nullptr;
    float *g_gate = nullptr, *g_sx = nullptr, *g_a = nullptr, *g_sa = nullptr, *g_part = nullptr;
    uint8_t *g_xq = nullptr, *g_aq = nullptr;
    uint8_t *g_xt = nullptr, *g_at = nullptr;  // operand-ordered codes for the wide kernels
    uint32_t *g_amax = nullptr, *g_work = nullptr;
    int batch_mode = MOE_FFN_FP8_BATCH_GROUPED;
    // the forward as one launch (hidden 5120, up to 8 tokens per launch, no fused norm)
    SingleFn single = nullptr;
    int single_lds = 0;
    int launch_mode = MOE_FFN_FP8_LAUNCH_THREE;
    std::vector<void*> allocations;
    int alloc_count = 0, fail_alloc_at = 0;  // the allocation-failure test hook (create)
    uint8_t* scratch = nullptr;  // this device's copy of `scratch` (allocation-free forward), or null
    // profiling
    bool prof_on = false;
    int prof_calls = 0;
    std::vector<hipEvent_t> events;  // kProfSlots x (stages + 1)
};

namespace {

int32_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_FFN_FP8_OK : MOE_FFN_FP8_ERR_HIP; }

// A device (or managed) pointer, aligned, with at least `bytes` bytes left in its
// allocation.  Host pointers and overruns are rejected before any launch.
bool device_range_ok(const void* p, size_t bytes, size_t align) {
    if (p == nullptr) return false;
    if (reinterpret_cast<uintptr_t>(p) % align != 0) return false;
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged) return false;
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    const uintptr_t b = reinterpret_cast<uintptr_t>(base), q = reinterpret_cast<uintptr_t>(p);
    return q >= b && q - b + bytes <= size;
}

bool dims_ok(const moe_ffn_fp8_dims& d) {
    return d.hidden >= 128 && d.hidden <= kMaxHidden && d.hidden % 128 == 0 &&
           d.inter >= 128 && d.inter <= kMaxInter && d.inter % 128 == 0 &&
           d.num_experts >= 0 && d.num_experts <= kMaxExperts && d.max_tokens >= 1 &&
           d.max_tokens <= kMaxBatch;
}

void free_all(moe_ffn_fp8_handle* h) {
    for (void* p : h->allocations) (void)hipFree(p);
    h->allocations.clear();
    for (hipEvent_t e : h->events) (void)hipEventDestroy(e);
    h->events.clear();
}

template <typename T>
bool alloc(moe_ffn_fp8_handle* h, T** out, size_t count) {
    void* p = nullptr;
    if (++h->alloc_count == h->fail_alloc_at) return false;  // as if the device were full
    if (hipMalloc(&p, std::max<size_t>(count * sizeof(T), 256)) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    h->allocations.push_back(p);
    *out = static_cast<T*>(p);
    return true;
}

int grid_for(uint64_t work, int per_block) {
    const uint64_t g = (work + per_block - 1) / per_block;
    return (int)std::min<uint64_t>(std::max<uint64_t>(g, 1), 1u << 20);
}

// A batch above one launch as grouped passes of up to h->gT tokens (group.hpp): each
// active expert is streamed once per pass.  The pass's tokens are consecutive rows.
int32_t launch_grouped(const uint16_t* x, const uint16_t* logits, moe_ffn_fp8_handle* h, uint16_t* out,
                       int32_t M, hipStream_t stream, const moe::Debug& dd) {
    const moe_ffn_fp8_dims& d = h->dims;
    const size_t K = d.hidden, I = d.inter;
    moe::GroupParams g{};
    g.w13p = h->w13p;
    g.w2p = h->w2p;
    g.s13 = h->s13;
    g.s2 = h->s2;
    g.w13_bytes = h->w13_bytes;
    g.w2_bytes = h->w2_bytes;
    g.K = d.hidden;
    g.I = d.inter;
    g.E = d.num_experts;
    g.S = h->gS;
    g.T = h->gT;
    g.nsplit = h->nsplit;
    g.route = h->g_route;
    g.gate = h->g_gate;
    g.sx = h->g_sx;
    g.xq = h->g_xq;
    g.amax = h->g_amax;
    g.a = h->g_a;
    g.aq = h->g_aq;
    g.sa = h->g_sa;
    g.part = h->g_part;
    g.work = h->g_work;
    const int npairs = (int)I / moe::kTile, per_slot = (int)(K / moe::kFc2Cols) * h->nsplit;
    hipError_t e = hipSuccess;
    // per-kernel events of a single-pass forward: FC13 + SwiGLU; re-quantisation + FC2; combine
    hipEvent_t* ev = nullptr;
    if (h->prof_on && h->prof_calls < kProfSlots && M <= h->gT)
        ev = &h->events[(size_t)h->prof_calls++ * (MOE_FFN_FP8_NUM_STAGES + 1)];
    auto mark = [&](int i) { return ev ? hipEventRecord(ev[i], stream) : hipSuccess; };
    for (int m0 = 0; m0 < M && e == hipSuccess; m0 += h->gT) {
        const int mc = std::min(h->gT, M - m0);
        g.M = mc;
        g.first = m0 == 0;
        g.x = x + (size_t)m0 * K;
        g.logits = logits ? logits + (size_t)m0 * d.num_experts : nullptr;
        g.out = out + (size_t)m0 * K;
        auto at = [&](auto* ptr, size_t per_token) { return ptr ? ptr + (size_t)m0 * per_token : ptr; };
        g.dbg = moe::Debug{at(dd.xq, K), at(dd.sx, 1), at(dd.expert, 1), at(dd.gate, 1), at(dd.aq_shared, I),
                           at(dd.sa_shared, 1), at(dd.aq_routed, I), at(dd.sa_routed, 1), dd.num_active};
        // a pass of many tokens gives the shared expert's GEMMs to the wide kernels; the
        // grouped ones then take the routed slots' items only (none without routed experts)
        const bool wide = h->gwide13 != nullptr && mc >= moe::kWideMin;
        const bool grouped = !wide || d.num_experts > 0;
        g.item0_13 = wide ? npairs : 0;
        g.item0_2 = wide ? per_slot : 0;
        g.xt = wide ? h->g_xt : nullptr;
        g.at = wide ? h->g_at : nullptr;
        void* args[] = {&g};
        const int rows = d.num_experts > 0 ? 2 * mc : mc;
        // the leading arguments of each kernel (preloaded into SGPRs; group.hpp)
        const uint32_t me = (uint32_t)mc | ((uint32_t)d.num_experts << 16), kk = (uint32_t)K;
        const uint32_t mk = (uint32_t)mc | ((uint32_t)K << 16);
        const uint32_t ig = (uint32_t)I | ((uint32_t)h->gwgrid13 << 16), tg = (uint32_t)h->gT | ((uint32_t)h->gwgrid2 << 16);
        const uint32_t mi = (uint32_t)mc | ((uint32_t)I << 16), in = (uint32_t)I | ((uint32_t)h->nsplit << 16);
        const uint32_t tn = (uint32_t)h->gT | ((uint32_t)h->nsplit << 16) | ((uint32_t)(d.num_experts > 0) << 31);
        const uint8_t* w13e = h->w13p + (uint64_t)d.num_experts * h->w13_bytes;
        const uint8_t* w2e = h->w2p + (uint64_t)d.num_experts * h->w2_bytes;
        const float* s13e = h->s13 + (size_t)d.num_experts * 2 * I;
        const float* s2e = h->s2 + (size_t)d.num_experts * K;
        void* prep_args[] = {&g.x, &g.logits, &g.xq, &g.xt, (void*)&me, (void*)&kk, &g};
        void* w13_args[] = {(void*)&w13e, &g.xt, &g.sx, (void*)&s13e, &g.a, &g.amax, (void*)&mk, (void*)&ig, &g};
        void* rq_args[] = {&g.a, &g.amax, &g.aq, &g.at, (void*)&mi, &g};
        void* w2_args[] = {(void*)&w2e, &g.at, &g.sa, (void*)&s2e, &g.part, (void*)&mk, (void*)&in, (void*)&tg, &g};
        void* comb_args[] = {&g.part, &g.out, &g.gate, (void*)&mk, (void*)&tn, &g};
        e = hipLaunchKernel((const void*)moe::gprep_kernel, dim3(mc), dim3(moe::kGroupPrepThreads), prep_args, 0,
                            stream);
        if (e == hipSuccess && grouped)  // the slot table (the wide kernels alone need none)
            e = hipLaunchKernel((const void*)moe::gorder_kernel, dim3(1), dim3(moe::kGroupOrderThreads), args,
                                moe::gorder_lds_bytes(mc, d.num_experts), stream);
        if (e == hipSuccess) e = mark(0);
        if (e == hipSuccess && wide)
            e = hipLaunchKernel((const void*)h->gwide13, dim3(h->gwgrid13), dim3(moe::kFc13Threads), w13_args,
                                h->gwlds, stream);
        if (e == hipSuccess && grouped)
            e = hipLaunchKernel((const void*)h->gfc13, dim3(h->ggrid13), dim3(moe::kFc13Threads), args, h->glds13,
                                stream);
        if (e == hipSuccess) e = mark(1);
        if (e == hipSuccess)
            e = hipLaunchKernel((const void*)moe::grequant_kernel, dim3(rows), dim3(moe::kGroupRequantThreads),
                                rq_args, 0, stream);
        if (e == hipSuccess && wide)
            e = hipLaunchKernel((const void*)h->gwide2, dim3(h->gwgrid2), dim3(moe::kFc2Threads), w2_args,
                                h->gwlds2, stream);
        if (e == hipSuccess && grouped)
            e = hipLaunchKernel((const void*)moe::gfc2_kernel, dim3(h->ggrid2), dim3(moe::kFc2Threads), args, h->glds2,
                                stream);
        if (e == hipSuccess) e = mark(2);
        if (e == hipSuccess)
            e = hipLaunchKernel((const void*)moe::gcombine_kernel, dim3(grid_for((size_t)mc * K / 4, 256)), dim3(256),
                                comb_args, 0, stream);
        if (e == hipSuccess) e = mark(3);
    }
    return hip_status(e);
}

// scratch_ws: the workspace of the allocation-free forward (one launch of the three decode
// kernels, after a clear of its work counters), instead of the handle's.
int32_t launch_forward(const uint16_t* x, const uint16_t* logits, moe_ffn_fp8_handle* h,
                       uint16_t* out, int32_t M, void* stream_ptr, const moe_ffn_fp8_debug* dbg,
                       const moe_ffn_fp8_variant* var = nullptr, const uint16_t* norm_w = nullptr,
                       float norm_eps = 0.0f, const moe::Workspace* scratch_ws = nullptr) {
    if (h == nullptr) return MOE_FFN_FP8_ERR_INVALID_ARG;
    const bool rms = norm_w != nullptr;
    if (rms) {
        if (!std::isfinite(norm_eps) || norm_eps < 0.0f) return MOE_FFN_FP8_ERR_INVALID_ARG;
        if (!device_range_ok(norm_w, (size_t)h->dims.hidden * 2, 16)) return MOE_FFN_FP8_ERR_INVALID_ARG;
        if (!h->rms_ok) return MOE_FFN_FP8_ERR_UNSUPPORTED;
    }
    moe_ffn_fp8_variant v{0, 0.0f, 0.0f};
    if (var) {
        v = *var;
        if ((v.gate_on_input != 0 && v.gate_on_input != 1) || !std::isfinite(v.x_scale) || v.x_scale < 0.0f ||
            !std::isfinite(v.a_scale) || v.a_scale < 0.0f)
            return MOE_FFN_FP8_ERR_INVALID_ARG;
    }
    const moe_ffn_fp8_dims& d = h->dims;
    if (M < 0 || M > d.max_tokens) return MOE_FFN_FP8_ERR_INVALID_ARG;
    if ((d.num_experts == 0) != (logits == nullptr)) return MOE_FFN_FP8_ERR_INVALID_ARG;
    if (M == 0) return MOE_FFN_FP8_OK;
    const size_t mk = (size_t)M * d.hidden, mi = (size_t)M * d.inter;
    if (!device_range_ok(x, mk * 2, 2) || !device_range_ok(out, mk * 2, 2)) return MOE_FFN_FP8_ERR_INVALID_ARG;
    if (logits && !device_range_ok(logits, (size_t)M * d.num_experts * 2, 2)) return MOE_FFN_FP8_ERR_INVALID_ARG;
    {  // the output may not overlap the inputs
        const uintptr_t o0 = reinterpret_cast<uintptr_t>(out), o1 = o0 + mk * 2;
        const uintptr_t x0 = reinterpret_cast<uintptr_t>(x), x1 = x0 + mk * 2;
        if (o0 < x1 && x0 < o1) return MOE_FFN_FP8_ERR_INVALID_ARG;
        if (logits) {
            const uintptr_t l0 = reinterpret_cast<uintptr_t>(logits), l1 = l0 + (size_t)M * d.num_experts * 2;
            if (o0 < l1 && l0 < o1) return MOE_FFN_FP8_ERR_INVALID_ARG;
        }
    }
    moe::Debug dd{};
    if (dbg) {
        dd = moe::Debug{dbg->xq, dbg->s_x, dbg->expert, dbg->gate, dbg->aq_shared,
                        dbg->s_a_shared, dbg->aq_routed, dbg->s_a_routed, dbg->num_active};
        if ((dd.xq && !device_range_ok(dd.xq, mk, 4)) ||
            (dd.sx && !device_range_ok(dd.sx, M * 4, 4)) ||
            (dd.expert && !device_range_ok(dd.expert, M * 4, 4)) ||
            (dd.gate && !device_range_ok(dd.gate, M * 4, 4)) ||
            (dd.aq_shared && !device_range_ok(dd.aq_shared, mi, 4)) ||
            (dd.sa_shared && !device_range_ok(dd.sa_shared, M * 4, 4)) ||
            (dd.aq_routed && !device_range_ok(dd.aq_routed, mi, 4)) ||
            (dd.sa_routed && !device_range_ok(dd.sa_routed, M * 4, 4)) ||
            (dd.num_active && !device_range_ok(dd.num_active, 4, 4)) ||
            (dbg->sync_timeouts && !device_range_ok(dbg->sync_timeouts, 4, 4)))
            return MOE_FFN_FP8_ERR_INVALID_ARG;
    }
    if (hipSetDevice(h->device) != hipSuccess) return MOE_FFN_FP8_ERR_HIP;
    if (h->gT > 0 && M > MOE_FFN_FP8_GROUP_FROM && var == nullptr && !rms && scratch_ws == nullptr &&
        h->batch_mode == MOE_FFN_FP8_BATCH_GROUPED) {
        int32_t st = launch_grouped(x, logits, h, out, M, static_cast<hipStream_t>(stream_ptr), dd);
        if (st == MOE_FFN_FP8_OK && dbg && dbg->sync_timeouts)
            st = hip_status(hipMemcpyAsync(dbg->sync_timeouts, h->ws.work + moe::kSyncTimeouts, 4,
                                           hipMemcpyDeviceToDevice, static_cast<hipStream_t>(stream_ptr)));
        return st;
    }

    const int C = h->chunk;  // tokens per launch
    moe::FwdParams p{};
    p.w13p = h->w13p;
    p.w2p = h->w2p;
    p.s13 = h->s13;
    p.s2 = h->s2;
    p.w13_bytes = h->w13_bytes;
    p.w2_bytes = h->w2_bytes;
    p.K = d.hidden;
    p.I = d.inter;
    p.E = d.num_experts;
    p.S = h->S;
    p.T = C;
    p.nsplit = h->nsplit;
    p.grid13 = h->grid13;
    p.ws = scratch_ws ? *scratch_ws : h->ws;
    p.gate_input = v.gate_on_input && d.num_experts > 0;
    p.x_scale = v.x_scale;
    p.a_scale = v.a_scale;
    p.norm_w = norm_w;
    p.norm_eps = norm_eps;

    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    const int lds2 = moe::fc2_lds(C, h->S, h->fc2_rows).total;
    hipEvent_t* ev = nullptr;
    if (h->prof_on && h->prof_calls < kProfSlots && M <= C)
        ev = &h->events[(size_t)h->prof_calls++ * (MOE_FFN_FP8_NUM_STAGES + 1)];
    auto mark = [&](int i) { return ev ? hipEventRecord(ev[i], stream) : hipSuccess; };
    // Every kernel takes, ahead of anything else, the few values its first loads need, as
    // scalar arguments that gfx950 preloads into SGPRs (the build's kernarg preload
    // count): the FwdParams struct behind them is fetched from memory at the kernel's
    // start, about a microsecond.  Small sizes are packed 8 or 16 bits to a word
    // (M, T, S, nsplit <= 255; K, I, E, grids <= 65535 by the limits checked at create).
    const uint32_t ki = (uint32_t)p.K | ((uint32_t)p.I << 16);

    hipError_t e = hipSuccess;
    if (scratch_ws) {  // the shared scratch keeps whatever the last call left in it
        hipLaunchKernelGGL(clear_words_kernel, dim3(1), dim3(64), 0, stream, p.ws.work, (int)moe::kWorkWords);
        e = hipGetLastError();
    }
    // a routed batch above one launch runs in expert order: launches index the batch's
    // rows through that order
    const bool ordered = M > C && d.num_experts > 0;
    if (ordered) {
        void* oargs[] = {&logits, &M, &p.E, &h->ws.order};
        e = hipLaunchKernel((const void*)moe::order_kernel, dim3(1), dim3(moe::kOrderThreads), oargs,
                            moe::order_lds_bytes(M, d.num_experts), stream);
    }
    for (int m0 = 0; m0 < M && e == hipSuccess; m0 += C) {
        const int mc = std::min(C, M - m0);
        const size_t K = d.hidden, I = d.inter;
        p.M = mc;
        p.first_chunk = m0 == 0;
        p.dbg = dd;
        if (ordered) {
            p.tok = h->ws.order + m0;
            p.x = x;
            p.logits = logits;
            p.out = out;
        } else {
            p.tok = nullptr;
            p.x = x + m0 * K;
            p.logits = logits ? logits + (size_t)m0 * d.num_experts : nullptr;
            p.out = out + m0 * K;
        }
        if (dbg && !ordered) {  // the chunk's rows of every debug array
            auto at = [&](auto* ptr, size_t per_token) { return ptr ? ptr + m0 * per_token : ptr; };
            p.dbg.xq = at(dd.xq, K);
            p.dbg.sx = at(dd.sx, 1);
            p.dbg.expert = at(dd.expert, 1);
            p.dbg.gate = at(dd.gate, 1);
            p.dbg.aq_shared = at(dd.aq_shared, I);
            p.dbg.sa_shared = at(dd.sa_shared, 1);
            p.dbg.aq_routed = at(dd.aq_routed, I);
            p.dbg.sa_routed = at(dd.sa_routed, 1);
        }
        const int lds13 = moe::fc13_lds(C, h->S, d.num_experts, mc, d.hidden, rms).total;
        e = mark(0);
        if (h->launch_mode == MOE_FFN_FP8_LAUNCH_SINGLE && !rms && !scratch_ws) {  // one launch, three phases
            const uint32_t grids = (uint32_t)h->grid13 | ((uint32_t)h->grid2 << 16);
            // combine blocks for the handle's largest launch, whatever this one's tokens: every
            // phase counts the same blocks in every launch
            const int ncomb = (int)grid_for((size_t)C * K / 4, moe::kFc13Threads);
            void* as[] = {&p, const_cast<uint32_t*>(&grids)};
            if (e == hipSuccess)
                e = hipLaunchKernel((const void*)h->single, dim3(h->grid13 + h->grid2 + ncomb),
                                    dim3(moe::kFc13Threads), as, h->single_lds, stream);
            for (int i = 1; i < 4 && e == hipSuccess; ++i) e = mark(i);
            continue;
        }
        if (e == hipSuccess) {  // FC13: x, token rows, logits, the shared expert's weights, norm weight
            const uint16_t* lx = p.x;
            const int32_t* ltok = p.tok;
            const uint16_t* llg = p.logits;
            const uint8_t* w13e = p.w13p + (uint64_t)p.E * p.w13_bytes;
            const uint16_t* lnw = p.norm_w;
            uint32_t mts = (uint32_t)p.M | ((uint32_t)p.T << 8) | ((uint32_t)p.S << 16) | ((uint32_t)rms << 24);
            uint32_t k_i = ki;
            uint32_t eg = (uint32_t)p.E | ((uint32_t)h->grid13 << 16);
            void* a13[] = {&lx, &ltok, &llg, &w13e, &lnw, &mts, &k_i, &eg, &p};
            e = hipLaunchKernel((const void*)h->fc13_m[rms ? 1 : 0][mc], dim3(h->grid13), dim3(moe::kFc13Threads),
                                a13, lds13, stream);
        }
        if (e == hipSuccess) e = mark(1);
        if (e == hipSuccess) {  // FC2: routing table, maxima, intermediate, the shared expert's W2 and s2
            const int32_t* route = p.ws.route;
            const uint32_t* amax = p.ws.amax;
            const float* a = p.ws.a;
            const float* s2e = p.s2 + (size_t)p.E * p.K;
            const uint8_t* w2e = p.w2p + (uint64_t)p.E * p.w2_bytes;
            uint32_t mts = (uint32_t)p.M | ((uint32_t)p.T << 8) | ((uint32_t)p.S << 16) | ((uint32_t)p.nsplit << 24);
            uint32_t k_i = ki;
            uint32_t grids = (uint32_t)p.grid13 | ((uint32_t)h->grid2 << 16);
            void* a2[] = {&route, &amax, &a, &s2e, &w2e, &mts, &k_i, &grids, &p};
            e = hipLaunchKernel((const void*)h->fc2, dim3(h->grid2), dim3(moe::kFc2Threads), a2, lds2, stream);
        }
        if (e == hipSuccess) e = mark(2);
        if (e == hipSuccess) {  // combine: scalar arguments only
            const int32_t* route = p.ws.route;
            const float* gate = p.ws.gate;
            const float* part = p.ws.part;
            uint16_t* o = p.out;
            uint32_t mtn = (uint32_t)p.M | ((uint32_t)p.T << 8) | ((uint32_t)p.nsplit << 16) |
                           ((uint32_t)(p.E > 0) << 24) | ((uint32_t)(p.gate_input != 0) << 25);
            int32_t S = p.S, Kc = p.K;
            void* ac[] = {&route, &gate, &part, &o, &mtn, &S, &Kc};
            e = hipLaunchKernel((const void*)moe::combine_kernel, dim3(grid_for((size_t)mc * K / 4, 256)),
                                dim3(256), ac, 0, stream);
        }
        if (e == hipSuccess) e = mark(3);
    }
    if (e == hipSuccess && dbg && dbg->sync_timeouts)  // the count of waits given up
        e = hipMemcpyAsync(dbg->sync_timeouts, p.ws.work + moe::kSyncTimeouts, 4, hipMemcpyDeviceToDevice, stream);
    return hip_status(e);
}

}  // namespace

MOE_API int32_t moe_ffn_fp8_create(const moe_ffn_fp8_dims* dims, moe_ffn_fp8_handle** out) {
    if (dims == nullptr || out == nullptr) return MOE_FFN_FP8_ERR_INVALID_ARG;
    *out = nullptr;
    if (!dims_ok(*dims)) return MOE_FFN_FP8_ERR_INVALID_ARG;
    const int K = dims->hidden, I = dims->inter, E = dims->num_experts;
    const int T = std::min(dims->max_tokens, kChunk);  // tokens per launch: sizes the workspace
    const int S = 1 + std::min(T, E);
    const int npairs = I / moe::kTile;
    const int nsplit = (I / moe::kKStep + moe::kFc2SplitSteps - 1) / moe::kFc2SplitSteps;
    const int ntiles = (K / moe::kFc2Cols) * nsplit;
    KernelFn fc13 = pick_fc13<false>(K / moe::kKStep);
    KernelFn fc13_rms = pick_fc13<true>(K / moe::kKStep);
    const int fc2_rows = T <= 4 ? 4 : T <= 8 ? 8 : 16;  // B rows of one slot (>= T)
    Fc2Fn fc2 = fc2_rows == 4 ? moe::fc2_kernel<4> : fc2_rows == 8 ? moe::fc2_kernel<8> : moe::fc2_kernel<16>;
    const int lds13_plain = moe::fc13_lds(T, S, E, T, K).total;
    const int lds13_rms = moe::fc13_lds(T, S, E, T, K, true).total;
    const bool rms_ok = lds13_rms <= kLdsBytes;
    const int lds13 = lds13_plain;
    const int lds2 = moe::fc2_lds(T, S, fc2_rows).total;
    const bool ordered = dims->max_tokens > T && E > 0;  // batches above one launch are ordered
    const int lds_order = ordered ? moe::order_lds_bytes(dims->max_tokens, E) : 0;
    if (fc13 == nullptr || lds13 > kLdsBytes || lds2 > kLdsBytes || lds_order > kLdsBytes)
        return MOE_FFN_FP8_ERR_UNSUPPORTED;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
        (void)hipGetLastError();
        return MOE_FFN_FP8_ERR_HIP;
    }
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(fc13), hipFuncAttributeMaxDynamicSharedMemorySize,
                            lds13) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(fc2),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds2) != hipSuccess ||
        (ordered && hipFuncSetAttribute(reinterpret_cast<const void*>(moe::order_kernel),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, lds_order) != hipSuccess) ||
        (rms_ok && hipFuncSetAttribute(reinterpret_cast<const void*>(fc13_rms),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds13_rms) != hipSuccess)) {
        (void)hipGetLastError();
        return MOE_FFN_FP8_ERR_UNSUPPORTED;
    }
    // the FC13 kernel of each launch size: the prologue compiled for its early chunks where one
    // is built (hidden 5120), else the general kernel
    KernelFn fc13_m[2][moe::kTile + 1] = {};
    for (int m = 1; m <= T; ++m) {
        KernelFn k0 = pick_fc13_m<false>(K / moe::kKStep, m), k1 = pick_fc13_m<true>(K / moe::kKStep, m);
        if (k0 && hipFuncSetAttribute(reinterpret_cast<const void*>(k0), hipFuncAttributeMaxDynamicSharedMemorySize,
                                      lds13) != hipSuccess)
            k0 = nullptr;
        if (k1 && (!rms_ok || hipFuncSetAttribute(reinterpret_cast<const void*>(k1),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, lds13_rms) != hipSuccess))
            k1 = nullptr;
        (void)hipGetLastError();
        fc13_m[0][m] = k0 ? k0 : fc13;
        fc13_m[1][m] = k1 ? k1 : fc13_rms;
    }
    // the single launch: hidden 5120 (5 full k-steps per wave), up to 8 rows per slot
    SingleFn single = nullptr;
    const int lds_single = std::max(lds13, lds2);
    if (K / moe::kKStep == 5 * moe::kFc13Waves && fc2_rows <= 8) {
        single = fc2_rows == 4 ? moe::single_kernel<5, true, 4> : moe::single_kernel<5, true, 8>;
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(single), hipFuncAttributeMaxDynamicSharedMemorySize,
                                lds_single) != hipSuccess) {
            (void)hipGetLastError();
            single = nullptr;
        }
    }
    // as many blocks as fit (one per CU), at most the items of the largest step (S slots):
    // at small I a block may start on a routed expert's items, after its prologue
    const int grid13 = persistent_grid(reinterpret_cast<const void*>(fc13), moe::kFc13Threads, lds13, S * npairs, cus);
    // FC2: one block per CU; more resident blocks only lengthen the memory queues.  Between one
    // and two items per CU (the shared expert alone at K = 5120: 320 items), half as many blocks
    // take two items each: no block waits at the end for a few others' second item (dense M=1
    // 29.97 -> 29.34 us, M=8 35.84 -> 35.18 us in an A/B on MI355X)
    const int items2 = S * ntiles;
    const int grid2 = std::min(persistent_grid(reinterpret_cast<const void*>(fc2), moe::kFc2Threads, lds2,
                                               items2 > cus && items2 <= 2 * cus ? (items2 + 1) / 2 : items2, cus),
                               cus);
    if (grid13 <= 0 || grid2 <= 0) return MOE_FFN_FP8_ERR_UNSUPPORTED;
    // grouped passes for batches above MOE_FFN_FP8_GROUP_FROM tokens
    GroupFn gfc13 = dims->max_tokens > MOE_FFN_FP8_GROUP_FROM ? pick_gfc13(K / moe::kKStep) : nullptr;
    const int gT = gfc13 ? std::min(dims->max_tokens, moe::kGroupMax) : 0;
    const int gS = 1 + std::min(gT, E);
    int glds13 = 0, glds2 = 0, ggrid13 = 0, ggrid2 = 0;
    if (gT) {
        glds13 = moe::gfc13_lds(gT, gS).total;
        glds2 = moe::gfc2_lds(gT, gS).total;
        if (glds13 > kLdsBytes || glds2 > kLdsBytes || moe::gorder_lds_bytes(gT, E) > kLdsBytes)
            return MOE_FFN_FP8_ERR_UNSUPPORTED;
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(gfc13), hipFuncAttributeMaxDynamicSharedMemorySize,
                                glds13) != hipSuccess ||
            hipFuncSetAttribute(reinterpret_cast<const void*>(moe::gfc2_kernel),
                                hipFuncAttributeMaxDynamicSharedMemorySize, glds2) != hipSuccess) {
            (void)hipGetLastError();
            return MOE_FFN_FP8_ERR_UNSUPPORTED;
        }
        // the first item of every block belongs to the shared expert: grid <= items of one slot
        ggrid13 = persistent_grid(reinterpret_cast<const void*>(gfc13), moe::kFc13Threads, glds13, npairs, cus);
        ggrid2 = std::min(persistent_grid(reinterpret_cast<const void*>(moe::gfc2_kernel), moe::kFc2Threads, glds2,
                                          ntiles, cus), 2 * cus);
        if (ggrid13 <= 0 || ggrid2 <= 0) return MOE_FFN_FP8_ERR_UNSUPPORTED;
    }
    // the wide kernels for the shared expert of passes of many tokens (a pass may hold that many)
    Wide13Fn gwide13 = nullptr;
    Wide2Fn gwide2 = nullptr;
    int gwgrid13 = 0, gwgrid2 = 0, gwlds = 0, gwlds2 = 0;
    if (gT >= moe::kWideMin && moe::wide_shape(K, I)) {
        gwide13 = pick_gwide13(K / moe::kKStep);
        const int sub = moe::wide2_sub(K, nsplit, cus);  // FC2 items in whole rounds of one per CU
        gwide2 = pick_gwide2(sub);
        gwlds = moe::wide_lds(gT, moe::wide13_stage_bytes()).total;
        gwlds2 = moe::wide_lds(gT, moe::wide2_stage_bytes(sub)).total;
        if (gwide13 && gwide2) {  // one block per CU (its registers), at most the items
            gwgrid13 = std::min(persistent_grid(reinterpret_cast<const void*>(gwide13), moe::kFc13Threads, gwlds,
                                                npairs / 2, cus), cus);
            gwgrid2 = std::min(persistent_grid(reinterpret_cast<const void*>(gwide2), moe::kFc2Threads, gwlds2,
                                               (int)(K / moe::kTile) / sub * nsplit, cus), cus);
        }
        if (gwgrid13 <= 0 || gwgrid2 <= 0) {
            gwide13 = nullptr;
            gwide2 = nullptr;
        }
    }

    auto* h = new (std::nothrow) moe_ffn_fp8_handle();
    if (h == nullptr) return MOE_FFN_FP8_ERR_OUT_OF_MEMORY;
    h->dims = *dims;
    h->device = dev;
    h->S = S;
    h->nsplit = nsplit;
    h->grid13 = grid13;
    h->grid2 = grid2;
    h->single = single;
    h->single_lds = lds_single;
    h->fc13 = fc13;
    for (int r = 0; r < 2; ++r)
        for (int m = 0; m <= moe::kTile; ++m) h->fc13_m[r][m] = fc13_m[r][m];
    h->fc2 = fc2;
    h->fc2_rows = fc2_rows;
    h->chunk = T;
    h->rms_ok = rms_ok;
    h->fc13_rms = fc13_rms;
    h->w13_bytes = (uint64_t)K * 2 * I;
    h->w2_bytes = (uint64_t)I * K;
    h->gT = gT;
    h->gS = gS;
    h->gfc13 = gfc13;
    h->glds13 = glds13;
    h->glds2 = glds2;
    h->ggrid13 = ggrid13;
    h->ggrid2 = ggrid2;
    h->gwide13 = gwide13;
    h->gwide2 = gwide2;
    h->gwgrid13 = gwgrid13;
    h->gwgrid2 = gwgrid2;
    h->gwlds = gwlds;
    h->gwlds2 = gwlds2;
    if (const char* f = std::getenv("MOE_FFN_FP8_FAIL_ALLOC")) h->fail_alloc_at = std::atoi(f);
    h->scratch = static_cast<uint8_t*>(scratch_address(dev));  // once per device, dev current
    const size_t n = (size_t)E + 1;
    moe::Workspace& ws = h->ws;
    const bool ok = alloc(h, &h->w13p, n * h->w13_bytes) && alloc(h, &h->w2p, n * h->w2_bytes) &&
                    alloc(h, &h->s13, n * 2 * I) && alloc(h, &h->s2, n * K) &&
                    alloc(h, &ws.route, moe::RouteLayout{T, S}.count()) && alloc(h, &ws.gate, T) &&
                    alloc(h, &ws.amax, (size_t)grid13 * 2 * T) && alloc(h, &ws.a, (size_t)2 * T * I) &&
                    alloc(h, &ws.part, (size_t)nsplit * 2 * T * K) && alloc(h, &ws.work, (size_t)moe::kWorkWords) &&
                    (!ordered || alloc(h, &ws.order, (size_t)dims->max_tokens)) &&
                    (!gT || (alloc(h, &h->g_route, (size_t)moe::GroupRoute{gT, gS}.count()) &&
                             alloc(h, &h->g_gate, gT) && alloc(h, &h->g_sx, gT) &&
                             alloc(h, &h->g_xq, (size_t)gT * K) && alloc(h, &h->g_amax, (size_t)2 * gT) &&
                             alloc(h, &h->g_a, (size_t)2 * gT * I) && alloc(h, &h->g_aq, (size_t)2 * gT * I) &&
                             alloc(h, &h->g_sa, (size_t)2 * gT) && alloc(h, &h->g_part, (size_t)nsplit * 2 * gT * K) &&
                             alloc(h, &h->g_work, 2))) &&
                    (!gwide13 || (alloc(h, &h->g_xt, (size_t)(gT + 15) / 16 * 16 * K) &&
                                  alloc(h, &h->g_at, (size_t)(gT + 15) / 16 * 16 * I)));
    if (!ok) {
        free_all(h);
        delete h;
        return MOE_FFN_FP8_ERR_OUT_OF_MEMORY;
    }
    // rows of the intermediate a forward does not write are read (and discarded) by FC2:
    // start them as zeros; the work counters start at zero
    if (hipMemset(ws.a, 0, (size_t)2 * T * I * 4) != hipSuccess ||
        hipMemset(ws.work, 0, (size_t)moe::kWorkWords * 4) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        (void)hipGetLastError();
        free_all(h);
        delete h;
        return MOE_FFN_FP8_ERR_HIP;
    }
    *out = h;
    return MOE_FFN_FP8_OK;
}

MOE_API int32_t moe_ffn_fp8_prepack_expert(moe_ffn_fp8_handle* h, int32_t slot, const uint8_t* w13,
                                           const float* s13, const uint8_t* w2, const float* s2,
                                           void* stream_ptr) {
    if (h == nullptr || slot < 0 || slot > h->dims.num_experts) return MOE_FFN_FP8_ERR_INVALID_ARG;
    const int K = h->dims.hidden, I = h->dims.inter;
    if (!device_range_ok(w13, h->w13_bytes, 1) || !device_range_ok(w2, h->w2_bytes, 1) ||
        !device_range_ok(s13, (size_t)2 * I * 4, 4) || !device_range_ok(s2, (size_t)K * 4, 4))
        return MOE_FFN_FP8_ERR_INVALID_ARG;
    if (hipSetDevice(h->device) != hipSuccess) return MOE_FFN_FP8_ERR_HIP;
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    uint8_t* d13 = h->w13p + (uint64_t)slot * h->w13_bytes;
    uint8_t* d2 = h->w2p + (uint64_t)slot * h->w2_bytes;
    hipLaunchKernelGGL(moe::pack_kernel<true>, dim3(grid_for(h->w13_bytes / 16, 256)), dim3(256), 0,
                       stream, w13, d13, K, I);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) {
        hipLaunchKernelGGL(moe::pack_kernel<false>, dim3(grid_for(h->w2_bytes / 16, 256)), dim3(256), 0,
                           stream, w2, d2, K, I);
        e = hipGetLastError();
    }
    if (e == hipSuccess)
        e = hipMemcpyAsync(h->s13 + (size_t)slot * 2 * I, s13, (size_t)2 * I * 4, hipMemcpyDeviceToDevice, stream);
    if (e == hipSuccess)
        e = hipMemcpyAsync(h->s2 + (size_t)slot * K, s2, (size_t)K * 4, hipMemcpyDeviceToDevice, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    return hip_status(e);
}

MOE_API int32_t moe_ffn_fp8_prepack(const moe_ffn_fp8_dims* dims, const uint8_t* w13, const uint8_t* w2,
                                    const float* s13, const float* s2, void* stream,
                                    moe_ffn_fp8_handle** out) {
    if (out == nullptr) return MOE_FFN_FP8_ERR_INVALID_ARG;
    *out = nullptr;
    moe_ffn_fp8_handle* h = nullptr;
    int32_t st = moe_ffn_fp8_create(dims, &h);
    if (st != MOE_FFN_FP8_OK) return st;
    const int K = dims->hidden, I = dims->inter;
    for (int slot = 0; slot <= dims->num_experts && st == MOE_FFN_FP8_OK; ++slot) {
        st = moe_ffn_fp8_prepack_expert(h, slot, w13 ? w13 + (uint64_t)slot * h->w13_bytes : nullptr,
                                        s13 ? s13 + (size_t)slot * 2 * I : nullptr,
                                        w2 ? w2 + (uint64_t)slot * h->w2_bytes : nullptr,
                                        s2 ? s2 + (size_t)slot * K : nullptr, stream);
    }
    if (st != MOE_FFN_FP8_OK) {
        moe_ffn_fp8_destroy(h);
        return st;
    }
    *out = h;
    return MOE_FFN_FP8_OK;
}

MOE_API int32_t moe_ffn_fp8_unpack_expert(const moe_ffn_fp8_handle* h, int32_t slot, uint8_t* w13,
                                          float* s13, uint8_t* w2, float* s2, void* stream_ptr) {
    if (h == nullptr || slot < 0 || slot > h->dims.num_experts) return MOE_FFN_FP8_ERR_INVALID_ARG;
    const int K = h->dims.hidden, I = h->dims.inter;
    if (!device_range_ok(w13, h->w13_bytes, 1) || !device_range_ok(w2, h->w2_bytes, 1) ||
        !device_range_ok(s13, (size_t)2 * I * 4, 4) || !device_range_ok(s2, (size_t)K * 4, 4))
        return MOE_FFN_FP8_ERR_INVALID_ARG;
    if (hipSetDevice(h->device) != hipSuccess) return MOE_FFN_FP8_ERR_HIP;
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    hipLaunchKernelGGL(moe::unpack_kernel<true>, dim3(grid_for(h->w13_bytes / 16, 256)), dim3(256), 0,
                       stream, h->w13p + (uint64_t)slot * h->w13_bytes, w13, K, I);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) {
        hipLaunchKernelGGL(moe::unpack_kernel<false>, dim3(grid_for(h->w2_bytes / 16, 256)), dim3(256), 0,
                           stream, h->w2p + (uint64_t)slot * h->w2_bytes, w2, K, I);
        e = hipGetLastError();
    }
    if (e == hipSuccess)
        e = hipMemcpyAsync(s13, h->s13 + (size_t)slot * 2 * I, (size_t)2 * I * 4, hipMemcpyDeviceToDevice, stream);
    if (e == hipSuccess)
        e = hipMemcpyAsync(s2, h->s2 + (size_t)slot * K, (size_t)K * 4, hipMemcpyDeviceToDevice, stream);
    return hip_status(e);
}

MOE_API int32_t moe_ffn_fp8_forward(const uint16_t* x_bf16, const uint16_t* router_logits_bf16,
                                    moe_ffn_fp8_handle* h, uint16_t* out_bf16, int32_t M, void* stream) {
    return launch_forward(x_bf16, router_logits_bf16, h, out_bf16, M, stream, nullptr);
}

MOE_API int32_t moe_ffn_fp8_forward_scratch(const uint16_t* x_bf16, const uint16_t* router_logits_bf16,
                                            moe_ffn_fp8_handle* h, uint16_t* out_bf16, int32_t M, void* stream) {
    if (h == nullptr || M < 0 || M > h->dims.max_tokens) return MOE_FFN_FP8_ERR_INVALID_ARG;
    if (M > h->chunk) return MOE_FFN_FP8_ERR_UNSUPPORTED;  // one launch of the decode kernels
    const moe_ffn_fp8_dims& d = h->dims;
    if (carve_workspace(nullptr, h->chunk, h->S, h->grid13, d.hidden, d.inter, h->nsplit, nullptr) > kScratchBytes)
        return MOE_FFN_FP8_ERR_UNSUPPORTED;
    if (h->scratch == nullptr) return MOE_FFN_FP8_ERR_HIP;
    moe::Workspace ws{};
    carve_workspace(h->scratch, h->chunk, h->S, h->grid13, d.hidden, d.inter, h->nsplit, &ws);
    return launch_forward(x_bf16, router_logits_bf16, h, out_bf16, M, stream, nullptr, nullptr, nullptr, 0.0f, &ws);
}

MOE_API int32_t moe_ffn_fp8_forward_debug(const uint16_t* x_bf16, const uint16_t* router_logits_bf16,
                                          moe_ffn_fp8_handle* h, uint16_t* out_bf16, int32_t M,
                                          void* stream, const moe_ffn_fp8_debug* dbg) {
    if (dbg == nullptr) return MOE_FFN_FP8_ERR_INVALID_ARG;
    return launch_forward(x_bf16, router_logits_bf16, h, out_bf16, M, stream, dbg);
}

MOE_API int32_t moe_ffn_fp8_forward_variant(const uint16_t* x_bf16, const uint16_t* router_logits_bf16,
                                            moe_ffn_fp8_handle* h, uint16_t* out_bf16, int32_t M, void* stream,
                                            const moe_ffn_fp8_variant* variant, const moe_ffn_fp8_debug* dbg) {
    if (variant == nullptr) return MOE_FFN_FP8_ERR_INVALID_ARG;
    return launch_forward(x_bf16, router_logits_bf16, h, out_bf16, M, stream, dbg, variant);
}

MOE_API int32_t moe_ffn_fp8_forward_rmsnorm(const uint16_t* h_bf16, const uint16_t* norm_w_bf16, float eps,
                                            const uint16_t* router_logits_bf16, moe_ffn_fp8_handle* h,
                                            uint16_t* out_bf16, int32_t M, void* stream,
                                            const moe_ffn_fp8_variant* variant, const moe_ffn_fp8_debug* dbg) {
    if (norm_w_bf16 == nullptr) return MOE_FFN_FP8_ERR_INVALID_ARG;
    return launch_forward(h_bf16, router_logits_bf16, h, out_bf16, M, stream, dbg, variant, norm_w_bf16, eps);
}

MOE_API int32_t moe_ffn_fp8_set_batch_mode(moe_ffn_fp8_handle* h, int32_t mode) {
    if (h == nullptr || (mode != MOE_FFN_FP8_BATCH_GROUPED && mode != MOE_FFN_FP8_BATCH_CHUNKED))
        return MOE_FFN_FP8_ERR_INVALID_ARG;
    h->batch_mode = mode;
    return MOE_FFN_FP8_OK;
}

MOE_API int32_t moe_ffn_fp8_set_launch_mode(moe_ffn_fp8_handle* h, int32_t mode) {
    if (h == nullptr || (mode != MOE_FFN_FP8_LAUNCH_THREE && mode != MOE_FFN_FP8_LAUNCH_SINGLE))
        return MOE_FFN_FP8_ERR_INVALID_ARG;
    if (mode == MOE_FFN_FP8_LAUNCH_SINGLE && h->single == nullptr) return MOE_FFN_FP8_ERR_UNSUPPORTED;
    h->launch_mode = mode;
    return MOE_FFN_FP8_OK;
}

MOE_API int32_t moe_ffn_fp8_profile_begin(moe_ffn_fp8_handle* h) {
    if (h == nullptr) return MOE_FFN_FP8_ERR_INVALID_ARG;
    if (hipSetDevice(h->device) != hipSuccess) return MOE_FFN_FP8_ERR_HIP;
    const size_t need = (size_t)kProfSlots * (MOE_FFN_FP8_NUM_STAGES + 1);
    while (h->events.size() < need) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) return MOE_FFN_FP8_ERR_HIP;
        h->events.push_back(e);
    }
    h->prof_calls = 0;
    h->prof_on = true;
    return MOE_FFN_FP8_OK;
}

MOE_API int32_t moe_ffn_fp8_profile_end(moe_ffn_fp8_handle* h, float* stage_ms, int32_t* calls) {
    if (h == nullptr || stage_ms == nullptr || calls == nullptr) return MOE_FFN_FP8_ERR_INVALID_ARG;
    h->prof_on = false;
    for (int s = 0; s < MOE_FFN_FP8_NUM_STAGES; ++s) stage_ms[s] = 0.0f;
    *calls = h->prof_calls;
    for (int c = 0; c < h->prof_calls; ++c) {
        hipEvent_t* ev = &h->events[(size_t)c * (MOE_FFN_FP8_NUM_STAGES + 1)];
        if (hipEventSynchronize(ev[MOE_FFN_FP8_NUM_STAGES]) != hipSuccess) return MOE_FFN_FP8_ERR_HIP;
        for (int s = 0; s < MOE_FFN_FP8_NUM_STAGES; ++s) {
            float ms = 0.0f;
            if (hipEventElapsedTime(&ms, ev[s], ev[s + 1]) != hipSuccess) return MOE_FFN_FP8_ERR_HIP;
            stage_ms[s] += ms;
        }
    }
    return MOE_FFN_FP8_OK;
}

MOE_API int32_t moe_ffn_fp8_destroy(moe_ffn_fp8_handle* h) {
    if (h == nullptr) return MOE_FFN_FP8_OK;
    (void)hipSetDevice(h->device);
    free_all(h);
    delete h;
    return MOE_FFN_FP8_OK;
}

MOE_API const char* moe_ffn_fp8_status_string(int32_t status) {
    switch (status) {
        case MOE_FFN_FP8_OK: return "ok";
        case MOE_FFN_FP8_ERR_INVALID_ARG: return "invalid argument";
        case MOE_FFN_FP8_ERR_UNSUPPORTED: return "unsupported size";
        case MOE_FFN_FP8_ERR_OUT_OF_MEMORY: return "out of device memory";
        case MOE_FFN_FP8_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

MOE_API int32_t moe_ffn_fp8_e4m3_encode(const float* in, uint8_t* out, int64_t n, void* stream) {
    if (n < 0) return MOE_FFN_FP8_ERR_INVALID_ARG;
    if (n == 0) return MOE_FFN_FP8_OK;
    if (!device_range_ok(in, (size_t)n * 4, 4) || !device_range_ok(out, (size_t)n, 1))
        return MOE_FFN_FP8_ERR_INVALID_ARG;
    hipLaunchKernelGGL(moe::encode_kernel, dim3(grid_for(n, 256)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), in, out, n);
    return hip_status(hipGetLastError());
}

MOE_API int32_t moe_ffn_fp8_e4m3_quantize(const float* in, float scale, uint8_t* out, int64_t n, void* stream) {
    if (n < 0 || !(scale > 0.0f) || !std::isfinite(scale)) return MOE_FFN_FP8_ERR_INVALID_ARG;
    if (n == 0) return MOE_FFN_FP8_OK;
    if (!device_range_ok(in, (size_t)n * 4, 4) || !device_range_ok(out, (size_t)n, 1))
        return MOE_FFN_FP8_ERR_INVALID_ARG;
    hipLaunchKernelGGL(moe::quantize_kernel, dim3(grid_for((n + 1) / 2, 256)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), in, scale, out, n);
    return hip_status(hipGetLastError());
}

MOE_API int32_t moe_ffn_fp8_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
    if (bytes <= 0 || bytes % 16 != 0) return MOE_FFN_FP8_ERR_INVALID_ARG;
    if (!device_range_ok(buf, (size_t)bytes, 16) || !device_range_ok(sink, 4, 4)) return MOE_FFN_FP8_ERR_INVALID_ARG;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
        (void)hipGetLastError();
        return MOE_FFN_FP8_ERR_HIP;
    }
    hipLaunchKernelGGL(moe::stream_read_kernel, dim3(cus), dim3(moe::kReadThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(buf), (uint64_t)bytes, sink);
    return hip_status(hipGetLastError());
}

MOE_API int32_t moe_ffn_fp8_e4m3_decode(const uint8_t* in, float* out, int64_t n, void* stream) {
    if (n < 0) return MOE_FFN_FP8_ERR_INVALID_ARG;
    if (n == 0) return MOE_FFN_FP8_OK;
    if (!device_range_ok(in, (size_t)n, 1) || !device_range_ok(out, (size_t)n * 4, 4))
        return MOE_FFN_FP8_ERR_INVALID_ARG;
    hipLaunchKernelGGL(moe::decode_kernel, dim3(grid_for(n, 256)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), in, out, n);
    return hip_status(hipGetLastError());
}
