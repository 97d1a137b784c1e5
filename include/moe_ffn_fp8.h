/*
 * moe_ffn_fp8.h -- C ABI of the FP8 mixture-of-experts feed-forward step for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (Blackwell 1,000 TPS/user blog, zh translation: the lead list and
 * the paragraph on FP8 for GEMM, MoE and attention; section "CUDA kernel
 * optimisation and fusion", items "GEMM weight swizzle" and "operator fusion"):
 * FP8 weights and activations with scales, the FC13 GEMM with SwiGLU fused onto
 * it, the quantisation of its result to FP8 in front of the FC2 GEMM, and a
 * mixture of experts with one shared expert and top-1 routing.  For M tokens,
 * hidden size K, intermediate size I and E routed experts:
 *
 *   s_x[m]  = fp32(max_k |x[m,k]| / 448),  xq = e4m3(x / s_x)         (per token)
 *   e[m]    = lowest index of the largest logit[m, :];  gate[m] = sigmoid(logit[m, e[m]])
 *   for the shared expert (all tokens) and for expert e[m] (token m only):
 *     h     = s_x[m] * s13[n] * sum_k dec(xq[m,k]) * dec(w13[k,n])     n in [0, 2I)
 *     a     = silu(h[:, 0:I]) * h[:, I:2I]                    (columns [0,I) = gate)
 *     s_a[m]= fp32(max_j |a[m,j]| / 448),  aq = e4m3(a / s_a)           (per token)
 *     y     = s_a[m] * s2[k] * sum_j dec(aq[m,j]) * dec(w2[j,k])
 *   out[m,k] = bf16_rne(y_shared[m,k] + gate[m] * y_e[m][m,k])    (y_shared if E == 0)
 *
 * e4m3 is the OCP 8-bit float (bias 7, max 448, NaN at 0x7F/0xFF, subnormals);
 * encoding rounds to nearest, ties to even, saturating at 448.  A token whose
 * row is all zero gets scale 0 and codes 0.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers (hipMalloc'd or torch tensors on the GPU)
 *    unless marked (host).  `stream` is a hipStream_t (NULL = default stream).
 *  - Every entry point returns a moe_ffn_fp8_status.  Arguments are checked on
 *    the host before any device work; a failed check enqueues nothing.  No C++
 *    exception crosses the ABI.  Launch failures return MOE_FFN_FP8_ERR_HIP.
 *  - Device-side faults surface at the caller's next synchronisation.
 *  - A handle serves one stream at a time: two forwards on one handle that overlap
 *    in time (different streams) race on its workspace.
 */
#ifndef MOE_FFN_FP8_H
#define MOE_FFN_FP8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_ffn_fp8_status {
    MOE_FFN_FP8_OK = 0,
    MOE_FFN_FP8_ERR_INVALID_ARG = -1,   /* null / misaligned pointer, bad size, host pointer */
    MOE_FFN_FP8_ERR_UNSUPPORTED = -2,   /* sizes outside what the kernels tile */
    MOE_FFN_FP8_ERR_OUT_OF_MEMORY = -3, /* device allocation failed (nothing leaked) */
    MOE_FFN_FP8_ERR_HIP = -4            /* a HIP runtime call or kernel launch failed */
} moe_ffn_fp8_status;

/* Sizes fixed when a handle is created.
 *  hidden      K, multiple of 128, 128..8192; also min(max_tokens, 16) * (K + 16) must
 *              fit the kernels' LDS budget (about 160 KB with the other tables)
 *  inter       I, multiple of 128, 128..32768
 *  num_experts E routed experts, 0..1024 (0 = plain dense FFN with the shared expert)
 *  max_tokens  largest M a forward may be called with, 1..65536.  Up to
 *              MOE_FFN_FP8_GROUP_FROM tokens run as one launch of the decode kernels.  A
 *              larger M runs as grouped passes of up to MOE_FFN_FP8_GROUP_MAX tokens
 *              (see moe_ffn_fp8_set_batch_mode): each pass streams the weights of the
 *              shared expert and of every distinct routed expert of its tokens once, for
 *              all of that expert's tokens.  Each token's result depends only on its own
 *              row, so the result is the same either way, all enqueued by the one call.
 *              A handle with max_tokens above MOE_FFN_FP8_GROUP_FROM also holds the grouped
 *              workspace, about (2 * nsplit * K * 4 + 2 * I * 5 + K) bytes per token of
 *              min(max_tokens, MOE_FFN_FP8_GROUP_MAX), nsplit = ceil(I / 2048).
 * Sizes outside these limits return MOE_FFN_FP8_ERR_INVALID_ARG, or
 * MOE_FFN_FP8_ERR_UNSUPPORTED for the LDS limit. */
#define MOE_FFN_FP8_CHUNK 16
#define MOE_FFN_FP8_GROUP_MAX 1024
/* Batches above this many tokens run grouped (measured on MI355X: at 12 and 16 tokens the
 * grouped pass is faster than one launch of the decode kernels, at 5 and 8 slower). */
#define MOE_FFN_FP8_GROUP_FROM 8
typedef struct moe_ffn_fp8_dims {
    int32_t hidden;
    int32_t inter;
    int32_t num_experts;
    int32_t max_tokens;
} moe_ffn_fp8_dims;

/* Opaque: owns the packed weights of E + 1 experts (slot E = shared expert) and the
 * forward workspace, all in device memory. */
typedef struct moe_ffn_fp8_handle moe_ffn_fp8_handle;

/* Number of kernels one forward launches, in order: router + activation
 * quantisation + FC13 + SwiGLU; re-quantisation + FC2 (split over I); combine. */
#define MOE_FFN_FP8_NUM_STAGES 3

/* Allocate a handle for `dims` (host) on the current device.  Packed weights are
 * uninitialised until every slot 0..E has been filled by moe_ffn_fp8_prepack_expert.
 * *out (host) receives the handle, or NULL on failure.  Allocation failure frees
 * everything allocated so far and returns MOE_FFN_FP8_ERR_OUT_OF_MEMORY.  For testing
 * that clean-up, the environment variable MOE_FFN_FP8_FAIL_ALLOC=n (n >= 1), read at each
 * call, makes the call's n-th device allocation fail as if the device were full. */
int32_t moe_ffn_fp8_create(const moe_ffn_fp8_dims* dims, moe_ffn_fp8_handle** out);

/* Offline weight prepack of one expert slot (0..E-1 routed, E shared): a pure
 * permutation of the codes into the order the matrix-core kernels read, so that
 * every lane issues contiguous 16-byte loads ("GEMM weight swizzle", same page and
 * section as above, re-derived for gfx950).  Inputs, all row-major, device:
 *   w13 uint8 [K][2I] e4m3 codes; columns [0,I) gate (FC1), [I,2I) up (FC3)
 *   s13 float [2I]    per-output-channel scales
 *   w2  uint8 [I][K]  e4m3 codes of the down projection
 *   s2  float [K]     per-output-channel scales
 * The library copies what it needs and synchronises `stream` before returning, so
 * the inputs may be freed right after.  Not for use inside a forward's stream order
 * on the same handle. */
int32_t moe_ffn_fp8_prepack_expert(moe_ffn_fp8_handle* h, int32_t slot,
                                   const uint8_t* w13, const float* s13,
                                   const uint8_t* w2, const float* s2, void* stream);

/* create + prepack of all E + 1 slots from stacked arrays:
 *   w13 [E+1][K][2I], w2 [E+1][I][K], s13 [E+1][2I], s2 [E+1][K] (device). */
int32_t moe_ffn_fp8_prepack(const moe_ffn_fp8_dims* dims, const uint8_t* w13,
                            const uint8_t* w2, const float* s13, const float* s2,
                            void* stream, moe_ffn_fp8_handle** out);

/* Inverse of the prepack for one slot, into caller buffers of the same shapes as
 * moe_ffn_fp8_prepack_expert's inputs (device).  For tests; enqueued on `stream`. */
int32_t moe_ffn_fp8_unpack_expert(const moe_ffn_fp8_handle* h, int32_t slot,
                                  uint8_t* w13, float* s13, uint8_t* w2, float* s2,
                                  void* stream);

/* One forward step, enqueued on `stream`; never allocates and never synchronises,
 * so it may be captured into a HIP graph.
 *   x_bf16             [M][K] bf16 bit patterns, 2-byte aligned
 *   router_logits_bf16 [M][E] bf16 bit patterns; must be NULL iff E == 0
 *   out_bf16           [M][K] bf16 result (may not alias the inputs)
 *   M                  0..max_tokens; M == 0 returns OK and launches nothing
 * Only the weights of the shared expert and of the distinct experts the tokens are
 * routed to are read; the set is found on the device.  With M above MOE_FFN_FP8_GROUP_FROM
 * that holds per grouped pass of up to MOE_FFN_FP8_GROUP_MAX consecutive tokens (or, in
 * the chunked batch mode, per chunk of MOE_FFN_FP8_CHUNK tokens, the chunks being
 * consecutive in routed-expert order: ascending expert, then ascending token). */
int32_t moe_ffn_fp8_forward(const uint16_t* x_bf16, const uint16_t* router_logits_bf16,
                            moe_ffn_fp8_handle* h, uint16_t* out_bf16, int32_t M,
                            void* stream);

/* moe_ffn_fp8_forward for callers that cannot allocate device memory or must not see an
 * allocation while they run: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It calls no allocating routine: the forward's workspace (routing
 * table, gates, row maxima, the float32 intermediate, the partial sums and the work
 * counters) lives in a static array of the library, MOE_FFN_FP8_SCRATCH_BYTES per device,
 * which every device the library runs on holds until the process ends (its address is
 * taken when a handle is first created on the device).  Every call on a device shares that
 * device's array and finds in it what the last call left; a first small kernel clears the
 * counters, then the three decode kernels run (always three, whatever the launch mode).
 * Calls that overlap in time on one device (different streams, or threads) race on it.
 * Same arguments and result as moe_ffn_fp8_forward, bit for bit, with two limits:
 *   M <= min(max_tokens, MOE_FFN_FP8_CHUNK) (one launch of the decode kernels), and the
 *   workspace of that launch, about (2 * nsplit * K * 4 + 2 * I * 4) bytes per token of
 *   min(max_tokens, MOE_FFN_FP8_CHUNK) plus the routing table and the row maxima, must fit
 *   MOE_FFN_FP8_SCRATCH_BYTES;
 * otherwise MOE_FFN_FP8_ERR_UNSUPPORTED.  MOE_FFN_FP8_ERR_HIP if HIP gave no address for
 * the array.  Other argument errors as moe_ffn_fp8_forward. */
#define MOE_FFN_FP8_SCRATCH_BYTES (8 << 20)
int32_t moe_ffn_fp8_forward_scratch(const uint16_t* x_bf16, const uint16_t* router_logits_bf16,
                                    moe_ffn_fp8_handle* h, uint16_t* out_bf16, int32_t M, void* stream);

/* Intermediate results of a forward, written when the pointer is not NULL (device):
 *   xq [M][K] uint8, s_x [M] float, expert [M] int32 (-1 when E == 0), gate [M] float,
 *   aq_shared [M][I] uint8, s_a_shared [M] float,
 *   aq_routed [M][I] uint8 and s_a_routed [M] float: row m belongs to expert[m];
 *   num_active [1] int32: number of distinct routed experts (with M above
 *     MOE_FFN_FP8_GROUP_FROM: summed over the grouped passes, or, in the chunked batch
 *     mode, over the chunks of MOE_FFN_FP8_CHUNK tokens; i.e. the routed experts streamed);
 *   sync_timeouts [1] uint32: the waits the handle's single launches have given up so far
 *     (see moe_ffn_fp8_set_launch_mode; nonzero means some result since was wrong), copied
 *     after the forward's kernels (when M > 0). */
typedef struct moe_ffn_fp8_debug {
    uint8_t* xq;
    float* s_x;
    int32_t* expert;
    float* gate;
    uint8_t* aq_shared;
    float* s_a_shared;
    uint8_t* aq_routed;
    float* s_a_routed;
    int32_t* num_active;
    uint32_t* sync_timeouts;
} moe_ffn_fp8_debug;

/* moe_ffn_fp8_forward that also writes the intermediates named in *dbg (host). */
int32_t moe_ffn_fp8_forward_debug(const uint16_t* x_bf16, const uint16_t* router_logits_bf16,
                                  moe_ffn_fp8_handle* h, uint16_t* out_bf16, int32_t M,
                                  void* stream, const moe_ffn_fp8_debug* dbg);

/* Variant readings of two points the pages leave open (host struct).  All zero is the
 * step as moe_ffn_fp8_forward computes it.
 *   gate_on_input  0: the gate multiplies the routed expert's output (out = y_shared +
 *                  gate * y_routed).  1: it multiplies the token before the routed
 *                  expert, and out = y_shared + y_routed.  The token enters the FFN
 *                  quantised once (the pages fuse the quantize step into the kernel in
 *                  front of it), so the gated input is gate * s_x * dec(xq): the same
 *                  codes, the token's scale times the gate (a float32 product).
 *   x_scale        0: per-token dynamic scale of x.  > 0: one static calibrated scale for
 *                  x (codes = e4m3(x / x_scale), saturating at +-448).
 *   a_scale        0: per-(token, expert) dynamic scale of the intermediate.  > 0: one
 *                  static calibrated scale for it (saturating likewise).
 * The static-scale reading takes the quantize step in front of a GEMM (Blackwell 1,000
 * TPS/user blog, zh translation, section "CUDA kernel optimisation and fusion", item
 * "operator fusion") with its scale fixed ahead of time.  Negative or non-finite scales, or
 * gate_on_input not 0 or 1, return MOE_FFN_FP8_ERR_INVALID_ARG. */
typedef struct moe_ffn_fp8_variant {
    int32_t gate_on_input;
    float x_scale;
    float a_scale;
} moe_ffn_fp8_variant;

/* moe_ffn_fp8_forward under the readings in *variant (host); dbg (host) may be NULL or
 * name intermediates to write as in moe_ffn_fp8_forward_debug (s_x and s_a then hold the
 * static scales where those are used). */
int32_t moe_ffn_fp8_forward_variant(const uint16_t* x_bf16, const uint16_t* router_logits_bf16,
                                    moe_ffn_fp8_handle* h, uint16_t* out_bf16, int32_t M,
                                    void* stream, const moe_ffn_fp8_variant* variant,
                                    const moe_ffn_fp8_debug* dbg);

/* The step with the RMSNorm in front of it fused into its first kernel (the pages fuse
 * the AllReduce with the RMSNorm that follows it and the quantize step into one kernel:
 * Blackwell 1,000 TPS/user blog, zh translation, section "CUDA kernel optimisation and
 * fusion", item "operator fusion"; one GPU has nothing to all-reduce).  The step computes
 * on x[m,k] = h[m,k] / sqrt(mean_k h[m,k]^2 + eps) * norm_w[k], in float32 from a float64
 * sum of squares, quantised per token from those unrounded values (never bf16).
 *   h_bf16       [M][K] bf16 hidden state (device), 2-byte aligned
 *   norm_w_bf16  [K] bf16 norm weight (device), 16-byte aligned; must not be NULL
 *   eps          finite, >= 0 (host)
 * The other arguments are those of moe_ffn_fp8_forward_variant (variant may be NULL for
 * the plain readings; dbg may be NULL; xq and s_x then describe the normalised x).
 * Returns MOE_FFN_FP8_ERR_UNSUPPORTED when the norm weight's LDS (2K bytes) does not fit
 * beside the handle's other LDS (min(max_tokens, 16) * (K + 16) bytes and the tables). */
int32_t moe_ffn_fp8_forward_rmsnorm(const uint16_t* h_bf16, const uint16_t* norm_w_bf16, float eps,
                                    const uint16_t* router_logits_bf16, moe_ffn_fp8_handle* h,
                                    uint16_t* out_bf16, int32_t M, void* stream,
                                    const moe_ffn_fp8_variant* variant, const moe_ffn_fp8_debug* dbg);

/* How a forward runs a batch above MOE_FFN_FP8_GROUP_FROM tokens.
 *   MOE_FFN_FP8_BATCH_GROUPED (the default): grouped passes of up to
 *     MOE_FFN_FP8_GROUP_MAX tokens; every active expert's weights are read once per
 *     pass (the pages build their MoE GEMMs to use the whole HBM bandwidth: Blackwell
 *     1,000 TPS/user blog, zh translation, section "CUDA kernel optimisation and
 *     fusion", item on spatial partitioning and efficient memory loads; a routed expert
 *     read once per launch of 16 tokens would be read several times per batch).
 *   MOE_FFN_FP8_BATCH_CHUNKED: one launch of the decode kernels up to MOE_FFN_FP8_CHUNK
 *     tokens, else consecutive launches of MOE_FFN_FP8_CHUNK tokens in routed-expert order.
 * Both give the same result.  The variant readings and the fused RMSNorm always run
 * chunked, and so does every batch when K is not a multiple of 1024 up to 5120 and above
 * 3072 (the grouped kernels keep one item per wave in registers).  Other values return MOE_FFN_FP8_ERR_INVALID_ARG.  Takes effect for the
 * forwards enqueued afterwards. */
#define MOE_FFN_FP8_BATCH_GROUPED 0
#define MOE_FFN_FP8_BATCH_CHUNKED 1
int32_t moe_ffn_fp8_set_batch_mode(moe_ffn_fp8_handle* h, int32_t mode);

/* How a launch of the decode kernels (up to MOE_FFN_FP8_CHUNK tokens) is enqueued.  The
 * pages overlap a kernel's preamble with the previous kernel's tail through programmatic
 * dependent launch (Blackwell 1,000 TPS/user blog, zh translation, section "Programmatic
 * dependent launch"); HIP has none, and this is its counterpart on one GPU.
 *   MOE_FFN_FP8_LAUNCH_THREE (default): three kernels on the stream (FC13 + SwiGLU,
 *     re-quantisation + FC2, combine).
 *   MOE_FFN_FP8_LAUNCH_SINGLE: one kernel whose blocks run the three as phases; the FC2
 *     blocks request their first weights while FC13's last blocks still run, then wait
 *     for them through counters in the handle's workspace (device-scope release and
 *     acquire).  The same arithmetic, so the same result bit for bit.  It relies on the
 *     in-order placement of a launch's workgroups, and its waits give up after 0.2 s
 *     (the results are then wrong; never expected; a debug forward's sync_timeouts
 *     reports the count).  The counters only grow, so a later launch is not disturbed
 *     by one whose waits gave up.  Calls on one handle must not overlap (as for every
 *     forward, the workspace is shared).
 * SINGLE is available for hidden 5120 and max_tokens up to 8; the fused RMSNorm, the
 * grouped passes and other sizes keep their kernels.  Returns
 * MOE_FFN_FP8_ERR_UNSUPPORTED for SINGLE on another handle, MOE_FFN_FP8_ERR_INVALID_ARG
 * for other values.  Takes effect for the forwards enqueued afterwards. */
#define MOE_FFN_FP8_LAUNCH_THREE 0
#define MOE_FFN_FP8_LAUNCH_SINGLE 1
int32_t moe_ffn_fp8_set_launch_mode(moe_ffn_fp8_handle* h, int32_t mode);

/* Per-kernel timing.  After profile_begin, each forward on the handle with M up to
 * MOE_FFN_FP8_CHUNK also records HIP events around each of its MOE_FFN_FP8_NUM_STAGES
 * kernels, and so does a forward of one grouped pass (up to MOE_FFN_FP8_GROUP_MAX
 * tokens), around its FC13 + SwiGLU kernel, its re-quantisation and FC2 kernels
 * together, and its combine (its routing and ordering kernels run before the first
 * event).  Up to 1024 forwards are kept; other forwards are not recorded.
 * profile_end synchronises those events and writes, to stage_ms (host,
 * MOE_FFN_FP8_NUM_STAGES floats), the summed milliseconds per kernel and to *calls
 * (host) the number of forwards recorded, then stops recording. */
int32_t moe_ffn_fp8_profile_begin(moe_ffn_fp8_handle* h);
int32_t moe_ffn_fp8_profile_end(moe_ffn_fp8_handle* h, float* stage_ms, int32_t* calls);

/* Free the handle and everything it owns.  NULL is accepted.  The caller makes sure
 * no work using the handle is still pending. */
int32_t moe_ffn_fp8_destroy(moe_ffn_fp8_handle* h);

/* Static string naming a status code. */
const char* moe_ffn_fp8_status_string(int32_t status);

/* The device's e4m3 codec over n elements (device buffers), for checking it against
 * the format definition: encode rounds to nearest, ties to even, saturating at 448;
 * decode gives NaN for 0x7F/0xFF. */
int32_t moe_ffn_fp8_e4m3_encode(const float* in, uint8_t* out, int64_t n, void* stream);
int32_t moe_ffn_fp8_e4m3_decode(const uint8_t* in, float* out, int64_t n, void* stream);

/* The forward's general quantiser (the quantize-before-GEMM step of the Blackwell 1,000
 * TPS/user blog, zh translation, section "CUDA kernel optimisation and fusion", item
 * "operator fusion"), over n elements: out[i] = the e4m3 code of the exact quotient
 * in[i] / scale, rounded to nearest with ties to even.  The forward applies it to the
 * float32 intermediate, to activations over a static scale or after the fused RMSNorm, and
 * to any row whose scale is below 2**-96 (scale and values lifted by 2**64 first).  The
 * plain forward's bf16 activations over their dynamic scale take a shortcut that gives the
 * same codes (ties resolved by the rounding of the scale), which this entry point does not
 * run.  in (device, float32, finite, |in / scale| <= 448 * (1 + 2**-22)), out (device, n
 * bytes), scale (host value) finite and > 0 (subnormal scales included), else
 * MOE_FFN_FP8_ERR_INVALID_ARG.  Enqueued on `stream`. */
int32_t moe_ffn_fp8_e4m3_quantize(const float* in, float scale, uint8_t* out, int64_t n, void* stream);

/* Measurement helper: reads `bytes` bytes of `buf` (device, 16-byte aligned; bytes a
 * positive multiple of 16) with the access pattern of the streaming GEMMs (one block
 * per CU, each wave reading its contiguous share of 160 KiB chunks, 16-byte loads) and
 * no arithmetic, enqueued on `stream`.  `sink` (device, 4 bytes) is written only in the
 * unlikely case that the XOR of the words one thread read equals a fixed value.  Timing it gives
 * the attainable read bandwidth that the forward's kernels are compared with, beside
 * the data-sheet HBM peak (the roofline the pages measure their GEMMs against: Blackwell
 * 1,000 TPS/user blog, zh translation, section "CUDA kernel optimisation and fusion",
 * the item on spatial partitioning and efficient memory loads). */
int32_t moe_ffn_fp8_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_FP8_H */
