/*
 * moe_decode.h -- C ABI of the output-centric ("warp decode") MoE decode layer
 * for AMD Instinct MI355X (gfx950).
 *
 * Source of the method: Cursor, "warp decode" blog post.  The MoE FFN of one
 * decode step is two kernels (section "What we changed"):
 *   moe_decode_gate_up  -- section "How the two kernels work", first two
 *       paragraphs: for each token b, routed slot j and intermediate neuron n,
 *       the gate and up rows of expert e = topk_ids[b,j] are streamed, their
 *       MXFP8 values converted to FP32 on the fly and dotted with x[b] in FP32;
 *       the neuron's value SiLU(gate) * up is written once.
 *   moe_decode_down     -- same section, third and fourth paragraphs: for each
 *       token b and output dimension o, the down rows of the token's k routed
 *       experts are streamed against h[b,j,:], each expert's router weight is
 *       folded into one FP32 accumulator, and y[b,o] is written once; the
 *       weighted top-k combine is part of the projection (no padding, no
 *       expert-major gather, no per-expert output buffer, no separate combine:
 *       sections "Stage elimination" and "Eliminating buffers").
 *
 * Number formats.  Weights are MXFP8 (OCP Microscaling v1.0): E4M3 element
 * codes (bias 7, max 448, S.1111.111 = NaN) with one E8M0 scale code
 * (value 2^(v-127), 0xFF = NaN) per 32 consecutive elements along the
 * reduction dimension.  Activations x, the intermediate h and the output y
 * are bf16 (stored as 16-bit patterns); results are rounded to nearest even.
 * Accumulation is FP32 in an unspecified order.  Router weights are FP32 and
 * are used as given (never renormalised).
 *
 * Layouts (all row-major, all contiguous):
 *   x            bf16   [B, H]
 *   topk_ids     int32  [B, k]   expert of slot j of token b
 *   topk_weights fp32   [B, k]   router weight of that slot
 *   w_gate, w_up uint8  [E, I, H]    E4M3 codes, row = one neuron of one expert
 *   s_gate, s_up uint8  [E, I, H/32] E8M0 codes, s[e,n,c/32] scales w[e,n,c]
 *   w_down       uint8  [E, H, I]    E4M3 codes, row = one output dim of one expert
 *   s_down       uint8  [E, H, I/32] E8M0 codes
 *   h            bf16   [B, k, I]    slot order = topk_ids order
 *   y            bf16   [B, H]
 *
 * Ownership and behaviour common to every call:
 *   - Every pointer is a device pointer owned by the caller.  The library
 *     allocates nothing, keeps no pointer after return and never synchronises.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the
 *     null stream).  The call returns as soon as the launch is enqueued; the
 *     caller synchronises the stream before reading outputs.
 *   - Calls are thread-safe.  The only state the library keeps is set once
 *     per device, before the first launch that needs it on that device, and
 *     is never changed afterwards: each matrix-core kernel's maximum dynamic
 *     LDS, set to the largest size its limits allow, and the device address
 *     of the no-allocation entry point's scratch array (whose concurrent
 *     calls on one device race; see moe_decode_conventional_noalloc).
 *   - Outputs are fully overwritten; every element is written exactly once.
 *   - Outputs must not overlap any input (checked on the host).
 *   - B == 0 is a valid no-op.
 *   - topk_ids outside [0, E) are not read through: every output that depends
 *     on such a slot is written as a quiet NaN.  Duplicate ids in one token
 *     are legal and are summed slot by slot.
 *   - E8M0 codes 0x00 (2^-127) and 0xFF (NaN) are honoured.
 * Return value: MOE_OK (0) once the launch is enqueued, else a negative code
 * below.  On any negative return other than MOE_ERR_LAUNCH nothing was
 * launched and no output was touched.
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_ERR_NULL (-1)        /* a required pointer is NULL (with B > 0)                    */
#define MOE_ERR_SHAPE (-2)       /* B<0, H/I/E/k<=0, k>E, H or I not a multiple of 32, or a   */
                                 /* shape beyond the supported range (H <= 8192,              */
                                 /* k*I <= 16384, E*I*H < 2^32 bytes per weight tensor)       */
#define MOE_ERR_ALIGN (-3)       /* x, h, w_* not 16-byte aligned; ids/weights not 4-byte     */
#define MOE_ERR_LAUNCH (-4)      /* the HIP runtime reported an error for the launch          */
#define MOE_ERR_ALIAS (-5)       /* an output range overlaps an input range                   */
#define MOE_ERR_ARG (-6)         /* an invalid tuning argument (see the _ex variants)         */
#define MOE_ERR_SCRATCH (-7)     /* the shape needs more scratch than the fixed buffer holds  */
                                 /* (moe_decode_conventional_noalloc only)                   */

/* Gate/up kernel: h[b,j,n] = bf16( SiLU(G) * U ), with
 *   G = sum_c dec(w_gate[e,n,c]) * 2^(s_gate[e,n,c/32]-127) * x[b,c],
 *   U = the same with w_up, s_up,  e = topk_ids[b,j].
 * Reads x [B,H], topk_ids [B,k], w_gate/s_gate/w_up/s_up of the routed experts only;
 * writes h_out [B,k,I]. */
int moe_decode_gate_up(const void *x, const int32_t *topk_ids,
                       const uint8_t *w_gate, const uint8_t *s_gate,
                       const uint8_t *w_up, const uint8_t *s_up,
                       void *h_out,
                       int B, int H, int I, int E, int k, void *stream);

/* Down kernel: y[b,o] = bf16( sum_j topk_weights[b,j] *
 *   sum_i dec(w_down[e_j,o,i]) * 2^(s_down[e_j,o,i/32]-127) * h[b,j,i] ),  e_j = topk_ids[b,j].
 * Reads h [B,k,I], topk_ids and topk_weights [B,k], w_down/s_down of the routed experts only;
 * writes y_out [B,H]. */
int moe_decode_down(const void *h, const int32_t *topk_ids, const float *topk_weights,
                    const uint8_t *w_down, const uint8_t *s_down,
                    void *y_out,
                    int B, int H, int I, int E, int k, void *stream);

/* Kernel variants of the gate/up call.
 *   MOE_GATE_UP_PER_SLOT: one wavefront per (R neurons, token slot) -- the
 *     blog post's organisation, one output set per warp ("How the two kernels
 *     work").  Best while few tokens share an expert.
 *   MOE_GATE_UP_EXPERT_GROUPED: the slots are sorted by expert on the device
 *     (inside the kernel, in LDS) and one wavefront takes R neurons of one
 *     routed expert for every slot routed to it, reading and converting the
 *     expert's rows once (section "Warp decode and Composer training": the
 *     regime where several tokens share an expert).  Same outputs; requires
 *     B*k <= 1024 and E <= 1024.
 *   MOE_GATE_UP_EXPERT_GROUPED_MFMA: the same grouping with the dot products
 *     on the matrix cores (v_mfma_f32_16x16x32_bf16): a workgroup takes 16
 *     neurons of one routed expert for up to 8 or 16 of its slots, streaming the
 *     rows and activations through LDS in 512-element chunks; the E8M0 scale
 *     is folded into the E4M3 -> bf16 conversion.  Same outputs within the
 *     same tolerance; requires H a multiple of 2048 up to 8192, B*k <= 1024,
 *     E <= 1024, and s_gate, s_up 16-byte aligned (MOE_ERR_ALIGN otherwise;
 *     rows_per_wave must be 0 or 16).
 * The plain call takes the matrix-core variant from 0.625 slots per expert
 * on (8*B*k >= 5E), or from half a slot at H >= 4096 (2*B*k >= E), when its
 * limits allow (with unaligned scales it takes the vector-unit grouped
 * variant instead); where they do not, the vector-unit grouped one from one
 * slot per expert on (B*k >= E), or half a slot at H >= 4096; else the
 * per-slot one.  At H = 4096 exactly, the vector-unit grouped variant from
 * 5/16 of a slot per expert up to 7/4 (16*B*k >= 5E, 4*B*k < 7E).  Each
 * choice is the fastest measured there. */
#define MOE_GATE_UP_PER_SLOT 1
#define MOE_GATE_UP_EXPERT_GROUPED 2
#define MOE_GATE_UP_EXPERT_GROUPED_MFMA 3

/* Kernel variants of the down call.
 *   MOE_DOWN_PER_TOKEN: one wavefront per (R output dimensions, token) --
 *     the blog post's organisation ("How the two kernels work").  Best while
 *     few tokens share an expert.
 *   MOE_DOWN_EXPERT_GROUPED: one workgroup per 8 output dimensions (4 for
 *     I > 1024) for every token; its wavefronts share out the routed experts
 *     (sorted on the device, in LDS), read each routed expert's rows once,
 *     and keep each slot's FP32 contribution in LDS until the workgroup adds
 *     every token's k contributions in slot order and writes y once.  No
 *     per-expert output buffer, no combine.  Same outputs; requires
 *     B <= 64, B*k <= 1024, E <= 1024 and I <= 2048.
 *   MOE_DOWN_EXPERT_GROUPED_MFMA: the same organisation (one workgroup per 8
 *     output dimensions for every token, work units of at most 8 slots of one
 *     expert, contributions added in slot order) with the dot products on the
 *     matrix cores (v_mfma_f32_4x4x4_16b_bf16): a wavefront converts its
 *     unit's 8 rows to bf16 once per 4 slots and forms the 8 x 4 dot products
 *     as 16-element chunk products, each scaled by its chunk's E8M0 scale
 *     (exact) before the chunks are summed.  Same outputs within the same
 *     tolerance; requires B*k <= 1024, E <= 1024 and I <= 2048
 *     (rows_per_wave must be 0 or 8).
 * The plain call takes the matrix-core grouped variant once 16*B*k >= 5E
 * (5/16 of a slot per expert on average) and its limits allow it, else the
 * per-token one: the fastest in each measured configuration but one (H =
 * 4096 with 5 tokens of uniform routing, where the per-token kernel is 3.5 %
 * faster; under skewed routing it is 6 % slower there).  The vector-unit
 * grouped variant runs on request only: its limits lie within the
 * matrix-core one's, which is faster wherever both run. */
#define MOE_DOWN_PER_TOKEN 1
#define MOE_DOWN_EXPERT_GROUPED 2
#define MOE_DOWN_EXPERT_GROUPED_MFMA 3

/* Tuning variants of the two calls: the same contract and results within the
 * same tolerance, with the launch shape given explicitly instead of taken
 * from the built-in table.  variant: 0 = the table's choice, else one of the
 * MOE_GATE_UP_* (gate/up) or MOE_DOWN_* (down) values.  rows_per_wave in
 * {1, 2, 4, 8} is the number of neurons (gate/up) or output dimensions (down)
 * one 64-lane wavefront owns (the grouped down kernel: 8 for I <= 1024,
 * else 4); 0 selects
 * the table's choice.  Combinations beyond the register budget (rows x
 * passes of 1024 elements: <= 16 per-slot, <= 8 grouped; per-token down:
 * passes x (5 rows + 8) <= 224), a grouped variant beyond its limits and
 * unknown variants return MOE_ERR_ARG. */
int moe_decode_gate_up_ex(const void *x, const int32_t *topk_ids,
                          const uint8_t *w_gate, const uint8_t *s_gate,
                          const uint8_t *w_up, const uint8_t *s_up,
                          void *h_out,
                          int B, int H, int I, int E, int k,
                          int variant, int rows_per_wave, void *stream);
int moe_decode_down_ex(const void *h, const int32_t *topk_ids, const float *topk_weights,
                       const uint8_t *w_down, const uint8_t *s_down,
                       void *y_out,
                       int B, int H, int I, int E, int k,
                       int variant, int rows_per_wave, void *stream);

/* Router step in front of the layer.  The blog post ("The traditional MoE
 * path") routes each token to a few of many experts (8 of 128 in one layer)
 * and gives no router details; these calls implement the plain top-k router:
 * from logits fp32 [B, E] (row-major, finite values), token b keeps its k
 * largest logits, largest first and the lower expert id first among equal
 * logits (-0 equals +0), so topk_ids[b, j] is its j-th selection; the routing
 * weight topk_weights[b, j] = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the
 * k selections (the softmax over all E renormalised over the kept k), in
 * FP32 with the device's expf.  Ids are always in [0, E), even for logits
 * that are not finite (their weights are then unspecified).
 * Limits: E <= 1024, k <= 64 and k <= E, B*E*4 < 2^31.  Pointers 4-byte
 * aligned; outputs disjoint from each other and from every input.
 *
 *   moe_decode_route: ids and weights only (one 64-lane wavefront per token).
 *   moe_decode_gate_up_routed: gate/up with the router step in front --
 *     reads logits instead of topk_ids, writes h_out as moe_decode_gate_up
 *     would for the ids it selects, and also writes topk_ids_out and
 *     topk_weights_out [B, k] for moe_decode_down.  For E <= 128 and
 *     B*k <= 16 (and whenever the _ex form asks for the per-slot variant
 *     with E <= 128) the selection is the per-slot kernel's prologue: each
 *     workgroup selects its token's experts itself, with no extra launch.
 *     Otherwise the router kernel runs first and the table's (or the asked)
 *     gate/up variant reads the ids it wrote: two launches on `stream`.  The
 *     _ex form takes variant and rows_per_wave as moe_decode_gate_up_ex
 *     does. */
int moe_decode_route(const float *logits, int32_t *topk_ids, float *topk_weights,
                     int B, int E, int k, void *stream);
int moe_decode_gate_up_routed(const void *x, const float *logits,
                              const uint8_t *w_gate, const uint8_t *s_gate,
                              const uint8_t *w_up, const uint8_t *s_up,
                              void *h_out, int32_t *topk_ids_out, float *topk_weights_out,
                              int B, int H, int I, int E, int k, void *stream);
int moe_decode_gate_up_routed_ex(const void *x, const float *logits,
                                 const uint8_t *w_gate, const uint8_t *s_gate,
                                 const uint8_t *w_up, const uint8_t *s_up,
                                 void *h_out, int32_t *topk_ids_out, float *topk_weights_out,
                                 int B, int H, int I, int E, int k,
                                 int variant, int rows_per_wave, void *stream);

/* The launch the built-in table picks for a call (for reports): writes the
 * variant, rows_per_wave and the number of workgroups; returns 0 or a
 * negative code. */
int moe_decode_gate_up_plan(int B, int H, int I, int E, int k, int *variant, int *rows_per_wave, int *workgroups);
int moe_decode_down_plan(int B, int H, int I, int E, int k, int *variant, int *rows_per_wave, int *workgroups);

/* The conventional, expert-centric path, for A/B comparison (blog post,
 * sections "The traditional MoE path", "Stage elimination", "Eliminating
 * buffers" and "Accuracy improvement").  Same layer as gate_up + down, but
 * computed the way an expert-centric pipeline does it, as seven launches on
 * `stream` through caller-provided device workspace: route (per-expert token
 * lists, each padded to a power of two), quantise x to MXFP8 (E4M3 codes and
 * one E8M0 scale 2^(floor(log2 amax) - 8) per 32 along H, saturating at 448),
 * scatter the quantised rows into an expert-major gather buffer, gate/up per
 * row (h = bf16(SiLU(G) * U)), quantise h to MXFP8 (blocks along I), down per
 * row into a bf16 per-expert output buffer, and the weighted combine y[b] =
 * bf16(sum_j w[b,j] * out[b,j]).  Padding rows are computed and discarded.
 * Inputs and y as for the two calls above; `workspace` is device memory of at
 * least the size moe_decode_conventional_workspace() reports, 256-byte
 * aligned, owned by the caller, disjoint from every input and from y, and
 * used only until the launches complete.  Limits: B*k <= 1024, E <= 1024,
 * H and I <= 8192.  Returns MOE_ERR_ARG if the workspace is too small;
 * otherwise the error codes above. */
int moe_decode_conventional_workspace(int B, int H, int I, int E, int k, size_t *bytes);
int moe_decode_conventional(const void *x, const int32_t *topk_ids, const float *topk_weights,
                            const uint8_t *w_gate, const uint8_t *s_gate,
                            const uint8_t *w_up, const uint8_t *s_up,
                            const uint8_t *w_down, const uint8_t *s_down,
                            void *y_out, void *workspace, size_t workspace_bytes,
                            int B, int H, int I, int E, int k, void *stream);

/* The conventional path of moe_decode_conventional for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid hipMalloc.  Same stages, kernels and results, but
 * instead of a caller's workspace the launches use a fixed 32 MiB device
 * buffer inside the library (one per device, resident from module load until
 * the process ends).  Nothing in that buffer needs to start at zero: the route
 * stage writes every entry the later stages read.  The call allocates and
 * frees nothing (no hipMalloc, hipFree or allocating library routine); its
 * first call on a device looks up that device's address of the buffer once.
 * Every call on one device shares that device's buffer and leaves its contents
 * behind, so calls that overlap in time on one device race: the caller orders
 * them (one stream, or events between streams).  Returns MOE_ERR_SCRATCH
 * (before any launch) when the shape's workspace,
 * moe_decode_conventional_workspace(), exceeds 32 MiB; otherwise the codes
 * and limits of moe_decode_conventional. */
int moe_decode_conventional_noalloc(const void *x, const int32_t *topk_ids, const float *topk_weights,
                                    const uint8_t *w_gate, const uint8_t *s_gate,
                                    const uint8_t *w_up, const uint8_t *s_up,
                                    const uint8_t *w_down, const uint8_t *s_down,
                                    void *y_out, int B, int H, int I, int E, int k, void *stream);

/* Bandwidth probes that set the denominator of the efficiency figure (blog
 * post, "Hardware efficiency": peak measured with a copy kernel over
 * contiguous memory).  copy: dst[0:bytes) = src[0:bytes); read: reads
 * src[0:bytes) and writes nothing unless an impossible checksum appears
 * (sink: one 4-byte device word).  bytes must be a positive multiple of 16,
 * pointers 16-byte aligned, src and dst disjoint.  Asynchronous on `stream`. */
int moe_decode_copy_peak(const void *src, void *dst, size_t bytes, void *stream);
int moe_decode_read_peak(const void *src, size_t bytes, void *sink, void *stream);

/* Static description of a return code (never NULL). */
const char *moe_decode_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DECODE_H */
