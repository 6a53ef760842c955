/*
 * moe_decode.h -- C ABI of the persistent MoE decode layer for MI355X (gfx950).
 *
 * One call of moe_decode_run computes, for T token rows x[T][H] (bf16):
 *
 *   logits[t][e] = sum_h x[t][h] * router_w[e][h] (+ router_bias[e])
 *   score        = sigmoid(logits); the K highest scores of each row are
 *                  selected (score descending, ties to the lower expert id)
 *                  and their weights w[t][k] renormalised to sum to 1
 *   rows are placed into 8-row tiles of their experts, in row order,
 *                  without a sort (per-expert row bitmaps + population counts)
 *   per selected expert e (and the shared expert, slot E, for every row):
 *       g = W_gate[e] x,  u = W_up[e] x,  h = bf16(silu(g) * u),  o_e = W_down[e] h
 *       (g and u clipped first when a limit is set: moe_decode_set_swiglu_limit)
 *       (expert weights in one of three formats, each with one scale per 32
 *        contiguous K elements: FP8 e4m3fn with fp32 scales, or the OCP
 *        microscaling formats MXFP8 (e4m3fn) and MXFP4 (e2m1) with E8M0 scales)
 *   y[t] = bf16( o_shared[t] + sum_k w[t][k] * o_{idx[t][k]}[t] )
 *
 * in ONE persistent kernel launch (moe_decode_run_block runs the same layer as a
 * pre-norm block: input RMSNorm before it, residual added after it, same
 * launch).  Sources (page titles and sections):
 *   - "SGLang's Low-Latency Mode Boosts DeepSeek-V4.1-Flash Speed by 1.56x on
 *     AMD": section "NVIDIA overlaps the dependency chain" (routing without
 *     sorting: 8-row tiles, bitmap and population counts, top-k preserved);
 *     section "AMD keeps the layer resident" (persistent kernel including
 *     the MoE, waits with deadlines); section "Four stages keep megakernels
 *     outside core" (Register / Guard / Build / Runtime, fallback).
 *   - "FlyDSL Mono Kernels for High-Interactivity LLM Serving in ATOM":
 *     sections "What FlyDSL Provides" and "MiniMax-M3: Connecting Attention
 *     and Experts" (blocks that stay resident and hand ready results on
 *     through tagged buffers, early weight loads, routed and shared expert
 *     up/gate and down projections fused in one path).
 *   - "Beyond Day-0: Optimizing DeepSeek-V4.1 Flash in SGLang", section 2.1
 *     (group32 FP8 weights and scales reorganised for the kernel; router
 *     emitting the downstream layout; fused weighted reduction of expert
 *     outputs plus shared-expert addition; scratch buffers reused across
 *     calls) and section 3.1 (fused SwiGLU keeping the intermediate rounding).
 *
 * Conventions: every pointer named "device" is a HIP device pointer on the
 * handle's device; streams are hipStream_t passed as void* (NULL = the null
 * stream).  No function prints, aborts or throws; all report moe_status.
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_DECODE_ABI_VERSION 5

typedef int32_t moe_status;
#define MOE_OK                0  /* success */
#define MOE_ERR_INVALID_ARG   1  /* NULL / misaligned pointer, T out of range, bad config */
#define MOE_ERR_UNSUPPORTED   2  /* shape outside what the kernel handles: use another path */
#define MOE_ERR_HIP           3  /* a HIP runtime call failed */
#define MOE_ERR_OUT_OF_MEMORY 4  /* device allocation failed in create */
#define MOE_ERR_TIMEOUT       5  /* an in-kernel wait passed its deadline (reported by check) */

/* Layer shape and limits, fixed at create time. */
typedef struct moe_decode_config {
  int32_t max_tokens;    /* largest T any run on the handle may pass; 1..512 */
  int32_t hidden;        /* H; multiple of 64, <= 16384 */
  int32_t num_experts;   /* E routed experts; 1..256 */
  int32_t top_k;         /* K experts per row; 1..min(E, 16) */
  int32_t intermediate;  /* I per expert; multiple of 32, <= 8192.  A width that is
                            not a multiple of 64 runs padded to the next one (in
                            every weight format): the padding rows and columns get
                            zero weights, so results are those of width I (the
                            per-GPU width 288 of TP8 padded to 320 for MXFP4
                            experts: "Beyond Day-0: Optimizing DeepSeek-V4.1 Flash
                            in SGLang", section 3.1) */
  int32_t num_shared;    /* S always-on shared experts; 0 or 1 */
  int32_t deadline_us;   /* bound on every in-kernel wait, microseconds; 0 = 1 s */
  uint32_t flags;        /* bits 0-1: expert weight format, MOE_WEIGHTS_*; bit 2:
                            MOE_FLAG_COOPERATIVE; other bits reserved, must be 0
                            (else MOE_ERR_INVALID_ARG) */
} moe_decode_config;

/*
 * Expert weight formats (config flags, bits 0-1).  All three quantise the
 * expert matrices along K (H for gate/up, I for down) in groups of 32
 * contiguous elements that share one scale; a weight is decode(q) * scale.
 *   MOE_WEIGHTS_FP8    e4m3fn codes, fp32 scales.
 *   MOE_WEIGHTS_MXFP8  e4m3fn codes, E8M0 scales (one byte e: 2^(e - 127); 255
 *                      is NaN and must not occur).  OCP Microscaling (MX)
 *                      v1.0 formats.
 *   MOE_WEIGHTS_MXFP4  e2m1 codes (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their
 *                      negatives), two per byte, element 2j in the low nibble
 *                      of byte j; E8M0 scales.
 * Sources: "Beyond Day-0: Optimizing DeepSeek-V4.1 Flash in SGLang", section
 * 2.1 (group-32 FP8 expert weights and scales) and the MXFP4 / MXFP8 expert
 * weights of the same model's checkpoints that the pages name.
 */
#define MOE_WEIGHTS_FP8   0u
#define MOE_WEIGHTS_MXFP8 1u
#define MOE_WEIGHTS_MXFP4 2u

/*
 * MOE_FLAG_COOPERATIVE: launch every run as a cooperative kernel.  The
 * kernel's hand-offs need every workgroup of its grid (sized to what the
 * device holds at once) to be resident together.  On an otherwise idle
 * device they are; when another kernel may hold compute units (a shared
 * device), a plain launch can leave some workgroups waiting for absent ones
 * until the deadline (MOE_ERR_TIMEOUT).  A cooperative launch instead either
 * runs the whole grid co-resident or fails (moe_decode_run returns
 * MOE_ERR_HIP).  It costs about 15 us per call on MI355X, so it is off by
 * default.  create returns MOE_ERR_UNSUPPORTED on a device without
 * cooperative launch.  Source: "FlyDSL Mono Kernels for High-Interactivity
 * LLM Serving in ATOM", section "What FlyDSL Provides" (enough cooperating
 * blocks must stay resident for progress).
 */
#define MOE_FLAG_COOPERATIVE 4u

/*
 * Weights, all device pointers, row-major and contiguous.  create() reads
 * them once (it re-lays the expert matrices out into the kernel's tile order
 * in memory the handle owns), so the caller may free them after create
 * returns.  B = bytes per row of K elements: K (FP8, MXFP8) or K / 2 (MXFP4).
 *   router_w    [E][H]               fp32
 *   router_bias [E]                  fp32, or NULL for no bias
 *   w13         [E+S][2I][B(H)]      expert codes; rows [0,I) gate, [I,2I) up
 *   s13         [E+S][2I][H/32]      scale of each 32 contiguous K elements:
 *                                    fp32 (FP8) or uint8 E8M0 (MX formats)
 *   w2          [E+S][H][B(I)]       expert codes (down projection)
 *   s2          [E+S][H][I/32]       fp32 or uint8 E8M0, as s13
 * Slot E (the last) is the shared expert when S = 1.  A weight's value is
 * decode(q) * scale; e4m3fn codes 0x7F/0xFF (NaN) must not occur.
 */
typedef struct moe_decode_weights {
  const float* router_w;
  const float* router_bias;
  const uint8_t* w13;
  const void* s13;
  const uint8_t* w2;
  const void* s2;
} moe_decode_weights;

/*
 * Optional copies of intermediate results (each pointer may be NULL; device
 * memory, written by the same kernel, valid once the run's stream reaches it):
 *   topk_idx     [T][K] int32  selected experts, score descending
 *   topk_w       [T][K] fp32   renormalised weights
 *   pair_rank    [T][K] int32  position of row t among the rows of expert
 *                              topk_idx[t][k] (tile = rank / 8, slot = rank % 8)
 *   expert_count [E]    int32  rows routed to each expert
 *   logits       [T][E] fp32   router logits including the bias
 */
typedef struct moe_decode_debug {
  int32_t* topk_idx;
  float* topk_w;
  int32_t* pair_rank;
  int32_t* expert_count;
  float* logits;
  /*
   * Per-workgroup timeline (profiling the waits).  trace is device memory of
   * int64 [trace_blocks][1 + trace_cap][4]; workgroups with index >=
   * trace_blocks record nothing.  Row 0 of a block: {kernel entry, exit,
   * items recorded, workgroups in the grid}; row 1 + i: {ticket | kind << 32,
   * ticket granted, inputs ready (after any wait), item done}.  Times are
   * the 100 MHz device wall clock.  kind: 0 router, 1 shared gate/up,
   * 2 top-k, 3 shared down, 4 routed gate/up, 5 routed down, 6 exit ticket,
   * 7 combine; 8 and 9 time the phases of the workgroup's own routing
   * (logits, top-k, placement); 12 follows a top-k item: {rounds of its
   * gather, ends of the first three rounds}.
   */
  int64_t* trace;
  int32_t trace_blocks;
  int32_t trace_cap;
  /*
   * Test control: nonzero makes every in-kernel wait of this run give up at its
   * first check, as if its deadline had passed.  The run then ends early with
   * MOE_ERR_TIMEOUT reported by moe_decode_check (y undefined); the next run on
   * the handle is unaffected.  0 for normal runs.
   */
  int32_t expire_waits;
  /*
   * [T][H] bf16: the normalised rows a pre-norm block run fed to the router
   * and the experts (moe_decode_run_block only; ignored by moe_decode_run).
   */
  uint16_t* norm_x;
} moe_decode_debug;

typedef struct moe_decode_handle moe_decode_handle;

/* Register: the ABI version this library implements (MOE_DECODE_ABI_VERSION). */
int32_t moe_decode_abi_version(void);

/*
 * Guard: MOE_OK if a handle created with cfg can run T rows, MOE_ERR_UNSUPPORTED
 * if the shape is outside the kernel's limits (the caller should fall back to
 * a general path), MOE_ERR_INVALID_ARG for a NULL cfg.  No device access.
 */
moe_status moe_decode_supported(const moe_decode_config* cfg, int32_t T);

/*
 * Build: allocate the handle's workspace (sized for cfg->max_tokens), copy the
 * router and re-lay the expert weights into tile order on device `device`.
 * Synchronous.  On success *out owns all of it until moe_decode_destroy.
 */
moe_status moe_decode_create(const moe_decode_config* cfg, const moe_decode_weights* w,
                             int32_t device, moe_decode_handle** out);

/*
 * Runtime: enqueue one layer call on hip_stream.  x and y are device pointers to
 * [T][H] bf16, 16-byte aligned, not overlapping; dbg may be NULL.  T = 0 is a
 * no-op; T > cfg.max_tokens gives MOE_ERR_UNSUPPORTED (the Guard's answer),
 * T < 0 MOE_ERR_INVALID_ARG, in both cases before any launch.
 * Asynchronous: no allocation, no host synchronisation, one kernel launch.
 * Runs on one handle must be ordered on one stream (they share the
 * workspace).
 *
 * Graph capture and replay: the launch carries no per-run state.  The run's
 * tag (checked by every hand-off inside the kernel) and its counter block
 * come from arrival counters in the handle's workspace that each launch
 * advances by a fixed amount, so a HIP graph that captured this call (or any
 * sequence of calls) can be replayed any number of times; each replay reads
 * x and writes y at the captured addresses, with the captured T.  Replays
 * must also be stream-ordered with every other run on the handle.  Source:
 * "SGLang's Low-Latency Mode Boosts DeepSeek-V4.1-Flash Speed by 1.56x on
 * AMD", section "AMD keeps the layer resident" (decode under HIP graphs).
 * Tags repeat after 2^32 - 1 runs of a handle; a hand-off word that no run
 * wrote for exactly that many runs would then pass as current.
 *
 * A wait that passes the deadline makes the kernel exit early (y is then
 * undefined) and is reported by moe_decode_check.
 */
moe_status moe_decode_run(moe_decode_handle* h, const void* x, int32_t T, void* y,
                          const moe_decode_debug* dbg, void* hip_stream);

/*
 * moe_decode_run with no workspace of the handle's: for callers that cannot
 * allocate device memory at any point of their path (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc) and want the
 * per-run scratch (counters, logits, top-k, h and expert outputs) to come
 * from memory the library already holds.  Same arguments, layouts, results
 * and errors as moe_decode_run; the handle still supplies the weights.
 *
 * The workspace is one array of 16 MiB in the library's code object, one
 * copy per GPU, held until the process ends; the call allocates and frees
 * nothing.  A run needs 4 * T * (K + S) * (I' + 2 H) bytes of h and output
 * scratch (I' = I rounded up to 64) plus 0.6 to 1 MiB of counters and
 * logits: at H 4096, I 512, K 8, S 1 that allows T <= 49.  A larger run
 * returns MOE_ERR_UNSUPPORTED before any device work.  Every call on a GPU, from any handle, shares that GPU's
 * array and keeps its contents for the next: the array's own run tags and
 * counters keep successive calls apart, but calls that overlap in time on
 * one GPU (two streams, two threads) race and must not be issued.  A
 * deadline failure sets the array's status word; moe_decode_check on the
 * same handle reports and clears it, and until then every call on that GPU
 * that waits gives up early.
 */
moe_status moe_decode_run_static(moe_decode_handle* h, const void* x, int32_t T, void* y,
                                 const moe_decode_debug* dbg, void* hip_stream);

/*
 * Pre-norm block form of the layer: the RMSNorm that feeds the MoE input and
 * the residual add after the combine, fused into the same single launch.
 * Sources: "SGLang's Low-Latency Mode Boosts DeepSeek-V4.1-Flash Speed by
 * 1.56x on AMD", section "AMD keeps the layer resident" (the MoE input is
 * normalised inside the resident kernel and each row is handed on to the
 * router and experts as soon as it is ready); "Beyond Day-0: Optimizing
 * DeepSeek-V4.1 Flash in SGLang", section 2.1 (the layer's output combined
 * into the next layer's input right after the MoE, without extra passes).
 *
 * set_input_norm: the RMSNorm weight gamma (device pointer, [H] fp32, copied:
 * the caller may free it on return) and epsilon (finite, > 0).  The first call
 * allocates the handle's normalised-row buffer ([max_tokens][H] bf16) and row
 * ready words; later calls replace the weight.  Synchronous: waits for the
 * handle's last run first.  MOE_ERR_INVALID_ARG for a NULL pointer or a bad
 * epsilon, MOE_ERR_OUT_OF_MEMORY / MOE_ERR_HIP on device errors.
 */
moe_status moe_decode_set_input_norm(moe_decode_handle* h, const float* norm_w, float eps);

/*
 * run_block: like moe_decode_run, but x [T][H] bf16 is the block input (the
 * residual stream) and
 *   xn[t] = bf16( x[t][h] * gamma[h] / sqrt(mean_h x[t][h]^2 + eps) )   (fp32 arithmetic)
 *   y[t]  = bf16( x[t] + o_shared[t] + sum_k w[t][k] * o_{idx[t][k]}[t] )  with the
 *           layer above run on xn (routing included): one rounding of the sum.
 * Each workgroup normalises rows in the kernel's prologue; a reader of a row
 * waits only for that row's ready word.  Same argument rules, ordering and
 * error reporting as moe_decode_run; MOE_ERR_INVALID_ARG if set_input_norm has
 * not been called.  dbg->norm_x, when set, receives xn.
 */
moe_status moe_decode_run_block(moe_decode_handle* h, const void* x, int32_t T, void* y,
                                const moe_decode_debug* dbg, void* hip_stream);

/*
 * Clipped SwiGLU, for the runs enqueued after this call (both forms):
 *   h = bf16( silu(min(g, L)) * clamp(u, -L, L) )
 * for every expert, routed and shared, with the rounding of h unchanged.
 * Source: "Beyond Day-0: Optimizing DeepSeek-V4.1 Flash in SGLang", section
 * 3.1 (fused clipped SwiGLU that keeps the original intermediate rounding;
 * the page gives neither the formula nor the limit, so the caller supplies L).
 * L > 0; L = +inf (the default) turns clipping off.  MOE_ERR_INVALID_ARG
 * for a NULL handle, L <= 0 or NaN.  No device work.
 */
moe_status moe_decode_set_swiglu_limit(moe_decode_handle* h, float limit);

/*
 * Kernel timing, for runs enqueued after this call (all three run forms):
 * with two events set, each run's single kernel launch records start_event
 * when the kernel starts and stop_event when it ends (hipExtLaunchKernel's
 * launch events: the times of the kernel itself, not of event records
 * queued around it).  Source: "SGLang's Low-Latency Mode Boosts
 * DeepSeek-V4.1-Flash Speed by 1.56x on AMD", section "AMD keeps the layer
 * resident" (the layer's latency per call, as the pages report it).
 * start_event and stop_event are hipEvent_t handles the caller created on the
 * handle's device and keeps alive while they are set; both NULL turns timing
 * off (the default).  MOE_ERR_INVALID_ARG for a NULL handle or exactly one
 * NULL event.  A run with events set on a handle created with
 * MOE_FLAG_COOPERATIVE returns MOE_ERR_UNSUPPORTED (a cooperative launch
 * takes no events), and so does a run with events set on a stream that is
 * capturing a graph (launch events time eager runs only).  No device work.
 */
moe_status moe_decode_set_launch_events(moe_decode_handle* h, void* start_event, void* stop_event);

/*
 * Wait for the last run's stream and report its in-kernel status:
 * MOE_OK, or MOE_ERR_TIMEOUT if a deadline fired (the status is then cleared,
 * so the next run starts clean).
 */
moe_status moe_decode_check(moe_decode_handle* h);

/* Free everything the handle owns (synchronises its device first). NULL is a no-op. */
void moe_decode_destroy(moe_decode_handle* h);

/* Static description of a status code. */
const char* moe_decode_status_string(moe_status s);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DECODE_H */
