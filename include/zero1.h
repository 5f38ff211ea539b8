/*
 * zero1.h -- C ABI of libzero1.so: one data-parallel rank's ZeRO-1 optimizer
 * step on one MI355X (gfx950), in hand-written HIP kernels.
 *
 * The step, for rank r of W data-parallel ranks, on r's contiguous shard of
 * the flat parameter vector (elements [begin, begin+len)):
 *   1. reduce    g = (sum over w = 0..W-1 of the bf16 gradient of replica w) / W,
 *                fp32 accumulation in rank order                   (zero1_shard_reduce)
 *   2. norm      this rank's sum of g^2 (fp64); the global norm is the square
 *                root of the rank partials added in rank order      (zero1_grad_norm)
 *   3. clip      if norm > max_norm, g *= max_norm / norm
 *   4. AdamW     m, v, update, then decoupled decay on the fp32 master
 *   5. bf16      the forward-pass parameter is the nearest-even bf16 of the
 *                new master                                          (3-5: zero1_adamw_step)
 *   1-5 fused over a ragged per-tensor list: zero1_mta_plan + zero1_mta_step.
 *
 * Sources (web pages; section names as they appear on each page):
 *   "并行训练" (notes.cassieliang.com):
 *       "一张卡上装了什么：混合精度与 AdamW" -- fp32 master, bf16 copy each step,
 *           AdamW code with the folded bias correction and decay after the update,
 *           16 B/param (12 B with bf16 m, v);
 *       "训练循环与 checkpoint" -- global L2-norm clipping of all gradients at max_norm,
 *           optimizer state (m, v, t) and t restarting at 1;
 *       "卡和卡怎么说话：集合通信" -- reduce-scatter: rank i receives the sum of block i;
 *       "数据并行与 ZeRO：按 batch 切，再把状态切碎" -- DDP averages replica gradients;
 *           ZeRO-1 reduce-scatters the gradients and updates only the own 1/W slice.
 *   "Stanford CS336 第八讲精读：并行（下）" sec. 五 (four-rank reduce example) and
 *       sec. 七 (all-reduce with AVG of each gradient).
 *   "Stanford CS336 第七讲精读：并行（上）" sec. 5.2 (ZeRO stage 1 steps).
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns every
 *     buffer; the library allocates no device memory.  All work is enqueued on
 *     `stream` (a hipStream_t, NULL = the null stream) and nothing synchronizes:
 *     results are ready when the stream reaches them, and a fault inside a kernel
 *     surfaces at the caller's next synchronization.  Setting the environment
 *     variable ZERO1_SYNC_CHECK=1 makes each call synchronize and check (tests;
 *     on a stream under graph capture it checks the launches only).
 *   - Graph capture: apart from zero1_mta_plan (a synchronous table upload),
 *     the entry points only launch kernels
 *     (no memset, copy or synchronization), so their work can be captured into
 *     a HIP graph.  The fp32 scalars derived from zero1_hparams -- the step t
 *     included -- are kernel arguments and are frozen into the graph, unless
 *     hp->device_scalars points them at device memory that the caller
 *     rewrites before each replay (zero1_step_scalars_derive).
 *   - bf16 values are passed as uint16_t bit patterns; fp32 as float.
 *   - Arguments are validated on the host before anything is launched; a
 *     rejected call launches nothing and returns an error status, with a
 *     message from zero1_last_error() (per host thread).
 *   - len == 0 is a valid no-op.
 *   - Non-finite values are not errors: they propagate by IEEE rules and
 *     zero1_norm_info.nonfinite is set when the norm is NaN or infinite.
 *   - Arithmetic: every fp32 operation is a single IEEE binary32 operation
 *     rounded to nearest-even (no fused multiply-add, correctly rounded divide
 *     and square root, subnormals kept); sums of squares are fp64; scalars
 *     derived from the hyper-parameters are formed in fp64 on the host and
 *     rounded once to fp32.
 *   - Calls that share a workspace must not overlap in time (same stream, or
 *     ordered by the caller).
 *   - Unknown flag bits are rejected (EINVAL); flags that do not concern an
 *     entry point are ignored by it, so one flag set can be passed to every
 *     call of a step.
 */
#ifndef ZERO1_H
#define ZERO1_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZERO1_ABI_VERSION 4
#define ZERO1_MAX_W 128          /* largest number of replicas per call */

typedef enum zero1_status {
    ZERO1_OK = 0,
    ZERO1_EINVAL = 1,            /* bad argument (message says which)            */
    ZERO1_EWORKSPACE = 2,        /* workspace NULL, too small or misaligned       */
    ZERO1_EHIP = 3,              /* a HIP runtime call failed (message has it)    */
    ZERO1_ENOTSUPPORTED = 4      /* current device is not gfx950                  */
} zero1_status;

/* flags (bitwise OR) */
#define ZERO1_SUM_ONLY     0x1u  /* reduce: keep the sum, do not divide by W        */
#define ZERO1_MV_BF16      0x2u  /* m and v are stored as bf16 (uint16_t)           */
#define ZERO1_RECOMPUTE_G  0x4u  /* step: the update re-reads the W slices          */
#define ZERO1_STORE_G      0x8u  /* step: the reduce stores fp32 g in the workspace
                                    and the update reads it back.  Neither design
                                    flag: STORE_G when W > 4 (fewer bytes than
                                    re-reading the slices), else RECOMPUTE_G.     */
/* 0x10u is unused (rejected as an unknown flag). */

/* Compatibility variants (not the pages' step; off by default):
 *   ZERO1_DECAY_FIRST  decay the master before the Adam update, the order
 *                      "并行训练" ("一张卡上装了什么：混合精度与 AdamW") attributes to
 *                      torch.optim.AdamW (differs by ~lr^2*lambda per step);
 *   ZERO1_CLIP_EPS     torch.nn.utils.clip_grad_norm_'s convention: coefficient
 *                      max_norm / (norm + 1e-6), applied when it is below 1;
 *   ZERO1_G_BF16       the reduced gradient is rounded to the nearest bf16
 *                      before the norm and the update (what a reduce-scatter
 *                      delivering bf16 hands to the optimizer); applies where
 *                      the library forms g (a g passed in is used as is). */
#define ZERO1_DECAY_FIRST  0x20u
#define ZERO1_CLIP_EPS     0x40u
#define ZERO1_G_BF16       0x80u

/* AdamW and clipping hyper-parameters of one step (host struct). */
typedef struct zero1_hparams {
    double lr;              /* >= 0                                             */
    double beta1;           /* in [0, 1)                                        */
    double beta2;           /* in [0, 1)                                        */
    double eps;             /* >= 0                                             */
    double weight_decay;    /* >= 0; decay factor 1 - lr*weight_decay           */
    double max_norm;        /* > 0; +inf disables clipping                      */
    int64_t step;           /* t >= 1 (bias correction uses beta^t)             */
    /* NULL, or the DEVICE address (8-byte aligned) of a zero1_step_scalars
     * that the kernels read when they run, in place of the values derived
     * from the fields above (which are then neither validated nor read): for a
     * step captured into a HIP graph and replayed with a new t or learning
     * rate each iteration (fill it with zero1_step_scalars_derive and copy it
     * to the device before each replay). */
    const void* device_scalars;
} zero1_hparams;

/* The per-step values every step call derives from zero1_hparams: each fp32
 * scalar is formed in fp64 and rounded once ("并行训练", mixed precision and
 * AdamW: step_size = lr*sqrt(1-beta2^t)/(1-beta1^t), decay = 1-lr*weight_decay),
 * and the clip threshold.  40 bytes. */
typedef struct zero1_step_scalars {
    float beta1, beta2;
    float one_minus_beta1, one_minus_beta2;
    float eps;
    float step_size;
    float decay;
    float reserved;
    double max_norm;
} zero1_step_scalars;

/* Fill *out (host memory) from *hp exactly as the step calls do (its
 * device_scalars field is ignored).  EINVAL for the same hyper-parameters the
 * step calls reject. */
zero1_status zero1_step_scalars_derive(const zero1_hparams* hp, zero1_step_scalars* out);

/* Result of the clip stage, written to device memory by the step calls. */
typedef struct zero1_norm_info {
    double sumsq_total;     /* sum over ranks of the partial sums of squares    */
    double norm;            /* sqrt(sumsq_total), fp64                          */
    float clip_coef;        /* fp32(max_norm / norm) when clip, else 1          */
    int32_t clip;           /* 1 when norm > max_norm                           */
    int32_t nonfinite;      /* 1 when norm is NaN or infinite                   */
    int32_t reserved;
} zero1_norm_info;

/* One tensor's part of this rank's shard (multi-tensor front end).
 * Elements [shard_offset, shard_offset + numel) of the shard belong to it;
 * its state and bf16 parameter are stored at the four pointers. */
typedef struct zero1_piece {
    int64_t numel;          /* > 0                                              */
    int64_t shard_offset;   /* position of its first element inside the shard   */
    uint16_t* param_bf16;   /* numel bf16, written                              */
    float* master;          /* numel fp32, read and written                     */
    void* m;                /* numel fp32 (bf16 with ZERO1_MV_BF16), r/w        */
    void* v;                /* numel fp32 (bf16 with ZERO1_MV_BF16), r/w        */
} zero1_piece;

/* A validated piece list uploaded into device memory by zero1_mta_plan.
 * Plain data owned by the caller; valid as long as the table memory is. */
typedef struct zero1_plan {
    void* table;            /* device: piece descriptors + chunk table          */
    int64_t shard_len;      /* sum of the pieces' numel                          */
    int32_t n_pieces;
    int32_t n_chunks;
    int32_t chunk_elems;    /* elements per chunk (pieces are cut into chunks)  */
    uint32_t flags;         /* ZERO1_MV_BF16 as given to zero1_mta_plan          */
    int32_t aligned;        /* 1 when every piece allows 16-byte vector access  */
    int32_t reserved;
} zero1_plan;

/* ---------------------------------------------------------------- misc */
int zero1_abi_version(void);
/* Message of the last failing call on this host thread ("" if none). */
const char* zero1_last_error(void);
const char* zero1_status_string(int status);

/* Host-only: rank's shard of an n_total-element flat vector cut into W
 * contiguous shards of S = ceil(n_total / W) elements (the last may be
 * short or empty): *begin = min(rank*S, n_total), *len = its length.
 * Rank i holding block i is the reduce-scatter convention of "并行训练",
 * section "卡和卡怎么说话：集合通信". */
zero1_status zero1_shard_range(int64_t n_total, int W, int rank,
                               int64_t* begin, int64_t* len);

/* Bytes of workspace needed by the flat entry points for a shard of `len`
 * elements (flags as passed to the call: ZERO1_STORE_G adds 4*len). */
size_t zero1_workspace_bytes(int64_t len, int W, uint32_t flags);

/* ---------------------------------------------------------------- step 1 (+2)
 * Reduce-scatter arithmetic on one rank's shard.
 * ("卡和卡怎么说话：集合通信" reduce-scatter; "Stanford CS336 第八讲精读" sec. 七 AVG.)
 *   grads     (host) array of W device pointers; grads[w] is replica w's flat
 *             gradient (bf16), indexed by flat position.
 *   W         1..ZERO1_MAX_W replicas.
 *   begin,len the shard [begin, begin+len) of the flat vector.
 *   flags     ZERO1_SUM_ONLY: output the sum instead of the average;
 *             ZERO1_G_BF16: round g to bf16 (compatibility variant).
 *   g_out     len fp32 outputs g[k] for flat element begin+k, or NULL.
 *             Must not overlap any gradient range.
 *   sumsq_out one double: sum of g[k]^2 over the shard (fp64, fixed order,
 *             deterministic), or NULL.  At least one of g_out, sumsq_out.
 *   ws        workspace of zero1_workspace_bytes(len, W, 0) bytes, 256-byte
 *             aligned (needed only when sumsq_out != NULL).
 * Accumulation: s = widen(G_0); s = s + widen(G_w) for w = 1..W-1; g = s / W. */
zero1_status zero1_shard_reduce(const uint16_t* const* grads, int W,
                                int64_t begin, int64_t len, uint32_t flags,
                                float* g_out, double* sumsq_out,
                                void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- step 2
 * This rank's partial of the global L2 norm ("训练循环与 checkpoint": the norm of
 * all gradients taken as one vector): *sumsq_out = sum of g[k]^2, k < len,
 * squares exact in fp64, fp64 adds in a fixed order (deterministic).
 *   g         len fp32 values.   ws: zero1_workspace_bytes(len, 1, 0) bytes. */
zero1_status zero1_grad_norm(const float* g, int64_t len, double* sumsq_out,
                             void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- steps 3-5
 * Clip and AdamW on a flat shard, then the bf16 copy
 * ("一张卡上装了什么：混合精度与 AdamW"; clip from "训练循环与 checkpoint").
 *   g           len fp32 reduced gradients, or NULL to recompute them from
 *               grads/W/begin (same arithmetic as zero1_shard_reduce).
 *   grads,W,begin  as for zero1_shard_reduce; ignored when g != NULL.
 *   master      len fp32, updated in place.
 *   m, v        len fp32 (or bf16 with ZERO1_MV_BF16), updated in place;
 *               zero before the first step.
 *   param_bf16  len bf16 outputs: nearest-even bf16 of the new master.
 *   hp          (host) hyper-parameters; hp->step is t (or hp->device_scalars).
 *   rank_sumsq  n_ranks doubles: every rank's partial sum of squares (this
 *               rank's included), added in rank order for the global norm.
 *   flags       ZERO1_MV_BF16; ZERO1_SUM_ONLY and ZERO1_G_BF16 (with g == NULL);
 *               ZERO1_DECAY_FIRST, ZERO1_CLIP_EPS (compatibility variants).
 *   info_out    one zero1_norm_info (device) or NULL; written even when len == 0.
 * Needs no workspace: every workgroup forms the norm from rank_sumsq itself.
 * Per element, with c the clip coefficient when clipping:
 *   g' = g*c;  m = b1*m + a1*g';  v = b2*v + a2*(g'*g');
 *   p = p - sigma*(m / (sqrt(v) + eps));  p = p*delta;  param = bf16(p)
 * where b1 = fp32(beta1), a1 = fp32(1-beta1), b2, a2 likewise, eps = fp32(eps),
 * sigma = fp32(lr*sqrt(1-beta2^t)/(1-beta1^t)), delta = fp32(1-lr*weight_decay).
 * The state buffers and param_bf16 must not overlap each other or g. */
zero1_status zero1_adamw_step(const float* g, const uint16_t* const* grads,
                              int W, int64_t begin, int64_t len,
                              float* master, void* m, void* v,
                              uint16_t* param_bf16, const zero1_hparams* hp,
                              const double* rank_sumsq, int n_ranks,
                              uint32_t flags, zero1_norm_info* info_out,
                              void* stream);

/* ---------------------------------------------------------------- fused step
 * Multi-tensor apply over a ragged per-tensor list (the parameter list the
 * training loop hands to clipping and the optimizer, "训练循环与 checkpoint").
 *
 * zero1_mta_table_bytes: device bytes the plan table needs for this list.
 * zero1_mta_plan: validates the pieces (numel > 0; together they tile
 *   [0, shard_len) exactly, in any order; no two buffers overlap), cuts them
 *   into chunks and copies the table into `table` (device, 256-byte aligned,
 *   table_bytes long).  Synchronous: call once per tensor-list layout and
 *   reuse the plan for every step.  `flags` may hold ZERO1_MV_BF16.
 * zero1_mta_workspace_bytes: step workspace for this plan and W.
 * zero1_mta_reduce: steps 1-2 for this rank: reduces the shard's gradient
 *   slices (grads, W, begin as for zero1_shard_reduce) and writes this rank's
 *   partial sum of squares to *sumsq_out (device).  With ZERO1_STORE_G the
 *   fp32 g is kept in the workspace for zero1_mta_update.
 * zero1_mta_update: steps 3-5: forms the global norm from rank_sumsq
 *   (n_ranks doubles, added in rank order), clips, and updates every piece.
 *   Must get the same grads, W, begin, plan, flags and workspace as the
 *   zero1_mta_reduce it follows.  A multi-GPU caller exchanges the ranks'
 *   partials between the two calls (one double per rank: the only data the
 *   step needs from other ranks once the gradients are reduced).
 * zero1_mta_step: the whole step (1-5) for rank my_rank when the other
 *   ranks' partials are already in rank_sumsq; entry my_rank is overwritten
 *   with this rank's partial: zero1_mta_reduce with sumsq_out =
 *   rank_sumsq + my_rank followed by zero1_mta_update.
 *   flags: ZERO1_STORE_G or ZERO1_RECOMPUTE_G (neither:
 *   the library picks, see zero1_mta_design), ZERO1_SUM_ONLY and the
 *   compatibility variants ZERO1_DECAY_FIRST, ZERO1_CLIP_EPS, ZERO1_G_BF16
 *   (ZERO1_MV_BF16 comes from the plan).
 * Every design gives bit-identical master, m, v and params for the same
 * clip coefficient; this rank's fp64 partial depends on the launch shape
 * only in its last bits (different fixed summation trees). */
size_t zero1_mta_table_bytes(const zero1_piece* pieces, int n_pieces);
zero1_status zero1_mta_plan(const zero1_piece* pieces, int n_pieces,
                            uint32_t flags, void* table, size_t table_bytes,
                            zero1_plan* plan_out);
size_t zero1_mta_workspace_bytes(const zero1_plan* plan, int W, uint32_t flags);
zero1_status zero1_mta_reduce(const uint16_t* const* grads, int W, int64_t begin,
                              const zero1_plan* plan, double* sumsq_out,
                              uint32_t flags, void* ws, size_t ws_bytes, void* stream);
zero1_status zero1_mta_update(const uint16_t* const* grads, int W, int64_t begin,
                              const zero1_plan* plan, const zero1_hparams* hp,
                              const double* rank_sumsq, int n_ranks, uint32_t flags,
                              zero1_norm_info* info_out, void* ws, size_t ws_bytes,
                              void* stream);
/* ---------------------------------------------------------------- buckets
 * Incremental reduction while backward still runs (reduce each bucket of
 * gradients as soon as it is produced, as ZeRO stage 2 does: "并行训练",
 * "数据并行与 ZeRO：按 batch 切，再把状态切碎"; "Stanford CS336 第七讲精读" 5.3), so
 * that only the update is left on the optimizer step's critical path:
 *   for each bucket k (any order):  zero1_mta_reduce_range(..., lo_k, hi_k,
 *                                     parts + k, ZERO1_STORE_G, ws, ...)
 *   zero1_partials_sum(parts, n_buckets, rank_sumsq + my_rank)
 *   (multi-GPU: exchange rank_sumsq)
 *   zero1_mta_update(..., ZERO1_STORE_G, ws, ...)
 * The buckets must cover the shard exactly once before the update. Every call
 * on one workspace reuses its partials area: issue them in order on one stream
 * (calls on different streams with the same workspace race).
 *
 * zero1_mta_reduce_range: steps 1-2 for shard elements [lo, hi): grads[w][k]
 *   is replica w's gradient of shard element lo + k (bf16, device); g for the
 *   range is stored in the workspace (sized by zero1_mta_workspace_bytes(plan,
 *   W, ZERO1_STORE_G)) and the range's fp64 sum of squares goes to *sumsq_out.
 *   flags: ZERO1_SUM_ONLY, ZERO1_G_BF16 (RECOMPUTE_G: EINVAL).
 * zero1_partials_sum: *sum_out = parts[0] + parts[1] + ... (n <= 8192 doubles,
 *   device), added in a fixed order (deterministic). */
zero1_status zero1_mta_reduce_range(const uint16_t* const* grads, int W,
                                    const zero1_plan* plan, int64_t lo, int64_t hi,
                                    double* sumsq_out, uint32_t flags, void* ws,
                                    size_t ws_bytes, void* stream);
zero1_status zero1_partials_sum(const double* parts, int n, double* sum_out,
                                void* stream);

/* Which design zero1_mta_step would run for these arguments on the current
 * device: ZERO1_STORE_G or ZERO1_RECOMPUTE_G; 0 when the arguments are
 * invalid or both design flags are given. */
int zero1_mta_design(const uint16_t* const* grads, int W, int64_t begin,
                     const zero1_plan* plan, uint32_t flags);
zero1_status zero1_mta_step(const uint16_t* const* grads, int W, int64_t begin,
                            const zero1_plan* plan, const zero1_hparams* hp,
                            double* rank_sumsq, int n_ranks, int my_rank,
                            uint32_t flags, zero1_norm_info* info_out,
                            void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- no allocation
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  zero1_mta_step_static is zero1_mta_step (same arguments, same
 * kernels, same results bit for bit) with its workspace in a static device
 * array of the library instead of a caller's buffer.
 *   - The array holds the workspace of a store-g step of up to
 *     ZERO1_STATIC_MAX_G_ELEMS shard elements (64 MiB of fp32 g plus 64.25 KiB
 *     of norm partials and info); every GPU the library runs on holds its own
 *     copy until the process ends.  A shard whose step needs more (the
 *     store-g design, chosen by default when W > 4, with a longer shard) is
 *     rejected with ZERO1_EINVAL before anything is launched; with
 *     ZERO1_RECOMPUTE_G any shard length fits.
 *   - The array's device address is looked up once per device, on the first
 *     call with that device current.  That first lookup is when the HIP
 *     runtime loads the code object holding the array onto the device (and
 *     maps its memory); later calls allocate nothing and only launch
 *     kernels, so a caller that captures the step into a graph makes one call
 *     on each device before capturing.
 *   - Each call writes every byte of the array it reads before reading it,
 *     so nothing needs to start at zero.  All calls on one GPU share its
 *     array: calls that overlap in time on one GPU (different streams, or
 *     several host threads) race and give wrong results.  The caller orders
 *     them (one stream, or events between streams).
 *   - The caller still owns the gradients, the plan table, the state
 *     buffers, rank_sumsq and info_out. */
#define ZERO1_STATIC_MAX_G_ELEMS 16777216
zero1_status zero1_mta_step_static(const uint16_t* const* grads, int W, int64_t begin,
                                   const zero1_plan* plan, const zero1_hparams* hp,
                                   double* rank_sumsq, int n_ranks, int my_rank,
                                   uint32_t flags, zero1_norm_info* info_out,
                                   void* stream);

/* ---------------------------------------------------------------- timing
 * Kernel-scoped timing of the step calls, for profiling.  After this call,
 * the first kernel launched by the calling thread's next call of a step entry
 * point (zero1_shard_reduce, zero1_grad_norm, zero1_adamw_step,
 * zero1_mta_reduce, zero1_mta_reduce_range, zero1_partials_sum,
 * zero1_mta_update, zero1_mta_step) records start_event when its execution
 * begins and stop_event when it ends; either may be NULL.  The stamps come
 * from that kernel's own dispatch (hipExtLaunchKernel), with no marker packets
 * around it, so hipEventElapsedTime(start, stop) is the kernel's duration as a
 * kernel trace reports it.  Which kernel is first: the reduce of the reduce
 * calls and of zero1_mta_step, the update of zero1_adamw_step
 * and zero1_mta_update, the sum of squares of zero1_grad_norm, the partials
 * sum of zero1_partials_sum (and of an empty zero1_shard_reduce /
 * zero1_grad_norm).  The request is dropped when that call returns, whether
 * or not it launched anything; a later request replaces an earlier one.
 *
 * The events are created and owned by the caller (hipEventCreate, timing
 * enabled, on the device the step runs on) and must outlive the kernel.
 * Errors surface in the step call: ZERO1_EHIP when its stream is being
 * captured into a graph (kernel-scoped events cannot be captured).
 * Host only; always ZERO1_OK. */
zero1_status zero1_time_next_launch(void* start_event, void* stop_event);

/* ---------------------------------------------------------------- arena
 * Placement of one rank's optimizer arrays inside one device allocation (the
 * arena).  On MI355X the HBM throughput of a kernel that streams several
 * arrays at once depends on how far apart the arrays are: the update's five
 * streams (the reduced gradient g -- or gradient slice 0 when g is recomputed
 * --, master, m, v and the shard's bf16 parameters) move 5.7-5.8 TB/s when
 * they are 24 GiB or more apart and 4.5-5.0 TB/s when they are 12 GiB or
 * less apart (1 GiB streams, a kernel that only moves them); on the step, the
 * Llama-7B/8 shard's update moves 6.1-6.2 TB/s in the arena against 5.0-6.0
 * TB/s with one allocation per array (that placement varies between
 * processes), and the whole 7e9-parameter W=1 step takes 33.7-33.8 ms
 * against 39.5-39.9.  The planner puts those five at one spacing D
 * (40 GiB, or more when an array is larger, or less when `capacity` is short)
 * and packs the remaining gradient buffers after the parameter buffer.  The
 * gaps between the spaced arrays are not used by the library: the caller may
 * place its other tensors there.
 *
 * Request: shard_len S >= 1; W in 1..ZERO1_MAX_W gradient buffers of
 * grad_elems bf16 each, this rank's shard starting at element grad_offset of
 * each (grad_offset = 0, grad_elems = S for buffers that hold only the shard;
 * the shard's begin and N for full replicas); the flat bf16 parameter buffer
 * of param_elems elements with the shard starting at param_offset; flags:
 * ZERO1_MV_BF16 (2-byte m, v) and the design (ZERO1_STORE_G, ZERO1_RECOMPUTE_G,
 * or neither for the one zero1_mta_step picks); capacity: the largest arena
 * the caller can allocate.
 *
 * Layout (byte offsets from the arena base, which must be 2 MiB aligned): the
 * workspace (ws_bytes = zero1_mta_workspace_bytes for that design; holds g),
 * master, m, v, the parameter buffer and each gradient buffer.  Every spaced
 * array's shard range starts on a 2 MiB boundary; the other buffers start on
 * 2 MiB boundaries.  Arrays never overlap; total_bytes <= capacity.
 * ZERO1_EINVAL when the request is invalid or even the packed layout (spacing
 * = the smallest that keeps the arrays apart) exceeds capacity.  Host only:
 * no device call. */
typedef struct zero1_arena_request {
    int64_t shard_len;
    int W;
    int64_t grad_elems;
    int64_t grad_offset;
    int64_t param_elems;
    int64_t param_offset;
    uint32_t flags;
    size_t capacity;
} zero1_arena_request;

typedef struct zero1_arena_layout {
    size_t total_bytes;
    size_t spacing;            /* D actually used */
    size_t ws, ws_bytes;
    size_t master, m, v;
    size_t params;             /* start of the parameter buffer (element 0) */
    size_t grads[ZERO1_MAX_W]; /* start of each gradient buffer (element 0) */
} zero1_arena_layout;

#define ZERO1_ARENA_SPACING ((size_t)40 << 30)   /* preferred spacing D */

zero1_status zero1_arena_plan(const zero1_arena_request* req, zero1_arena_layout* out);

#ifdef __cplusplus
}
#endif

#endif /* ZERO1_H */
