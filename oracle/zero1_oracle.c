/*
 * zero1_oracle.c -- plain CPU oracle for one data-parallel rank's ZeRO-1
 * optimizer step.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * bench's CPU-baseline leg use it to decide what the GPU library must produce.
 * The product path never calls it, and it shares no code, header or table with
 * the GPU library.
 *
 * Pages cited (all read as data, restated here in my own words):
 *   [PT]  "并行训练" (parallel-training notes, notes.cassieliang.com)
 *         sec. "一张卡上装了什么：混合精度与 AdamW"   (mixed precision + AdamW)
 *         sec. "训练循环与 checkpoint"               (training loop, clipping)
 *         sec. "卡和卡怎么说话：集合通信"             (collectives)
 *         sec. "数据并行与 ZeRO：按 batch 切，再把状态切碎" (DDP / ZeRO)
 *   [L8]  "Stanford CS336 第八讲精读：并行（下）" sec. 五 (four-rank experiment),
 *         sec. 七 (data parallel: all-reduce AVG of every gradient)
 *   [L7]  "Stanford CS336 第七讲精读：并行（上）" sec. 5.1 (16 B/param bill),
 *         sec. 5.2 (ZeRO stage 1 algorithm)
 *
 * Precision contract: every float operation below is one IEEE-754 binary32
 * operation rounded to nearest-even (build with -O2 -fno-fast-math
 * -ffp-contract=off, x86-64 SSE, no FMA contraction).  Sums of squares are
 * fp64.  Subnormals are kept (the entry points refuse to run if the x87/SSE
 * control word flushes them).
 *
 * Parity pins: each function is pinned by tests under tests/ (worked examples,
 * closed forms, exact-rational re-evaluation, library RNE).  Nothing here is
 * "parity unpinned" except the exact 100-step AdamW-vs-torch figure on [PT]
 * (the page gives neither its quadratic nor its hyper-parameters; only the
 * order of magnitude is pinned, under a stated reading of both).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>
#include <xmmintrin.h>

#define ORACLE_NORM_BLOCK 65536 /* fixed block of the fp64 sum of squares */

/* ---------------------------------------------------------------------- */
/* Number formats                                                          */
/* ---------------------------------------------------------------------- */

/* bf16 -> fp32 is exact: a bf16 value is the upper half of a binary32. */
static float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t f32_bits(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    return u;
}

/*
 * fp32 -> bf16, round to nearest, ties to even ([PT] mixed precision: the
 * fp32 master is copied to bf16 for the forward pass every step).
 * Written from the definition: the two bf16 neighbours of x are the value
 * with the low 16 bits cleared (toward zero) and the next bf16 away from
 * zero; pick the nearer one, and on an exact tie the one with an even last
 * bit.  Distances are exact in double.  Overflow follows IEEE: the neighbour
 * above the largest finite bf16 is 2^128, which then becomes infinity.
 * NaN stays NaN (quiet, sign kept); +-0 and +-inf are unchanged.
 */
uint16_t oracle_f32_to_bf16(float x)
{
    uint32_t u = f32_bits(x);
    uint32_t mag = u & 0x7fffffffu;
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (mag > 0x7f800000u) /* NaN */
        return (uint16_t)((u >> 16) | 0x0040u);
    if (mag == 0x7f800000u) /* infinity */
        return (uint16_t)(u >> 16);
    uint32_t lo_bits = mag & 0xffff0000u;             /* toward zero   */
    uint32_t hi_bits = lo_bits + 0x00010000u;         /* away from zero */
    double ax = fabs((double)x);
    double lo = (double)bf16_to_f32((uint16_t)(lo_bits >> 16));
    double hi = (hi_bits == 0x7f800000u) ? ldexp(1.0, 128)
                                          : (double)bf16_to_f32((uint16_t)(hi_bits >> 16));
    double d_lo = ax - lo;
    double d_hi = hi - ax;
    uint32_t pick;
    if (d_lo < d_hi)
        pick = lo_bits;
    else if (d_hi < d_lo)
        pick = hi_bits;
    else /* exact tie: even last bit of the bf16 significand */
        pick = ((lo_bits >> 16) & 1u) ? hi_bits : lo_bits;
    return (uint16_t)(sign | (uint16_t)(pick >> 16));
}

float oracle_bf16_to_f32(uint16_t h) { return bf16_to_f32(h); }

void oracle_f32_to_bf16_array(const float* x, uint16_t* out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f32_to_bf16(x[i]);
}

/* 1 when the SSE control word keeps subnormals (FTZ bit 15 and DAZ bit 6 off). */
int oracle_fp_env_ok(void)
{
    unsigned int csr = _mm_getcsr();
    return ((csr & 0x8000u) == 0) && ((csr & 0x0040u) == 0);
}

/* ---------------------------------------------------------------------- */
/* O1: the reduce-scatter arithmetic on this rank's shard                  */
/* ---------------------------------------------------------------------- */

/*
 * Rank r of a reduce-scatter receives, at each position of its own slice, the
 * sum over all W ranks of that position ([PT] collectives: rank i gets the sum
 * of the i-th block; [L8] sec. 五 shows [0,1,2,3]+rank reducing to 6,10,14,18).
 * DDP divides that sum by W ([L8] sec. 七: all-reduce with AVG; [PT] DDP: the
 * average of the replica gradients equals the full-batch gradient).
 *
 * Reading adopted (the pages do not fix it): the W bf16 values are widened to
 * fp32 and added one at a time in rank order 0..W-1 into an fp32 accumulator,
 * then divided once by W (an IEEE division, not a reciprocal multiply).
 * grads[w] points at replica w's gradient of shard element 0.
 */
void oracle_shard_reduce(const uint16_t* const* grads, int W, int64_t len,
                         int average, float* g)
{
    const float fw = (float)W;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < len; ++i) {
        float s = bf16_to_f32(grads[0][i]);
        for (int w = 1; w < W; ++w)
            s = s + bf16_to_f32(grads[w][i]);
        g[i] = average ? s / fw : s;
    }
}

/* ---------------------------------------------------------------------- */
/* O2: global L2 norm                                                      */
/* ---------------------------------------------------------------------- */

/*
 * Clipping treats all gradients as one long vector and takes its L2 norm
 * ([PT] training loop).  Under ZeRO-1 each rank holds only its shard of the
 * reduced gradient, so the square of the global norm is the sum of the ranks'
 * partial sums of squares.
 *
 * Each square of a binary32 value is exact in fp64.  The adds are fp64, in a
 * fixed order: sequentially inside consecutive blocks of ORACLE_NORM_BLOCK
 * elements (blocks counted from the shard's first element), then the block
 * sums one after another.  `total_in` lets a caller stream a shard through in
 * block-aligned pieces and obtain the same value as one call.
 */
double oracle_sumsq(const float* g, int64_t len, double total_in)
{
    int64_t nblk = (len + ORACLE_NORM_BLOCK - 1) / ORACLE_NORM_BLOCK;
    double total = total_in;
    /* block sums are independent; compute them in parallel, add them in order */
    enum { CHUNK = 256 };
    double part[CHUNK];
    for (int64_t b0 = 0; b0 < nblk; b0 += CHUNK) {
        int64_t nb = nblk - b0 < CHUNK ? nblk - b0 : CHUNK;
#pragma omp parallel for schedule(static)
        for (int64_t b = 0; b < nb; ++b) {
            int64_t lo = (b0 + b) * ORACLE_NORM_BLOCK;
            int64_t hi = lo + ORACLE_NORM_BLOCK < len ? lo + ORACLE_NORM_BLOCK : len;
            double s = 0.0;
            for (int64_t i = lo; i < hi; ++i) {
                double x = (double)g[i];
                s = s + x * x;
            }
            part[b] = s;
        }
        for (int64_t b = 0; b < nb; ++b)
            total = total + part[b];
    }
    return total;
}

/*
 * Global norm from the W ranks' partial sums of squares, added in rank order,
 * then the fp64 square root.
 */
double oracle_global_norm(const double* rank_sumsq, int n_ranks)
{
    double q = 0.0;
    for (int r = 0; r < n_ranks; ++r)
        q = q + rank_sumsq[r];
    return sqrt(q);
}

/* ---------------------------------------------------------------------- */
/* O3: clip coefficient                                                    */
/* ---------------------------------------------------------------------- */

/*
 * If the norm exceeds max_norm, every gradient is scaled by max_norm/norm, so
 * the direction is kept ([PT] training loop).  Readings adopted: a strict ">"
 * test, no epsilon in the denominator, the quotient formed in fp64 and rounded
 * once to fp32.  Returns 1 when the gradients must be multiplied by *coef.
 * A NaN norm fails the test (no clip); an infinite norm gives coef 0.
 */
int oracle_clip_coef(double norm, double max_norm, float* coef)
{
    if (norm > max_norm) {
        *coef = (float)(max_norm / norm);
        return 1;
    }
    *coef = 1.0f;
    return 0;
}

/* ---------------------------------------------------------------------- */
/* O4: the AdamW scalars of step t                                         */
/* ---------------------------------------------------------------------- */

typedef struct {
    float b1, b2;   /* beta1, beta2 as binary32                          */
    float a1, a2;   /* 1-beta1, 1-beta2 formed in fp64, rounded once     */
    float eps;      /* eps                                               */
    float sigma;    /* lr*sqrt(1-beta2^t)/(1-beta1^t), fp64, rounded once */
    float delta;    /* 1-lr*weight_decay, fp64, rounded once             */
} oracle_scalars;

/*
 * [PT] mixed precision + AdamW: the two bias corrections are folded into one
 * step size lr*sqrt(1-beta2^t)/(1-beta1^t), and decoupled weight decay
 * multiplies the parameter by 1-lr*weight_decay.  The page's code applies
 * Python floats to fp32 tensors, so each scalar is formed in double and used
 * as the nearest binary32.  t counts from 1 ([PT] checkpoint: bias correction
 * restarts at t = 1).
 */
void oracle_adamw_scalars(double lr, double beta1, double beta2, double eps,
                          double weight_decay, int64_t t, oracle_scalars* s)
{
    s->b1 = (float)beta1;
    s->b2 = (float)beta2;
    s->a1 = (float)(1.0 - beta1);
    s->a2 = (float)(1.0 - beta2);
    s->eps = (float)eps;
    double bc1 = 1.0 - pow(beta1, (double)t);
    double bc2 = 1.0 - pow(beta2, (double)t);
    s->sigma = (float)(lr * sqrt(bc2) / bc1);
    s->delta = (float)(1.0 - lr * weight_decay);
}

/* ---------------------------------------------------------------------- */
/* O5-O7: AdamW on the shard, then the bf16 copy                           */
/* ---------------------------------------------------------------------- */

/*
 * One element of AdamW with decoupled weight decay, as [PT] "一张卡上装了什么：
 * 混合精度与 AdamW" defines it, in this file's notation (g already clipped,
 * sigma_t and delta from oracle_adamw_scalars):
 *   m_t = b1 m_{t-1} + a1 g                 (first moment, a1 = 1 - beta1)
 *   v_t = b2 v_{t-1} + a2 (g g)             (second moment, a2 = 1 - beta2)
 *   p_t = (p_{t-1} - sigma_t m_t / (sqrt(v_t) + eps)) delta
 * The decay factor delta multiplies the master after the Adam move (the
 * section's order); each operation is one binary32 operation, evaluated left
 * to right as written.  decay_first = 1 applies delta before the move
 * instead: the order the section attributes to torch.optim.AdamW, which it
 * says differs by a term of order lr^2 * lambda per step.  The bf16 parameter
 * of the forward pass is then the nearest bf16 of p_t (same section: the fp32
 * master takes the update, a bf16 copy is made every step).
 */
static void adamw_one(float g, float* p, float* m, float* v,
                      const oracle_scalars* s, int decay_first)
{
    float mn = s->b1 * *m + s->a1 * g;
    float vn = s->b2 * *v + s->a2 * (g * g);
    float d = sqrtf(vn) + s->eps;
    float q = mn / d;
    float pn;
    if (decay_first) {
        pn = *p * s->delta;
        pn = pn - s->sigma * q;
    } else {
        pn = *p - s->sigma * q;
        pn = pn * s->delta;
    }
    *m = mn;
    *v = vn;
    *p = pn;
}

/*
 * AdamW over a flat shard.  `clip` and `coef` come from oracle_clip_coef:
 * when clip is 1 the gradient is multiplied by coef first.  With mv_bf16 the
 * moments are stored as bf16 ([PT] notes that some setups keep m and v in
 * bf16, 12 B/param in total); reading adopted: the stored bf16 moments are
 * widened, the step runs in fp32 exactly as above, and the new moments are
 * stored as their nearest bf16; the parameter update uses the fp32 moments.
 */
void oracle_adamw_v(const float* g, float* master, void* m, void* v,
                    uint16_t* param_bf16, int64_t len, const oracle_scalars* s,
                    int clip, float coef, int mv_bf16, int decay_first)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < len; ++i) {
        float gi = clip ? g[i] * coef : g[i];
        if (mv_bf16) {
            uint16_t* mb = (uint16_t*)m;
            uint16_t* vb = (uint16_t*)v;
            float mi = bf16_to_f32(mb[i]);
            float vi = bf16_to_f32(vb[i]);
            adamw_one(gi, &master[i], &mi, &vi, s, decay_first);
            mb[i] = oracle_f32_to_bf16(mi);
            vb[i] = oracle_f32_to_bf16(vi);
        } else {
            adamw_one(gi, &master[i], &((float*)m)[i], &((float*)v)[i], s, decay_first);
        }
        param_bf16[i] = oracle_f32_to_bf16(master[i]);
    }
}

void oracle_adamw(const float* g, float* master, float* m, float* v,
                  uint16_t* param_bf16, int64_t len, const oracle_scalars* s,
                  int clip, float coef)
{
    oracle_adamw_v(g, master, m, v, param_bf16, len, s, clip, coef, 0, 0);
}

void oracle_adamw_bf16mv(const float* g, float* master, uint16_t* m_bf16,
                         uint16_t* v_bf16, uint16_t* param_bf16, int64_t len,
                         const oracle_scalars* s, int clip, float coef)
{
    oracle_adamw_v(g, master, m_bf16, v_bf16, param_bf16, len, s, clip, coef, 1, 0);
}

/* Decay first, then the Adam update (no bf16 copy): used by the pin of the
 * page's remark about the two orders. */
void oracle_adamw_decay_first(const float* g, float* master, float* m, float* v,
                              int64_t len, const oracle_scalars* s)
{
    for (int64_t i = 0; i < len; ++i)
        adamw_one(g[i], &master[i], &m[i], &v[i], s, 1);
}

/*
 * Clip coefficient with the convention of torch.nn.utils.clip_grad_norm_
 * (not the pages'): coef = max_norm / (norm + 1e-6), clamped at 1, i.e. the
 * gradients are scaled only when that quotient is below 1.  Formed in fp64,
 * rounded once to fp32.
 */
int oracle_clip_coef_eps(double norm, double max_norm, float* coef)
{
    double c = max_norm / (norm + 1e-6);
    if (c < 1.0) {
        *coef = (float)c;
        return 1;
    }
    *coef = 1.0f;
    return 0;
}

/* The reduced gradient rounded to bf16 (nearest even) and widened back: what
 * a reduce-scatter that delivers bf16 would hand to the optimizer. */
void oracle_round_to_bf16(float* g, int64_t len)
{
    for (int64_t i = 0; i < len; ++i)
        g[i] = bf16_to_f32(oracle_f32_to_bf16(g[i]));
}

/* ---------------------------------------------------------------------- */
/* The whole step on a flat shard                                          */
/* ---------------------------------------------------------------------- */

/*
 * One rank's ZeRO-1 step ([L7] sec. 5.2 and [PT] ZeRO-1: reduce-scatter the
 * gradients, update only this rank's slice with this rank's optimizer state;
 * the parameter all-gather that follows is outside this step):
 *   g = reduce(grads);  rank_sumsq[my_rank] = sum g^2;
 *   norm = sqrt(sum over ranks);  clip;  AdamW;  bf16 copy.
 * rank_sumsq holds the other ranks' partials on entry (zero where unknown).
 * g_scratch has len floats.  info_out receives {norm, clip coef, clip flag,
 * this rank's partial}.  variant: bit 0 decay first, bit 1 the torch clip
 * convention, bit 2 the reduced gradient rounded to bf16 (compatibility
 * variants; 0 is the pages' step).  Returns 0, or -1 when subnormals would be
 * flushed.
 */
int oracle_step_v(const uint16_t* const* grads, int W, int64_t len, int average,
                  float* master, void* m, void* v, int mv_bf16,
                  uint16_t* param_bf16, double lr, double beta1, double beta2,
                  double eps, double weight_decay, double max_norm, int64_t t,
                  double* rank_sumsq, int n_ranks, int my_rank, float* g_scratch,
                  double* info_out, unsigned variant)
{
    if (!oracle_fp_env_ok())
        return -1;
    oracle_shard_reduce(grads, W, len, average, g_scratch);
    if (variant & 4u)
        oracle_round_to_bf16(g_scratch, len);
    rank_sumsq[my_rank] = oracle_sumsq(g_scratch, len, 0.0);
    double norm = oracle_global_norm(rank_sumsq, n_ranks);
    float coef;
    int clip = (variant & 2u) ? oracle_clip_coef_eps(norm, max_norm, &coef)
                              : oracle_clip_coef(norm, max_norm, &coef);
    oracle_scalars s;
    oracle_adamw_scalars(lr, beta1, beta2, eps, weight_decay, t, &s);
    oracle_adamw_v(g_scratch, master, m, v, param_bf16, len, &s, clip, coef,
                   mv_bf16, (int)(variant & 1u));
    info_out[0] = norm;
    info_out[1] = (double)coef;
    info_out[2] = (double)clip;
    info_out[3] = rank_sumsq[my_rank];
    return 0;
}

int oracle_step(const uint16_t* const* grads, int W, int64_t len, int average,
                float* master, void* m, void* v, int mv_bf16,
                uint16_t* param_bf16, double lr, double beta1, double beta2,
                double eps, double weight_decay, double max_norm, int64_t t,
                double* rank_sumsq, int n_ranks, int my_rank, float* g_scratch,
                double* info_out)
{
    return oracle_step_v(grads, W, len, average, master, m, v, mv_bf16, param_bf16,
                         lr, beta1, beta2, eps, weight_decay, max_norm, t,
                         rank_sumsq, n_ranks, my_rank, g_scratch, info_out, 0u);
}

/* ---------------------------------------------------------------------- */
/* Memory accounting ([PT] ZeRO table; [L7] sec. 5.1)                      */
/* ---------------------------------------------------------------------- */

/*
 * Bytes per GPU for psi parameters, K bytes of optimizer state per parameter,
 * bf16 params and grads (2 B each), n_d data-parallel ranks:
 *   stage 0 (DDP): (2+2+K) psi
 *   stage 1: 2 psi + 2 psi + K psi / n_d
 *   stage 2: 2 psi + (2+K) psi / n_d
 *   stage 3: (2+2+K) psi / n_d
 */
double oracle_zero_bytes_per_gpu(double psi, double K, double n_d, int stage)
{
    switch (stage) {
    case 0: return (2.0 + 2.0 + K) * psi;
    case 1: return 2.0 * psi + 2.0 * psi + K * psi / n_d;
    case 2: return 2.0 * psi + (2.0 + K) * psi / n_d;
    case 3: return (2.0 + 2.0 + K) * psi / n_d;
    default: return -1.0;
    }
}

/* ---------------------------------------------------------------------- */
/* Harness helper (no arithmetic)                                          */
/* ---------------------------------------------------------------------- */

/* Sets the number of OpenMP threads the loops above use when n > 0 and
 * returns the number in effect (the CPU baseline times 1 and N threads). */
int oracle_threads(int n)
{
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
}
