/* A plain C11 program that runs ZeRO-1 steps through libzero1.so with the HIP
 * runtime only (no Python, no torch): the GPU test tests/test_gpu_parity.py
 * writes its inputs, runs it, and compares its outputs with the oracle.
 *
 * usage: step_demo IN OUT
 * IN  (little-endian binary): int64 n_tensors, W, rank, steps; int64 sizes[n];
 *     double partials[steps][W] (every rank's fp64 sum of squares);
 *     float master[S] (this rank's shard of the fp32 master);
 *     uint16 grads[steps][W][N] (bf16 replica gradients, N = sum of sizes).
 * OUT: float master[S], m[S], v[S]; uint16 params[S] (the shard's bf16
 *     parameters, gathered from the per-tensor buffers); then per step the
 *     zero1_norm_info (32 bytes).
 * Exit status 0 on success; messages on stderr otherwise. */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zero1.h"

#define HIPCHK(x)                                                               \
    do {                                                                        \
        hipError_t e_ = (x);                                                    \
        if (e_ != hipSuccess) {                                                 \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));             \
            return 1;                                                           \
        }                                                                       \
    } while (0)
#define ZCHK(x)                                                                 \
    do {                                                                        \
        zero1_status s_ = (x);                                                  \
        if (s_ != ZERO1_OK) {                                                   \
            fprintf(stderr, "%s: %s: %s\n", #x, zero1_status_string(s_), zero1_last_error()); \
            return 1;                                                           \
        }                                                                       \
    } while (0)

static int rd(FILE* f, void* p, size_t n)
{
    return fread(p, 1, n, f) == n ? 0 : 1;
}

int main(int argc, char** argv)
{
    if (argc != 3) {
        fprintf(stderr, "usage: step_demo IN OUT\n");
        return 2;
    }
    FILE* in = fopen(argv[1], "rb");
    if (!in) {
        fprintf(stderr, "cannot open %s\n", argv[1]);
        return 1;
    }
    int64_t hdr[4];
    if (rd(in, hdr, sizeof hdr)) return 1;
    const int64_t nt = hdr[0], W = hdr[1], rank = hdr[2], steps = hdr[3];
    if (nt < 1 || nt > 1 << 20 || W < 1 || W > ZERO1_MAX_W || rank < 0 || rank >= W || steps < 1 || steps > 100) {
        fprintf(stderr, "bad header\n");
        return 1;
    }
    int64_t* sizes = malloc(sizeof(int64_t) * (size_t)nt);
    double* partials = malloc(sizeof(double) * (size_t)(steps * W));
    if (!sizes || !partials || rd(in, sizes, sizeof(int64_t) * (size_t)nt) ||
        rd(in, partials, sizeof(double) * (size_t)(steps * W)))
        return 1;
    int64_t N = 0;
    for (int64_t i = 0; i < nt; ++i) N += sizes[i];
    int64_t begin = 0, S = 0;
    ZCHK(zero1_shard_range(N, (int)W, (int)rank, &begin, &S));

    /* device buffers: W replica gradients, flat master/m/v of the shard, one
     * bf16 buffer per tensor, the chunk table, the workspace, rank partials */
    uint16_t* hgrads = malloc(2 * (size_t)(N * W));
    float* hmaster = malloc(4 * (size_t)S);
    if (!hgrads || !hmaster) return 1;
    uint16_t* dgrads[ZERO1_MAX_W];
    for (int64_t w = 0; w < W; ++w) HIPCHK(hipMalloc((void**)&dgrads[w], 2 * (size_t)N));
    float *master, *m, *v;
    HIPCHK(hipMalloc((void**)&master, 4 * (size_t)S));
    HIPCHK(hipMalloc((void**)&m, 4 * (size_t)S));
    HIPCHK(hipMalloc((void**)&v, 4 * (size_t)S));
    HIPCHK(hipMemset(m, 0, 4 * (size_t)S));
    HIPCHK(hipMemset(v, 0, 4 * (size_t)S));
    uint16_t** params = malloc(sizeof(uint16_t*) * (size_t)nt);
    if (!params) return 1;
    for (int64_t i = 0; i < nt; ++i) {
        HIPCHK(hipMalloc((void**)&params[i], 2 * (size_t)sizes[i]));
        HIPCHK(hipMemset(params[i], 0, 2 * (size_t)sizes[i]));
    }

    /* the pieces: every tensor's part inside [begin, begin + S) */
    zero1_piece* pieces = malloc(sizeof(zero1_piece) * (size_t)nt);
    int np = 0;
    int64_t t0 = 0;
    for (int64_t i = 0; i < nt; ++i) {
        const int64_t t1 = t0 + sizes[i];
        const int64_t lo = t0 > begin ? t0 : begin, hi = t1 < begin + S ? t1 : begin + S;
        if (lo < hi) {
            zero1_piece p;
            p.numel = hi - lo;
            p.shard_offset = lo - begin;
            p.param_bf16 = params[i] + (lo - t0);
            p.master = master + (lo - begin);
            p.m = m + (lo - begin);
            p.v = v + (lo - begin);
            pieces[np++] = p;
        }
        t0 = t1;
    }
    const size_t tb = zero1_mta_table_bytes(pieces, np);
    void* table;
    HIPCHK(hipMalloc(&table, tb));
    zero1_plan plan;
    ZCHK(zero1_mta_plan(pieces, np, 0, table, tb, &plan));
    const size_t wsb = zero1_mta_workspace_bytes(&plan, (int)W, 0);
    void* ws;
    HIPCHK(hipMalloc(&ws, wsb));
    double* rank_sumsq;
    HIPCHK(hipMalloc((void**)&rank_sumsq, sizeof(double) * (size_t)W));
    zero1_norm_info* info;
    HIPCHK(hipMalloc((void**)&info, sizeof(zero1_norm_info) * (size_t)steps));
    if (rd(in, hmaster, 4 * (size_t)S)) return 1;
    HIPCHK(hipMemcpy(master, hmaster, 4 * (size_t)S, hipMemcpyHostToDevice));

    for (int64_t t = 1; t <= steps; ++t) {
        if (rd(in, hgrads, 2 * (size_t)(N * W))) {
            fprintf(stderr, "short input\n");
            return 1;
        }
        for (int64_t w = 0; w < W; ++w)
            HIPCHK(hipMemcpy(dgrads[w], hgrads + w * N, 2 * (size_t)N, hipMemcpyHostToDevice));
        HIPCHK(hipMemcpy(rank_sumsq, partials + (t - 1) * W, sizeof(double) * (size_t)W, hipMemcpyHostToDevice));
        const zero1_hparams hp = {1e-3, 0.9, 0.95, 1e-8, 0.1, 1.0, t, NULL};
        ZCHK(zero1_mta_step((const uint16_t* const*)dgrads, (int)W, begin, &plan, &hp, rank_sumsq, (int)W, (int)rank,
                            0, info + (t - 1), ws, wsb, NULL));
        HIPCHK(hipDeviceSynchronize());
    }
    fclose(in);

    FILE* out = fopen(argv[2], "wb");
    if (!out) return 1;
    float* h = malloc(4 * (size_t)S);
    uint16_t* hp16 = malloc(2 * (size_t)S);
    zero1_norm_info* hinfo = malloc(sizeof(zero1_norm_info) * (size_t)steps);
    if (!h || !hp16 || !hinfo) return 1;
    const float* arrs[3] = {master, m, v};
    for (int k = 0; k < 3; ++k) {
        HIPCHK(hipMemcpy(h, arrs[k], 4 * (size_t)S, hipMemcpyDeviceToHost));
        fwrite(h, 4, (size_t)S, out);
    }
    for (int i = 0; i < np; ++i)
        HIPCHK(hipMemcpy(hp16 + pieces[i].shard_offset, pieces[i].param_bf16, 2 * (size_t)pieces[i].numel,
                         hipMemcpyDeviceToHost));
    fwrite(hp16, 2, (size_t)S, out);
    HIPCHK(hipMemcpy(hinfo, info, sizeof(zero1_norm_info) * (size_t)steps, hipMemcpyDeviceToHost));
    fwrite(hinfo, sizeof(zero1_norm_info), (size_t)steps, out);
    fclose(out);
    fprintf(stderr, "step_demo: W=%lld rank=%lld shard=%lld pieces=%d steps=%lld done\n", (long long)W,
            (long long)rank, (long long)S, np, (long long)steps);
    return 0;
}
