/* Runs the oracle's whole step (oracle_step_v, oracle/zero1_oracle.c) over a
 * case read from a file, so that the oracle can be built and run under the
 * address and undefined-behaviour sanitizers by tests/test_sanitizers.py; the
 * test compares what this program writes with the regular oracle build.
 *
 * Input (native byte order):
 *   int32 W, mv_bf16, variant, steps, n_ranks, my_rank;  int64 len, t0;
 *   double lr, beta1, beta2, eps, weight_decay, max_norm;
 *   double rank_sumsq[n_ranks];  float master[len];
 *   then per step: uint16 grads[W][len].
 * Output: per step double info[4] (norm, clip coefficient, clip flag, this
 * rank's partial), then master (float[len]), m and v (float or bf16 bits
 * [len]) and the bf16 parameters (uint16[len]). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_step_v(const uint16_t* const* grads, int W, int64_t len, int average, float* master, void* m,
                  void* v, int mv_bf16, uint16_t* param_bf16, double lr, double beta1, double beta2,
                  double eps, double weight_decay, double max_norm, int64_t t, double* rank_sumsq,
                  int n_ranks, int my_rank, float* g_scratch, double* info_out, unsigned variant);

static int read_all(FILE* f, void* p, size_t n)
{
    return n == 0 || fread(p, 1, n, f) == n;
}

int main(int argc, char** argv)
{
    if (argc != 3) {
        fprintf(stderr, "usage: %s case.bin out.bin\n", argv[0]);
        return 2;
    }
    FILE* in = fopen(argv[1], "rb");
    FILE* out = fopen(argv[2], "wb");
    if (!in || !out) {
        fprintf(stderr, "cannot open files\n");
        return 2;
    }
    int32_t hdr[6];
    int64_t len_t0[2];
    double hp[6];
    if (!read_all(in, hdr, sizeof hdr) || !read_all(in, len_t0, sizeof len_t0) || !read_all(in, hp, sizeof hp)) {
        fprintf(stderr, "short header\n");
        return 2;
    }
    const int W = hdr[0], mv_bf16 = hdr[1], steps = hdr[3], n_ranks = hdr[4], my_rank = hdr[5];
    const unsigned variant = (unsigned)hdr[2];
    const int64_t len = len_t0[0], t0 = len_t0[1];
    if (W < 1 || W > 128 || steps < 1 || n_ranks < 1 || my_rank < 0 || my_rank >= n_ranks || len < 0) {
        fprintf(stderr, "bad header\n");
        return 2;
    }
    const size_t n = (size_t)len, mvb = mv_bf16 ? 2 : 4;
    double* rs = malloc(sizeof(double) * (size_t)n_ranks);
    float* master = malloc(4 * n + 4);
    void* m = calloc(n + 1, mvb);
    void* v = calloc(n + 1, mvb);
    uint16_t* param = calloc(n + 1, 2);
    float* scratch = malloc(4 * n + 4);
    uint16_t* gbuf = malloc(2 * n * (size_t)W + 2);
    const uint16_t** gp = malloc(sizeof(uint16_t*) * (size_t)W);
    if (!rs || !master || !m || !v || !param || !scratch || !gbuf || !gp) {
        fprintf(stderr, "out of memory\n");
        return 2;
    }
    if (!read_all(in, rs, sizeof(double) * (size_t)n_ranks) || !read_all(in, master, 4 * n)) {
        fprintf(stderr, "short state\n");
        return 2;
    }
    for (int w = 0; w < W; ++w) gp[w] = gbuf + (size_t)w * n;
    for (int k = 0; k < steps; ++k) {
        if (!read_all(in, gbuf, 2 * n * (size_t)W)) {
            fprintf(stderr, "short gradients at step %d\n", k);
            return 2;
        }
        double info[4];
        if (oracle_step_v(gp, W, len, 1, master, m, v, mv_bf16, param, hp[0], hp[1], hp[2], hp[3], hp[4], hp[5],
                          t0 + k, rs, n_ranks, my_rank, scratch, info, variant) != 0) {
            fprintf(stderr, "oracle refused (subnormals flushed)\n");
            return 3;
        }
        fwrite(info, sizeof info, 1, out);
    }
    fwrite(master, 4, n, out);
    fwrite(m, mvb, n, out);
    fwrite(v, mvb, n, out);
    fwrite(param, 2, n, out);
    fclose(out);
    fclose(in);
    free(rs);
    free(master);
    free(m);
    free(v);
    free(param);
    free(scratch);
    free(gbuf);
    free(gp);
    return 0;
}
