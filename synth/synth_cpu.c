/*
 * synth_cpu.c -- seeded synthetic inputs (CPU side).
 *
 * The only code that both the oracle side and the GPU side use: it draws the
 * gradients and master weights that a test or the bench feeds to both.  It
 * holds none of the optimizer's arithmetic.  synth_gpu.hip implements the same
 * definition on the GPU, bit for bit; tests compare the two.
 *
 * Definition (counter-based, so any element can be drawn on its own):
 *   SplitMix64 (Steele, Lea & Flood, OOPSLA 2014; the public-domain reference
 *   by S. Vigna): state advances by the golden-ratio gamma 0x9E3779B97F4A7C15
 *   and each output is the state passed through the 64-bit finalizer
 *       z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
 *       z ^= z >> 27; z *= 0x94D049BB133111EB;  z ^= z >> 31.
 *   at(key, i)  = finalizer(key + (i+1)*gamma)   (output i of a generator seeded with key)
 *   key(seed, a, b, c) = at(at(at(seed, a), b), c)
 * Value of element i under key k with scale sigma:
 *   h = at(k, i);  U = sum over the four 16-bit fields f of h of (2f+1)
 *   z = U * 2^-17 - 2          (Irwin-Hall of 4 uniforms, centred; exact in fp32)
 *   x = (z * 1.7320508f) * sigma   (two binary32 products; variance sigma^2)
 *   outliers: if at(k ^ 0x5A5A5A5A5A5A5A5A, i) mod 100 < pct, x = x * 100.
 * fp32 inputs store x; bf16 inputs store the upper 16 bits of x (truncation,
 * so the stored gradient is exactly a bf16 value; no rounding rule involved).
 */
#include <stdint.h>
#include <string.h>

#define SM_GAMMA 0x9E3779B97F4A7C15ULL
#define OUTLIER_SALT 0x5A5A5A5A5A5A5A5AULL

static uint64_t finalize64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t synth_at(uint64_t key, uint64_t i) { return finalize64(key + (i + 1) * SM_GAMMA); }

uint64_t synth_key(uint64_t seed, uint64_t a, uint64_t b, uint64_t c)
{
    return synth_at(synth_at(synth_at(seed, a), b), c);
}

float synth_value(uint64_t key, uint64_t i, float sigma, int outlier_pct)
{
    uint64_t h = synth_at(key, i);
    uint32_t u = 0;
    for (int k = 0; k < 4; ++k)
        u += 2u * (uint32_t)((h >> (16 * k)) & 0xFFFFu) + 1u;
    float z = (float)u * 0x1p-17f - 2.0f;
    float x = (z * 1.7320508f) * sigma;
    if (outlier_pct > 0 && synth_at(key ^ OUTLIER_SALT, i) % 100u < (uint64_t)outlier_pct)
        x = x * 100.0f;
    return x;
}

void synth_fill_f32(float* out, int64_t n, uint64_t key, uint64_t i0, float sigma, int outlier_pct)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j)
        out[j] = synth_value(key, i0 + (uint64_t)j, sigma, outlier_pct);
}

void synth_fill_bf16(uint16_t* out, int64_t n, uint64_t key, uint64_t i0, float sigma, int outlier_pct)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        float x = synth_value(key, i0 + (uint64_t)j, sigma, outlier_pct);
        uint32_t u;
        memcpy(&u, &x, sizeof u);
        out[j] = (uint16_t)(u >> 16);
    }
}

/* Draws at arbitrary global indices (for sampled checks of huge shards). */
void synth_gather_f32(float* out, const int64_t* idx, int64_t n, uint64_t key, float sigma, int outlier_pct)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j)
        out[j] = synth_value(key, (uint64_t)idx[j], sigma, outlier_pct);
}

void synth_gather_bf16(uint16_t* out, const int64_t* idx, int64_t n, uint64_t key, float sigma, int outlier_pct)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        float x = synth_value(key, (uint64_t)idx[j], sigma, outlier_pct);
        uint32_t u;
        memcpy(&u, &x, sizeof u);
        out[j] = (uint16_t)(u >> 16);
    }
}
