// kernels.hip -- gfx950 kernels of one rank's ZeRO-1 optimizer step.
//
// Everything here is HBM-bound elementwise work (about 0.5 flop per byte), so
// the design rules are those of a streaming kernel on CDNA4: 16-byte coalesced
// accesses (8 bf16 or 4 fp32 per lane), enough workgroups per CU to keep loads
// in flight, one pass over each array per phase, no atomics, no MFMA.
//
// Arithmetic contract (matches the page's AdamW code on "并行训练", section
// "一张卡上装了什么：混合精度与 AdamW", applied one binary32 operation at a time):
// built with -ffp-contract=off and the pragma below, so no multiply-add is
// fused; fp32 '/' and sqrtf are the correctly rounded HIP defaults; subnormals
// are kept.  fp64 is used only for sums of squares (each square is exact in
// fp64, so fma(x, x, acc) rounds exactly like acc + x*x).
//
// Determinism: every workgroup owns a fixed set of tiles, every lane adds its
// own elements in index order, and partial sums are combined by a fixed tree
// (wave butterfly, then the four waves in order), so a rerun with the same
// launch shape reproduces every bit, including the norm.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

#pragma clang fp contract(off)

namespace z1 {
namespace {

// ------------------------------------------------------------- number formats
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Nearest-even bf16 of an fp32 value: add half an ulp of the bf16 result
// (minus one when the kept last bit is even) and truncate; carries into the
// exponent give the right result, including overflow to infinity.  NaNs are
// kept as quiet NaNs with their sign.
__device__ __forceinline__ uint32_t bf16_rne_bits(float x)
{
    uint32_t u = __float_as_uint(x);
    uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    return ((u & 0x7fffffffu) > 0x7f800000u) ? ((u >> 16) | 0x40u) : r;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return bf16_rne_bits(lo) | (bf16_rne_bits(hi) << 16);
}

// ------------------------------------------------------------- reduction
// g[0..V) for V consecutive elements starting at e of every slice.
// Accumulation order: s = G_0; s = s + G_w for w = 1..W-1; then the average.
template <int V>
__device__ __forceinline__ void reduce_group(const Reduce& r, int64_t e, float (&s)[V])
{
    if constexpr (V == kVec) {
        uint4 buf[8];
        const uint4 a = *reinterpret_cast<const uint4*>(r.gp.p[0] + e);
        s[0] = bf16_lo(a.x); s[1] = bf16_hi(a.x);
        s[2] = bf16_lo(a.y); s[3] = bf16_hi(a.y);
        s[4] = bf16_lo(a.z); s[5] = bf16_hi(a.z);
        s[6] = bf16_lo(a.w); s[7] = bf16_hi(a.w);
        for (int w0 = 1; w0 < r.W; w0 += 8) {
            const int nb = r.W - w0 < 8 ? r.W - w0 : 8;
            // issue up to eight 16-byte loads before the first dependent add
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (k < nb) buf[k] = *reinterpret_cast<const uint4*>(r.gp.p[w0 + k] + e);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if (k < nb) {
                    s[0] = s[0] + bf16_lo(buf[k].x); s[1] = s[1] + bf16_hi(buf[k].x);
                    s[2] = s[2] + bf16_lo(buf[k].y); s[3] = s[3] + bf16_hi(buf[k].y);
                    s[4] = s[4] + bf16_lo(buf[k].z); s[5] = s[5] + bf16_hi(buf[k].z);
                    s[6] = s[6] + bf16_lo(buf[k].w); s[7] = s[7] + bf16_hi(buf[k].w);
                }
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < V; ++j) {
            float a = bf16_to_f32(r.gp.p[0][e + j]);
            for (int w = 1; w < r.W; ++w)
                a = a + bf16_to_f32(r.gp.p[w][e + j]);
            s[j] = a;
        }
    }
    if (r.mode == kAvgMulPow2) {
#pragma unroll
        for (int j = 0; j < V; ++j) s[j] = s[j] * r.inv_w;
    } else if (r.mode == kAvgDiv) {
#pragma unroll
        for (int j = 0; j < V; ++j) s[j] = s[j] / r.f_w;
    }
}

__device__ __forceinline__ float reduce_one(const Reduce& r, int64_t e)
{
    float a = bf16_to_f32(r.gp.p[0][e]);
    for (int w = 1; w < r.W; ++w)
        a = a + bf16_to_f32(r.gp.p[w][e]);
    if (r.mode == kAvgMulPow2) a = a * r.inv_w;
    else if (r.mode == kAvgDiv) a = a / r.f_w;
    return a;
}

// ------------------------------------------------------------- block sum (fp64)
// Fixed-order workgroup sum: butterfly inside each 64-lane wave, then the four
// wave results in order.  Returns the total in lane 0 of wave 0.
__device__ __forceinline__ double block_sum(double x)
{
    __shared__ double wsum[kThreads / 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        x += __shfl_xor(x, off, 64);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) wsum[wave] = x;
    __syncthreads();
    double t = 0.0;
    if (threadIdx.x == 0) {
        t = wsum[0];
#pragma unroll
        for (int k = 1; k < kThreads / 64; ++k) t = t + wsum[k];
    }
    return t;
}

// ------------------------------------------------------------- phase 1
template <int V, bool STORE, bool NORM>
__global__ __launch_bounds__(kThreads) void reduce_kernel(Reduce r, int64_t len, float* __restrict__ g_out,
                                                          double* __restrict__ partials)
{
    double acc = 0.0;
    const int64_t tile = (int64_t)kThreads * V;
    const int64_t ntiles = (len + tile - 1) / tile;
    for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const int64_t e = t * tile + (int64_t)threadIdx.x * V;
        if (V > 1 && e + V <= len) {
            float s[V];
            reduce_group<V>(r, e, s);
            if constexpr (STORE) {
                float4* o = reinterpret_cast<float4*>(g_out + e);
                o[0] = make_float4(s[0], s[1], s[2], s[3]);
                o[1] = make_float4(s[4], s[5], s[6], s[7]);
            }
            if constexpr (NORM) {
#pragma unroll
                for (int j = 0; j < V; ++j) acc = fma((double)s[j], (double)s[j], acc);
            }
        } else {
            for (int j = 0; j < V && e + j < len; ++j) {
                const float x = reduce_one(r, e + j);
                if constexpr (STORE) g_out[e + j] = x;
                if constexpr (NORM) acc = fma((double)x, (double)x, acc);
            }
        }
    }
    if constexpr (NORM) {
        const double b = block_sum(acc);
        if (threadIdx.x == 0) partials[blockIdx.x] = b;
    }
}

template <int V>
__global__ __launch_bounds__(kThreads) void sumsq_kernel(const float* __restrict__ g, int64_t len,
                                                         double* __restrict__ partials)
{
    double acc = 0.0;
    const int64_t tile = (int64_t)kThreads * V;
    const int64_t ntiles = (len + tile - 1) / tile;
    for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const int64_t e = t * tile + (int64_t)threadIdx.x * V;
        if (V > 1 && e + V <= len) {
            const float4* p = reinterpret_cast<const float4*>(g + e);
            const float4 a = p[0], b = p[1];
            const float s[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) acc = fma((double)s[j], (double)s[j], acc);
        } else {
            for (int j = 0; j < V && e + j < len; ++j) {
                const double x = (double)g[e + j];
                acc = fma(x, x, acc);
            }
        }
    }
    const double b = block_sum(acc);
    if (threadIdx.x == 0) partials[blockIdx.x] = b;
}

// ------------------------------------------------------------- finalize
// One workgroup adds the per-workgroup partials of phase 1 in a fixed order:
// each lane sums a strided subset sequentially, then a fixed LDS tree.
__global__ __launch_bounds__(kThreads) void finalize_kernel(const double* __restrict__ partials, int nb,
                                                            double* __restrict__ q_out)
{
    __shared__ double sh[kThreads];
    double a = 0.0;
    for (int i = threadIdx.x; i < nb; i += kThreads) a = a + partials[i];
    sh[threadIdx.x] = a;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) sh[threadIdx.x] = sh[threadIdx.x] + sh[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) *q_out = sh[0];
}

// Global norm and clip decision from the ranks' partial sums of squares
// ("训练循环与 checkpoint": clip all gradients as one vector when the L2 norm
// exceeds max_norm).  The partials are added in rank order, so every
// workgroup that evaluates this gets the same bits.
__device__ __forceinline__ NormInfo clip_info(const double* rank_sumsq, int n_ranks, double max_norm)
{
    NormInfo ni;
    double tot = 0.0;
    for (int q = 0; q < n_ranks; ++q) tot = tot + rank_sumsq[q];
    ni.sumsq_total = tot;
    ni.norm = sqrt(tot);
    if (ni.norm > max_norm) {
        ni.clip = 1;
        ni.clip_coef = (float)(max_norm / ni.norm);
    } else {
        ni.clip = 0;
        ni.clip_coef = 1.0f;
    }
    ni.nonfinite = (isnan(ni.norm) || isinf(ni.norm)) ? 1 : 0;
    ni.reserved = 0;
    return ni;
}

// Prologue of every update kernel: lane 0 forms the clip decision, workgroup 0
// publishes it, and the whole workgroup reads it from LDS.
struct ClipArgs {
    const double* rank_sumsq;
    int n_ranks;
    double max_norm;
    NormInfo* info_out;   // may be null
};

__device__ __forceinline__ void block_clip(const ClipArgs& ca, bool& clip, float& coef)
{
    __shared__ NormInfo sh;
    if (threadIdx.x == 0) {
        sh = clip_info(ca.rank_sumsq, ca.n_ranks, ca.max_norm);
        if (blockIdx.x == 0 && ca.info_out) *ca.info_out = sh;
    }
    __syncthreads();
    clip = sh.clip != 0;
    coef = sh.clip_coef;
}

// ------------------------------------------------------------- phase 2
// One element of AdamW in the page's order: moments, update, then decay.
__device__ __forceinline__ void adamw_elem(float g, float& p, float& m, float& v, const Scal& c)
{
    const float mn = c.b1 * m + c.a1 * g;
    const float vn = c.b2 * v + c.a2 * (g * g);
    const float d = sqrtf(vn) + c.eps;
    const float q = mn / d;
    float pn = p - c.sigma * q;
    pn = pn * c.delta;
    m = mn;
    v = vn;
    p = pn;
}

// Update n (<= V) consecutive elements.  gsrc: 0 = read g from `g` at shard
// index gi, 1 = recompute g from the slices at shard index gi.  State index si.
template <int V, int GSRC, bool MVBF16>
__device__ __forceinline__ void step_group(const float* __restrict__ g, const Reduce& r, int64_t gi,
                                           float* __restrict__ master, void* __restrict__ mp,
                                           void* __restrict__ vp, uint16_t* __restrict__ param,
                                           int64_t si, int n, const Scal& c, bool clip, float coef)
{
    if (V > 1 && n == V) {
        float gv[8], p[8], m[8], v[8];
        if constexpr (GSRC == 0) {
            const float4* gp = reinterpret_cast<const float4*>(g + gi);
            const float4 a = gp[0], b = gp[1];
            gv[0] = a.x; gv[1] = a.y; gv[2] = a.z; gv[3] = a.w;
            gv[4] = b.x; gv[5] = b.y; gv[6] = b.z; gv[7] = b.w;
        } else {
            reduce_group<8>(r, gi, gv);
        }
        const float4* pp = reinterpret_cast<const float4*>(master + si);
        const float4 p0 = pp[0], p1 = pp[1];
        p[0] = p0.x; p[1] = p0.y; p[2] = p0.z; p[3] = p0.w;
        p[4] = p1.x; p[5] = p1.y; p[6] = p1.z; p[7] = p1.w;
        if constexpr (MVBF16) {
            const uint4 mb = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(mp) + si);
            const uint4 vb = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(vp) + si);
            m[0] = bf16_lo(mb.x); m[1] = bf16_hi(mb.x); m[2] = bf16_lo(mb.y); m[3] = bf16_hi(mb.y);
            m[4] = bf16_lo(mb.z); m[5] = bf16_hi(mb.z); m[6] = bf16_lo(mb.w); m[7] = bf16_hi(mb.w);
            v[0] = bf16_lo(vb.x); v[1] = bf16_hi(vb.x); v[2] = bf16_lo(vb.y); v[3] = bf16_hi(vb.y);
            v[4] = bf16_lo(vb.z); v[5] = bf16_hi(vb.z); v[6] = bf16_lo(vb.w); v[7] = bf16_hi(vb.w);
        } else {
            const float4* mq = reinterpret_cast<const float4*>(static_cast<const float*>(mp) + si);
            const float4* vq = reinterpret_cast<const float4*>(static_cast<const float*>(vp) + si);
            const float4 m0 = mq[0], m1 = mq[1], v0 = vq[0], v1 = vq[1];
            m[0] = m0.x; m[1] = m0.y; m[2] = m0.z; m[3] = m0.w;
            m[4] = m1.x; m[5] = m1.y; m[6] = m1.z; m[7] = m1.w;
            v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
            v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float gj = clip ? gv[j] * coef : gv[j];
            adamw_elem(gj, p[j], m[j], v[j], c);
        }
        float4* po = reinterpret_cast<float4*>(master + si);
        po[0] = make_float4(p[0], p[1], p[2], p[3]);
        po[1] = make_float4(p[4], p[5], p[6], p[7]);
        if constexpr (MVBF16) {
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(mp) + si) =
                make_uint4(pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3]),
                           pack_bf16x2(m[4], m[5]), pack_bf16x2(m[6], m[7]));
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(vp) + si) =
                make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                           pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
        } else {
            float4* mo = reinterpret_cast<float4*>(static_cast<float*>(mp) + si);
            float4* vo = reinterpret_cast<float4*>(static_cast<float*>(vp) + si);
            mo[0] = make_float4(m[0], m[1], m[2], m[3]);
            mo[1] = make_float4(m[4], m[5], m[6], m[7]);
            vo[0] = make_float4(v[0], v[1], v[2], v[3]);
            vo[1] = make_float4(v[4], v[5], v[6], v[7]);
        }
        *reinterpret_cast<uint4*>(param + si) =
            make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                       pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));
    } else {
        for (int j = 0; j < n; ++j) {
            float gj = (GSRC == 0) ? g[gi + j] : reduce_one(r, gi + j);
            if (clip) gj = gj * coef;
            float p = master[si + j], m, v;
            if constexpr (MVBF16) {
                m = bf16_to_f32(static_cast<const uint16_t*>(mp)[si + j]);
                v = bf16_to_f32(static_cast<const uint16_t*>(vp)[si + j]);
            } else {
                m = static_cast<const float*>(mp)[si + j];
                v = static_cast<const float*>(vp)[si + j];
            }
            adamw_elem(gj, p, m, v, c);
            master[si + j] = p;
            if constexpr (MVBF16) {
                static_cast<uint16_t*>(mp)[si + j] = (uint16_t)bf16_rne_bits(m);
                static_cast<uint16_t*>(vp)[si + j] = (uint16_t)bf16_rne_bits(v);
            } else {
                static_cast<float*>(mp)[si + j] = m;
                static_cast<float*>(vp)[si + j] = v;
            }
            param[si + j] = (uint16_t)bf16_rne_bits(p);
        }
    }
}

template <int V, int GSRC, bool MVBF16>
__global__ __launch_bounds__(kThreads) void adamw_flat_kernel(const float* __restrict__ g, Reduce r,
                                                              int64_t len, float* __restrict__ master,
                                                              void* __restrict__ m, void* __restrict__ v,
                                                              uint16_t* __restrict__ param, Scal c,
                                                              ClipArgs ca)
{
    bool clip;
    float coef;
    block_clip(ca, clip, coef);
    const int64_t tile = (int64_t)kThreads * V;
    const int64_t ntiles = (len + tile - 1) / tile;
    for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const int64_t e = t * tile + (int64_t)threadIdx.x * V;
        if (e >= len) continue;
        const int n = (int)(len - e < V ? len - e : V);
        step_group<V, GSRC, MVBF16>(g, r, e, master, m, v, param, e, n, c, clip, coef);
    }
}

template <int V, int GSRC, bool MVBF16>
__global__ __launch_bounds__(kThreads) void adamw_mta_kernel(const float* __restrict__ g, Reduce r,
                                                             const PieceDesc* __restrict__ pieces,
                                                             const ChunkDesc* __restrict__ chunks,
                                                             int n_chunks, Scal c,
                                                             ClipArgs ca)
{
    bool clip;
    float coef;
    block_clip(ca, clip, coef);
    for (int k = blockIdx.x; k < n_chunks; k += gridDim.x) {
        const ChunkDesc ch = chunks[k];
        const PieceDesc pc = pieces[ch.piece];
        const int64_t g0 = pc.shard_offset + ch.offset;
        float* master = pc.master + ch.offset;
        void* m = MVBF16 ? (void*)(static_cast<uint16_t*>(pc.m) + ch.offset)
                         : (void*)(static_cast<float*>(pc.m) + ch.offset);
        void* v = MVBF16 ? (void*)(static_cast<uint16_t*>(pc.v) + ch.offset)
                         : (void*)(static_cast<float*>(pc.v) + ch.offset);
        uint16_t* param = pc.param + ch.offset;
        for (int e = threadIdx.x * V; e < ch.len; e += kThreads * V) {
            const int n = ch.len - e < V ? ch.len - e : V;
            step_group<V, GSRC, MVBF16>(g, r, g0 + e, master, m, v, param, e, n, c, clip, coef);
        }
    }
}

}  // namespace

// ------------------------------------------------------------- launchers
hipError_t launch_reduce(const Reduce& r, int64_t len, bool vec, float* g_out, double* partials,
                         int nblocks, hipStream_t s)
{
    const dim3 grid(nblocks), block(kThreads);
    const bool store = g_out != nullptr, norm = partials != nullptr;
#define Z1_REDUCE(V, ST, NO) hipLaunchKernelGGL((reduce_kernel<V, ST, NO>), grid, block, 0, s, r, len, g_out, partials)
    if (vec) {
        if (store && norm) Z1_REDUCE(kVec, true, true);
        else if (store) Z1_REDUCE(kVec, true, false);
        else Z1_REDUCE(kVec, false, true);
    } else {
        if (store && norm) Z1_REDUCE(1, true, true);
        else if (store) Z1_REDUCE(1, true, false);
        else Z1_REDUCE(1, false, true);
    }
#undef Z1_REDUCE
    return hipGetLastError();
}

hipError_t launch_sumsq(const float* g, int64_t len, bool vec, double* partials, int nblocks, hipStream_t s)
{
    if (vec)
        hipLaunchKernelGGL((sumsq_kernel<kVec>), dim3(nblocks), dim3(kThreads), 0, s, g, len, partials);
    else
        hipLaunchKernelGGL((sumsq_kernel<1>), dim3(nblocks), dim3(kThreads), 0, s, g, len, partials);
    return hipGetLastError();
}

hipError_t launch_finalize(const double* partials, int nblocks, double* q_out, hipStream_t s)
{
    hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(kThreads), 0, s, partials, nblocks, q_out);
    return hipGetLastError();
}

hipError_t launch_adamw_flat(const float* g, const Reduce& r, int64_t len, bool vec, bool mv_bf16,
                             float* master, void* m, void* v, uint16_t* param, const Scal& sc,
                             const double* rank_sumsq, int n_ranks, double max_norm, NormInfo* info_out,
                             int nblocks, hipStream_t s)
{
    const dim3 grid(nblocks), block(kThreads);
    const ClipArgs ca{rank_sumsq, n_ranks, max_norm, info_out};
#define Z1_FLAT(V, GS, MV) hipLaunchKernelGGL((adamw_flat_kernel<V, GS, MV>), grid, block, 0, s, g, r, len, master, m, v, param, sc, ca)
    const int gs = g ? 0 : 1;
    if (vec) {
        if (gs == 0) { if (mv_bf16) Z1_FLAT(kVec, 0, true); else Z1_FLAT(kVec, 0, false); }
        else         { if (mv_bf16) Z1_FLAT(kVec, 1, true); else Z1_FLAT(kVec, 1, false); }
    } else {
        if (gs == 0) { if (mv_bf16) Z1_FLAT(1, 0, true); else Z1_FLAT(1, 0, false); }
        else         { if (mv_bf16) Z1_FLAT(1, 1, true); else Z1_FLAT(1, 1, false); }
    }
#undef Z1_FLAT
    return hipGetLastError();
}

hipError_t launch_adamw_mta(const float* g, const Reduce& r, const PieceDesc* pieces, const ChunkDesc* chunks,
                            int n_chunks, bool vec, bool mv_bf16, const Scal& sc, const double* rank_sumsq,
                            int n_ranks, double max_norm, NormInfo* info_out, int nblocks, hipStream_t s)
{
    const dim3 grid(nblocks), block(kThreads);
    const ClipArgs ca{rank_sumsq, n_ranks, max_norm, info_out};
#define Z1_MTA(V, GS, MV) hipLaunchKernelGGL((adamw_mta_kernel<V, GS, MV>), grid, block, 0, s, g, r, pieces, chunks, n_chunks, sc, ca)
    const int gs = g ? 0 : 1;
    if (vec) {
        if (gs == 0) { if (mv_bf16) Z1_MTA(kVec, 0, true); else Z1_MTA(kVec, 0, false); }
        else         { if (mv_bf16) Z1_MTA(kVec, 1, true); else Z1_MTA(kVec, 1, false); }
    } else {
        if (gs == 0) { if (mv_bf16) Z1_MTA(1, 0, true); else Z1_MTA(1, 0, false); }
        else         { if (mv_bf16) Z1_MTA(1, 1, true); else Z1_MTA(1, 1, false); }
    }
#undef Z1_MTA
    return hipGetLastError();
}

}  // namespace z1
