// kernels.hip -- gfx950 kernels of one rank's ZeRO-1 optimizer step.
//
// Everything here is HBM-bound elementwise work (about 0.5 flop per byte), so
// the rules are those of a streaming kernel on CDNA4:
//   * Work is cut into tiles of 2048 elements per 256-lane workgroup.  Inside a
//     tile, wave w owns elements [512w, 512w+512) and lane l of it the two
//     quads [512w+4l, +4) and [512w+256+4l, +4), so every load or store
//     instruction of a wave covers one contiguous run (512 B of bf16, 1 KiB of
//     fp32): fully coalesced for both element sizes.
//   * Every array but g is touched once per step, so those accesses carry the
//     non-temporal hint (global_load/store ... nt): streaming data should not
//     displace anything in L2/MALL.  On MI355X this is worth ~1.5-2x over
//     plain accesses for these kernels.  g, written by the reduce and read
//     back by the update, is stored with the sc1 policy and read with the
//     default one while it fits the MALL.
//   * Workgroups are dispatched to the 8 XCDs round-robin (workgroup b runs
//     on XCD b % 8), and each XCD has its own L2 and address-translation
//     caches.  So the tiles are split into 8 contiguous eighths and XCD x's
//     workgroups walk eighth x with a stride of their own count: each XCD
//     streams through one compact window of every array instead of all 8
//     XCDs touching every page (+10-15% on MI355X, most at multi-GB shards).
//     No atomics, no MFMA (nothing here is a contraction).
//   * Tiles that run past the end, and shards whose pointers are not 16-byte
//     aligned, take an element path (lane t handles t, t+256, ...).
//
// Arithmetic contract: AdamW with the folded bias correction and the decay
// after the Adam move, as "并行训练" defines it in "一张卡上装了什么：混合精度与
// AdamW", evaluated one binary32 operation at a time: built with -ffp-contract=off and the pragma below, so no multiply-add is
// fused; fp32 '/' and sqrtf are the correctly rounded HIP defaults; subnormals
// are kept.  fp64 is used only for sums of squares (each square is exact in
// fp64, so fma(x, x, acc) rounds exactly like acc + x*x).
//
// Determinism: every workgroup owns a fixed set of tiles, every lane adds its
// own elements in a fixed order, a workgroup's lanes are combined by a fixed
// tree (wave butterfly, then the four waves in order) and the workgroups'
// partials by another (finalize_kernel: strided lane sums, then an LDS
// halving tree), so a rerun with the same launch shape reproduces every bit,
// including the norm.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

#include "internal.h"

#pragma clang fp contract(off)

namespace z1 {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------- memory access
// Every buffer the kernels touch is device (global) memory.  Pointers that
// arrive through memory -- the multi-tensor piece descriptors -- are generic
// to the compiler, which then emits FLAT instructions (they also count
// against the LDS/scalar-load counter and go through the aperture check);
// casting to the global address space gives GLOBAL instructions (the
// multi-tensor update measured ~1 % faster on the GPT-2-small shard).
template <typename T>
using gptr = __attribute__((address_space(1))) T*;
template <typename T>
__device__ __forceinline__ gptr<const T> gbl(const T* p) { return (gptr<const T>)p; }
template <typename T>
__device__ __forceinline__ gptr<T> gbl(T* p) { return (gptr<T>)p; }

template <typename T>
__device__ __forceinline__ T ld_nt(const T* p) { return __builtin_nontemporal_load(gbl(p)); }
template <typename T>
__device__ __forceinline__ void st_nt(T* p, T v) { __builtin_nontemporal_store(v, gbl(p)); }

// The reduced gradient g (store-g design) is written by one kernel and read
// back by the next.  The update reads it with the default cache policy, so a
// g that fits in the 256 MB MALL is re-read mostly from there (GPT-2 small
// W=8 shard: update kernel 82 -> 75 us); the reduce stores such a g with sc1
// buffer stores (st8_g_sc1 below; a ragged tail with plain stores) and a
// larger one with the non-temporal hint (NT), where it cannot stay resident
// anyway.
template <bool NT = false, typename T>
__device__ __forceinline__ T ld_g(const T* p)
{
    if constexpr (NT) return __builtin_nontemporal_load(gbl(p)); else return *gbl(p);
}
template <bool NT = false, typename T>
__device__ __forceinline__ void st_g(T* p, T v)
{
    if constexpr (NT) __builtin_nontemporal_store(v, gbl(p)); else *gbl(p) = v;
}

// Offset of this lane's first quad inside a tile (the second is 256 further).
__device__ __forceinline__ int quad_a() { return 512 * (int)(threadIdx.x >> 6) + 4 * (int)(threadIdx.x & 63); }

// ------------------------------------------------------------- work mapping
// The units [lo, hi) and stride of this workgroup when n units are split into
// `split` contiguous parts (8: one per XCD; 1: a plain grid stride).  The
// grid is a multiple of split.
struct Units {
    int64_t lo, hi, step;
};

__device__ __forceinline__ Units xcd_units(int64_t n, int split)
{
    const int64_t G = gridDim.x, b = blockIdx.x;
    const int64_t nx = (split > 1 && G % split == 0) ? split : 1;
    const int64_t x = b % nx, j = b / nx, per = (n + nx - 1) / nx;
    const int64_t lo = x * per;
    const int64_t hi = lo + per < n ? lo + per : n;
    return Units{lo + j, hi, G / nx};
}

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

// Eight values of this lane in a tile starting at p: quad a then quad b.
__device__ __forceinline__ void ld8_bf16(const uint16_t* p, float (&x)[8])
{
    const int a = quad_a();
    const u32x2 u = ld_nt(reinterpret_cast<const u32x2*>(p + a));
    const u32x2 w = ld_nt(reinterpret_cast<const u32x2*>(p + a + 256));
    x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x); x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
    x[4] = bf16_lo(w.x); x[5] = bf16_hi(w.x); x[6] = bf16_lo(w.y); x[7] = bf16_hi(w.y);
}

__device__ __forceinline__ void st8_bf16(uint16_t* p, const float (&x)[8])
{
    const int a = quad_a();
    const u32x2 u = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    const u32x2 w = {pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
    st_nt(reinterpret_cast<u32x2*>(p + a), u);
    st_nt(reinterpret_cast<u32x2*>(p + a + 256), w);
}

__device__ __forceinline__ void ld8_f32(const float* p, float (&x)[8])
{
    const int a = quad_a();
    const f32x4 u = ld_nt(reinterpret_cast<const f32x4*>(p + a));
    const f32x4 w = ld_nt(reinterpret_cast<const f32x4*>(p + a + 256));
    x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
    x[4] = w.x; x[5] = w.y; x[6] = w.z; x[7] = w.w;
}

template <bool NT = false>
__device__ __forceinline__ void st8_g(float* p, const float (&x)[8])
{
    const int a = quad_a();
    const f32x4 u = {x[0], x[1], x[2], x[3]};
    const f32x4 w = {x[4], x[5], x[6], x[7]};
    st_g<NT>(reinterpret_cast<f32x4*>(p + a), u);
    st_g<NT>(reinterpret_cast<f32x4*>(p + a + 256), w);
}

// g kept for the update to re-read (small enough for the MALL) is stored
// through a buffer descriptor with the sc1 policy bit rather than a plain
// store: measured ~2.5 us less per reduce at the GPT-2-small W=8 shard, with
// the same update time (the lines leave L2 as they are written instead of
// waiting, dirty, for the write-back at the end of the kernel).  One
// descriptor per tile (base = the tile, 8 KiB), so offsets stay small for any
// shard size.
constexpr int kBufSc1 = 16;                   // cache-policy operand of buffer stores: sc1
constexpr int kBufDword3 = 0x00020000;        // gfx9 buffer descriptor word 3 (raw, untyped)

// The lane's 8 values of the tile that starts at `tile`.
__device__ __forceinline__ void st8_g_sc1(float* tile, const float (&x)[8])
{
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(tile, 0, kTile * 4, kBufDword3);
    const int a = quad_a();
    const f32x4 u = {x[0], x[1], x[2], x[3]};
    const f32x4 w = {x[4], x[5], x[6], x[7]};
    __builtin_amdgcn_raw_buffer_store_b128(u, rs, a * 4, 0, kBufSc1);
    __builtin_amdgcn_raw_buffer_store_b128(w, rs, (a + 256) * 4, 0, kBufSc1);
}

__device__ __forceinline__ void ld8_g(const float* p, float (&x)[8])
{
    const int a = quad_a();
    const f32x4 u = ld_g(reinterpret_cast<const f32x4*>(p + a));
    const f32x4 w = ld_g(reinterpret_cast<const f32x4*>(p + a + 256));
    x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
    x[4] = w.x; x[5] = w.y; x[6] = w.z; x[7] = w.w;
}

__device__ __forceinline__ void st8_f32(float* p, const float (&x)[8])
{
    const int a = quad_a();
    const f32x4 u = {x[0], x[1], x[2], x[3]};
    const f32x4 w = {x[4], x[5], x[6], x[7]};
    st_nt(reinterpret_cast<f32x4*>(p + a), u);
    st_nt(reinterpret_cast<f32x4*>(p + a + 256), w);
}

// ------------------------------------------------------------- reduction
// Accumulation order for every element: s = G_0; s = s + G_w for w = 1..W-1;
// then the average (multiply by the exact 2^-k, or an IEEE division).
__device__ __forceinline__ float average(const Reduce& r, float s)
{
    if (r.mode == kAvgMulPow2) s = s * r.inv_w;
    else if (r.mode == kAvgDiv) s = s / r.f_w;
    // compatibility variant: the reduced gradient as a bf16 reduce-scatter
    // would deliver it (nearest even), widened back for the update
    if (r.round_bf16) s = __uint_as_float(bf16_rne_bits(s) << 16);
    return s;
}

// One slice's share of a tile for this lane, as loaded: two 8-byte words of
// four bf16 each (quad a, quad a+256).  Kept packed until the add so that a
// batch of eight slices holds 32 registers, not 64.
struct Raw {
    u32x2 a, b;
};

__device__ __forceinline__ Raw ld_raw(const uint16_t* p)
{
    const int a = quad_a();
    return Raw{ld_nt(reinterpret_cast<const u32x2*>(p + a)), ld_nt(reinterpret_cast<const u32x2*>(p + a + 256))};
}

__device__ __forceinline__ void raw_init(float (&s)[8], const Raw& x)
{
    s[0] = bf16_lo(x.a.x); s[1] = bf16_hi(x.a.x); s[2] = bf16_lo(x.a.y); s[3] = bf16_hi(x.a.y);
    s[4] = bf16_lo(x.b.x); s[5] = bf16_hi(x.b.x); s[6] = bf16_lo(x.b.y); s[7] = bf16_hi(x.b.y);
}

__device__ __forceinline__ void raw_add(float (&s)[8], const Raw& x)
{
    s[0] = s[0] + bf16_lo(x.a.x); s[1] = s[1] + bf16_hi(x.a.x);
    s[2] = s[2] + bf16_lo(x.a.y); s[3] = s[3] + bf16_hi(x.a.y);
    s[4] = s[4] + bf16_lo(x.b.x); s[5] = s[5] + bf16_hi(x.b.x);
    s[6] = s[6] + bf16_lo(x.b.y); s[7] = s[7] + bf16_hi(x.b.y);
}

// Slices [w0, w0+B) of the tile at e: all B loads are issued before the first
// add.  The first batch starts the sum (s = G_0) and runs mid() right after
// its loads are issued: the caller's stores placed there leave the memory
// queue behind this tile's loads, so waiting for the loads does not also wait
// for the stores (loads and stores retire through one in-order counter).
template <int B, bool FIRST, typename Mid>
__device__ __forceinline__ void reduce_batch(const Reduce& r, int w0, int64_t e, float (&s)[8], Mid& mid)
{
    Raw x[B];
#pragma unroll
    for (int k = 0; k < B; ++k) x[k] = ld_raw(r.gp.p[w0 + k] + e);
    if constexpr (FIRST) mid();
#pragma unroll
    for (int k = 0; k < B; ++k) {
        if (FIRST && k == 0) raw_init(s, x[0]);
        else raw_add(s, x[k]);
    }
}

// This lane's 8 reduced values of the tile at shard index e (vector path):
// s = G_0 + G_1 + ... + G_{W-1} in rank order, in batches of eight slices,
// then one of four, two, then single slices; then the average.
template <typename Mid>
__device__ __forceinline__ void reduce8(const Reduce& r, int64_t e, float (&s)[8], Mid mid)
{
    int w0;
    if (r.W >= 8) {
        reduce_batch<8, true>(r, 0, e, s, mid);
        for (w0 = 8; w0 + 8 <= r.W; w0 += 8) reduce_batch<8, false>(r, w0, e, s, mid);
    } else if (r.W >= 4) {
        reduce_batch<4, true>(r, 0, e, s, mid);
        w0 = 4;
    } else {
        reduce_batch<1, true>(r, 0, e, s, mid);
        w0 = 1;
    }
    if (w0 + 4 <= r.W) { reduce_batch<4, false>(r, w0, e, s, mid); w0 += 4; }
    if (w0 + 2 <= r.W) { reduce_batch<2, false>(r, w0, e, s, mid); w0 += 2; }
    if (w0 < r.W) reduce_batch<1, false>(r, w0, e, s, mid);
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] = average(r, s[j]);
}

__device__ __forceinline__ void reduce8(const Reduce& r, int64_t e, float (&s)[8])
{
    reduce8(r, e, s, [] {});
}

__device__ __forceinline__ float reduce1(const Reduce& r, int64_t e)
{
    float a = bf16_to_f32(ld_nt(r.gp.p[0] + e));
    for (int w = 1; w < r.W; ++w)
        a = a + bf16_to_f32(ld_nt(r.gp.p[w] + e));
    return average(r, a);
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

// The sum-of-squares pass that stores nothing (the first pass of the
// recompute design) over whole tiles when there are few slices: one tile of
// WS slices is only 8*WS bytes per lane, too little in flight to keep HBM
// busy, so the loads of U tiles are issued together (U = 4 for one or two
// slices, 2 for three or four; with the grid of kFewPerCu workgroups per CU,
// the shape measured best on MI355X).  The tiles are then reduced and
// squared in tile order, so acc
// takes the same sequence of values as one tile at a time.  Returns the
// first tile not processed.
template <int WS, int U>
__device__ __forceinline__ int64_t norm_tiles(const Reduce& r, int64_t t, int64_t end, int64_t step, double& acc)
{
    for (; t + (U - 1) * step < end; t += U * step) {
        Raw x[U][WS];
#pragma unroll
        for (int k = 0; k < U; ++k) {
#pragma unroll
            for (int w = 0; w < WS; ++w) x[k][w] = ld_raw(r.gp.p[w] + (t + k * step) * kTile);
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            float sv[8];
            raw_init(sv, x[k][0]);
#pragma unroll
            for (int w = 1; w < WS; ++w) raw_add(sv, x[k][w]);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                sv[j] = average(r, sv[j]);
                acc = fma((double)sv[j], (double)sv[j], acc);
            }
        }
    }
    return t;
}

// ------------------------------------------------------------- phase 1
// W-slice reduce over the workgroup's tiles; optionally stores g (GNT: with
// the non-temporal hint, for g larger than the MALL) and accumulates this
// lane's fp64 sum of squares.  Full tiles run a software pipeline: tile t's g
// is stored only after tile t+step's loads are issued.  A ragged last tile
// takes the element path.  FEW (1..4, sum of squares only): the launch has
// exactly that many slices and the whole tiles go through norm_tiles (a
// separate instantiation, so that its registers do not lower the occupancy
// of the general kernel).
template <bool VEC, bool STORE, bool NORM, bool GNT, int FEW>
__global__ __launch_bounds__(kThreads) void reduce_kernel(Reduce r, int64_t len, float* __restrict__ g_out,
                                                          double* __restrict__ partials, int split)
{
    double acc = 0.0;
    const int64_t ntiles = (len + kTile - 1) / kTile;
    const Units u = xcd_units(ntiles, split);
    int64_t t = u.lo;
    const int64_t full_end = VEC ? (u.hi < len / kTile ? u.hi : len / kTile) : u.lo;
    static_assert(FEW == 0 || (VEC && !STORE && NORM && FEW <= 4), "few-slice pass: vector, sum of squares only");
    if constexpr (FEW > 0) t = norm_tiles<FEW, FEW <= 2 ? 4 : 2>(r, t, full_end, u.step, acc);
    if (VEC && t < full_end) {
        float sp[8];                // the previous tile's g, stored after the next tile's loads
        int64_t tp = t;
        reduce8(r, t * kTile, sp);
        if constexpr (NORM) {
#pragma unroll
            for (int j = 0; j < 8; ++j) acc = fma((double)sp[j], (double)sp[j], acc);
        }
        for (t += u.step; t < full_end; t += u.step) {
            float s[8];
            reduce8(r, t * kTile, s, [&] {
                if constexpr (STORE && GNT) st8_g<true>(g_out + tp * kTile, sp);
                if constexpr (STORE && !GNT) st8_g_sc1(g_out + tp * kTile, sp);
            });
            if constexpr (NORM) {
#pragma unroll
                for (int j = 0; j < 8; ++j) acc = fma((double)s[j], (double)s[j], acc);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) sp[j] = s[j];
            tp = t;
        }
        if constexpr (STORE && GNT) st8_g<true>(g_out + tp * kTile, sp);
        if constexpr (STORE && !GNT) st8_g_sc1(g_out + tp * kTile, sp);
    }
    for (; t < u.hi; t += u.step) {
        const int64_t base = t * kTile;
        for (int64_t e = base + threadIdx.x; e < base + kTile && e < len; e += kThreads) {
            const float x = reduce1(r, e);
            if constexpr (STORE) st_g<GNT>(g_out + e, x);
            if constexpr (NORM) acc = fma((double)x, (double)x, acc);
        }
    }
    if constexpr (NORM) {
        const double b = block_sum(acc);
        if (threadIdx.x == 0) partials[blockIdx.x] = b;
    }
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void sumsq_kernel(const float* __restrict__ g, int64_t len,
                                                         double* __restrict__ partials, int split)
{
    double acc = 0.0;
    const int64_t ntiles = (len + kTile - 1) / kTile;
    const Units u = xcd_units(ntiles, split);
    for (int64_t t = u.lo; t < u.hi; t += u.step) {
        const int64_t base = t * kTile;
        if (VEC && base + kTile <= len) {
            float s[8];
            ld8_f32(g + base, s);
#pragma unroll
            for (int j = 0; j < 8; ++j) acc = fma((double)s[j], (double)s[j], acc);
        } else {
            for (int64_t e = base + threadIdx.x; e < base + kTile && e < len; e += kThreads) {
                const double x = (double)ld_nt(g + e);
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
    // the lane's strided subset in order; loads issued 8 at a time so that
    // their latencies overlap (the adds stay in the same order)
    for (int i0 = threadIdx.x; i0 < nb; i0 += 8 * kThreads) {
        double x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int i = i0 + k * kThreads;
            x[k] = i < nb ? partials[i] : 0.0;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (i0 + k * kThreads < nb) a = a + x[k];
    }
    sh[threadIdx.x] = a;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) sh[threadIdx.x] = sh[threadIdx.x] + sh[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) *q_out = sh[0];
}

// Global norm and clip decision from the sum of the ranks' partial sums of
// squares ("训练循环与 checkpoint": clip all gradients as one vector when the
// L2 norm exceeds max_norm).  clip_eps selects the torch convention instead:
// coefficient max_norm / (norm + 1e-6), applied when it is below 1.
__device__ __forceinline__ NormInfo norm_info(double tot, double max_norm, int clip_eps)
{
    NormInfo ni;
    ni.sumsq_total = tot;
    ni.norm = sqrt(tot);
    const double c = clip_eps ? max_norm / (ni.norm + 1e-6) : max_norm / ni.norm;
    const bool clip = clip_eps ? (c < 1.0) : (ni.norm > max_norm);
    ni.clip = clip ? 1 : 0;
    ni.clip_coef = clip ? (float)c : 1.0f;
    ni.nonfinite = (isnan(ni.norm) || isinf(ni.norm)) ? 1 : 0;
    ni.reserved = 0;
    return ni;
}

// The partials are added in rank order, so every workgroup that evaluates
// this gets the same bits.
__device__ __forceinline__ NormInfo clip_info(const double* rank_sumsq, int n_ranks, double max_norm,
                                              int clip_eps)
{
    double tot = 0.0;
    for (int q = 0; q < n_ranks; ++q) tot = tot + rank_sumsq[q];
    return norm_info(tot, max_norm, clip_eps);
}

// Steps replayed from a captured graph carry their per-step scalars in device
// memory: every update kernel swaps them in before anything else.
__device__ __forceinline__ void use_device_scalars(Scal& c, double& max_norm)
{
    if (c.dev) {
        const StepScal d = *c.dev;
        c.b1 = d.b1; c.b2 = d.b2; c.a1 = d.a1; c.a2 = d.a2;
        c.eps = d.eps; c.sigma = d.sigma; c.delta = d.delta;
        max_norm = d.max_norm;
    }
}

// Prologue of every update kernel: lane 0 forms the clip decision, workgroup 0
// publishes it, and the whole workgroup reads it from LDS.
struct ClipArgs {
    const double* rank_sumsq;
    int n_ranks;
    double max_norm;
    int clip_eps;
    NormInfo* info_out;   // may be null
};

__device__ __forceinline__ void block_clip(const ClipArgs& ca, bool& clip, float& coef)
{
    __shared__ NormInfo sh;
    if (threadIdx.x == 0) {
        sh = clip_info(ca.rank_sumsq, ca.n_ranks, ca.max_norm, ca.clip_eps);
        if (blockIdx.x == 0 && ca.info_out) *ca.info_out = sh;
    }
    __syncthreads();
    clip = sh.clip != 0;
    coef = sh.clip_coef;
}

// ------------------------------------------------------------- phase 2
// One element of AdamW: m = b1 m + a1 g, v = b2 v + a2 (g g), then the
// master moves by sigma m / (sqrt(v) + eps) and is multiplied by the decay
// factor (decay after the move; decay_first swaps the two).
__device__ __forceinline__ void adamw_elem(float g, float& p, float& m, float& v, const Scal& c)
{
    const float mn = c.b1 * m + c.a1 * g;
    const float vn = c.b2 * v + c.a2 * (g * g);
    const float d = sqrtf(vn) + c.eps;
    const float q = mn / d;
    float pn;
    if (c.decay_first) {   // compatibility variant: decay, then update
        pn = p * c.delta;
        pn = pn - c.sigma * q;
    } else {
        pn = p - c.sigma * q;
        pn = pn * c.delta;
    }
    m = mn;
    v = vn;
    p = pn;
}

// Where the update finds its arrays: g (fp32 buffer; unused when the gradient
// is recomputed from the slices) and the state and param of one span.
struct Span {
    const float* g;
    float* master;
    void* m;
    void* v;
    uint16_t* param;
};

// The lane's 8 elements of a full tile at state index si, given their g.
template <bool MVBF16>
__device__ __forceinline__ void update8(const Span& sp, int64_t si, const float (&gv)[8], const Scal& c, bool clip,
                                        float coef)
{
    float p[8], m[8], v[8];
    ld8_f32(sp.master + si, p);
    if constexpr (MVBF16) {
        ld8_bf16(static_cast<const uint16_t*>(sp.m) + si, m);
        ld8_bf16(static_cast<const uint16_t*>(sp.v) + si, v);
    } else {
        ld8_f32(static_cast<const float*>(sp.m) + si, m);
        ld8_f32(static_cast<const float*>(sp.v) + si, v);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float gj = clip ? gv[j] * coef : gv[j];
        adamw_elem(gj, p[j], m[j], v[j], c);
    }
    st8_f32(sp.master + si, p);
    if constexpr (MVBF16) {
        st8_bf16(static_cast<uint16_t*>(sp.m) + si, m);
        st8_bf16(static_cast<uint16_t*>(sp.v) + si, v);
    } else {
        st8_f32(static_cast<float*>(sp.m) + si, m);
        st8_f32(static_cast<float*>(sp.v) + si, v);
    }
    st8_bf16(sp.param + si, p);
}

// One element at state index si, given its g.
template <bool MVBF16>
__device__ __forceinline__ void update1(const Span& sp, int64_t si, float gj, const Scal& c, bool clip, float coef)
{
    if (clip) gj = gj * coef;
    float p = ld_nt(sp.master + si), m, v;
    if constexpr (MVBF16) {
        m = bf16_to_f32(ld_nt(static_cast<const uint16_t*>(sp.m) + si));
        v = bf16_to_f32(ld_nt(static_cast<const uint16_t*>(sp.v) + si));
    } else {
        m = ld_nt(static_cast<const float*>(sp.m) + si);
        v = ld_nt(static_cast<const float*>(sp.v) + si);
    }
    adamw_elem(gj, p, m, v, c);
    st_nt(sp.master + si, p);
    if constexpr (MVBF16) {
        st_nt(static_cast<uint16_t*>(sp.m) + si, (uint16_t)bf16_rne_bits(m));
        st_nt(static_cast<uint16_t*>(sp.v) + si, (uint16_t)bf16_rne_bits(v));
    } else {
        st_nt(static_cast<float*>(sp.m) + si, m);
        st_nt(static_cast<float*>(sp.v) + si, v);
    }
    st_nt(sp.param + si, (uint16_t)bf16_rne_bits(p));
}

// One tile [0, n) of a span (n <= kTile), g at shard index gi, state at si:
// vector path when the whole tile is present (and VEC), element path otherwise.
template <bool VEC, int GSRC, bool MVBF16>
__device__ __forceinline__ void update_tile(const Span& sp, const Reduce& r, int64_t gi, int64_t si, int n,
                                            const Scal& c, bool clip, float coef)
{
    if (VEC && n == kTile) {
        float gv[8];
        if constexpr (GSRC == 0) ld8_g(sp.g + gi, gv);
        else reduce8(r, gi, gv);
        update8<MVBF16>(sp, si, gv, c, clip, coef);
    } else {
        for (int j = threadIdx.x; j < n; j += kThreads) {
            const float gj = (GSRC == 0) ? ld_g(sp.g + gi + j) : reduce1(r, gi + j);
            update1<MVBF16>(sp, si + j, gj, c, clip, coef);
        }
    }
}

template <bool VEC, int GSRC, bool MVBF16>
__global__ __launch_bounds__(kThreads) void adamw_flat_kernel(Span sp, Reduce r, int64_t len, Scal c,
                                                              ClipArgs ca, int split)
{
    use_device_scalars(c, ca.max_norm);
    bool clip;
    float coef;
    block_clip(ca, clip, coef);
    const int64_t ntiles = (len + kTile - 1) / kTile;
    const Units u = xcd_units(ntiles, split);
    for (int64_t t = u.lo; t < u.hi; t += u.step) {
        const int64_t base = t * kTile;
        const int n = (int)(len - base < kTile ? len - base : kTile);
        update_tile<VEC, GSRC, MVBF16>(sp, r, base, base, n, c, clip, coef);
    }
}

// Span of one chunk's piece, starting at the chunk.
template <bool MVBF16>
__device__ __forceinline__ Span chunk_span(const PieceDesc& pc, const ChunkDesc& ch)
{
    const size_t mvb = MVBF16 ? 2 : 4;
    Span sp;
    sp.g = nullptr;
    sp.master = pc.master + ch.offset;
    sp.m = static_cast<char*>(pc.m) + mvb * ch.offset;
    sp.v = static_cast<char*>(pc.v) + mvb * ch.offset;
    sp.param = pc.param + ch.offset;
    return sp;
}

template <bool VEC, int GSRC, bool MVBF16>
__global__ __launch_bounds__(kThreads) void adamw_mta_kernel(const float* __restrict__ g, Reduce r,
                                                             const PieceDesc* __restrict__ pieces,
                                                             const ChunkDesc* __restrict__ chunks,
                                                             int n_chunks, Scal c, ClipArgs ca, int split)
{
    use_device_scalars(c, ca.max_norm);
    bool clip;
    float coef;
    block_clip(ca, clip, coef);
    const Units u = xcd_units(n_chunks, split);
    for (int64_t k = u.lo; k < u.hi; k += u.step) {
        const ChunkDesc ch = chunks[k];
        const PieceDesc pc = pieces[ch.piece];
        Span sp = chunk_span<MVBF16>(pc, ch);
        sp.g = g;
        const int64_t g0 = pc.shard_offset + ch.offset;
        for (int sub = 0; sub < ch.len; sub += kTile) {
            const int n = ch.len - sub < kTile ? ch.len - sub : kTile;
            update_tile<VEC, GSRC, MVBF16>(sp, r, g0 + sub, sub, n, c, clip, coef);
        }
    }
}

// ------------------------------------------------------------- launch helper
// Timing events requested for the next launch on this thread
// (zero1_time_next_launch): the first kernel launched after the request takes
// them, stamped by its own dispatch.
thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;

// Launches kernel<<<grid, kThreads, 0, s>>>(args...), with the arguments
// converted to the kernel's parameter types; with a timing request pending,
// through hipExtLaunchKernel so that the events bracket this kernel alone
// (refused while s is being captured into a graph).
template <typename... P, typename... A>
hipError_t run(void (*kernel)(P...), dim3 grid, hipStream_t s, const A&... args)
{
    static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
    std::tuple<P...> formal{args...};
    void* argv[sizeof...(P)];
    std::apply([&argv](auto&... x) {
        int i = 0;
        ((argv[i++] = static_cast<void*>(&x)), ...);
    }, formal);
    const void* f = reinterpret_cast<const void*>(kernel);
    if (t_ev_start || t_ev_stop) {
        const hipEvent_t a = t_ev_start, b = t_ev_stop;
        t_ev_start = t_ev_stop = nullptr;
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        const hipError_t e = hipStreamIsCapturing(s, &cs);
        if (e != hipSuccess) return e;
        if (cs != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
        return hipExtLaunchKernel(f, grid, dim3(kThreads), argv, 0, s, a, b, 0);
    }
    return hipLaunchKernel(f, grid, dim3(kThreads), argv, 0, s);
}

}  // namespace

void set_launch_events(hipEvent_t start, hipEvent_t stop)
{
    t_ev_start = start;
    t_ev_stop = stop;
}

// ------------------------------------------------------------- launchers
hipError_t launch_reduce(const Reduce& r, int64_t len, bool vec, float* g_out, double* partials,
                         int nblocks, int split, bool g_nt, hipStream_t s)
{
    const dim3 grid(nblocks);
    const bool store = g_out != nullptr, norm = partials != nullptr;
    hipError_t e;
    if (few_slice_pass(vec, store, norm, r.W)) {
        switch (r.W) {
        case 1: return run(reduce_kernel<true, false, true, false, 1>, grid, s, r, len, g_out, partials, split);
        case 2: return run(reduce_kernel<true, false, true, false, 2>, grid, s, r, len, g_out, partials, split);
        case 3: return run(reduce_kernel<true, false, true, false, 3>, grid, s, r, len, g_out, partials, split);
        default: return run(reduce_kernel<true, false, true, false, 4>, grid, s, r, len, g_out, partials, split);
        }
    }
#define Z1_REDUCE(V, ST, NO, NT) e = run(reduce_kernel<V, ST, NO, NT, 0>, grid, s, r, len, g_out, partials, split)
#define Z1_REDUCE_V(V)                                                  \
    do {                                                                \
        if (store && norm) {                                            \
            if (g_nt) Z1_REDUCE(V, true, true, true);                   \
            else Z1_REDUCE(V, true, true, false);                       \
        } else if (store) {                                             \
            if (g_nt) Z1_REDUCE(V, true, false, true);                  \
            else Z1_REDUCE(V, true, false, false);                      \
        } else {                                                        \
            Z1_REDUCE(V, false, true, false);                           \
        }                                                               \
    } while (0)
    if (vec) Z1_REDUCE_V(true);
    else Z1_REDUCE_V(false);
#undef Z1_REDUCE_V
#undef Z1_REDUCE
    return e;
}

hipError_t launch_sumsq(const float* g, int64_t len, bool vec, double* partials, int nblocks, int split,
                        hipStream_t s)
{
    if (vec) return run(sumsq_kernel<true>, dim3(nblocks), s, g, len, partials, split);
    return run(sumsq_kernel<false>, dim3(nblocks), s, g, len, partials, split);
}

hipError_t launch_finalize(const double* partials, int nblocks, double* q_out, hipStream_t s)
{
    return run(finalize_kernel, dim3(1), s, partials, nblocks, q_out);
}

hipError_t launch_adamw_flat(const float* g, const Reduce& r, int64_t len, bool vec, bool mv_bf16,
                             float* master, void* m, void* v, uint16_t* param, const Scal& sc,
                             const double* rank_sumsq, int n_ranks, double max_norm, int clip_eps,
                             NormInfo* info_out, int nblocks, int split, hipStream_t s)
{
    const dim3 grid(nblocks);
    const ClipArgs ca{rank_sumsq, n_ranks, max_norm, clip_eps, info_out};
    const Span sp{g, master, m, v, param};
    hipError_t e;
#define Z1_FLAT(V, GS, MV) e = run(adamw_flat_kernel<V, GS, MV>, grid, s, sp, r, len, sc, ca, split)
    const int gs = g ? 0 : 1;
    if (vec) {
        if (gs == 0) { if (mv_bf16) Z1_FLAT(true, 0, true); else Z1_FLAT(true, 0, false); }
        else         { if (mv_bf16) Z1_FLAT(true, 1, true); else Z1_FLAT(true, 1, false); }
    } else {
        if (gs == 0) { if (mv_bf16) Z1_FLAT(false, 0, true); else Z1_FLAT(false, 0, false); }
        else         { if (mv_bf16) Z1_FLAT(false, 1, true); else Z1_FLAT(false, 1, false); }
    }
#undef Z1_FLAT
    return e;
}

hipError_t launch_adamw_mta(const float* g, const Reduce& r, const PieceDesc* pieces, const ChunkDesc* chunks,
                            int n_chunks, bool vec, bool mv_bf16, const Scal& sc, const double* rank_sumsq,
                            int n_ranks, double max_norm, int clip_eps, NormInfo* info_out, int nblocks,
                            int split, hipStream_t s)
{
    const dim3 grid(nblocks);
    const ClipArgs ca{rank_sumsq, n_ranks, max_norm, clip_eps, info_out};
    hipError_t e;
#define Z1_MTA(V, GS, MV) e = run(adamw_mta_kernel<V, GS, MV>, grid, s, g, r, pieces, chunks, n_chunks, sc, ca, split)
    const int gs = g ? 0 : 1;
    if (vec) {
        if (gs == 0) { if (mv_bf16) Z1_MTA(true, 0, true); else Z1_MTA(true, 0, false); }
        else         { if (mv_bf16) Z1_MTA(true, 1, true); else Z1_MTA(true, 1, false); }
    } else {
        if (gs == 0) { if (mv_bf16) Z1_MTA(false, 0, true); else Z1_MTA(false, 0, false); }
        else         { if (mv_bf16) Z1_MTA(false, 1, true); else Z1_MTA(false, 1, false); }
    }
#undef Z1_MTA
    return e;
}

}  // namespace z1
