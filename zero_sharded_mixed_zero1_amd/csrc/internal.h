// internal.h -- declarations shared by the C-ABI host code (api.cpp) and the
// gfx950 kernels (kernels.hip) of libzero1.so.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace z1 {

constexpr int kMaxW = 128;          // == ZERO1_MAX_W
constexpr int kThreads = 256;       // threads per workgroup (4 waves of 64)
constexpr int kVec = 8;             // alignment unit (elements) of the vector path
constexpr int kTile = 2048;         // elements per workgroup tile: 256 lanes x 8
constexpr int kMaxPartials = 8192;  // capacity of the per-workgroup norm partials
constexpr int kChunkElems = 2048;   // multi-tensor chunk: one tile

// Launch shape and cache-policy thresholds, fixed at build time (the values
// measured best on MI355X).  The grid shapes decide how the fp64 sum of
// squares is split into partials, so they are constants of the library, not
// run-time settings: the same build gives the same bits in every process.
#ifndef Z1_REDUCE_PER_CU
#define Z1_REDUCE_PER_CU 8          // reduce: persistent grid of 8 workgroups per CU
#endif
#ifndef Z1_FEW_PER_CU
#define Z1_FEW_PER_CU 6             // sum-of-squares pass over 1-4 slices: 6 workgroups per CU
#endif
#ifndef Z1_UPDATE_PER_CU
#define Z1_UPDATE_PER_CU 8          // update past kMaxPartials units: 8 workgroups per CU
#endif
#ifndef Z1_G_NT_BYTES
#define Z1_G_NT_BYTES (128ll << 20) // g larger than this is stored non-temporally
#endif
// Workspace layout (zero1_workspace_bytes): the norm info, the per-workgroup
// fp64 partials, then the fp32 g of the store-g design.
constexpr size_t kInfoBytes = 256;
constexpr size_t kPartialBytes = sizeof(double) * kMaxPartials;
constexpr size_t kGOffset = kInfoBytes + kPartialBytes;   // multiple of 256

constexpr int kReducePerCu = Z1_REDUCE_PER_CU;
constexpr int kFewPerCu = Z1_FEW_PER_CU;
constexpr int kUpdatePerCu = Z1_UPDATE_PER_CU;
constexpr long long kGNtBytes = Z1_G_NT_BYTES;

// W gradient slice pointers, passed by value in the kernel arguments (1 KiB).
struct GradPtrs {
    const uint16_t* p[kMaxW];
};

// Per-step fp32 scalars, formed in fp64 on the host and rounded once.
// The device copy of one step's scalars (zero1_step_scalars).
struct StepScal {
    float b1, b2, a1, a2, eps, sigma, delta, reserved;
    double max_norm;
};

struct Scal {
    float b1, b2, a1, a2, eps, sigma, delta;
    int decay_first;        // 1: decay the master before the Adam update
    const StepScal* dev;    // non-null: read b1..delta and max_norm from here at run time
};

// How the W-slice sum becomes g: keep it, multiply by the exact 2^-k (W a
// power of two: identical to dividing), or divide by W.
enum AvgMode : int { kAvgNone = 0, kAvgMulPow2 = 1, kAvgDiv = 2 };

struct Reduce {
    GradPtrs gp;   // already offset to the shard's first element
    int W;
    int mode;      // AvgMode
    float inv_w;   // 2^-k for kAvgMulPow2
    float f_w;     // (float)W for kAvgDiv
    int round_bf16;  // 1: g is rounded to the nearest bf16 after the average
};

// Same layout as zero1_norm_info.
struct NormInfo {
    double sumsq_total;
    double norm;
    float clip_coef;
    int32_t clip;
    int32_t nonfinite;
    int32_t reserved;
};

// Device-side piece descriptor (48 bytes) and chunk descriptor (16 bytes).
struct PieceDesc {
    int64_t numel;
    int64_t shard_offset;
    uint16_t* param;
    float* master;
    void* m;
    void* v;
};

struct ChunkDesc {
    int32_t piece;
    int32_t len;
    int64_t offset;   // element offset inside the piece
};

// ---- error state of the calling thread (zero1_last_error): records the
// message and returns st (a zero1_status).
int set_error(int st, const char* msg);

// ---- timing request for the next launch on the calling thread
// (zero1_time_next_launch): the next kernel the launchers below start takes
// the events (start and stop stamped by its own dispatch) and clears them.
void set_launch_events(hipEvent_t start, hipEvent_t stop);

// ---- launchers (kernels.hip); each returns the launch's status.
// Phase 1: g = reduce(slices) over [0, len); optional fp32 store of g and one
// fp64 partial sum of squares per workgroup (nblocks of them).
// `split`: 8 splits the units into one contiguous part per XCD, 1 is a plain
// grid stride (nblocks must be a multiple of split).  g_nt: store g with the
// non-temporal hint.
hipError_t launch_reduce(const Reduce& r, int64_t len, bool vec, float* g_out,
                         double* partials, int nblocks, int split, bool g_nt, hipStream_t s);
// launch_reduce runs the few-slice sum-of-squares kernel (loads of several
// tiles issued together, its own grid of kFewPerCu workgroups per CU) when it
// only sums squares on the vector path over at most four slices.
inline bool few_slice_pass(bool vec, bool store_g, bool norm, int W) { return vec && norm && !store_g && W <= 4; }
// Sum of squares of an fp32 vector, one partial per workgroup.
hipError_t launch_sumsq(const float* g, int64_t len, bool vec, double* partials,
                        int nblocks, int split, hipStream_t s);
// One workgroup: add the per-workgroup partials in a fixed order into *q_out.
hipError_t launch_finalize(const double* partials, int nblocks, double* q_out, hipStream_t s);
// Phase 2 over a flat shard.  g == nullptr: recompute g from r.  Every
// workgroup first forms the global norm from rank_sumsq[0..n_ranks) (in rank
// order) and the clip decision for max_norm; workgroup 0 writes it to info_out.
// clip_eps selects the torch clip convention (max_norm / (norm + 1e-6) < 1).
hipError_t launch_adamw_flat(const float* g, const Reduce& r, int64_t len, bool vec,
                             bool mv_bf16, float* master, void* m, void* v,
                             uint16_t* param, const Scal& sc, const double* rank_sumsq,
                             int n_ranks, double max_norm, int clip_eps, NormInfo* info_out,
                             int nblocks, int split, hipStream_t s);
// Phase 2 over a multi-tensor plan (same prologue).
hipError_t launch_adamw_mta(const float* g, const Reduce& r, const PieceDesc* pieces,
                            const ChunkDesc* chunks, int n_chunks, bool vec,
                            bool mv_bf16, const Scal& sc, const double* rank_sumsq,
                            int n_ranks, double max_norm, int clip_eps, NormInfo* info_out,
                            int nblocks, int split, hipStream_t s);

}  // namespace z1
