// calib.hip -- bandwidth calibration kernels for measurement (libzero1_calib.so).
//
// Not part of the optimizer step: these kernels move bytes in the exact access
// pattern of the step kernels and compute nothing, so that their time is what
// HBM delivers for that traffic mix and that placement of the arrays.  A step
// kernel's time over the matching calibration time is then its efficiency
// against an achievable ceiling, next to its fraction of the nominal 8 TB/s.
//
// Access pattern (the same as the step kernels): tiles of 2048 elements per
// 256-lane workgroup; lane l of wave w owns the quads [512w + 4l, +4) and
// [512w + 256 + 4l, +4) of a tile, so every wave instruction covers one
// contiguous run (512 B of a 2-byte stream, 1 KiB of a 4-byte one); loads and
// stores carry the non-temporal hint; read streams are loaded in batches of up
// to eight before any is used; with split = 8 the tiles are split into eight
// contiguous parts, one per XCD (workgroup b runs on XCD b % 8), each walked
// with a stride of that XCD's workgroup count; with split = 1, one grid stride.
//
// Every read stream is folded into a per-lane XOR (so no load can be dropped)
// and every write stream receives that XOR, so the bytes moved are exactly
// tiles * 2048 * (sum of the streams' element sizes).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 2048;
constexpr int kMaxRd = 128;
constexpr int kMaxWr = 8;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Streams {
    const void* rd[kMaxRd];
    void* wr[kMaxWr];
    uint8_t rd_bytes[kMaxRd];   // 2 or 4 bytes per element
    uint8_t wr_bytes[kMaxWr];
    int n_rd, n_wr;
};

template <typename T>
using gptr = __attribute__((address_space(1))) T*;

__device__ __forceinline__ int quad_a() { return 512 * (int)(threadIdx.x >> 6) + 4 * (int)(threadIdx.x & 63); }

// The lane's 8 elements of one stream in the tile at element e, as four
// 32-bit words (a 2-byte stream fills words 0-1 of each quad's pair, the
// upper two are zero), xor-folded into acc.
__device__ __forceinline__ void ld_fold(const void* base, int bytes, int64_t e, u32x4 (&acc)[2])
{
    const int a = quad_a();
    if (bytes == 4) {
        const uint32_t* p = static_cast<const uint32_t*>(base) + e;
        const u32x4 x = __builtin_nontemporal_load((gptr<const u32x4>)(p + a));
        const u32x4 y = __builtin_nontemporal_load((gptr<const u32x4>)(p + a + 256));
        acc[0] ^= x;
        acc[1] ^= y;
    } else {
        const uint16_t* p = static_cast<const uint16_t*>(base) + e;
        const u32x2 x = __builtin_nontemporal_load((gptr<const u32x2>)(p + a));
        const u32x2 y = __builtin_nontemporal_load((gptr<const u32x2>)(p + a + 256));
        acc[0].x ^= x.x;
        acc[0].y ^= x.y;
        acc[1].x ^= y.x;
        acc[1].y ^= y.y;
    }
}

__device__ __forceinline__ void st_acc(void* base, int bytes, int64_t e, const u32x4 (&acc)[2], uint32_t salt)
{
    const int a = quad_a();
    if (bytes == 4) {
        uint32_t* p = static_cast<uint32_t*>(base) + e;
        __builtin_nontemporal_store(acc[0] ^ salt, (gptr<u32x4>)(p + a));
        __builtin_nontemporal_store(acc[1] ^ salt, (gptr<u32x4>)(p + a + 256));
    } else {
        uint16_t* p = static_cast<uint16_t*>(base) + e;
        const u32x2 x = {acc[0].x ^ acc[0].z ^ salt, acc[0].y ^ acc[0].w};
        const u32x2 y = {acc[1].x ^ acc[1].z ^ salt, acc[1].y ^ acc[1].w};
        __builtin_nontemporal_store(x, (gptr<u32x2>)(p + a));
        __builtin_nontemporal_store(y, (gptr<u32x2>)(p + a + 256));
    }
}

__global__ __launch_bounds__(kThreads) void stream_kernel(Streams s, int64_t ntiles, int split, uint32_t* sink)
{
    const int64_t G = gridDim.x, b = blockIdx.x;
    const int64_t nx = (split > 1 && G % split == 0) ? split : 1;
    const int64_t x = b % nx, per = (ntiles + nx - 1) / nx;
    const int64_t lo = x * per, hi = lo + per < ntiles ? lo + per : ntiles;
    u32x4 tot = {0u, 0u, 0u, 0u};
    for (int64_t t = lo + b / nx; t < hi; t += G / nx) {
        const int64_t e = t * kTile;
        u32x4 acc[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
        // batches of up to eight streams: all loads issued before the folds
        for (int k0 = 0; k0 < s.n_rd; k0 += 8) {
            u32x4 part[8][2];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                part[k][0] = part[k][1] = u32x4{0u, 0u, 0u, 0u};
                if (k0 + k < s.n_rd) ld_fold(s.rd[k0 + k], s.rd_bytes[k0 + k], e, part[k]);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                acc[0] ^= part[k][0];
                acc[1] ^= part[k][1];
            }
        }
        for (int k = 0; k < s.n_wr; ++k) st_acc(s.wr[k], s.wr_bytes[k], e, acc, (uint32_t)k);
        tot ^= acc[0] ^ acc[1];
    }
    // keeps the loads of a read-only pass alive; the condition never holds
    // for data that is not crafted for it, so nothing is written in practice
    if (s.n_wr == 0 && tot.x == 0x9e3779b9u && tot.y == 0x7f4a7c15u && tot.z == 0x85ebca6bu)
        sink[blockIdx.x] = tot.w;
}

}  // namespace

extern "C" {

// One pass over n_tiles * 2048 elements of every stream.
//   rd[n_rd], rd_bytes[n_rd]: read streams (device pointers, 16-byte aligned)
//     and their element sizes (2 or 4); n_rd <= 128.
//   wr[n_wr], wr_bytes[n_wr]: write streams likewise; n_wr <= 8.
//   grid, split: workgroups, and 8 (one contiguous part of the tiles per XCD;
//     grid a multiple of 8) or 1 (a plain grid stride).
//   sink: grid uint32 words of device memory (written only in a case that
//     does not occur; it keeps a read-only pass from being optimized away).
// Returns 0, 1 for a bad argument, or 2 + the HIP error code of the launch.
int zcal_stream(const void* const* rd, const int* rd_bytes, int n_rd, void* const* wr, const int* wr_bytes,
                int n_wr, int64_t n_tiles, int grid, int split, void* sink, void* stream)
{
    if (n_rd < 0 || n_rd > kMaxRd || n_wr < 0 || n_wr > kMaxWr || n_tiles < 0 || grid < 1 || !sink ||
        (split != 1 && split != 8))
        return 1;
    Streams s{};
    for (int k = 0; k < n_rd; ++k) {
        if (!rd[k] || (rd_bytes[k] != 2 && rd_bytes[k] != 4) || reinterpret_cast<uintptr_t>(rd[k]) % 16) return 1;
        s.rd[k] = rd[k];
        s.rd_bytes[k] = (uint8_t)rd_bytes[k];
    }
    for (int k = 0; k < n_wr; ++k) {
        if (!wr[k] || (wr_bytes[k] != 2 && wr_bytes[k] != 4) || reinterpret_cast<uintptr_t>(wr[k]) % 16) return 1;
        s.wr[k] = wr[k];
        s.wr_bytes[k] = (uint8_t)wr_bytes[k];
    }
    s.n_rd = n_rd;
    s.n_wr = n_wr;
    if (n_tiles == 0) return 0;
    hipLaunchKernelGGL(stream_kernel, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream), s, n_tiles,
                       split, static_cast<uint32_t*>(sink));
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 0 : 2 + (int)e;
}

}  // extern "C"
