// api.cpp -- C ABI of libzero1.so (declared in include/zero1.h): argument
// validation, fp64 derivation of the per-step fp32 scalars, workspace layout,
// the multi-tensor plan builder, and the launch sequence of each entry point.
// No entry point allocates device memory or synchronizes (except
// zero1_mta_plan, which copies its table once, and ZERO1_SYNC_CHECK=1).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstddef>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/zero1.h"
#include "internal.h"

using namespace z1;

static_assert(sizeof(NormInfo) == sizeof(zero1_norm_info), "norm info layout");
static_assert(sizeof(PieceDesc) == 48 && sizeof(ChunkDesc) == 16, "descriptor layout");
static_assert(kMaxW == ZERO1_MAX_W, "max W");
static_assert(sizeof(StepScal) == sizeof(zero1_step_scalars) && sizeof(StepScal) == 40 &&
                  offsetof(StepScal, max_norm) == offsetof(zero1_step_scalars, max_norm) &&
                  offsetof(StepScal, delta) == offsetof(zero1_step_scalars, decay),
              "step scalars layout");

namespace {

// ------------------------------------------------------------------ errors
thread_local std::string g_last_error;

zero1_status fail(zero1_status st, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

zero1_status ok()
{
    g_last_error.clear();
    return ZERO1_OK;
}

#define Z1_HIP(call)                                                                       \
    do {                                                                                   \
        hipError_t e_ = (call);                                                            \
        if (e_ != hipSuccess)                                                              \
            return fail(ZERO1_EHIP, "%s failed: %s", #call, hipGetErrorString(e_));       \
    } while (0)

bool sync_check_enabled()
{
    static const bool on = [] {
        const char* s = std::getenv("ZERO1_SYNC_CHECK");
        return s && s[0] && s[0] != '0';
    }();
    return on;
}

zero1_status finish(hipStream_t s)
{
    if (sync_check_enabled()) {
        // a stream being captured into a graph cannot be synchronized: check
        // the launches only
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        Z1_HIP(hipStreamIsCapturing(s, &cs));
        if (cs == hipStreamCaptureStatusNone) Z1_HIP(hipStreamSynchronize(s));
        Z1_HIP(hipGetLastError());
    }
    return ok();
}

// ------------------------------------------------------------------ device
struct DevInfo {
    bool probed = false;
    bool gfx950 = false;
    int cus = 0;
    char arch[64] = {0};
};

std::mutex g_dev_mu;
DevInfo g_dev[64];

zero1_status current_device(DevInfo& out)
{
    int dev = 0;
    Z1_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= 64) return fail(ZERO1_ENOTSUPPORTED, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_dev_mu);
    DevInfo& d = g_dev[dev];
    if (!d.probed) {
        hipDeviceProp_t p;
        Z1_HIP(hipGetDeviceProperties(&p, dev));
        std::snprintf(d.arch, sizeof d.arch, "%s", p.gcnArchName);
        d.gfx950 = std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
        d.cus = p.multiProcessorCount;
        d.probed = true;
    }
    if (!d.gfx950) return fail(ZERO1_ENOTSUPPORTED, "device %d is %s; libzero1 is built for gfx950", dev, d.arch);
    out = d;
    return ZERO1_OK;
}

// ------------------------------------------------------------------ layout

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Ws {
    NormInfo* info;
    double* partials;
    float* g;   // nullptr unless the design stores g
};

zero1_status carve(void* ws, size_t bytes, size_t need, bool want_g, Ws& out)
{
    if (!ws) return fail(ZERO1_EWORKSPACE, "workspace is NULL (need %zu bytes)", need);
    if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(ZERO1_EWORKSPACE, "workspace must be 256-byte aligned");
    if (bytes < need) return fail(ZERO1_EWORKSPACE, "workspace has %zu bytes, needs %zu", bytes, need);
    char* b = static_cast<char*>(ws);
    out.info = reinterpret_cast<NormInfo*>(b);
    out.partials = reinterpret_cast<double*>(b + kInfoBytes);
    out.g = want_g ? reinterpret_cast<float*>(b + kGOffset) : nullptr;
    return ZERO1_OK;
}

// Workgroups for a grid-stride pass over `units` tiles: enough to fill every
// CU several times over, never more than there are tiles.
int grid_for(int64_t units, const DevInfo& d, int per_cu)
{
    int64_t cap = per_cu > 0 ? (int64_t)d.cus * per_cu : units;   // per_cu <= 0: one workgroup per unit
    if (cap > kMaxPartials) cap = kMaxPartials;
    int64_t n = units < cap ? units : cap;
    // a multiple of 8 (the kernels split the work over the 8 XCDs); spare
    // workgroups find no units and exit
    if (n > 8) n = (n + 7) / 8 * 8;
    return (int)(n > 0 ? n : 1);
}

int64_t tiles(int64_t len, bool /*vec*/) { return (len + kTile - 1) / kTile; }

// Launch shape of the streaming kernels, measured on MI355X (GPT-2 small and
// Llama-7B W=8 shards, 7e9 W=1): up to a few thousand units, one workgroup
// per unit with a plain stride is best; past that, a persistent grid of 8
// workgroups per CU with each XCD walking its own contiguous eighth of the
// units wins by 2-4%.
struct Shape {
    int grid;
    int split;
};

Shape update_shape(int64_t units, const DevInfo& d)
{
    const bool big = units > kMaxPartials;
    return Shape{grid_for(units, d, big ? kUpdatePerCu : 0), big ? 8 : 1};
}

// few: the few-slice sum-of-squares pass (few_slice_pass), whose loads of
// several tiles at once keep enough in flight with 6 workgroups per CU: the
// W=1 pass over a 7e9 shard takes 2.14 ms there and 2.39 ms at 8 per CU.
Shape reduce_shape(int64_t tiles, const DevInfo& d, bool few)
{
    const int grid = grid_for(tiles, d, few ? kFewPerCu : kReducePerCu);
    return Shape{grid, tiles >= 16 * (int64_t)grid ? 8 : 1};
}

// The reduce stores g with the non-temporal hint when g is larger than
// kGNtBytes (it cannot stay in the 256 MB MALL until the update reads it back;
// measured 3-6% faster reduce at the 7.5e9/64 and Llama-7B/8 shards, 5% slower
// update at the GPT-2-small shard if applied there).
bool g_store_nt(int64_t g_elems)
{
    return (double)g_elems * sizeof(float) > (double)kGNtBytes;
}

// ------------------------------------------------------------------ checks
bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

zero1_status check_grads(const uint16_t* const* grads, int W, int64_t begin, int64_t len, Reduce& r,
                         uint32_t flags, bool& vec_ok)
{
    if (W < 1 || W > kMaxW) return fail(ZERO1_EINVAL, "W=%d must be in [1, %d]", W, kMaxW);
    if (len < 0) return fail(ZERO1_EINVAL, "len=%lld is negative", (long long)len);
    if (begin < 0) return fail(ZERO1_EINVAL, "begin=%lld is negative", (long long)begin);
    if (!grads) return fail(ZERO1_EINVAL, "grads (host array of W pointers) is NULL");
    vec_ok = true;
    std::memset(&r, 0, sizeof r);
    for (int w = 0; w < W; ++w) {
        if (!grads[w]) return fail(ZERO1_EINVAL, "grads[%d] is NULL", w);
        r.gp.p[w] = grads[w] + begin;
        if (!aligned16(r.gp.p[w])) vec_ok = false;
    }
    r.W = W;
    r.round_bf16 = (flags & ZERO1_G_BF16) ? 1 : 0;
    if ((flags & ZERO1_SUM_ONLY) || W == 1) {
        r.mode = kAvgNone;
    } else if ((W & (W - 1)) == 0) {
        r.mode = kAvgMulPow2;   // s * 2^-k == s / W exactly for a power of two
        r.inv_w = 1.0f / (float)W;
    } else {
        r.mode = kAvgDiv;
        r.f_w = (float)W;
    }
    return ZERO1_OK;
}

constexpr uint32_t kAllFlags = ZERO1_SUM_ONLY | ZERO1_MV_BF16 | ZERO1_RECOMPUTE_G | ZERO1_STORE_G |
                               ZERO1_DECAY_FIRST | ZERO1_CLIP_EPS | ZERO1_G_BF16;

zero1_status check_flags(uint32_t flags, uint32_t allowed, const char* fn)
{
    if (flags & ~kAllFlags) return fail(ZERO1_EINVAL, "%s: unknown flag bits 0x%x", fn, flags & ~kAllFlags);
    if (flags & ~allowed) return fail(ZERO1_EINVAL, "%s: flags 0x%x do not apply here", fn, flags & ~allowed);
    return ZERO1_OK;
}

zero1_status check_hparam_values(const zero1_hparams* hp);

zero1_status check_hparams(const zero1_hparams* hp)
{
    if (!hp) return fail(ZERO1_EINVAL, "hp is NULL");
    if (hp->device_scalars) {   // the values come from device memory; the fields are not read
        if (reinterpret_cast<uintptr_t>(hp->device_scalars) % 8)
            return fail(ZERO1_EINVAL, "hp->device_scalars must be 8-byte aligned");
        return ZERO1_OK;
    }
    return check_hparam_values(hp);
}

zero1_status check_hparam_values(const zero1_hparams* hp)
{
    if (!(hp->lr >= 0.0) || std::isinf(hp->lr)) return fail(ZERO1_EINVAL, "lr=%g must be finite and >= 0", hp->lr);
    if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0)) return fail(ZERO1_EINVAL, "beta1=%g must be in [0, 1)", hp->beta1);
    if (!(hp->beta2 >= 0.0 && hp->beta2 < 1.0)) return fail(ZERO1_EINVAL, "beta2=%g must be in [0, 1)", hp->beta2);
    if (!(hp->eps >= 0.0) || std::isinf(hp->eps)) return fail(ZERO1_EINVAL, "eps=%g must be finite and >= 0", hp->eps);
    if (!(hp->weight_decay >= 0.0) || std::isinf(hp->weight_decay))
        return fail(ZERO1_EINVAL, "weight_decay=%g must be finite and >= 0", hp->weight_decay);
    if (!(hp->max_norm > 0.0)) return fail(ZERO1_EINVAL, "max_norm=%g must be > 0 (inf disables clipping)", hp->max_norm);
    if (hp->step < 1) return fail(ZERO1_EINVAL, "step=%lld must be >= 1", (long long)hp->step);
    return ZERO1_OK;
}

// The page's AdamW applies Python floats to fp32 tensors: each scalar is formed
// in double and used as the nearest binary32 ("并行训练", section on mixed
// precision and AdamW: step_size = lr*sqrt(1-beta2^t)/(1-beta1^t), decay 1-lr*wd).
Scal scalars(const zero1_hparams* hp, uint32_t flags)
{
    Scal s;
    std::memset(&s, 0, sizeof s);
    s.decay_first = (flags & ZERO1_DECAY_FIRST) ? 1 : 0;
    if (hp->device_scalars) {   // read by the kernels when they run
        s.dev = static_cast<const StepScal*>(hp->device_scalars);
        return s;
    }
    s.b1 = (float)hp->beta1;
    s.b2 = (float)hp->beta2;
    s.a1 = (float)(1.0 - hp->beta1);
    s.a2 = (float)(1.0 - hp->beta2);
    s.eps = (float)hp->eps;
    const double t = (double)hp->step;
    const double bc1 = 1.0 - std::pow(hp->beta1, t);
    const double bc2 = 1.0 - std::pow(hp->beta2, t);
    s.sigma = (float)(hp->lr * std::sqrt(bc2) / bc1);
    s.delta = (float)(1.0 - hp->lr * hp->weight_decay);
    return s;
}

struct Range {
    uintptr_t lo, hi;
    const char* what;
    int idx;
};

// Reject any two overlapping non-empty byte ranges.
zero1_status check_disjoint(std::vector<Range>& v)
{
    std::sort(v.begin(), v.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
    for (size_t i = 1; i < v.size(); ++i)
        if (v[i].lo < v[i - 1].hi)
            return fail(ZERO1_EINVAL, "buffers overlap: %s[%d] and %s[%d]", v[i - 1].what, v[i - 1].idx,
                        v[i].what, v[i].idx);
    return ZERO1_OK;
}

// A timing request (zero1_time_next_launch) lives until the next step entry
// point returns: that call's first launch takes it, and it is dropped at
// return whether or not anything was launched.
struct LaunchRequestScope {
    LaunchRequestScope() = default;
    LaunchRequestScope(const LaunchRequestScope&) = delete;
    LaunchRequestScope& operator=(const LaunchRequestScope&) = delete;
    ~LaunchRequestScope() { set_launch_events(nullptr, nullptr); }
};

}  // namespace

int z1::set_error(int st, const char* msg)
{
    g_last_error = msg;
    return st;
}

// ====================================================================== ABI
extern "C" {

int zero1_abi_version(void) { return ZERO1_ABI_VERSION; }

const char* zero1_last_error(void) { return g_last_error.c_str(); }

const char* zero1_status_string(int st)
{
    switch (st) {
    case ZERO1_OK: return "ZERO1_OK";
    case ZERO1_EINVAL: return "ZERO1_EINVAL";
    case ZERO1_EWORKSPACE: return "ZERO1_EWORKSPACE";
    case ZERO1_EHIP: return "ZERO1_EHIP";
    case ZERO1_ENOTSUPPORTED: return "ZERO1_ENOTSUPPORTED";
    default: return "ZERO1_UNKNOWN";
    }
}

zero1_status zero1_shard_range(int64_t n_total, int W, int rank, int64_t* begin, int64_t* len)
{
    if (n_total < 0) return fail(ZERO1_EINVAL, "n_total=%lld is negative", (long long)n_total);
    if (W < 1) return fail(ZERO1_EINVAL, "W=%d must be >= 1", W);
    if (rank < 0 || rank >= W) return fail(ZERO1_EINVAL, "rank=%d must be in [0, %d)", rank, W);
    if (!begin || !len) return fail(ZERO1_EINVAL, "begin/len outputs are NULL");
    const int64_t S = n_total / W + (n_total % W != 0);
    const int64_t b = std::min<int64_t>((int64_t)rank * S, n_total);
    *begin = b;
    *len = std::min<int64_t>(b + S, n_total) - b;
    return ok();
}

size_t zero1_workspace_bytes(int64_t len, int W, uint32_t flags)
{
    (void)W;
    size_t n = kGOffset;
    if ((flags & ZERO1_STORE_G) && len > 0) n += round_up((size_t)len * sizeof(float), 256);
    return n;
}

zero1_status zero1_shard_reduce(const uint16_t* const* grads, int W, int64_t begin, int64_t len,
                                uint32_t flags, float* g_out, double* sumsq_out, void* ws,
                                size_t ws_bytes, void* stream)
{
    LaunchRequestScope timing_scope;
    if (zero1_status fs = check_flags(flags, kAllFlags, "zero1_shard_reduce")) return fs;
    Reduce r;
    bool vec = false;
    zero1_status st = check_grads(grads, W, begin, len, r, flags, vec);
    if (st) return st;
    if (!g_out && !sumsq_out) return fail(ZERO1_EINVAL, "g_out and sumsq_out are both NULL");
    if (g_out) {
        if (!aligned16(g_out)) vec = false;
        std::vector<Range> rg;
        rg.push_back({(uintptr_t)g_out, (uintptr_t)(g_out + len), "g_out", 0});
        for (int w = 0; w < W; ++w)
            rg.push_back({(uintptr_t)(grads[w] + begin), (uintptr_t)(grads[w] + begin + len), "grads", w});
        if (len > 0 && (st = check_disjoint(rg))) return st;
    }
    DevInfo d;
    if ((st = current_device(d))) return st;
    Ws w;
    if (sumsq_out && (st = carve(ws, ws_bytes, zero1_workspace_bytes(len, W, 0), false, w))) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (len == 0) {   // empty shard: the sum of no squares is 0 (a kernel, not a memset)
        if (sumsq_out) Z1_HIP(launch_finalize(w.partials, 0, sumsq_out, s));
        return finish(s);
    }
    const Shape sh = reduce_shape(tiles(len, vec), d, few_slice_pass(vec, g_out != nullptr, sumsq_out != nullptr, W));
    const int nb = sh.grid;
    Z1_HIP(launch_reduce(r, len, vec, g_out, sumsq_out ? w.partials : nullptr, nb, sh.split, g_store_nt(len), s));
    if (sumsq_out) Z1_HIP(launch_finalize(w.partials, nb, sumsq_out, s));
    return finish(s);
}

zero1_status zero1_grad_norm(const float* g, int64_t len, double* sumsq_out, void* ws, size_t ws_bytes,
                             void* stream)
{
    LaunchRequestScope timing_scope;
    if (len < 0) return fail(ZERO1_EINVAL, "len=%lld is negative", (long long)len);
    if (!sumsq_out) return fail(ZERO1_EINVAL, "sumsq_out is NULL");
    if (!g && len > 0) return fail(ZERO1_EINVAL, "g is NULL");
    zero1_status st;
    DevInfo d;
    if ((st = current_device(d))) return st;
    Ws w;
    if ((st = carve(ws, ws_bytes, zero1_workspace_bytes(len, 1, 0), false, w))) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (len == 0) {
        Z1_HIP(launch_finalize(w.partials, 0, sumsq_out, s));
        return finish(s);
    }
    const bool vec = aligned16(g);
    const Shape sh = reduce_shape(tiles(len, vec), d, false);
    const int nb = sh.grid;
    Z1_HIP(launch_sumsq(g, len, vec, w.partials, nb, sh.split, s));
    Z1_HIP(launch_finalize(w.partials, nb, sumsq_out, s));
    return finish(s);
}

zero1_status zero1_adamw_step(const float* g, const uint16_t* const* grads, int W, int64_t begin, int64_t len,
                              float* master, void* m, void* v, uint16_t* param_bf16, const zero1_hparams* hp,
                              const double* rank_sumsq, int n_ranks, uint32_t flags, zero1_norm_info* info_out,
                              void* stream)
{
    LaunchRequestScope timing_scope;
    if (zero1_status fs = check_flags(flags, kAllFlags, "zero1_adamw_step")) return fs;
    zero1_status st;
    if ((st = check_hparams(hp))) return st;
    if (len < 0) return fail(ZERO1_EINVAL, "len=%lld is negative", (long long)len);
    if (n_ranks < 1) return fail(ZERO1_EINVAL, "n_ranks=%d must be >= 1", n_ranks);
    if (!rank_sumsq) return fail(ZERO1_EINVAL, "rank_sumsq is NULL");
    const bool mv_bf16 = (flags & ZERO1_MV_BF16) != 0;
    Reduce r;
    std::memset(&r, 0, sizeof r);
    bool vec = true;
    if (!g) {
        if ((st = check_grads(grads, W, begin, len, r, flags, vec))) return st;
    } else if (!aligned16(g)) {
        vec = false;
    }
    if (len > 0 && (!master || !m || !v || !param_bf16))
        return fail(ZERO1_EINVAL, "master, m, v and param_bf16 must be non-NULL");
    const size_t mvb = mv_bf16 ? 2 : 4;
    if (!aligned16(master) || !aligned16(m) || !aligned16(v) || !aligned16(param_bf16)) vec = false;
    if (len > 0) {
        std::vector<Range> rg = {
            {(uintptr_t)master, (uintptr_t)master + 4 * (size_t)len, "master", 0},
            {(uintptr_t)m, (uintptr_t)m + mvb * (size_t)len, "m", 0},
            {(uintptr_t)v, (uintptr_t)v + mvb * (size_t)len, "v", 0},
            {(uintptr_t)param_bf16, (uintptr_t)param_bf16 + 2 * (size_t)len, "param_bf16", 0}};
        if (g) rg.push_back({(uintptr_t)g, (uintptr_t)g + 4 * (size_t)len, "g", 0});
        if ((st = check_disjoint(rg))) return st;
    }
    DevInfo d;
    if ((st = current_device(d))) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // always launched (also for len == 0) so that info_out is written
    const Scal sc = scalars(hp, flags);
    const Shape sh = update_shape(tiles(len, vec), d);
    const int nb = sh.grid;
    Z1_HIP(launch_adamw_flat(g, r, len, vec, mv_bf16, master, m, v, param_bf16, sc, rank_sumsq, n_ranks,
                             hp->max_norm, (flags & ZERO1_CLIP_EPS) ? 1 : 0,
                             reinterpret_cast<NormInfo*>(info_out), nb, sh.split, s));
    return finish(s);
}

// ------------------------------------------------------------------ multi-tensor
// Elements per multi-tensor chunk: one 2048-element tile.
static int64_t plan_chunk_elems() { return kChunkElems; }

size_t zero1_mta_table_bytes(const zero1_piece* pieces, int n_pieces)
{
    if (!pieces || n_pieces <= 0) return 0;
    const int64_t chunk = plan_chunk_elems();
    size_t chunks = 0;
    for (int i = 0; i < n_pieces; ++i)
        if (pieces[i].numel > 0) chunks += (size_t)((pieces[i].numel + chunk - 1) / chunk);
    return round_up(sizeof(PieceDesc) * (size_t)n_pieces, 256) + sizeof(ChunkDesc) * chunks;
}

zero1_status zero1_mta_plan(const zero1_piece* pieces, int n_pieces, uint32_t flags, void* table,
                            size_t table_bytes, zero1_plan* plan_out)
{
    if (zero1_status fs = check_flags(flags, kAllFlags, "zero1_mta_plan")) return fs;
    if (!plan_out) return fail(ZERO1_EINVAL, "plan_out is NULL");
    if (!pieces || n_pieces < 1) return fail(ZERO1_EINVAL, "need at least one piece");
    const bool mv_bf16 = (flags & ZERO1_MV_BF16) != 0;
    std::vector<int> order(n_pieces);
    for (int i = 0; i < n_pieces; ++i) {
        const zero1_piece& p = pieces[i];
        if (p.numel <= 0) return fail(ZERO1_EINVAL, "piece %d: numel=%lld must be > 0", i, (long long)p.numel);
        if (p.shard_offset < 0) return fail(ZERO1_EINVAL, "piece %d: negative shard_offset", i);
        if (!p.param_bf16 || !p.master || !p.m || !p.v) return fail(ZERO1_EINVAL, "piece %d: NULL buffer", i);
        if (p.numel > (int64_t)1 << 40) return fail(ZERO1_EINVAL, "piece %d: numel too large", i);
        order[i] = i;
    }
    std::sort(order.begin(), order.end(),
              [&](int a, int b) { return pieces[a].shard_offset < pieces[b].shard_offset; });
    int64_t pos = 0;
    for (int k = 0; k < n_pieces; ++k) {
        const zero1_piece& p = pieces[order[k]];
        if (p.shard_offset != pos)
            return fail(ZERO1_EINVAL, "pieces do not tile the shard: piece %d starts at %lld, expected %lld",
                        order[k], (long long)p.shard_offset, (long long)pos);
        pos += p.numel;
    }
    const size_t mvb = mv_bf16 ? 2 : 4;
    std::vector<Range> rg;
    rg.reserve(4 * (size_t)n_pieces);
    bool aligned = true;
    for (int i = 0; i < n_pieces; ++i) {
        const zero1_piece& p = pieces[i];
        const size_t n = (size_t)p.numel;
        rg.push_back({(uintptr_t)p.param_bf16, (uintptr_t)p.param_bf16 + 2 * n, "param_bf16", i});
        rg.push_back({(uintptr_t)p.master, (uintptr_t)p.master + 4 * n, "master", i});
        rg.push_back({(uintptr_t)p.m, (uintptr_t)p.m + mvb * n, "m", i});
        rg.push_back({(uintptr_t)p.v, (uintptr_t)p.v + mvb * n, "v", i});
        if (p.shard_offset % kVec || !aligned16(p.param_bf16) || !aligned16(p.master) || !aligned16(p.m) ||
            !aligned16(p.v))
            aligned = false;
    }
    zero1_status st;
    if ((st = check_disjoint(rg))) return st;
    const size_t need = zero1_mta_table_bytes(pieces, n_pieces);
    if (!table) return fail(ZERO1_EWORKSPACE, "table is NULL (need %zu bytes)", need);
    if (reinterpret_cast<uintptr_t>(table) % 256) return fail(ZERO1_EWORKSPACE, "table must be 256-byte aligned");
    if (table_bytes < need) return fail(ZERO1_EWORKSPACE, "table has %zu bytes, needs %zu", table_bytes, need);
    DevInfo d;
    if ((st = current_device(d))) return st;

    const size_t chunk_off = round_up(sizeof(PieceDesc) * (size_t)n_pieces, 256);
    const int64_t chunk = plan_chunk_elems();
    std::vector<char> host(need, 0);
    PieceDesc* pd = reinterpret_cast<PieceDesc*>(host.data());
    ChunkDesc* cd = reinterpret_cast<ChunkDesc*>(host.data() + chunk_off);
    int64_t nc = 0;
    for (int k = 0; k < n_pieces; ++k) {   // shard order, so chunk k covers shard positions in order
        const zero1_piece& p = pieces[order[k]];
        pd[k] = PieceDesc{p.numel, p.shard_offset, p.param_bf16, p.master, p.m, p.v};
        for (int64_t off = 0; off < p.numel; off += chunk) {
            const int64_t l = std::min<int64_t>(chunk, p.numel - off);
            cd[nc++] = ChunkDesc{k, (int32_t)l, off};
        }
    }
    if (nc > INT32_MAX) return fail(ZERO1_EINVAL, "too many chunks");
    Z1_HIP(hipMemcpy(table, host.data(), need, hipMemcpyHostToDevice));
    plan_out->table = table;
    plan_out->shard_len = pos;
    plan_out->n_pieces = n_pieces;
    plan_out->n_chunks = (int32_t)nc;
    plan_out->chunk_elems = (int32_t)chunk;
    plan_out->flags = flags & ZERO1_MV_BF16;
    plan_out->aligned = aligned ? 1 : 0;
    plan_out->reserved = 0;
    return ok();
}

static bool use_store_g(uint32_t flags, int W)
{
    if (flags & ZERO1_STORE_G) return true;
    if (flags & ZERO1_RECOMPUTE_G) return false;
    return W > 4;   // 2W+34 bytes/param beats 4W+26 once W > 4
}

size_t zero1_mta_workspace_bytes(const zero1_plan* plan, int W, uint32_t flags)
{
    if (!plan) return 0;
    return zero1_workspace_bytes(plan->shard_len, W, use_store_g(flags, W) ? ZERO1_STORE_G : 0);
}

// Shared checks of the two mta phases.
static zero1_status mta_common(const uint16_t* const* grads, int W, int64_t begin, const zero1_plan* plan,
                               uint32_t flags, void* ws, size_t ws_bytes, Reduce& r, bool& vec, bool& store_g,
                               DevInfo& d, Ws& w)
{
    zero1_status st;
    if (!plan || !plan->table) return fail(ZERO1_EINVAL, "plan is NULL or has no table");
    if ((flags & ZERO1_STORE_G) && (flags & ZERO1_RECOMPUTE_G))
        return fail(ZERO1_EINVAL, "ZERO1_STORE_G and ZERO1_RECOMPUTE_G are exclusive");
    if ((st = check_grads(grads, W, begin, plan->shard_len, r, flags, vec))) return st;
    vec = vec && plan->aligned;
    store_g = use_store_g(flags, W);
    if ((st = current_device(d))) return st;
    return carve(ws, ws_bytes, zero1_mta_workspace_bytes(plan, W, flags), store_g, w);
}

zero1_status zero1_mta_reduce(const uint16_t* const* grads, int W, int64_t begin, const zero1_plan* plan,
                              double* sumsq_out, uint32_t flags, void* ws, size_t ws_bytes, void* stream)
{
    LaunchRequestScope timing_scope;
    if (zero1_status fs = check_flags(flags, kAllFlags, "zero1_mta_reduce")) return fs;
    Reduce r;
    bool vec = false, store_g = false;
    DevInfo d;
    Ws w;
    if (!sumsq_out) return fail(ZERO1_EINVAL, "sumsq_out is NULL");
    zero1_status st = mta_common(grads, W, begin, plan, flags, ws, ws_bytes, r, vec, store_g, d, w);
    if (st) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Shape sh = reduce_shape(tiles(plan->shard_len, vec), d, few_slice_pass(vec, w.g != nullptr, true, W));
    const int nb = sh.grid;
    Z1_HIP(launch_reduce(r, plan->shard_len, vec, w.g, w.partials, nb, sh.split, g_store_nt(plan->shard_len), s));
    Z1_HIP(launch_finalize(w.partials, nb, sumsq_out, s));
    return finish(s);
}

zero1_status zero1_mta_reduce_range(const uint16_t* const* grads, int W, const zero1_plan* plan, int64_t lo,
                                   int64_t hi, double* sumsq_out, uint32_t flags, void* ws, size_t ws_bytes,
                                   void* stream)
{
    LaunchRequestScope timing_scope;
    if (zero1_status fs = check_flags(flags, kAllFlags, "zero1_mta_reduce_range")) return fs;
    zero1_status st;
    if (!plan || !plan->table) return fail(ZERO1_EINVAL, "plan is NULL or has no table");
    if (!sumsq_out) return fail(ZERO1_EINVAL, "sumsq_out is NULL");
    if (lo < 0 || hi < lo || hi > plan->shard_len)
        return fail(ZERO1_EINVAL, "range [%lld, %lld) is not inside the shard [0, %lld)", (long long)lo,
                    (long long)hi, (long long)plan->shard_len);
    if (flags & ZERO1_RECOMPUTE_G)
        return fail(ZERO1_EINVAL, "zero1_mta_reduce_range stores g: it pairs with ZERO1_STORE_G only");
    Reduce r;
    bool vec = false;
    if ((st = check_grads(grads, W, 0, hi - lo, r, flags, vec))) return st;
    DevInfo d;
    if ((st = current_device(d))) return st;
    Ws w;
    if ((st = carve(ws, ws_bytes, zero1_mta_workspace_bytes(plan, W, ZERO1_STORE_G), true, w))) return st;
    float* g = w.g + lo;
    if (reinterpret_cast<uintptr_t>(g) % 16) vec = false;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Shape sh = reduce_shape(tiles(hi - lo, vec), d, false);   // stores g: never the few-slice pass
    if (hi > lo)
        Z1_HIP(launch_reduce(r, hi - lo, vec, g, w.partials, sh.grid, sh.split, g_store_nt(plan->shard_len), s));
    Z1_HIP(launch_finalize(w.partials, hi > lo ? sh.grid : 0, sumsq_out, s));
    return finish(s);
}

zero1_status zero1_partials_sum(const double* parts, int n, double* sum_out, void* stream)
{
    LaunchRequestScope timing_scope;
    if (n < 0 || n > kMaxPartials) return fail(ZERO1_EINVAL, "n=%d must be in [0, %d]", n, kMaxPartials);
    if ((!parts && n > 0) || !sum_out) return fail(ZERO1_EINVAL, "parts or sum_out is NULL");
    zero1_status st;
    DevInfo d;
    if ((st = current_device(d))) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Z1_HIP(launch_finalize(parts, n, sum_out, s));
    return finish(s);
}

zero1_status zero1_mta_update(const uint16_t* const* grads, int W, int64_t begin, const zero1_plan* plan,
                              const zero1_hparams* hp, const double* rank_sumsq, int n_ranks, uint32_t flags,
                              zero1_norm_info* info_out, void* ws, size_t ws_bytes, void* stream)
{
    LaunchRequestScope timing_scope;
    if (zero1_status fs = check_flags(flags, kAllFlags, "zero1_mta_update")) return fs;
    zero1_status st;
    if ((st = check_hparams(hp))) return st;
    if (n_ranks < 1) return fail(ZERO1_EINVAL, "n_ranks=%d must be >= 1", n_ranks);
    if (!rank_sumsq) return fail(ZERO1_EINVAL, "rank_sumsq is NULL");
    Reduce r;
    bool vec = false, store_g = false;
    DevInfo d;
    Ws w;
    if ((st = mta_common(grads, W, begin, plan, flags, ws, ws_bytes, r, vec, store_g, d, w))) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const char* tb = static_cast<const char*>(plan->table);
    const PieceDesc* pd = reinterpret_cast<const PieceDesc*>(tb);
    const ChunkDesc* cd = reinterpret_cast<const ChunkDesc*>(tb + round_up(sizeof(PieceDesc) * plan->n_pieces, 256));
    const Shape sh = update_shape(plan->n_chunks, d);
    const int nb = sh.grid;
    Z1_HIP(launch_adamw_mta(w.g, r, pd, cd, plan->n_chunks, vec, (plan->flags & ZERO1_MV_BF16) != 0, scalars(hp, flags),
                            rank_sumsq, n_ranks, hp->max_norm, (flags & ZERO1_CLIP_EPS) ? 1 : 0,
                            reinterpret_cast<NormInfo*>(info_out), nb, sh.split, s));
    return finish(s);
}

int zero1_mta_design(const uint16_t* const* grads, int W, int64_t begin, const zero1_plan* plan, uint32_t flags)
{
    if (!plan || !plan->table) return 0;
    if ((flags & ZERO1_STORE_G) && (flags & ZERO1_RECOMPUTE_G)) return 0;
    Reduce r;
    bool vec = false;
    if (check_grads(grads, W, begin, plan->shard_len, r, 0, vec) != ZERO1_OK) return 0;
    return use_store_g(flags, W) ? ZERO1_STORE_G : ZERO1_RECOMPUTE_G;
}

zero1_status zero1_mta_step(const uint16_t* const* grads, int W, int64_t begin, const zero1_plan* plan,
                            const zero1_hparams* hp, double* rank_sumsq, int n_ranks, int my_rank,
                            uint32_t flags, zero1_norm_info* info_out, void* ws, size_t ws_bytes, void* stream)
{
    LaunchRequestScope timing_scope;
    if (zero1_status fs = check_flags(flags, kAllFlags, "zero1_mta_step")) return fs;
    zero1_status st;
    if ((st = check_hparams(hp))) return st;
    if (n_ranks < 1 || my_rank < 0 || my_rank >= n_ranks)
        return fail(ZERO1_EINVAL, "my_rank=%d must be in [0, n_ranks=%d)", my_rank, n_ranks);
    if (!rank_sumsq) return fail(ZERO1_EINVAL, "rank_sumsq is NULL");
    if ((st = zero1_mta_reduce(grads, W, begin, plan, rank_sumsq + my_rank, flags, ws, ws_bytes, stream))) return st;
    return zero1_mta_update(grads, W, begin, plan, hp, rank_sumsq, n_ranks, flags, info_out, ws, ws_bytes, stream);
}

zero1_status zero1_time_next_launch(void* start_event, void* stop_event)
{
    set_launch_events(static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event));
    return ok();
}

zero1_status zero1_step_scalars_derive(const zero1_hparams* hp, zero1_step_scalars* out)
{
    if (!hp || !out) return fail(ZERO1_EINVAL, "hp or out is NULL");
    zero1_status st;
    if ((st = check_hparam_values(hp))) return st;
    zero1_hparams h = *hp;
    h.device_scalars = nullptr;
    const Scal c = scalars(&h, 0);
    zero1_step_scalars o;
    std::memset(&o, 0, sizeof o);
    o.beta1 = c.b1;
    o.beta2 = c.b2;
    o.one_minus_beta1 = c.a1;
    o.one_minus_beta2 = c.a2;
    o.eps = c.eps;
    o.step_size = c.sigma;
    o.decay = c.delta;
    o.max_norm = hp->max_norm;
    *out = o;
    return ok();
}

zero1_status zero1_arena_plan(const zero1_arena_request* req, zero1_arena_layout* out)
{
    if (!req || !out) return fail(ZERO1_EINVAL, "request or layout is NULL");
    const zero1_arena_request& q = *req;
    if (zero1_status fs = check_flags(q.flags, kAllFlags, "zero1_arena_plan")) return fs;
    if ((q.flags & ZERO1_STORE_G) && (q.flags & ZERO1_RECOMPUTE_G))
        return fail(ZERO1_EINVAL, "ZERO1_STORE_G and ZERO1_RECOMPUTE_G are exclusive");
    if (q.shard_len < 1) return fail(ZERO1_EINVAL, "shard_len=%lld must be >= 1", (long long)q.shard_len);
    if (q.W < 1 || q.W > kMaxW) return fail(ZERO1_EINVAL, "W=%d must be in [1, %d]", q.W, kMaxW);
    if (q.grad_offset < 0 || q.grad_elems < q.grad_offset + q.shard_len)
        return fail(ZERO1_EINVAL, "gradient buffers of %lld elements cannot hold the shard at %lld",
                    (long long)q.grad_elems, (long long)q.grad_offset);
    if (q.param_offset < 0 || q.param_elems < q.param_offset + q.shard_len)
        return fail(ZERO1_EINVAL, "the parameter buffer of %lld elements cannot hold the shard at %lld",
                    (long long)q.param_elems, (long long)q.param_offset);
    const size_t unit = (size_t)2 << 20;
    const size_t S = (size_t)q.shard_len;
    const bool store_g = use_store_g(q.flags, q.W);
    const size_t mvb = (q.flags & ZERO1_MV_BF16) ? 2 : 4;
    const size_t ws_bytes = zero1_workspace_bytes(q.shard_len, q.W, store_g ? ZERO1_STORE_G : 0);
    const size_t grad_bytes = round_up((size_t)q.grad_elems * 2, unit);

    // the five spaced slots: bytes of each buffer before and after its shard start
    struct Slot { size_t before, after; };
    const Slot slot[5] = {
        store_g ? Slot{0, ws_bytes} : Slot{(size_t)q.grad_offset * 2, (size_t)(q.grad_elems - q.grad_offset) * 2},
        {0, S * 4},
        {0, S * mvb},
        {0, S * mvb},
        {(size_t)q.param_offset * 2, (size_t)(q.param_elems - q.param_offset) * 2},
    };
    const size_t base = round_up(slot[0].before, unit);   // shard start of slot 0
    size_t d_min = 0;
    for (int k = 0; k < 4; ++k) d_min = std::max(d_min, slot[k].after + slot[k + 1].before);
    d_min = round_up(d_min, unit);
    // what follows the parameter buffer: the gradient buffers not spaced, and
    // the workspace when it is not slot 0
    size_t tail = (size_t)(store_g ? q.W : q.W - 1) * grad_bytes + (store_g ? 0 : round_up(ws_bytes, unit));
    const size_t fixed = base + round_up(slot[4].after, unit) + tail;   // everything but 4 D
    size_t d = std::max(d_min, (size_t)ZERO1_ARENA_SPACING);
    if (fixed + 4 * d > q.capacity) {
        if (q.capacity < fixed + 4 * d_min)
            return fail(ZERO1_EINVAL, "capacity %zu bytes is below the packed layout's %zu", q.capacity,
                        fixed + 4 * d_min);
        d = (q.capacity - fixed) / 4 / unit * unit;
    }
    zero1_arena_layout L;
    std::memset(&L, 0, sizeof L);
    L.spacing = d;
    L.ws_bytes = ws_bytes;
    L.master = base + d;
    L.m = base + 2 * d;
    L.v = base + 3 * d;
    L.params = base + 4 * d - slot[4].before;
    size_t next = round_up(base + 4 * d + slot[4].after, unit);
    int w0 = 0;
    if (store_g) {
        L.ws = base;
    } else {
        L.grads[0] = base - slot[0].before;
        w0 = 1;
        L.ws = next;
        next += round_up(ws_bytes, unit);
    }
    for (int w = w0; w < q.W; ++w) {
        L.grads[w] = next;
        next += grad_bytes;
    }
    L.total_bytes = next;
    *out = L;
    return ok();
}

}  // extern "C"
