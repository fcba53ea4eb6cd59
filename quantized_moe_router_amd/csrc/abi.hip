// Host side of libmoe_int4.so: argument checks, workspace map, and the
// extern "C" entry points declared in include/moe_int4.h.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "common.h"
#include "moe_int4.h"

namespace moe {

hipError_t launch_decode_forward(const uint16_t *x, const uint16_t *router_w, const ExpertArgs &a,
                                 const Dims &d, const Workspace &ws, hipEvent_t ev_route,
                                 hipEvent_t ev_mid, hipStream_t st);
hipError_t launch_decode_experts(const ExpertArgs &a, const int32_t *ids, const float *wts,
                                 const Dims &d, const Workspace &ws, hipStream_t st);
hipError_t launch_quantize_int4(const uint16_t *w, int rows, int K, int group, int32_t *packed,
                                uint16_t *scales, hipStream_t st);

namespace {

thread_local std::string g_error;

int32_t fail(int32_t code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return code;
}

constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
    size_t dec_keys, ctrl, logits, ids, weights, counts, offsets, sorted_slots,
        slot_pos, active, chunk_hist, tiles, h, y, shared_gate, sh_h, xh, xp, xs, total;
};

Layout layout(const Dims &d)
{
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += round_up(bytes);
        return o;
    };
    const size_t S = (size_t)d.S, T = (size_t)d.T;
    const size_t chunk = (size_t)perm_chunk(d.S), nchunks = (S + chunk - 1) / chunk;
    L.dec_keys = take(kKeysBytes);   // the control prefix: same place and size for every shape
    L.ctrl = take(kCtrlBytes);
    L.logits = take(4 * T * d.E * (size_t)(d.T > kDecodeMaxTokens ? router_ksplit(d) : 1));
    L.ids = take(4 * S);
    L.weights = take(4 * S);
    L.counts = take(4 * (size_t)d.E);
    L.offsets = take(4 * ((size_t)d.E + 1));
    L.sorted_slots = take(4 * S);
    L.slot_pos = take(4 * S);
    L.active = take(4 * ((size_t)d.E + 1));
    L.chunk_hist = take(4 * nchunks * d.E);
    L.tiles = take(16 * routed_tile_slots(d));
    L.h = take(2 * S * d.I);
    // y: fp16 rows per slot (many tokens), fp32 per slot and shared row (decode)
    L.y = take((d.T <= kDecodeMaxTokens ? 4 : 2) * T * ((size_t)d.k + 1) * d.H);
    L.shared_gate = take(4 * T);
    L.sh_h = take(2 * T * (size_t)d.sh_I);
    L.xh = take(d.T > kDecodeMaxTokens ? 2 * T * (size_t)d.H : 0);
    L.xp = take(d.T <= kDecodeMaxTokens ? 2 * T * (size_t)d.H : 0);
    L.xs = take(d.T <= kDecodeMaxTokens ? 4 * T * (size_t)(d.H / 32) : 0);
    L.total = off;
    return L;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// One-time check per device that it is a gfx950 part.
int32_t check_device()
{
    static std::mutex mu;
    static int checked[64] = {0};  // 0 unknown, 1 ok, -1 bad
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return fail(MOE_INT4_EDEVICE, "no HIP device is current");
    std::lock_guard<std::mutex> lock(mu);
    if (checked[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return fail(MOE_INT4_EDEVICE, "hipGetDeviceProperties failed for device %d", dev);
        checked[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        if (checked[dev] < 0)
            return fail(MOE_INT4_EDEVICE, "device %d is %s; this library is built for gfx950",
                        dev, prop.gcnArchName);
    }
    if (checked[dev] < 0) return fail(MOE_INT4_EDEVICE, "device %d is not gfx950", dev);
    return MOE_INT4_OK;
}

int32_t check_shape(const moe_int4_shape *s, const moe_shared_int6 *sh, Dims *d)
{
    if (!s) return fail(MOE_INT4_EINVAL, "shape is NULL");
    if (s->tokens < 0 || s->tokens > (1 << 20))
        return fail(MOE_INT4_EINVAL, "tokens=%d outside [0, 1048576]", s->tokens);
    if (s->group != 128 && s->group != 64)
        return fail(MOE_INT4_EINVAL, "group=%d, INT4 supports 128 and 64", s->group);
    if (s->hidden <= 0 || s->hidden % 256 || s->hidden > 4096)
        return fail(MOE_INT4_EINVAL, "hidden=%d must be a positive multiple of 256, at most 4096",
                    s->hidden);
    if (s->inter <= 0 || s->inter % 128 || s->inter > 1024)
        return fail(MOE_INT4_EINVAL, "inter=%d must be a positive multiple of 128, at most 1024",
                    s->inter);
    if (s->experts <= 0 || s->experts > kMaxExperts)
        return fail(MOE_INT4_EINVAL, "experts=%d outside [1, %d]", s->experts, kMaxExperts);
    int kmax = s->experts < kMaxTopK ? s->experts : kMaxTopK;
    if (s->top_k < 1 || s->top_k > kmax)
        return fail(MOE_INT4_EINVAL, "top_k=%d outside [1, %d]", s->top_k, kmax);
    d->T = s->tokens;
    d->H = s->hidden;
    d->E = s->experts;
    d->I = s->inter;
    d->k = s->top_k;
    d->S = s->tokens * s->top_k;
    d->gsh = s->group == 64 ? 1 : 2;
    d->sh_I = 0;
    if (sh) {
        if (sh->group != kShGroup)
            return fail(MOE_INT4_EINVAL, "shared expert group=%d, only 64 is supported", sh->group);
        if (sh->inter <= 0 || sh->inter % 128 || sh->inter > 1024)
            return fail(MOE_INT4_EINVAL,
                        "shared expert inter=%d must be a positive multiple of 128, at most 1024",
                        sh->inter);
        if (!sh->gate_w || !sh->w13_packed || !sh->w13_scales || !sh->w2_packed || !sh->w2_scales)
            return fail(MOE_INT4_EINVAL, "a shared-expert pointer is NULL");
        if (!aligned16(sh->gate_w) || !aligned16(sh->w13_packed) || !aligned16(sh->w13_scales) ||
            !aligned16(sh->w2_packed) || !aligned16(sh->w2_scales))
            return fail(MOE_INT4_EALIGN, "a shared-expert pointer is not 16-byte aligned");
        d->sh_I = sh->inter;
    }
    // element offsets inside one activation buffer are 32-bit in the kernels
    const size_t lim = (size_t)1 << 31;
    if ((size_t)d->T * d->H >= lim || (size_t)d->S * d->I >= lim || (size_t)d->T * d->sh_I >= lim)
        return fail(MOE_INT4_EINVAL,
                    "tokens=%d too many for one call: tokens*hidden and tokens*top_k*inter must stay "
                    "below 2^31 (split the batch)", d->T);
    return MOE_INT4_OK;
}

struct PtrCheck {
    const char *name;
    const void *p;
};

int32_t check_ptrs(std::initializer_list<PtrCheck> ps)
{
    for (const PtrCheck &c : ps) {
        if (!c.p) return fail(MOE_INT4_EINVAL, "%s is NULL", c.name);
        if (!aligned16(c.p)) return fail(MOE_INT4_EALIGN, "%s is not 16-byte aligned", c.name);
    }
    return MOE_INT4_OK;
}

int32_t check_workspace(const Dims &d, void *ws, size_t bytes, Workspace *out)
{
    Layout L = layout(d);
    if (!ws) return fail(MOE_INT4_EINVAL, "workspace is NULL");
    if (!aligned16(ws)) return fail(MOE_INT4_EALIGN, "workspace is not 16-byte aligned");
    if (bytes < L.total)
        return fail(MOE_INT4_EWORKSPACE, "workspace has %zu bytes, %zu needed", bytes, L.total);
    char *b = static_cast<char *>(ws);
    Workspace w{};
    w.dec_keys = reinterpret_cast<uint32_t *>(b + L.dec_keys);
    w.ctrl = reinterpret_cast<uint32_t *>(b + L.ctrl);
    w.status = w.ctrl;
    w.logits = reinterpret_cast<float *>(b + L.logits);
    w.ids = reinterpret_cast<int32_t *>(b + L.ids);
    w.weights = reinterpret_cast<float *>(b + L.weights);
    w.counts = reinterpret_cast<int32_t *>(b + L.counts);
    w.offsets = reinterpret_cast<int32_t *>(b + L.offsets);
    w.sorted_slots = reinterpret_cast<int32_t *>(b + L.sorted_slots);
    w.slot_pos = reinterpret_cast<int32_t *>(b + L.slot_pos);
    w.active = reinterpret_cast<int32_t *>(b + L.active);
    w.chunk_hist = reinterpret_cast<int32_t *>(b + L.chunk_hist);
    w.tiles = reinterpret_cast<int4 *>(b + L.tiles);
    w.h = reinterpret_cast<uint16_t *>(b + L.h);
    w.y = reinterpret_cast<uint16_t *>(b + L.y);
    w.shared_gate = reinterpret_cast<float *>(b + L.shared_gate);
    w.sh_h = reinterpret_cast<uint16_t *>(b + L.sh_h);
    w.xh = reinterpret_cast<uint16_t *>(b + L.xh);
    w.xp = reinterpret_cast<uint16_t *>(b + L.xp);
    w.xs = reinterpret_cast<float *>(b + L.xs);
    w.bytes = L.total;
    *out = w;
    return MOE_INT4_OK;
}

int32_t launched(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(MOE_INT4_ELAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
    return MOE_INT4_OK;
}

int32_t check_int8_shape(int32_t tokens, int32_t n, int32_t k, int32_t group)
{
    if (group != 64 && group != 128)
        return fail(MOE_INT4_EINVAL, "group=%d, INT8 supports 64 and 128", group);
    if (tokens < 0 || tokens > (1 << 20))
        return fail(MOE_INT4_EINVAL, "tokens=%d outside [0, 1048576]", tokens);
    if (n <= 0 || n > (1 << 24))
        return fail(MOE_INT4_EINVAL, "n=%d outside [1, 16777216]", n);
    if (k <= 0 || k % group || k > 65536)
        return fail(MOE_INT4_EINVAL, "k=%d must be a positive multiple of group=%d, at most 65536", k, group);
    if ((long long)tokens * n >= (1LL << 31) || (long long)tokens * k >= (1LL << 31))
        return fail(MOE_INT4_EINVAL, "tokens * n and tokens * k must stay below 2^31");
    return MOE_INT4_OK;
}

}  // namespace

size_t workspace_size(const Dims &d) { return layout(d).total; }

static_assert(kKeysBytes == MOE_INT4_WS_STATUS_OFFSET, "status word follows the router keys");
static_assert(kKeysBytes + kCtrlBytes == MOE_INT4_WS_PREFIX_BYTES, "control prefix size");
static_assert(kStatusKeyWait == MOE_INT4_STATUS_KEY_WAIT && kStatusRouteWait == MOE_INT4_STATUS_ROUTE_WAIT &&
                  kStatusHWait == MOE_INT4_STATUS_H_WAIT,
              "status bits");

// ---------------------------------------------------------------------------
// Static scratch of moe_int4_forward_noalloc: the workspace as a file-scope
// device array, so that the entry point allocates nothing.  Each device the
// library runs on holds its own copy (kScratchBytes) until the process ends;
// host code uses only the per-device address from hipGetSymbolAddress (the
// array's name in host code is a host-side stand-in, not a device address).
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)MOE_INT4_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];   // device address of `scratch` per device, null until set up

__global__ void zero_words_kernel(uint32_t *p, int n)
{
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// The current device's scratch, set up on its first use: the symbol's
// address on that device, then its control prefix cleared by a fill kernel
// on the caller's stream, ahead of the first call's kernels.
int32_t device_scratch(hipStream_t st, void **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return fail(MOE_INT4_EDEVICE, "no HIP device is current");
    if (st) {
        int sdev = -1;
        if (hipStreamGetDevice(st, &sdev) != hipSuccess)
            return fail(MOE_INT4_EINVAL, "hipStreamGetDevice failed for the given stream");
        if (sdev != dev)
            return fail(MOE_INT4_EINVAL, "the stream belongs to device %d, the current device is %d", sdev, dev);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(MOE_INT4_EDEVICE, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                        hipGetErrorString(e));
        const int words = (int)(MOE_INT4_WS_PREFIX_BYTES / 4);
        zero_words_kernel<<<(words + 255) / 256, 256, 0, st>>>(reinterpret_cast<uint32_t *>(p), words);
        int32_t rc = launched(hipGetLastError(), "scratch clear");
        if (rc) return rc;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return MOE_INT4_OK;
}

// A second stream per device, with a fork and a join event, on which a
// many-token forward runs its shared expert: that work needs only x and the
// shared gate logits (both written by the top-k kernel), so it overlaps the
// permutation (a few workgroups) and the routed GEMMs' tails instead of
// following them.  Made on the first forward that can use it; a forward whose
// stream is being captured before then, or that may not allocate, runs the
// shared expert on its own stream.  The mutex keeps each forward's fork,
// shared launches and join together when several host threads enqueue.
struct SideStream {
    hipStream_t st = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];

const SideStream *side_stream(hipStream_t main)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    SideStream &s = g_side[dev];
    if (s.st) return &s;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(main, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
    SideStream n;
    if (hipStreamCreateWithFlags(&n.st, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&n.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&n.join, hipEventDisableTiming) != hipSuccess) {
        if (n.fork) (void)hipEventDestroy(n.fork);
        (void)hipStreamDestroy(n.st);
        return nullptr;
    }
    s = n;
    return &s;
}

}  // namespace

}  // namespace moe

using namespace moe;

extern "C" {

const char *moe_int4_version(void) { return "moe_int4 0.1 gfx950"; }

const char *moe_int4_last_error(void) { return g_error.c_str(); }

int32_t moe_int4_workspace_bytes(const moe_int4_shape *shape, const moe_shared_int6 *shared,
                                 size_t *bytes)
{
    Dims d;
    int32_t rc = check_shape(shape, shared, &d);
    if (rc) return rc;
    if (!bytes) return fail(MOE_INT4_EINVAL, "bytes is NULL");
    *bytes = workspace_size(d);
    return MOE_INT4_OK;
}

int32_t moe_int4_route(const uint16_t *x, const uint16_t *router_w, const moe_int4_shape *shape,
                       int32_t *topk_ids, float *topk_w, int32_t *expert_counts,
                       int32_t *expert_offsets, int32_t *sorted_slots, void *workspace,
                       size_t workspace_bytes, void *hip_stream)
{
    g_error.clear();
    Dims d;
    int32_t rc = check_shape(shape, nullptr, &d);
    if (rc) return rc;
    if (d.T == 0) return MOE_INT4_OK;
    rc = check_ptrs({{"x", x}, {"router_w", router_w}, {"topk_ids", topk_ids},
                     {"topk_w", topk_w}, {"expert_counts", expert_counts},
                     {"expert_offsets", expert_offsets}, {"sorted_slots", sorted_slots}});
    if (rc) return rc;
    Workspace ws;
    if ((rc = check_workspace(d, workspace, workspace_bytes, &ws))) return rc;
    if ((rc = check_device())) return rc;
    RouteOut ro{topk_ids, topk_w, expert_counts, expert_offsets, sorted_slots};
    return launched(launch_route(x, router_w, d, ws, ro, (hipStream_t)hip_stream), "route");
}

int32_t moe_int4_experts(const uint16_t *x, const int32_t *topk_ids, const float *topk_w,
                         const int32_t *w13_packed, const uint16_t *w13_scales,
                         const int32_t *w2_packed, const uint16_t *w2_scales,
                         const moe_int4_shape *shape, const moe_shared_int6 *shared,
                         uint16_t *out, void *workspace, size_t workspace_bytes, void *hip_stream)
{
    g_error.clear();
    Dims d;
    int32_t rc = check_shape(shape, shared, &d);
    if (rc) return rc;
    if (d.T == 0) return MOE_INT4_OK;
    rc = check_ptrs({{"x", x}, {"topk_ids", topk_ids}, {"topk_w", topk_w},
                     {"w13_packed", w13_packed}, {"w13_scales", w13_scales},
                     {"w2_packed", w2_packed}, {"w2_scales", w2_scales}, {"out", out}});
    if (rc) return rc;
    if ((const void *)out == (const void *)x) return fail(MOE_INT4_EINVAL, "out aliases x");
    Workspace ws;
    if ((rc = check_workspace(d, workspace, workspace_bytes, &ws))) return rc;
    if ((rc = check_device())) return rc;
    hipStream_t st = (hipStream_t)hip_stream;
    ExpertArgs a{x, w13_packed, w13_scales, w2_packed, w2_scales, topk_w, out,
                 shared ? shared->gate_w : nullptr, shared ? shared->w13_packed : nullptr,
                 shared ? shared->w13_scales : nullptr, shared ? shared->w2_packed : nullptr,
                 shared ? shared->w2_scales : nullptr};
    if (d.T <= kDecodeMaxTokens)
        return launched(launch_decode_experts(a, topk_ids, topk_w, d, ws, st), "experts");
    RouteOut ro{const_cast<int32_t *>(topk_ids), const_cast<float *>(topk_w), ws.counts,
                ws.offsets, ws.sorted_slots};
    if ((rc = launched(launch_permute(d, ws, ro, st), "permute"))) return rc;
    return launched(launch_prefill_experts(a, d, ws, ro, st, nullptr), "experts");
}

// The host checks of the whole-layer entry points that do not involve the
// workspace (T = 0 passes without pointer checks: it is a no-op).
static int32_t forward_args(const uint16_t *x, const uint16_t *router_w, const int32_t *w13_packed,
                            const uint16_t *w13_scales, const int32_t *w2_packed,
                            const uint16_t *w2_scales, int32_t top_k, const uint16_t *out,
                            const moe_int4_shape *shape, const moe_shared_int6 *shared, Dims *d)
{
    int32_t rc = check_shape(shape, shared, d);
    if (rc) return rc;
    if (top_k != shape->top_k)
        return fail(MOE_INT4_EINVAL, "top_k=%d differs from shape->top_k=%d", top_k, shape->top_k);
    if (d->T == 0) return MOE_INT4_OK;
    rc = check_ptrs({{"x", x}, {"router_w", router_w}, {"w13_packed", w13_packed},
                     {"w13_scales", w13_scales}, {"w2_packed", w2_packed},
                     {"w2_scales", w2_scales}, {"out", out}});
    if (rc) return rc;
    if ((const void *)out == (const void *)x) return fail(MOE_INT4_EINVAL, "out aliases x");
    return MOE_INT4_OK;
}

static int32_t forward_impl(const uint16_t *x, const uint16_t *router_w,
                           const int32_t *w13_packed, const uint16_t *w13_scales,
                           const int32_t *w2_packed, const uint16_t *w2_scales, int32_t top_k,
                           uint16_t *out, const moe_int4_shape *shape,
                           const moe_shared_int6 *shared, void *workspace,
                           size_t workspace_bytes, void *hip_stream, void *const *events,
                           uint32_t *status = nullptr, bool side = true)
{
    g_error.clear();
    Dims d;
    int32_t rc = forward_args(x, router_w, w13_packed, w13_scales, w2_packed, w2_scales, top_k, out,
                              shape, shared, &d);
    if (rc || d.T == 0) return rc;
    Workspace ws;
    if ((rc = check_workspace(d, workspace, workspace_bytes, &ws))) return rc;
    if (status) ws.status = status;
    if ((rc = check_device())) return rc;
    hipStream_t st = (hipStream_t)hip_stream;
    hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
    if (events)
        for (int i = 0; i < 4; ++i) {
            if (!events[i]) return fail(MOE_INT4_EINVAL, "events[%d] is NULL", i);
            ev[i] = (hipEvent_t)events[i];
        }
    if (ev[0] && (rc = launched(hipEventRecord(ev[0], st), "event"))) return rc;
    ExpertArgs a{x, w13_packed, w13_scales, w2_packed, w2_scales, ws.weights, out,
                 shared ? shared->gate_w : nullptr, shared ? shared->w13_packed : nullptr,
                 shared ? shared->w13_scales : nullptr, shared ? shared->w2_packed : nullptr,
                 shared ? shared->w2_scales : nullptr};
    if (d.T <= kDecodeMaxTokens) {
        if ((rc = launched(launch_decode_forward(x, router_w, a, d, ws, ev[1], ev[2], st), "decode")))
            return rc;
    } else {
        RouteOut ro{ws.ids, ws.weights, ws.counts, ws.offsets, ws.sorted_slots};
        std::unique_lock<std::mutex> lock(g_side_mu, std::defer_lock);
        const SideStream *ss = nullptr;
        if (side && d.sh_I > 0) {
            lock.lock();
            ss = side_stream(st);
        }
        if ((rc = launched(launch_route(x, router_w, d, ws, ro, st, true, a.sh_gate, ss ? ss->fork : nullptr),
                           "route")))
            return rc;
        if (ss) {
            // the shared expert on the side stream from the top-k kernel on
            if ((rc = launched(hipStreamWaitEvent(ss->st, ss->fork, 0), "side stream wait"))) return rc;
            if ((rc = launched(launch_shared_expert(a, d, ws, ss->st, true), "shared expert"))) return rc;
            if ((rc = launched(hipEventRecord(ss->join, ss->st), "event"))) return rc;
        }
        if (ev[1] && (rc = launched(hipEventRecord(ev[1], st), "event"))) return rc;
        if ((rc = launched(launch_prefill_experts(a, d, ws, ro, st, ev[2], true, ss ? ss->join : nullptr),
                           "experts")))
            return rc;
    }
    if (ev[3] && (rc = launched(hipEventRecord(ev[3], st), "event"))) return rc;
    return MOE_INT4_OK;
}

int32_t moe_int4_forward(const uint16_t *x, const uint16_t *router_w, const int32_t *w13_packed,
                         const uint16_t *w13_scales, const int32_t *w2_packed,
                         const uint16_t *w2_scales, int32_t top_k, uint16_t *out,
                         const moe_int4_shape *shape, const moe_shared_int6 *shared,
                         void *workspace, size_t workspace_bytes, void *hip_stream)
{
    return forward_impl(x, router_w, w13_packed, w13_scales, w2_packed, w2_scales, top_k, out,
                        shape, shared, workspace, workspace_bytes, hip_stream, nullptr);
}

int32_t moe_int4_forward_traced(const uint16_t *x, const uint16_t *router_w,
                                const int32_t *w13_packed, const uint16_t *w13_scales,
                                const int32_t *w2_packed, const uint16_t *w2_scales,
                                int32_t top_k, uint16_t *out, const moe_int4_shape *shape,
                                const moe_shared_int6 *shared, void *workspace,
                                size_t workspace_bytes, void *hip_stream, void *const *events)
{
    if (!events) return fail(MOE_INT4_EINVAL, "events is NULL");
    return forward_impl(x, router_w, w13_packed, w13_scales, w2_packed, w2_scales, top_k, out,
                        shape, shared, workspace, workspace_bytes, hip_stream, events);
}

int32_t moe_int4_forward_noalloc(const uint16_t *x, const uint16_t *router_w,
                                 const int32_t *w13_packed, const uint16_t *w13_scales,
                                 const int32_t *w2_packed, const uint16_t *w2_scales,
                                 int32_t top_k, uint16_t *out, const moe_int4_shape *shape,
                                 const moe_shared_int6 *shared, uint32_t *status,
                                 void *hip_stream)
{
    g_error.clear();
    Dims d;
    int32_t rc = forward_args(x, router_w, w13_packed, w13_scales, w2_packed, w2_scales, top_k, out,
                              shape, shared, &d);
    if (rc) return rc;
    const size_t need = workspace_size(d);
    if (need > kScratchBytes)
        return fail(MOE_INT4_EWORKSPACE,
                    "this shape needs %zu bytes of workspace; the static scratch of "
                    "moe_int4_forward_noalloc holds %zu (use moe_int4_forward with a workspace)",
                    need, kScratchBytes);
    if (status && ((uintptr_t)status & 3u)) return fail(MOE_INT4_EALIGN, "status is not 4-byte aligned");
    if (d.T == 0) return MOE_INT4_OK;
    if ((rc = check_device())) return rc;
    void *ws = nullptr;
    if ((rc = device_scratch((hipStream_t)hip_stream, &ws))) return rc;
    // everything on the caller's stream: no side stream is made here
    return forward_impl(x, router_w, w13_packed, w13_scales, w2_packed, w2_scales, top_k, out, shape,
                        shared, ws, kScratchBytes, hip_stream, nullptr, status, false);
}

int32_t moe_int4_quantize(const uint16_t *w, int32_t rows, int32_t cols, int32_t group,
                          int32_t *packed, uint16_t *scales, void *hip_stream)
{
    g_error.clear();
    if (group != 128 && group != 64) return fail(MOE_INT4_EINVAL, "group=%d, INT4 supports 128 and 64", group);
    if (rows < 0 || cols <= 0 || cols % group)
        return fail(MOE_INT4_EINVAL, "rows=%d cols=%d: rows >= 0 and cols a positive multiple of %d",
                    rows, cols, group);
    if ((long long)rows * cols >= (1LL << 31))
        return fail(MOE_INT4_EINVAL, "rows * cols = %lld must stay below 2^31", (long long)rows * cols);
    if (rows == 0) return MOE_INT4_OK;
    int32_t rc = check_ptrs({{"w", w}, {"packed", packed}, {"scales", scales}});
    if (rc) return rc;
    if ((rc = check_device())) return rc;
    return launched(launch_quantize_int4(w, rows, cols, group, packed, scales, (hipStream_t)hip_stream),
                    "quantize");
}

int32_t moe_int8_linear_workspace_bytes(int32_t tokens, int32_t n, int32_t k, int32_t group,
                                        size_t *bytes)
{
    g_error.clear();
    int32_t rc = check_int8_shape(tokens, n, k, group);
    if (rc) return rc;
    if (!bytes) return fail(MOE_INT4_EINVAL, "bytes is NULL");
    *bytes = int8_plan(tokens, n, k, group).part_bytes;
    return MOE_INT4_OK;
}

int32_t moe_int8_linear(const uint16_t *x, const int32_t *w_packed, const uint16_t *w_scales,
                        int32_t tokens, int32_t n, int32_t k, int32_t group, uint16_t *out,
                        void *workspace, size_t workspace_bytes, void *hip_stream)
{
    g_error.clear();
    int32_t rc = check_int8_shape(tokens, n, k, group);
    if (rc) return rc;
    if (tokens == 0) return MOE_INT4_OK;
    rc = check_ptrs({{"x", x}, {"w_packed", w_packed}, {"w_scales", w_scales}, {"out", out}});
    if (rc) return rc;
    const size_t need = int8_plan(tokens, n, k, group).part_bytes;
    if (need) {
        if (!workspace) return fail(MOE_INT4_EINVAL, "workspace is NULL (%zu bytes needed)", need);
        if (!aligned16(workspace)) return fail(MOE_INT4_EALIGN, "workspace is not 16-byte aligned");
        if (workspace_bytes < need)
            return fail(MOE_INT4_EWORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
    }
    if ((rc = check_device())) return rc;
    return launched(launch_int8_linear(x, w_packed, w_scales, tokens, n, k, group, out, workspace,
                                       (hipStream_t)hip_stream),
                    "int8 linear");
}

}  // extern "C"
