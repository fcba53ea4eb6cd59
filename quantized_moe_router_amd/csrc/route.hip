// Routing kernels: router logits, top-k with renormalised softmax, and the
// stable grouping of token slots by expert.
//
// Method ("Running 125B MoE on Three 3090s - vLLM Optimization Edition",
// section 3.3, "MoE block (decode-05)"):
//   * the router is one GEMV over the bf16 router rows;
//   * the page's router hands its logits to its last CTA, which does the
//     top-k, the renormalisation and the grouping of slots by expert; here
//     the few-token router (decode.hip) publishes its logits as keys that a
//     routing workgroup of the same launch polls, and the many-token path
//     below runs a top-k kernel and a permutation after the router GEMM;
//   * top-k keys pack an order-preserving integer image of the logit above
//     the inverted expert id, so one max yields value and id and equal
//     logits resolve to the lower id;
//   * with renormalisation the full softmax denominator cancels, so the
//     weights are a softmax over the k selected logits.
// Logits stay fp32 (the page keys on bf16 logits; fp32 avoids manufacturing
// ties).  Everything here is integer-exact except the fp32 sums and exp.
#include "permute.h"
#include "tiles.h"
#include "topk.h"

namespace moe {

// ---------------------------------------------------------------------------
// Prefill routing
// ---------------------------------------------------------------------------

// One wave per token.
// The logits arrive as nsplit partial sums over H ([split][T][E]), added here
// in split order.
// With xh given, the wave also writes its token's x row to xh in the gate/up
// GEMMs' fp16 pair order: the row's loads are issued with the logits' loads,
// so the conversion rides on their latency instead of taking a kernel of its
// own, and the row is stored before the selection, which then runs without
// the row's registers.  With gate_w given as well, it also forms the shared
// expert's gate logit x . gate_w from the same registers (bf16 products, fp32
// sums in the order of the stand-alone gate kernel).  KPL = ceil(E / 64) and
// NB (the logit splits loaded per pass) are template arguments, so a launch
// holds the registers of its own variant only.
template <int KPL, int NB>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int nsplit, Dims d,
                                                   int32_t *ids, float *weights,
                                                   const uint16_t *__restrict__ x, uint16_t *__restrict__ xh,
                                                   const uint16_t *__restrict__ gate_w,
                                                   float *__restrict__ gate_out)
{
    __shared__ uint32_t s_topk[4][kTopkLds];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    if (t >= d.T) return;
    constexpr int kXo = kMaxHidden / 8 / kWave;   // octets of a row per lane
    const int n8 = d.H / 8;
    const bool gate = xh && gate_w;
    uint4 xo[kXo], gv[kXo];
    if (xh) {
        const uint4 *src = reinterpret_cast<const uint4 *>(x + (size_t)t * d.H);
#pragma unroll
        for (int j = 0; j < kXo; ++j) xo[j] = src[min(lane + kWave * j, n8 - 1)];
        if (gate) {
#pragma unroll
            for (int j = 0; j < kXo; ++j) gv[j] = reinterpret_cast<const uint4 *>(gate_w)[min(lane + kWave * j, n8 - 1)];
        }
    }
    uint32_t val[KPL];
    logit_keys<KPL, NB>(logits + (size_t)t * d.E, nsplit, (size_t)d.T * d.E, d.E, lane, val);
    if (xh) {
        uint4 *dst = reinterpret_cast<uint4 *>(xh + (size_t)t * d.H);
#pragma unroll
        for (int j = 0; j < kXo; ++j)
            if (lane + kWave * j < n8) dst[lane + kWave * j] = bf16_octet_to_f16_pairs(xo[j]);
        if (gate) {
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < kXo; ++j) {
                if (lane + kWave * j < n8) {
                    acc = dot2(gv[j].x, xo[j].x, acc);
                    acc = dot2(gv[j].y, xo[j].y, acc);
                    acc = dot2(gv[j].z, xo[j].z, acc);
                    acc = dot2(gv[j].w, xo[j].w, acc);
                }
            }
            acc = wave_sum(acc);
            if (lane == 0) gate_out[t] = acc;
        }
    }
    const TopkLane r = wave_topk_keys<KPL>(val, d.k, lane, s_topk[wave]);
    if (lane < d.k) {
        ids[(size_t)t * d.k + lane] = r.id;
        weights[(size_t)t * d.k + lane] = r.w;
    }
}

template <int KPL>
static void launch_topk_kpl(const float *logits, int nsplit, const Dims &d, int32_t *ids, float *weights,
                            const uint16_t *x, uint16_t *xh, const uint16_t *gate_w, float *gate_out,
                            hipStream_t st)
{
    const unsigned grid = (unsigned)((d.T + 3) / 4);
    if (nsplit <= 1)
        topk_kernel<KPL, 1><<<grid, 256, 0, st>>>(logits, nsplit, d, ids, weights, x, xh, gate_w, gate_out);
    else if (nsplit == 2)
        topk_kernel<KPL, 2><<<grid, 256, 0, st>>>(logits, nsplit, d, ids, weights, x, xh, gate_w, gate_out);
    else
        topk_kernel<KPL, 4><<<grid, 256, 0, st>>>(logits, nsplit, d, ids, weights, x, xh, gate_w, gate_out);
}

static void launch_topk(const float *logits, int nsplit, const Dims &d, int32_t *ids, float *weights,
                        const uint16_t *x, uint16_t *xh, const uint16_t *gate_w, float *gate_out, hipStream_t st)
{
    if (d.E <= 64) launch_topk_kpl<1>(logits, nsplit, d, ids, weights, x, xh, gate_w, gate_out, st);
    else if (d.E <= 128) launch_topk_kpl<2>(logits, nsplit, d, ids, weights, x, xh, gate_w, gate_out, st);
    else if (d.E <= 256) launch_topk_kpl<4>(logits, nsplit, d, ids, weights, x, xh, gate_w, gate_out, st);
    else if (d.E <= 512) launch_topk_kpl<8>(logits, nsplit, d, ids, weights, x, xh, gate_w, gate_out, st);
    else launch_topk_kpl<16>(logits, nsplit, d, ids, weights, x, xh, gate_w, gate_out, st);
}

// Small permutation (one wave): used when routing is given by the caller.
__global__ __launch_bounds__(kWave) void permute_small_kernel(const int32_t *__restrict__ ids,
                                                              Dims d, Workspace ws, RouteOut ro)
{
    __shared__ int32_t s_run[kMaxExperts];
    wave_permute(ids, d.S, d.E, threadIdx.x, s_run, ro.counts, ro.offsets, ro.sorted_slots,
                 ws.slot_pos, ws.active);
}

// Mid-size permutation (kPermChunk < S <= kPermMidWaves * kPermChunk): one
// workgroup of 16 waves runs the three passes of the large path without a
// kernel boundary.  Wave w counts the slots [w * chunk, + chunk) into its own
// LDS histogram (LDS atomics: a count needs no ranking); thread e then sums expert e over the chunks, the workgroup
// scans the totals, and expert e's base in each chunk replaces the count;
// each wave finally scatters its chunk from those bases (in slot order:
// stable).
static_assert(kPermMidWaves * kWave >= kMaxExperts, "one thread per expert in the scan");

__global__ __launch_bounds__(kPermMidWaves * kWave) void permute_mid_kernel(const int32_t *__restrict__ ids,
                                                                            Dims d, Workspace ws, RouteOut ro,
                                                                            int nslots, int mt)
{
    __shared__ int32_t s_run[kPermMidWaves][kMaxExperts];
    __shared__ int s_sum[kPermMidWaves], s_nz[kPermMidWaves];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int E = d.E, S = d.S;
    const int chunk = (S + kPermMidWaves - 1) / kPermMidWaves;   // <= kPermChunk
    const int beg = min(S, wave * chunk), end = min(S, beg + chunk);
    // the chunk's ids stay in registers for the scatter; the count needs no
    // ranking, so it is one LDS atomic per slot
    int idv[kPermPer];
    load_chunk_ids(ids, beg, end, E, lane, idv);
    for (int e = lane; e < E; e += kWave) s_run[wave][e] = 0;
#pragma unroll
    for (int j = 0; j < kPermPer; ++j) {
        if (beg + kWave * j >= end) break;   // uniform
        if (beg + kWave * j + lane < end) atomicAdd(&s_run[wave][idv[j]], 1);
    }
    __syncthreads();
    const int e = tid;   // kPermMidWaves * kWave = 1024 = kMaxExperts threads
    int total = 0;
    if (e < E)
        for (int w = 0; w < kPermMidWaves; ++w) total += s_run[w][e];
    const int nz = (e < E && total > 0) ? 1 : 0;
    const int incl = wave_incl_scan(total, lane), nz_incl = wave_incl_scan(nz, lane);
    if (lane == kWave - 1) {
        s_sum[wave] = incl;
        s_nz[wave] = nz_incl;
    }
    __syncthreads();
    int base = 0, nz_base = 0;
    for (int w = 0; w < wave; ++w) {
        base += s_sum[w];
        nz_base += s_nz[w];
    }
    const int off = base + incl - total, nz_pos = nz_base + nz_incl - nz;
    if (e < E) {
        ro.counts[e] = total;
        ro.offsets[e] = off;
        if (nz) ws.active[1 + nz_pos] = e;
        int run = off;
        for (int w = 0; w < kPermMidWaves; ++w) {
            const int c = s_run[w][e];
            s_run[w][e] = run;
            run += c;
        }
    }
    if (e == E - 1) {
        ro.offsets[E] = S;
        ws.active[0] = nz_pos + nz;
    }
    __syncthreads();
    wave_scatter_ids(idv, beg, end, E, lane, s_run[wave], ro.sorted_slots, ws.slot_pos);
    // the grouped GEMMs' tile list from this thread's (expert e's) count and
    // offset
    build_tile_list(e < E ? total : 0, e < E ? off : 0, nslots, mt, ws.tiles, s_sum);
}

// Large permutation, pass 1: per-chunk histograms (one wave per chunk).
__global__ __launch_bounds__(kWave) void perm_hist_kernel(const int32_t *__restrict__ ids, Dims d,
                                                          Workspace ws)
{
    __shared__ int32_t s_run[kMaxExperts];
    const int c = blockIdx.x, lane = threadIdx.x;
    for (int e = lane; e < d.E; e += kWave) s_run[e] = 0;
    const int chunk = perm_chunk(d.S);
    int beg = c * chunk, end = min(d.S, beg + chunk);
    // a count needs no ranking: one LDS atomic per slot
    int idv[kPermPer];
    load_chunk_ids(ids, beg, end, d.E, lane, idv);
#pragma unroll
    for (int j = 0; j < kPermPer; ++j) {
        if (beg + kWave * j >= end) break;   // uniform
        if (beg + kWave * j + lane < end) atomicAdd(&s_run[idv[j]], 1);
    }
    for (int e = lane; e < d.E; e += kWave) ws.chunk_hist[(size_t)c * d.E + e] = s_run[e];
}

// Pass 2: per-expert totals, offsets, active list, and each chunk's base.
// One workgroup of 1024 threads, thread e owns expert e.
__global__ __launch_bounds__(1024) void perm_scan_kernel(Dims d, Workspace ws, RouteOut ro,
                                                         int nchunks, int nslots, int mt)
{
    __shared__ int s_sum[16], s_nz[16];
    const int e = threadIdx.x, lane = e & (kWave - 1), wave = e >> 6;
    const int ec = e < d.E ? e : 0;
    // Up to kScanKeep chunks: every count of the expert loaded at once and
    // kept in registers for the bases (two 16-bit counts per register: a
    // count is at most kPermChunk), so the pass costs one round of loads
    // instead of one per batch and pass.  More chunks: kScanBatch loads in
    // flight per batch (clamped addresses), summed in order, and loaded again
    // for the bases.
    constexpr int kScanKeep = 128, kScanBatch = 32;
    static_assert(kPermChunk < 65536, "16-bit counts");
    const bool keep = nchunks <= kScanKeep;
    uint32_t kv[kScanKeep / 2];
    int total = 0;
    if (keep) {
#pragma unroll
        for (int u = 0; u < kScanKeep / 2; ++u) {
            const int c = 2 * u;
            const uint32_t a = (uint32_t)ws.chunk_hist[(size_t)min(c, nchunks - 1) * d.E + ec];
            const uint32_t b = (uint32_t)ws.chunk_hist[(size_t)min(c + 1, nchunks - 1) * d.E + ec];
            kv[u] = (c < nchunks ? a : 0u) | ((c + 1 < nchunks ? b : 0u) << 16);
        }
#pragma unroll
        for (int u = 0; u < kScanKeep / 2; ++u) total += (int)(kv[u] & 0xFFFFu) + (int)(kv[u] >> 16);
    } else {
        for (int c0 = 0; c0 < nchunks; c0 += kScanBatch) {
            int v[kScanBatch];
#pragma unroll
            for (int u = 0; u < kScanBatch; ++u) v[u] = ws.chunk_hist[(size_t)min(c0 + u, nchunks - 1) * d.E + ec];
#pragma unroll
            for (int u = 0; u < kScanBatch; ++u) total += c0 + u < nchunks ? v[u] : 0;
        }
    }
    if (e >= d.E) total = 0;
    int nz = (e < d.E && total > 0) ? 1 : 0;
    int incl = wave_incl_scan(total, lane), nz_incl = wave_incl_scan(nz, lane);
    if (lane == kWave - 1) { s_sum[wave] = incl; s_nz[wave] = nz_incl; }
    __syncthreads();
    int base = 0, nz_base = 0;
    for (int w = 0; w < wave; ++w) { base += s_sum[w]; nz_base += s_nz[w]; }
    int off = base + incl - total;
    int nz_pos = nz_base + nz_incl - nz;
    if (e < d.E) {
        ro.counts[e] = total;
        ro.offsets[e] = off;
        if (nz) ws.active[1 + nz_pos] = e;
        int run = off;
        if (keep) {
#pragma unroll
            for (int u = 0; u < kScanKeep / 2; ++u) {
                const int c = 2 * u;
                if (c < nchunks) ws.chunk_hist[(size_t)c * d.E + e] = run;
                run += (int)(kv[u] & 0xFFFFu);
                if (c + 1 < nchunks) ws.chunk_hist[(size_t)(c + 1) * d.E + e] = run;
                run += (int)(kv[u] >> 16);
            }
        } else {
            for (int c0 = 0; c0 < nchunks; c0 += kScanBatch) {
                int v[kScanBatch];
#pragma unroll
                for (int u = 0; u < kScanBatch; ++u) v[u] = ws.chunk_hist[(size_t)min(c0 + u, nchunks - 1) * d.E + e];
#pragma unroll
                for (int u = 0; u < kScanBatch; ++u)
                    if (c0 + u < nchunks) {
                        ws.chunk_hist[(size_t)(c0 + u) * d.E + e] = run;
                        run += v[u];
                    }
            }
        }
    }
    if (e == d.E - 1) {
        ro.offsets[d.E] = d.S;
        ws.active[0] = nz_pos + nz;
    }
    // the grouped GEMMs' tile list from this thread's (expert e's) count and
    // offset
    build_tile_list(e < d.E ? total : 0, e < d.E ? off : 0, nslots, mt, ws.tiles, s_sum);
}

// Pass 3: scatter each chunk's slots from its per-expert bases.
__global__ __launch_bounds__(kWave) void perm_scatter_kernel(const int32_t *__restrict__ ids,
                                                             Dims d, Workspace ws, RouteOut ro)
{
    __shared__ int32_t s_run[kMaxExperts];
    const int c = blockIdx.x, lane = threadIdx.x;
    for (int e = lane; e < d.E; e += kWave) s_run[e] = ws.chunk_hist[(size_t)c * d.E + e];
    const int chunk = perm_chunk(d.S);
    int beg = c * chunk, end = min(d.S, beg + chunk);
    wave_scatter(ids, beg, end, d.E, lane, s_run, ro.sorted_slots, ws.slot_pos);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_permute(const Dims &d, const Workspace &ws, const RouteOut &ro, hipStream_t st)
{
    if (d.S <= kPermChunk) {
        permute_small_kernel<<<1, kWave, 0, st>>>(ro.ids, d, ws, ro);
        return hipGetLastError();
    }
    if (d.S <= kPermMidWaves * kPermChunk) {
        permute_mid_kernel<<<1, kPermMidWaves * kWave, 0, st>>>(ro.ids, d, ws, ro, (int)routed_tile_slots(d),
                                                                routed_tile_rows(d));
        return hipGetLastError();
    }
    const int chunk = perm_chunk(d.S), nchunks = (d.S + chunk - 1) / chunk;
    perm_hist_kernel<<<nchunks, kWave, 0, st>>>(ro.ids, d, ws);
    perm_scan_kernel<<<1, 1024, 0, st>>>(d, ws, ro, nchunks, (int)routed_tile_slots(d), routed_tile_rows(d));
    perm_scatter_kernel<<<nchunks, kWave, 0, st>>>(ro.ids, d, ws, ro);
    return hipGetLastError();
}

hipError_t launch_decode_route(const uint16_t *x, const uint16_t *router_w, const Dims &d,
                               const Workspace &ws, const RouteOut &ro, hipStream_t st);
hipError_t launch_router_mfma(const uint16_t *x, const uint16_t *router_w, const Dims &d,
                              float *logits, hipStream_t st);

hipError_t launch_route(const uint16_t *x, const uint16_t *router_w, const Dims &d,
                        const Workspace &ws, const RouteOut &ro, hipStream_t st, bool convert_x,
                        const uint16_t *gate_w, hipEvent_t ev_topk)
{
    if (d.T <= kDecodeMaxTokens) return launch_decode_route(x, router_w, d, ws, ro, st);
    hipError_t e = launch_router_mfma(x, router_w, d, ws.logits, st);
    if (e != hipSuccess) return e;
    launch_topk(ws.logits, router_ksplit(d), d, ro.ids, ro.weights, x, convert_x ? ws.xh : nullptr,
                convert_x ? gate_w : nullptr, ws.shared_gate, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ev_topk && (e = hipEventRecord(ev_topk, st)) != hipSuccess) return e;
    return launch_permute(d, ws, ro, st);
}

}  // namespace moe
