// Routing kernels: router logits, top-k with renormalised softmax, and the
// stable grouping of token slots by expert.
//
// Method ("Running 125B MoE on Three 3090s - vLLM Optimization Edition",
// section 3.3, "MoE block (decode-05)"):
//   * the router is one GEMV over the bf16 router rows;
//   * the workgroup that finishes last (found with an acquire-release ticket
//     taken after its stores) does the top-k, the renormalisation and the
//     grouping of slots by expert, so no grid-wide barrier kernel is needed;
//   * top-k keys pack an order-preserving integer image of the logit above
//     the inverted expert id, so one max yields value and id and equal
//     logits resolve to the lower id;
//   * with renormalisation the full softmax denominator cancels, so the
//     weights are a softmax over the k selected logits.
// Logits stay fp32 (the page keys on bf16 logits; fp32 avoids manufacturing
// ties).  Everything here is integer-exact except the fp32 sums and exp.
#include "common.h"

namespace moe {

// ---------------------------------------------------------------------------
// wave-level helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        uint64_t o = __shfl_xor(v, off, kWave);
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane)
{
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int o = __shfl_up(v, off, kWave);
        if (lane >= off) v += o;
    }
    return v;
}

// Order-preserving map of a finite float onto uint32 (-0 and +0 coincide).
__device__ __forceinline__ uint32_t float_order(float l)
{
    uint32_t u = __float_as_uint(l == 0.f ? 0.f : l);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_float(uint32_t o)
{
    uint32_t u = (o & 0x80000000u) ? (o ^ 0x80000000u) : ~o;
    return __uint_as_float(u);
}

// Top-k of one token's logits by one wave.  KPL = ceil(E/64) keys per lane.
// Writes ids/weights (global) and, if lds_ids != nullptr, the ids to LDS.
template <int KPL>
__device__ void wave_topk(const float *lrow, int E, int k, int lane, int32_t *ids,
                          float *weights, int32_t *lds_ids)
{
    uint64_t key[KPL];
    uint64_t lmax = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        int e = lane + kWave * i;
        key[i] = 0;
        if (e < E) {
            uint64_t o = float_order(lrow[e]);
            key[i] = (o << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
        }
        lmax = key[i] > lmax ? key[i] : lmax;
    }
    int my_e = 0;
    float my_l = 0.f, first_l = 0.f;
    for (int r = 0; r < k; ++r) {
        uint64_t m = wave_max_u64(lmax);
        int e = (int)(0xFFFFFFFFu - (uint32_t)m);
        float l = order_float((uint32_t)(m >> 32));
        if (r == 0) first_l = l;
        if (lane == r) { my_e = e; my_l = l; }
        if ((e & (kWave - 1)) == lane) {
            lmax = 0;
#pragma unroll
            for (int i = 0; i < KPL; ++i) {
                if (i == (e >> 6)) key[i] = 0;
                lmax = key[i] > lmax ? key[i] : lmax;
            }
        }
    }
    float ex = lane < k ? expf(my_l - first_l) : 0.f;
    float sum = wave_sum(ex);
    if (lane < k) {
        ids[lane] = my_e;
        weights[lane] = ex / sum;
        if (lds_ids) lds_ids[lane] = my_e;
    }
}

__device__ void topk_any(const float *lrow, int E, int k, int lane, int32_t *ids, float *w,
                         int32_t *lds_ids)
{
    if (E <= 64) wave_topk<1>(lrow, E, k, lane, ids, w, lds_ids);
    else if (E <= 128) wave_topk<2>(lrow, E, k, lane, ids, w, lds_ids);
    else if (E <= 256) wave_topk<4>(lrow, E, k, lane, ids, w, lds_ids);
    else if (E <= 512) wave_topk<8>(lrow, E, k, lane, ids, w, lds_ids);
    else wave_topk<16>(lrow, E, k, lane, ids, w, lds_ids);
}

// Lanes holding the same (valid) id as this lane, as a 64-bit mask.
__device__ __forceinline__ uint64_t match_id(int id, bool valid, int nbits)
{
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        bool bit = (id >> b) & 1;
        uint64_t bal = __ballot(valid && bit);
        m &= bit ? bal : ~bal;
    }
    return m;
}

// Caller-given ids outside [0, E) are clamped so that no access leaves its
// buffer (the results for such input are unspecified).
__device__ __forceinline__ int clamp_id(int id, int E) { return id < 0 ? 0 : (id >= E ? E - 1 : id); }

__device__ __forceinline__ int id_bits(int E)
{
    int b = 1;
    while ((1 << b) < E) ++b;
    return b;
}

// Count slots per expert over slots [beg, end) into run[] (LDS, E ints, must
// be zero on entry).  One wave.
__device__ void wave_count(const int32_t *ids, int beg, int end, int E, int lane, int32_t *run)
{
    const int nbits = id_bits(E);
    for (int base = beg; base < end; base += kWave) {
        int s = base + lane;
        bool valid = s < end;
        int id = valid ? clamp_id(ids[s], E) : 0;
        uint64_t m = match_id(id, valid, nbits);
        bool leader = valid && ((m & ((1ull << lane) - 1)) == 0);
        if (leader) run[id] += __popcll(m);
    }
}

// Place slots [beg, end) at run[id] + (rank among equal ids), advancing run[].
__device__ void wave_scatter(const int32_t *ids, int beg, int end, int E, int lane, int32_t *run,
                             int32_t *sorted_slots, int32_t *slot_pos)
{
    const int nbits = id_bits(E);
    for (int base = beg; base < end; base += kWave) {
        int s = base + lane;
        bool valid = s < end;
        int id = valid ? clamp_id(ids[s], E) : 0;
        uint64_t m = match_id(id, valid, nbits);
        uint64_t below = m & ((1ull << lane) - 1);
        int pos = valid ? run[id] + __popcll(below) : 0;
        if (valid) {
            sorted_slots[pos] = s;
            slot_pos[s] = pos;
        }
        if (valid && below == 0) run[id] += __popcll(m);
    }
}

// counts -> offsets (exclusive) and the active-expert list; turns run[] into
// the per-expert write cursor.  One wave; run[] holds the counts on entry.
__device__ void wave_offsets(int E, int S, int lane, int32_t *run, int32_t *counts,
                             int32_t *offsets, int32_t *active)
{
    const int per = (E + kWave - 1) / kWave;
    const int e0 = lane * per;
    int local = 0, nz = 0;
    for (int i = 0; i < per; ++i) {
        int e = e0 + i;
        if (e < E) {
            local += run[e];
            nz += run[e] > 0;
        }
    }
    int excl = wave_incl_scan(local, lane) - local;
    int nz_excl = wave_incl_scan(nz, lane) - nz;
    for (int i = 0; i < per; ++i) {
        int e = e0 + i;
        if (e < E) {
            int c = run[e];
            counts[e] = c;
            offsets[e] = excl;
            run[e] = excl;
            if (c > 0) active[1 + nz_excl++] = e;
            excl += c;
        }
    }
    if (lane == kWave - 1) {
        offsets[E] = S;
        active[0] = nz_excl;
    }
}

// The whole permutation by one wave (small S).  run: LDS, E ints.
__device__ void wave_permute(const int32_t *ids, int S, int E, int lane, int32_t *run,
                             int32_t *counts, int32_t *offsets, int32_t *sorted_slots,
                             int32_t *slot_pos, int32_t *active)
{
    for (int e = lane; e < E; e += kWave) run[e] = 0;
    wave_count(ids, 0, S, E, lane, run);
    wave_offsets(E, S, lane, run, counts, offsets, active);
    wave_scatter(ids, 0, S, E, lane, run, sorted_slots, slot_pos);
}

// ---------------------------------------------------------------------------
// Decode routing: one kernel.  Each wave computes one expert's logits for all
// T tokens; the last workgroup to finish selects and permutes.
// ---------------------------------------------------------------------------
constexpr int kRouterWaves = 2;

template <int CPL>
__global__ __launch_bounds__(kRouterWaves * kWave) void router_decode_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ router_w, Dims d, Workspace ws,
    RouteOut ro)
{
    __shared__ int32_t s_ids[kDecodeMaxTokens * kMaxTopK];
    __shared__ int32_t s_run[kMaxExperts];
    __shared__ int s_last;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int e = blockIdx.x * kRouterWaves + wave;
    const int nck = d.H / 8;  // 16-byte chunks per row

    if (e < d.E) {
        uint4 wr[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            int idx = lane + kWave * c;
            if (idx < nck)
                wr[c] = reinterpret_cast<const uint4 *>(router_w + (size_t)e * d.H)[idx];
        }
        for (int t = 0; t < d.T; ++t) {
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                int idx = lane + kWave * c;
                if (idx < nck) {
                    uint4 xv = reinterpret_cast<const uint4 *>(x + (size_t)t * d.H)[idx];
                    acc = dot2(wr[c].x, xv.x, acc);
                    acc = dot2(wr[c].y, xv.y, acc);
                    acc = dot2(wr[c].z, xv.z, acc);
                    acc = dot2(wr[c].w, xv.w, acc);
                }
            }
            acc = wave_sum(acc);
            if (lane == 0) ws.logits[(size_t)t * d.E + e] = acc;
        }
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t ticket = atomicAdd(ws.route_ticket, 1u);
        s_last = (ticket == gridDim.x - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    for (int t = wave; t < d.T; t += kRouterWaves)
        topk_any(ws.logits + (size_t)t * d.E, d.E, d.k, lane, ro.ids + (size_t)t * d.k,
                 ro.weights + (size_t)t * d.k, s_ids + t * d.k);
    __syncthreads();
    if (wave == 0)
        wave_permute(s_ids, d.S, d.E, lane, s_run, ro.counts, ro.offsets, ro.sorted_slots,
                     ws.slot_pos, ws.active);
    if (threadIdx.x == 0) *ws.route_ticket = 0;
}

// ---------------------------------------------------------------------------
// Prefill routing
// ---------------------------------------------------------------------------

// Router GEMM for many tokens: 64 tokens x 64 experts per workgroup, fp32
// FMA over LDS-staged tiles.
constexpr int kRG_T = 64, kRG_E = 64, kRG_K = 32;

__global__ __launch_bounds__(256) void router_gemm_kernel(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ router_w,
                                                          Dims d, float *__restrict__ logits)
{
    __shared__ float sa[kRG_K][kRG_T + 1];
    __shared__ float sb[kRG_K][kRG_E + 1];
    const int t0 = blockIdx.x * kRG_T, e0 = blockIdx.y * kRG_E;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < d.H; k0 += kRG_K) {
        for (int i = threadIdx.x; i < kRG_T * kRG_K; i += 256) {
            int r = i / kRG_K, c = i % kRG_K;
            int t = t0 + r, e = e0 + r;
            sa[c][r] = t < d.T ? bf16_to_f32(x[(size_t)t * d.H + k0 + c]) : 0.f;
            sb[c][r] = e < d.E ? bf16_to_f32(router_w[(size_t)e * d.H + k0 + c]) : 0.f;
        }
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < kRG_K; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = sa[kk][ty * 4 + i];
                b[i] = sb[kk][tx * 4 + i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int t = t0 + ty * 4 + i;
        if (t >= d.T) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int e = e0 + tx * 4 + j;
            if (e < d.E) logits[(size_t)t * d.E + e] = acc[i][j];
        }
    }
}

// One wave per token.
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, Dims d,
                                                   int32_t *ids, float *weights)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= d.T) return;
    topk_any(logits + (size_t)t * d.E, d.E, d.k, lane, ids + (size_t)t * d.k,
             weights + (size_t)t * d.k, nullptr);
}

// Small permutation (one wave): used when routing is given by the caller.
__global__ __launch_bounds__(kWave) void permute_small_kernel(const int32_t *__restrict__ ids,
                                                              Dims d, Workspace ws, RouteOut ro)
{
    __shared__ int32_t s_run[kMaxExperts];
    wave_permute(ids, d.S, d.E, threadIdx.x, s_run, ro.counts, ro.offsets, ro.sorted_slots,
                 ws.slot_pos, ws.active);
}

// Large permutation, pass 1: per-chunk histograms (one wave per chunk).
__global__ __launch_bounds__(kWave) void perm_hist_kernel(const int32_t *__restrict__ ids, Dims d,
                                                          Workspace ws)
{
    __shared__ int32_t s_run[kMaxExperts];
    const int c = blockIdx.x, lane = threadIdx.x;
    for (int e = lane; e < d.E; e += kWave) s_run[e] = 0;
    int beg = c * kPermChunk, end = min(d.S, beg + kPermChunk);
    wave_count(ids, beg, end, d.E, lane, s_run);
    for (int e = lane; e < d.E; e += kWave) ws.chunk_hist[(size_t)c * d.E + e] = s_run[e];
}

// Pass 2: per-expert totals, offsets, active list, and each chunk's base.
// One workgroup of 1024 threads, thread e owns expert e.
__global__ __launch_bounds__(1024) void perm_scan_kernel(Dims d, Workspace ws, RouteOut ro,
                                                         int nchunks)
{
    __shared__ int s_sum[16], s_nz[16];
    const int e = threadIdx.x, lane = e & (kWave - 1), wave = e >> 6;
    int total = 0;
    if (e < d.E)
        for (int c = 0; c < nchunks; ++c) total += ws.chunk_hist[(size_t)c * d.E + e];
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
        for (int c = 0; c < nchunks; ++c) {
            int v = ws.chunk_hist[(size_t)c * d.E + e];
            ws.chunk_hist[(size_t)c * d.E + e] = run;
            run += v;
        }
    }
    if (e == d.E - 1) {
        ro.offsets[d.E] = d.S;
        ws.active[0] = nz_pos + nz;
    }
}

// Pass 3: scatter each chunk's slots from its per-expert bases.
__global__ __launch_bounds__(kWave) void perm_scatter_kernel(const int32_t *__restrict__ ids,
                                                             Dims d, Workspace ws, RouteOut ro)
{
    __shared__ int32_t s_run[kMaxExperts];
    const int c = blockIdx.x, lane = threadIdx.x;
    for (int e = lane; e < d.E; e += kWave) s_run[e] = ws.chunk_hist[(size_t)c * d.E + e];
    int beg = c * kPermChunk, end = min(d.S, beg + kPermChunk);
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
    int nchunks = (d.S + kPermChunk - 1) / kPermChunk;
    perm_hist_kernel<<<nchunks, kWave, 0, st>>>(ro.ids, d, ws);
    perm_scan_kernel<<<1, 1024, 0, st>>>(d, ws, ro, nchunks);
    perm_scatter_kernel<<<nchunks, kWave, 0, st>>>(ro.ids, d, ws, ro);
    return hipGetLastError();
}

hipError_t launch_route(const uint16_t *x, const uint16_t *router_w, const Dims &d,
                        const Workspace &ws, const RouteOut &ro, hipStream_t st)
{
    if (d.T <= kDecodeMaxTokens) {
        int grid = (d.E + kRouterWaves - 1) / kRouterWaves;
        int cpl = (d.H / 8 + kWave - 1) / kWave;
#define MOE_ROUTER_CASE(N) \
    case N: router_decode_kernel<N><<<grid, kRouterWaves * kWave, 0, st>>>(x, router_w, d, ws, ro); break;
        switch (cpl) {
            MOE_ROUTER_CASE(1) MOE_ROUTER_CASE(2) MOE_ROUTER_CASE(3) MOE_ROUTER_CASE(4)
            MOE_ROUTER_CASE(5) MOE_ROUTER_CASE(6) MOE_ROUTER_CASE(7) MOE_ROUTER_CASE(8)
            default: return hipErrorInvalidValue;
        }
#undef MOE_ROUTER_CASE
        return hipGetLastError();
    }
    dim3 grid((d.T + kRG_T - 1) / kRG_T, (d.E + kRG_E - 1) / kRG_E);
    router_gemm_kernel<<<grid, 256, 0, st>>>(x, router_w, d, ws.logits);
    topk_kernel<<<(d.T + 3) / 4, 256, 0, st>>>(ws.logits, d, ro.ids, ro.weights);
    return launch_permute(d, ws, ro, st);
}

}  // namespace moe
