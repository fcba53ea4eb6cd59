// Decode path (few tokens): three kernels.
//
//   1. router_kernel        logits[t][e] = x_t . router_w[e]  (bf16, fp32 sum),
//                           plus the shared-expert gate logit as one more row;
//                           one extra workgroup selects every token's experts
//                           (and builds the permutation for the routing-only
//                           entry point)
//   2. w13_slot_kernel      per (slot, 16-output tile): the INT4 gate/up GEMV
//                           and a = silu(g) * u -> fp16 (w13_shared_kernel:
//                           the INT6 shared expert's gate/up per token)
//   3. w2_rows_kernel       each workgroup owns 8 output rows and sums, in a
//                           fixed order, every slot's down projection weighted
//                           by its routing weight (plus sigmoid(gate) times the
//                           shared expert), then rounds once to bf16
//
// Method ("Running 125B MoE on Three 3090s - vLLM Optimization Edition",
// section 3.3, "MoE block (decode-05)"): router and shared gate as one GEMV
// whose last CTA does the top-k and renormalisation; routed experts; shared
// expert added as sigmoid(gate) x shared; down projection fused with the
// final combine.
#include "int6.h"
#include "permute.h"
#include "topk.h"

namespace moe {

__device__ __forceinline__ int clamp_expert(int id, int E)
{
    return id < 0 ? 0 : (id >= E ? E - 1 : id);
}

// ---------------------------------------------------------------------------
// 1. Router GEMV with the routing tail in one extra workgroup.
//    Producer workgroups hold one router row per wave (8 per workgroup; row E
//    is the shared-expert gate when present) and compute it for every token,
//    NT tokens' activations in flight at a time.  A producer publishes the 8
//    logits of a token with one 32-byte coherent store, as order-preserving
//    keys, which are never zero; then it is done (no wait, no counter).
//    The last workgroup, dispatched after every producer, first converts x to
//    nibble-pair order with its chunk sums (for the gate/up kernel), then
//    reads each token's keys until none is zero, selects the experts, and
//    sets the keys back to zero for the next call; for the routing-only
//    entry point it then builds the expert permutation.  With fewer tokens
//    than waves, several waves watch a token with staggered polls: one
//    coherent load round trip (about 1.2 us on this part) is the largest
//    step of the routing, and staggering shortens the wait from the last key
//    landing to a poll that sees it.  ("MoE block (decode-05)": the router's
//    last CTA does the top-k, the renormalisation and the block alignment,
//    with no separate kernel.)  The keys live in a fixed zeroed region of the
//    workspace that no other path writes.  The wait for them is bounded, so
//    the kernel always ends; every producer is resident or done by the time
//    the last workgroup runs (workgroups are dispatched in block order), so
//    the bound is not reached in practice, and a wait that does reach it sets
//    kStatusKeyWait.
// ---------------------------------------------------------------------------
constexpr int kRtWaves = 8;
constexpr uint32_t kKeySpinLimit = 1u << 22;   // reads of a token's keys before giving up
enum RouteTail { kTailNone = 0, kTailTopk = 1, kTailPermute = 2 };

struct RouterArgs {
    const uint16_t *x, *router_w, *gate_w;
    int nrouted;     // router rows: E, or 0 when only the gate logit is wanted
    Dims d;
    Workspace ws;
    RouteOut ro;     // tail outputs: ids, weights (+ counts, offsets, sorted_slots)
    int tail;        // RouteTail
};

// Key of a logit: the order-preserving map, never 0 (0 marks "not yet written").
__device__ __forceinline__ uint32_t logit_key(float l)
{
    const uint32_t k = float_order(l);
    return k == 0u ? 1u : k;
}

// One token's routing from its published keys.  Several waves may watch
// one token: each polls the keys (its first poll delayed by `delay` short
// sleeps, so that the waves' polls are spread over one load round trip
// instead of arriving together), the first to see every key claims the token
// in LDS and routes it, and the others stop at their next poll.  Returns true
// on the wave that routed (`out` is valid there).  A wave that gives up
// waiting claims the token as well, sets kStatusKeyWait in the sticky status
// word and routes on the keys it has (absent keys read as 0, below every
// logit).
constexpr int kPollRoundTrip = 48;   // s_sleep(1) periods in about one coherent load round trip

template <int KPL>
__device__ bool route_token(uint32_t *keys, int E, int k, int lane, uint32_t *lds, uint32_t *status,
                            int *claim, int delay, TopkLane &out)
{
    for (int i = 0; i < delay; ++i) __builtin_amdgcn_s_sleep(1);
    uint32_t val[KPL];
    bool missing = true;
    for (uint32_t spin = 0; spin < kKeySpinLimit; ++spin) {
        if (__builtin_amdgcn_readfirstlane(*reinterpret_cast<volatile int *>(claim))) return false;
        bool miss = false;
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
            const int e = lane + kWave * i;
            const uint32_t v = load_coherent(keys + min(e, E - 1));
            val[i] = e < E ? v : 0u;
            miss |= e < E && v == 0u;
        }
        missing = __ballot(miss) != 0;
        if (!missing) break;
    }
    int won = 0;
    if (lane == 0) won = atomicCAS(claim, 0, 1) == 0;
    if (!__builtin_amdgcn_readfirstlane(won)) return false;
    if (missing && lane == 0) set_status(status, kStatusKeyWait);
    out = wave_topk_keys<KPL>(val, k, lane, lds);
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int e = lane + kWave * i;
        if (e < E) store_coherent(keys + e, 0u);   // ready for the next call
    }
    return true;
}

__device__ __forceinline__ bool route_token_any(uint32_t *keys, int E, int k, int lane, uint32_t *lds,
                                                uint32_t *status, int *claim, int delay, TopkLane &out)
{
    if (E <= 64) return route_token<1>(keys, E, k, lane, lds, status, claim, delay, out);
    if (E <= 128) return route_token<2>(keys, E, k, lane, lds, status, claim, delay, out);
    if (E <= 256) return route_token<4>(keys, E, k, lane, lds, status, claim, delay, out);
    if (E <= 512) return route_token<8>(keys, E, k, lane, lds, status, claim, delay, out);
    return route_token<16>(keys, E, k, lane, lds, status, claim, delay, out);
}

// x of the T tokens in nibble-pair order (ws.xp) with the sums of its 32-value
// chunks (ws.xs).  One 16-byte piece per thread and pass, four passes' loads
// in flight; a chunk is 4 consecutive pieces, i.e. a lane quad.
__device__ __forceinline__ void transform_x(const uint16_t *x, const Dims &d, const Workspace &ws,
                                            int tid)
{
    const int npieces = d.T * d.H / 8;
    const uint4 *src = reinterpret_cast<const uint4 *>(x);
    uint4 *dst = reinterpret_cast<uint4 *>(ws.xp);
    constexpr int kStep = kRtWaves * kWave;
    for (int p0 = 0; p0 < npieces; p0 += 4 * kStep) {
        const int pa = p0 + tid, pb = pa + kStep, pc = pb + kStep, pd = pc + kStep;
        const uint4 va = src[min(pa, npieces - 1)], vb = src[min(pb, npieces - 1)];
        const uint4 vc = src[min(pc, npieces - 1)], vd = src[min(pd, npieces - 1)];
        auto piece = [&](int pi, const uint4 v) {
            const uint32_t in[4] = {v.x, v.y, v.z, v.w};
            uint32_t pr[4];
            octet_to_pair_order(in, pr);
            float sum = 0.f;
            sum = dot2(in[0], 0x3F803F80u, sum);  // bf16 (1.0, 1.0)
            sum = dot2(in[1], 0x3F803F80u, sum);
            sum = dot2(in[2], 0x3F803F80u, sum);
            sum = dot2(in[3], 0x3F803F80u, sum);
            sum = quad_sum(sum);                   // the whole 32-value chunk
            if (pi < npieces) {
                dst[pi] = make_uint4(pr[0], pr[1], pr[2], pr[3]);
                if ((pi & 3) == 0) ws.xs[pi >> 2] = sum;
            }
        };
        piece(pa, va); piece(pb, vb); piece(pc, vc); piece(pd, vd);
    }
}

template <int CPL, int NT>
__global__ __launch_bounds__(kRtWaves *kWave) void router_kernel(RouterArgs r)
{
    __shared__ float s_lg[kDecodeMaxTokens][kRtWaves];
    __shared__ uint32_t s_topk[kRtWaves][kTopkLds];
    __shared__ int32_t s_ids[kDecodeMaxTokens * kMaxTopK];
    __shared__ int32_t s_run[kMaxExperts];
    __shared__ int s_claim[kDecodeMaxTokens];
    const Dims &d = r.d;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const bool publish = r.tail != kTailNone;

    if (blockIdx.x == gridDim.x - 1) {
        // ---- routing workgroup ----
        // (the barrier before the stores of transform_x: a barrier after
        // them would wait for the stores to complete)
        if (tid < kDecodeMaxTokens) s_claim[tid] = 0;
        __syncthreads();
        transform_x(r.x, d, r.ws, tid);
        if (!publish) return;
        // with fewer tokens than waves, kRtWaves / T waves watch each token
        const int per = d.T >= kRtWaves ? 1 : kRtWaves / d.T;
        for (int t = wave / per; t < d.T; t += kRtWaves / per) {
            TopkLane tk;
            const bool mine = route_token_any(r.ws.dec_keys + (size_t)t * d.E, d.E, d.k, lane, s_topk[wave],
                                              r.ws.status, &s_claim[t], (wave % per) * (kPollRoundTrip / per), tk);
            if (mine && lane < d.k) {
                const int id = clamp_expert(tk.id, d.E);
                r.ro.ids[t * d.k + lane] = id;
                r.ro.weights[t * d.k + lane] = tk.w;
                s_ids[t * d.k + lane] = id;
            }
        }
        if (r.tail == kTailPermute) {
            __syncthreads();
            if (wave == 0)
                wave_permute(s_ids, d.S, d.E, lane, s_run, r.ro.counts, r.ro.offsets,
                             r.ro.sorted_slots, r.ws.slot_pos, r.ws.active);
        }
        return;
    }

    // ---- producer workgroup ----
    const int row = blockIdx.x * kRtWaves + wave;
    const bool gate = r.gate_w != nullptr && row == r.nrouted;
    if (row < r.nrouted || gate) {
        const uint16_t *wrow = gate ? r.gate_w : r.router_w + (size_t)row * d.H;
        const int nck = d.H / 8;
        uint4 wr[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            // unconditional loads; a chunk past the row end re-reads chunk 0, zeroed
            const int idx = lane + kWave * c, ok = idx < nck;
            const uint4 v = reinterpret_cast<const uint4 *>(wrow)[ok ? idx : 0];
            wr[c] = ok ? v : make_uint4(0, 0, 0, 0);
        }
        for (int t0 = 0; t0 < d.T; t0 += NT) {
            uint4 xv[NT][CPL];
#pragma unroll
            for (int u = 0; u < NT; ++u) {
                const int t = min(t0 + u, d.T - 1);
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const int idx = lane + kWave * c;
                    xv[u][c] = reinterpret_cast<const uint4 *>(r.x + (size_t)t * d.H)[idx < nck ? idx : 0];
                }
            }
#pragma unroll
            for (int u = 0; u < NT; ++u) {
                float acc = 0.f;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    acc = dot2(wr[c].x, xv[u][c].x, acc);
                    acc = dot2(wr[c].y, xv[u][c].y, acc);
                    acc = dot2(wr[c].z, xv[u][c].z, acc);
                    acc = dot2(wr[c].w, xv[u][c].w, acc);
                }
                acc = wave_sum(acc);
                if (lane == 0 && t0 + u < d.T) {
                    if (gate) r.ws.shared_gate[t0 + u] = acc;
                    else s_lg[t0 + u][wave] = acc;
                }
            }
        }
    }
    if (!publish) return;
    __syncthreads();
    // the workgroup's keys of token t are 8 consecutive words: one 32-byte store
    if (tid < kRtWaves * d.T) {
        const int t = tid / kRtWaves, j = tid % kRtWaves, rr = blockIdx.x * kRtWaves + j;
        if (rr < r.nrouted)
            store_coherent(r.ws.dec_keys + (size_t)t * d.E + rr, logit_key(s_lg[t][j]));
    }
}

// ---------------------------------------------------------------------------
// 2. gate/up projection per slot.  Lane groups of 16 handle the rows gate i,
//    gate i+1, up i, up i+1; lane q reads 16-byte chunks q + 16c of its row,
//    so each load instruction reads 256 contiguous bytes of four rows and a
//    lane's activation chunks are fixed (kept in registers).
// ---------------------------------------------------------------------------
constexpr int kTileOut = 16;  // outputs of a per workgroup (4 waves x 2 quads x 2)


// Shared expert (INT6, group 64) gate/up for one token: same lane layout, 32
// codes (six words) per chunk.
template <int CPL>
__device__ __forceinline__ void w13_int6_tile(const ExpertArgs &a, const Dims &d, int t,
                                              uint16_t *hrow, int i0, int lane)
{
    const int grp = lane >> 4, q = lane & 15;
    const int nck = d.H / 32, words = d.H / 32 * 6, nsc = d.H / kShGroup;
    ActRaw raw[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int kc = q + 16 * c, kcl = kc < nck ? kc : 0;
        raw[c] = load_act_raw(a.x + (size_t)t * d.H + kcl * 32);
    }
    uint32_t w[2][CPL][7];
    float sc[2][CPL];
#pragma unroll
    for (int qd = 0; qd < 2; ++qd) {
        const int i = i0 + 2 * qd;
        const int row = (grp < 2) ? i + grp : d.sh_I + i + (grp - 2);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int kc = q + 16 * c, ok = kc < nck, kcl = ok ? kc : 0;
            load_block6(a.sh_w13p + (size_t)row * words + kcl * 6, w[qd][c]);
            const float s = bf16_to_f32(a.sh_w13s[(size_t)row * nsc + kcl / 2]);
            sc[qd][c] = ok ? s : 0.f;
        }
    }
#pragma unroll
    for (int qd = 0; qd < 2; ++qd) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            uint32_t xv[16];
#pragma unroll
            for (int o = 0; o < 4; ++o) {
                xv[4 * o] = raw[c].v[o].x; xv[4 * o + 1] = raw[c].v[o].y;
                xv[4 * o + 2] = raw[c].v[o].z; xv[4 * o + 3] = raw[c].v[o].w;
            }
            float xs = 0.f;
#pragma unroll
            for (int u = 0; u < 16; ++u) xs = dot2(xv[u], 0x3F803F80u, xs);
            acc = fmaf(sc[qd][c], chunk_dot6<false>(w[qd][c], xv) - 160.f * xs, acc);
        }
        // rows: lanes 0-15 gate i, 16-31 gate i+1, 32-47 up i, 48-63 up i+1
        acc = row_sum(acc);
        const float g0 = read_lane(acc, 0), g1 = read_lane(acc, 16);
        const float u0 = read_lane(acc, 32), u1 = read_lane(acc, 48);
        if (lane == 0 || lane == 16)
            hrow[i0 + 2 * qd + grp] = (uint16_t)f32_to_f16_sat(lane == 0 ? silu(g0) * u0 : silu(g1) * u1);
    }
}

// Shared expert gate/up: grid (sh_I / 16, T).
template <int CPL>
__global__ __launch_bounds__(256) void w13_shared_kernel(ExpertArgs a, Dims d, Workspace ws)
{
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
    const int t = blockIdx.y;
    w13_int6_tile<CPL>(a, d, t, ws.sh_h + (size_t)t * d.sh_I, blockIdx.x * kTileOut + wave * 4, lane);
}

// Routed gate/up: grid (I / 16, S); expert ids of the slots from `ids`
// (written by the router's tail, or given by the caller).
// Routed slots: wave w computes h[i] for i in [i0, i0 + 4), i0 = 16 x + 4 w:
// the weight chunks are requested first, then the token's activations (already
// in nibble-pair order, with their chunk sums) are staged in LDS, which keeps
// them out of registers and lets more workgroups share a CU.  h is stored in
// nibble-pair order (0,4)(1,5)(2,6)(3,7) within each 8-block: the order in
// which the down projection's weight nibbles come out of a word.
template <int CPL>
__global__ __launch_bounds__(256) void w13_slot_kernel(ExpertArgs a, Dims d, Workspace ws,
                                                       const int32_t *__restrict__ ids)
{
    __shared__ __align__(16) uint16_t s_x[kMaxHidden];   // 256 threads x 2 chunks of 16 bytes
    __shared__ float s_xs[256];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int s = blockIdx.y;
    if (s >= d.S) {
        // second half of the grid (one token): read slice x of the
        // down-projection weights of slot s - S's expert, so that they come
        // from the last-level cache when the down projection runs; the bytes
        // are folded into a value stored only for an impossible token count
        const int sp = s - d.S;
        const int e = clamp_expert(__builtin_amdgcn_readfirstlane((int)load_coherent(reinterpret_cast<const uint32_t *>(ids) + sp)), d.E);
        const size_t per = (size_t)d.H * d.I / 2 / 16 / gridDim.x;   // 16-byte pieces per workgroup
        const uint4 *src = reinterpret_cast<const uint4 *>(a.w2p + (size_t)e * d.H * d.I / 8) + blockIdx.x * per;
        uint32_t fold = 0;
        for (size_t i = tid; i < per; i += 256) {
            const uint4 v = src[i];
            fold ^= v.x ^ v.y ^ v.z ^ v.w;
        }
        if (d.T < 0) ws.h[tid] = (uint16_t)fold;
        return;
    }
    const int i0 = blockIdx.x * kTileOut + wave * 4;
    if (blockIdx.x * kTileOut >= d.I) return;
    // the expert id as a vector load, used only after the activation loads are
    // issued: a scalar load would make the wait for the kernel arguments
    // (scalar loads complete out of order) wait for it too, and hold the
    // activation loads back by a memory round trip
    const int t = s / d.k;
    const uint32_t e_raw = load_coherent(reinterpret_cast<const uint32_t *>(ids) + s);
    const int grp = lane >> 4, q = lane & 15;
    const int nck = d.H / 32, words = d.H / 8, nsc = d.H >> (d.gsh + 5);
    // the token's activations first, then the weights: loads complete in
    // issue order, so the LDS store of x then waits for x alone.  Every load
    // and store here is unconditional (clamped indices; copies past the row end
    // land in unused LDS), which keeps the compiler from serialising them.
    static_assert(kMaxHidden / 8 == 2 * 256, "two 16-byte chunks of x per thread");
    const uint4 *xsrc = reinterpret_cast<const uint4 *>(ws.xp + (size_t)t * d.H);
    const uint4 xr0 = xsrc[min(tid, d.H / 8 - 1)];
    const uint4 xr1 = xsrc[min(tid + 256, d.H / 8 - 1)];
    const float xsr = ws.xs[(size_t)t * nck + min(tid, nck - 1)];
    __builtin_amdgcn_sched_barrier(0);
    const int e = clamp_expert(__builtin_amdgcn_readfirstlane((int)e_raw), d.E);
    uint4 w[2][CPL];
    float sc[2][CPL];
#pragma unroll
    for (int qd = 0; qd < 2; ++qd) {
        const int i = i0 + 2 * qd;
        const int row = (grp < 2) ? i + grp : d.I + i + (grp - 2);
        const size_t r = (size_t)e * 2 * d.I + row;
        const uint4 *wrow = reinterpret_cast<const uint4 *>(a.w13p + r * words);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int kc = q + 16 * c, ok = kc < nck, kcl = ok ? kc : 0;
            w[qd][c] = load_stream(wrow + kcl);
            const float sv = bf16_to_f32(a.w13s[r * nsc + (kcl >> d.gsh)]);
            sc[qd][c] = ok ? sv : 0.f;
        }
    }
    __builtin_amdgcn_sched_barrier(0);   // every weight load issued before the wait for x
    reinterpret_cast<uint4 *>(s_x)[tid] = xr0;
    reinterpret_cast<uint4 *>(s_x)[tid + 256] = xr1;
    s_xs[tid] = xsr;
    __syncthreads();
    uint16_t *hrow = ws.h + (size_t)s * d.I;
    // chunk-outer: each x chunk is read from LDS once for both row sets
    struct XChunk {
        uint32_t v[16];
        float sum;
    };
    auto read_x = [&](int c, XChunk &xc) {
        const int kc = q + 16 * c, kcl = kc < nck ? kc : 0;
        const uint4 *xp4 = reinterpret_cast<const uint4 *>(s_x + kcl * 32);
#pragma unroll
        for (int o = 0; o < 4; ++o) {
            const uint4 v = xp4[o];
            xc.v[4 * o] = v.x; xc.v[4 * o + 1] = v.y; xc.v[4 * o + 2] = v.z; xc.v[4 * o + 3] = v.w;
        }
        xc.sum = s_xs[kcl];
    };
    float accs[2] = {0.f, 0.f};
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        XChunk xc;
        read_x(c, xc);
#pragma unroll
        for (int qd = 0; qd < 2; ++qd)
            accs[qd] = fmaf(sc[qd][c], chunk_dot(w[qd][c], xc.v) - 136.f * xc.sum, accs[qd]);
    }
#pragma unroll
    for (int qd = 0; qd < 2; ++qd) {
        // rows: lanes 0-15 gate i, 16-31 gate i+1, 32-47 up i, 48-63 up i+1
        const float acc = row_sum(accs[qd]);
        const float g0 = read_lane(acc, 0), g1 = read_lane(acc, 16);
        const float u0 = read_lane(acc, 32), u1 = read_lane(acc, 48);
        if (lane == 0 || lane == 16) {
            const int i = i0 + 2 * qd + grp;
            hrow[(i & ~7) | pair_pos(i & 7)] =
                (uint16_t)f32_to_f16_sat(lane == 0 ? silu(g0) * u0 : silu(g1) * u1);
        }
    }
}

// ---------------------------------------------------------------------------
// 3a. down projection + combine for one token.  Each workgroup owns kDnRows output rows and
//    every slot.  A lane group of 32 lanes takes one slot at a time (4 lanes
//    per row; lane q reads chunks q + 4c of the row), 2 groups per wave, so a
//    workgroup has 16 groups; group g takes the slots g, g + 16, ...  Each
//    group keeps its own partial sum per (token, row), and the partials are
//    added in group order at the end (a fixed order: deterministic).  The
//    activations and the first slot's weights are in flight together, and a
//    group's next expert id is in flight with its current weights.  h arrives in nibble-pair
//    order; each 32-value chunk's sum (for the +8 code bias) is formed once
//    while staging, not once per output row.
// ---------------------------------------------------------------------------
constexpr int kDnWaves = 8;
constexpr int kDnRows = 8;
constexpr int kDnGroups = kDnWaves * 2;    // 32-lane slot groups per workgroup
constexpr int kDnHBytes = 64 * 1024;      // LDS for staged activations (holds k * I fp16 for k <= 32, I <= 1024)
constexpr int kDnMaxGroup = 16;           // tokens per LDS group

template <int CPL, int SHCPL>
__global__ __launch_bounds__(kDnWaves *kWave, (CPL <= 5 && SHCPL <= 5) ? 4 : 2) void w2_rows_kernel(ExpertArgs a, Dims d,
                                                                 Workspace ws,
                                                                 const int32_t *__restrict__ ids,
                                                                 const float *__restrict__ wts)
{
    __shared__ __align__(16) uint16_t s_h[kDnHBytes / 2];
    __shared__ float s_hs[kDnHBytes / 64];                  // chunk sums (32 values each)
    __shared__ float s_part[kDnGroups][kDnMaxGroup][kDnRows];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int grp = wave * 2 + (lane >> 5), rl = (lane >> 2) & 7, q = lane & 3;
    const int row = blockIdx.x * kDnRows + rl;
    const int nck = d.I / 32, words = d.I / 8, nsc = d.I >> (d.gsh + 5);
    const int slots_per_group = kDnHBytes / (2 * d.I);
    int tg = slots_per_group / d.k;
    tg = tg < 1 ? 1 : (tg > kDnMaxGroup ? kDnMaxGroup : tg);

    for (int t0 = 0; t0 < d.T; t0 += tg) {
        const int nt = min(tg, d.T - t0);
        const int s0 = t0 * d.k, ns = nt * d.k;
        for (int i = tid; i < kDnGroups * kDnMaxGroup * kDnRows; i += kDnWaves * kWave)
            (&s_part[0][0][0])[i] = 0.f;
        int sr = grp;
        int sg = s0 + min(sr, ns - 1);
        int e = clamp_expert(ids[sg], d.E);
        float rw = wts[sg];
        const uint4 *src = reinterpret_cast<const uint4 *>(ws.h + (size_t)s0 * d.I);
        const int n16 = ns * d.I / 8;
        auto load_weights = [&](int ex, uint4 (&w)[CPL], float (&sc)[CPL]) {
            const size_t r = (size_t)ex * d.H + row;
            const uint4 *wrow = reinterpret_cast<const uint4 *>(a.w2p + r * words);
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int kc = q + 4 * c, ok = kc < nck, kcl = ok ? kc : 0;
                w[c] = load_stream(wrow + kcl);
                const float sv = bf16_to_f32(a.w2s[r * nsc + (kcl >> d.gsh)]);
                sc[c] = ok ? sv : 0.f;
            }
        };
        auto accumulate = [&](int slot, float wt, const uint4 (&w)[CPL], const float (&sc)[CPL]) {
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int kc = q + 4 * c, kcl = kc < nck ? kc : 0;
                const uint4 *hp = reinterpret_cast<const uint4 *>(s_h + (size_t)slot * d.I + kcl * 32);
                uint32_t hv[16];
#pragma unroll
                for (int o = 0; o < 4; ++o) {
                    const uint4 v = hp[o];
                    hv[4 * o] = v.x; hv[4 * o + 1] = v.y; hv[4 * o + 2] = v.z; hv[4 * o + 3] = v.w;
                }
                const float hs = s_hs[slot * nck + kcl];
                acc = fmaf(sc[c], chunk_dot_h(w[c], hv) - 136.f * hs, acc);
            }
            acc = quad_sum(acc);
            if (q == 0) s_part[grp][slot / d.k][rl] += wt * acc;
        };
        // first slot, with the staging of the activations
        uint4 w[CPL];
        float sc[CPL];
        load_weights(e, w, sc);
        // the group's next slot's routing, in flight with these weights
        int sn = sr + kDnGroups;
        int sgn = s0 + min(sn, ns - 1);
        int en = clamp_expert(ids[sgn], d.E);
        float rwn = wts[sgn];
        // the activations straight to LDS (no registers held), issued after
        // every load whose result is needed before the barrier: a wait on a
        // load issued before these copies would also wait for the copies.
        // Wave w copies the 16-byte chunks [64 w + 512 j, + 64) below n16; lanes
        // past n16 re-read the last chunk into unused LDS (n16 <= 4096 chunks).
        __builtin_amdgcn_sched_barrier(0);
        {
            uint4 *dst = reinterpret_cast<uint4 *>(s_h);
            for (int base = wave * kWave; base < n16; base += kDnWaves * kWave)
                __builtin_amdgcn_global_load_lds(src + min(base + lane, n16 - 1), dst + base, 16, 0, 0);
        }
        {
            // the token group's activations (ns x I fp16, nibble-pair order) are
            // in LDS once this wave's copies have landed; then the chunk sums
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies
            __syncthreads();
            for (int i = tid; i < ns * nck; i += kDnWaves * kWave) {
                const uint4 *cp = reinterpret_cast<const uint4 *>(s_h + (size_t)i * 32);
                float hs = 0.f;
#pragma unroll
                for (int o = 0; o < 4; ++o) {
                    const uint4 v = cp[o];
                    hs = dot2h(v.x, 0x3C003C00u, hs); hs = dot2h(v.y, 0x3C003C00u, hs);
                    hs = dot2h(v.z, 0x3C003C00u, hs); hs = dot2h(v.w, 0x3C003C00u, hs);
                }
                s_hs[i] = hs;
            }
            __syncthreads();
        }
        if (sr < ns) accumulate(sr, rw, w, sc);
        // the group's remaining slots
        while (sn < ns) {
            sr = sn; e = en; rw = rwn;
            load_weights(e, w, sc);
            sn = sr + kDnGroups;
            sgn = s0 + min(sn, ns - 1);
            en = clamp_expert(ids[sgn], d.E);
            rwn = wts[sgn];
            accumulate(sr, rw, w, sc);
        }
        // shared expert: one extra slot per token, INT6 rows of the same outputs
        // (SHCPL = 0: compiled without, for layers that have none)
        if (SHCPL > 0 && d.sh_I > 0) {
            const int snck = d.sh_I / 32, swords = d.sh_I / 32 * 6, snsc = d.sh_I / kShGroup;
            for (int tl = grp; tl < nt; tl += kDnGroups) {
                const int t = t0 + tl;
                float acc = 0.f;
#pragma unroll
                for (int c = 0; c < SHCPL; ++c) {
                    const int kc = q + 4 * c, ok = kc < snck, kcl = ok ? kc : 0;
                    uint32_t wv[7];
                    load_block6(a.sh_w2p + (size_t)row * swords + kcl * 6, wv);
                    const float s = bf16_to_f32(a.sh_w2s[(size_t)row * snsc + kcl / 2]);
                    uint32_t hv[16];
                    const float hs = load_act_natural<true>(ws.sh_h + (size_t)t * d.sh_I + kcl * 32, hv);
                    acc = fmaf(ok ? s : 0.f, chunk_dot6<true>(wv, hv) - 160.f * hs, acc);
                }
                acc = quad_sum(acc);
                const float g = 1.f / (1.f + expf(-ws.shared_gate[t]));
                if (q == 0) s_part[grp][tl][rl] += g * acc;
            }
        }
        __syncthreads();
        for (int i = tid; i < nt * kDnRows; i += kDnWaves * kWave) {
            const int tl = i / kDnRows, r = i % kDnRows;
            float acc = 0.f;
            for (int g2 = 0; g2 < kDnGroups; ++g2) acc += s_part[g2][tl][r];
            a.out[(size_t)(t0 + tl) * d.H + blockIdx.x * kDnRows + r] = (uint16_t)f32_to_bf16(acc);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// 3b. down projection per slot, then the combine (two or more tokens).  Grid (H / 64, S + T_sh):
//    workgroup (x, s) computes rows [64 x, 64 x + 64) of slot s's expert (4
//    waves of 16 rows, 4 lanes per row, lane q reading chunks q + 4c), times
//    the slot's routing weight, into yp[s] (fp32); slot S + t holds the shared
//    expert's rows of token t (INT6, weight sigmoid(gate)).  Each workgroup
//    issues its weight loads at once, so the projection costs one round of
//    memory latency however many slots a token group has; then
//    w2_combine_kernel sums each token's k (+1) rows in slot order and rounds
//    once to bf16 (a fixed order: deterministic).  h arrives in nibble-pair
//    order; each 32-value chunk's sum (for the +8 code bias) is formed once,
//    by the four threads that stage the chunk.
// ---------------------------------------------------------------------------
constexpr int kDsRows = 64;

template <int CPL, int SHCPL>
__global__ __launch_bounds__(256) void w2_slot_kernel(ExpertArgs a, Dims d, Workspace ws,
                                                      const int32_t *__restrict__ ids,
                                                      const float *__restrict__ wts, float *__restrict__ yp)
{
    __shared__ __align__(16) uint16_t s_h[1024];   // one slot's h (I <= 1024)
    __shared__ float s_hs[32];                      // its chunk sums
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int rl = lane >> 2, q = lane & 3;
    const int row = blockIdx.x * kDsRows + wave * 16 + rl;
    const int s = blockIdx.y;
    if (s < d.S) {
        // the expert id as a vector load, used only after the activation load
        // is issued (a scalar load would hold the activation load back)
        const uint32_t e_raw = load_coherent(reinterpret_cast<const uint32_t *>(ids) + s);
        const float wt = wts[s];
        const int nck = d.I / 32, words = d.I / 8, nsc = d.I >> (d.gsh + 5), n16 = d.I / 8;
        const uint4 hv = reinterpret_cast<const uint4 *>(ws.h + (size_t)s * d.I)[min(tid, n16 - 1)];
        __builtin_amdgcn_sched_barrier(0);
        const int e = clamp_expert(__builtin_amdgcn_readfirstlane((int)e_raw), d.E);
        const size_t r = (size_t)e * d.H + row;
        const uint4 *wrow = reinterpret_cast<const uint4 *>(a.w2p + r * words);
        uint4 w[CPL];
        float sc[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int kc = q + 4 * c, ok = kc < nck, kcl = ok ? kc : 0;
            w[c] = load_stream(wrow + kcl);
            const float sv = bf16_to_f32(a.w2s[r * nsc + (kcl >> d.gsh)]);
            sc[c] = ok ? sv : 0.f;
        }
        __builtin_amdgcn_sched_barrier(0);   // every weight load issued before the wait for h
        // threads 4c .. 4c + 3 hold chunk c: its sum over the quad
        float hsum = dot2h(hv.x, 0x3C003C00u, 0.f);
        hsum = dot2h(hv.y, 0x3C003C00u, hsum);
        hsum = dot2h(hv.z, 0x3C003C00u, hsum);
        hsum = dot2h(hv.w, 0x3C003C00u, hsum);
        hsum = quad_sum(hsum);
        if (tid < n16) {
            reinterpret_cast<uint4 *>(s_h)[tid] = hv;
            if ((tid & 3) == 0) s_hs[tid >> 2] = hsum;
        }
        __syncthreads();
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int kc = q + 4 * c, kcl = kc < nck ? kc : 0;
            const uint4 *hp = reinterpret_cast<const uint4 *>(s_h + kcl * 32);
            uint32_t hw[16];
#pragma unroll
            for (int o = 0; o < 4; ++o) {
                const uint4 v = hp[o];
                hw[4 * o] = v.x; hw[4 * o + 1] = v.y; hw[4 * o + 2] = v.z; hw[4 * o + 3] = v.w;
            }
            acc = fmaf(sc[c], chunk_dot_h(w[c], hw) - 136.f * s_hs[kcl], acc);
        }
        acc = quad_sum(acc);
        if (q == 0) yp[(size_t)s * d.H + row] = wt * acc;
    } else if constexpr (SHCPL > 0) {
        // the shared expert's rows for token t (INT6 in groups of 64, h in natural order)
        const int t = s - d.S;
        const int snck = d.sh_I / 32, swords = d.sh_I / 32 * 6, snsc = d.sh_I / kShGroup;
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < SHCPL; ++c) {
            const int kc = q + 4 * c, ok = kc < snck, kcl = ok ? kc : 0;
            uint32_t wv[7];
            load_block6(a.sh_w2p + (size_t)row * swords + kcl * 6, wv);
            const float sv = bf16_to_f32(a.sh_w2s[(size_t)row * snsc + kcl / 2]);
            uint32_t hw[16];
            const float hs = load_act_natural<true>(ws.sh_h + (size_t)t * d.sh_I + kcl * 32, hw);
            acc = fmaf(ok ? sv : 0.f, chunk_dot6<true>(wv, hw) - 160.f * hs, acc);
        }
        acc = quad_sum(acc);
        const float g = 1.f / (1.f + expf(-ws.shared_gate[t]));
        if (q == 0) yp[(size_t)s * d.H + row] = g * acc;
    }
}

// out[t][n] = bf16(sum_j yp[t k + j][n] (+ yp[S + t][n])), j ascending, the
// shared row last; four columns per thread.
__global__ __launch_bounds__(256) void w2_combine_kernel(const float *__restrict__ yp, Dims d,
                                                         uint16_t *__restrict__ out)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int n4 = d.H / 4;
    if (i >= d.T * n4) return;
    const int t = i / n4, c = i - t * n4;
    const float4 *col = reinterpret_cast<const float4 *>(yp) + c;
    // rows of slots t k .. t k + k - 1, then the shared row: twelve loads in
    // flight at a time (top-10 and the shared row in one round trip; clamped,
    // unconditional; a clamped duplicate is not added), summed in slot order
    const int nrows = d.k + (d.sh_I > 0 ? 1 : 0);
    auto row_of = [&](int j) { return j < d.k ? (size_t)(t * d.k + j) : (size_t)(d.S + t); };
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < nrows; j0 += 12) {
        float4 v[12];
#pragma unroll
        for (int u = 0; u < 12; ++u) v[u] = col[row_of(min(j0 + u, nrows - 1)) * n4];
#pragma unroll
        for (int u = 0; u < 12; ++u)
            if (j0 + u < nrows) {
                acc.x += v[u].x; acc.y += v[u].y; acc.z += v[u].z; acc.w += v[u].w;
            }
    }
    uint2 o;
    o.x = f32x2_to_bf16x2(acc.x, acc.y);
    o.y = f32x2_to_bf16x2(acc.z, acc.w);
    reinterpret_cast<uint2 *>(out + (size_t)t * d.H)[c] = o;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static int cpl_of(int chunks, int lanes) { return (chunks + lanes - 1) / lanes; }

static hipError_t launch_router(const RouterArgs &r, hipStream_t st)
{
    const int rows = r.nrouted + (r.gate_w ? 1 : 0);
    const int grid = (rows + kRtWaves - 1) / kRtWaves + 1;   // producers + the routing workgroup
    const bool one = r.d.T == 1;
    switch (cpl_of(r.d.H / 8, kWave)) {
#define MOE_CASE(N) \
    case N:                                                                                   \
        if (one) router_kernel<N, 1><<<grid, kRtWaves * kWave, 0, st>>>(r);                  \
        else router_kernel<N, 4><<<grid, kRtWaves * kWave, 0, st>>>(r);                      \
        break;
        MOE_CASE(1) MOE_CASE(2) MOE_CASE(3) MOE_CASE(4) MOE_CASE(5) MOE_CASE(6) MOE_CASE(7) MOE_CASE(8)
#undef MOE_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode_route(const uint16_t *x, const uint16_t *router_w, const Dims &d,
                               const Workspace &ws, const RouteOut &ro, hipStream_t st)
{
    return launch_router(RouterArgs{x, router_w, nullptr, d.E, d, ws, ro, kTailPermute}, st);
}

static hipError_t launch_w13_slots(const ExpertArgs &a, const Dims &d, const Workspace &ws,
                                   const int32_t *ids, hipStream_t st)
{
    const int cpl = cpl_of(d.H / 32, 16);
    // one token: as many workgroups again read the down projection's weights
    // ahead of it (the gate/up launch is latency-bound there; per layer, same
    // box: down stage 8.15 -> 7.3 us, gate/up 7.96 -> 8.44 us, layer 20.1 ->
    // 19.9 us; at two tokens the gate/up launch lost more than the down gained)
    dim3 grid(d.I / kTileOut, d.T == 1 ? 2 * d.S : d.S);
    switch (cpl) {
#define MOE_CASE(N) \
    case N: w13_slot_kernel<N><<<grid, 256, 0, st>>>(a, d, ws, ids); break;
        MOE_CASE(1) MOE_CASE(2) MOE_CASE(3) MOE_CASE(4) MOE_CASE(5) MOE_CASE(6) MOE_CASE(7) MOE_CASE(8)
#undef MOE_CASE
    default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || d.sh_I == 0) return e;
    dim3 sgrid(d.sh_I / kTileOut, d.T);
    switch (cpl) {
#define MOE_CASE(N) \
    case N: w13_shared_kernel<N><<<sgrid, 256, 0, st>>>(a, d, ws); break;
        MOE_CASE(1) MOE_CASE(2) MOE_CASE(3) MOE_CASE(4) MOE_CASE(5) MOE_CASE(6) MOE_CASE(7) MOE_CASE(8)
#undef MOE_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

static hipError_t launch_w2_rows(const ExpertArgs &a, const Dims &d, const Workspace &ws,
                                 const int32_t *ids, const float *wts, hipStream_t st)
{
    const int grid = d.H / kDnRows;
    const int cpl = cpl_of(d.I / 32, 4);
    const int shcpl = d.sh_I ? cpl_of(d.sh_I / 32, 4) : 0;
#define MOE_CASE(N, M) \
    if (cpl == N && shcpl == M) { w2_rows_kernel<N, M><<<grid, kDnWaves * kWave, 0, st>>>(a, d, ws, ids, wts); return hipGetLastError(); }
#define MOE_ROW(N) MOE_CASE(N, 0) MOE_CASE(N, 1) MOE_CASE(N, 2) MOE_CASE(N, 3) MOE_CASE(N, 4) MOE_CASE(N, 5) MOE_CASE(N, 6) MOE_CASE(N, 7) MOE_CASE(N, 8)
    MOE_ROW(1) MOE_ROW(2) MOE_ROW(3) MOE_ROW(4) MOE_ROW(5) MOE_ROW(6) MOE_ROW(7) MOE_ROW(8)
#undef MOE_ROW
#undef MOE_CASE
    return hipErrorInvalidValue;
}

static hipError_t launch_w2_slots(const ExpertArgs &a, const Dims &d, const Workspace &ws,
                                  const int32_t *ids, const float *wts, hipStream_t st)
{
    float *yp = reinterpret_cast<float *>(ws.y);
    dim3 grid(d.H / kDsRows, d.S + (d.sh_I > 0 ? d.T : 0));
    const int cpl = cpl_of(d.I / 32, 4);
    const int shcpl = d.sh_I ? cpl_of(d.sh_I / 32, 4) : 0;
    bool launched = false;
#define MOE_CASE(N, M) \
    if (cpl == N && shcpl == M) { w2_slot_kernel<N, M><<<grid, 256, 0, st>>>(a, d, ws, ids, wts, yp); launched = true; }
#define MOE_ROW(N) MOE_CASE(N, 0) MOE_CASE(N, 1) MOE_CASE(N, 2) MOE_CASE(N, 3) MOE_CASE(N, 4) MOE_CASE(N, 5) MOE_CASE(N, 6) MOE_CASE(N, 7) MOE_CASE(N, 8)
    MOE_ROW(1) MOE_ROW(2) MOE_ROW(3) MOE_ROW(4) MOE_ROW(5) MOE_ROW(6) MOE_ROW(7) MOE_ROW(8)
#undef MOE_ROW
#undef MOE_CASE
    if (!launched) return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n4 = d.T * d.H / 4;
    w2_combine_kernel<<<(n4 + 255) / 256, 256, 0, st>>>(yp, d, a.out);
    return hipGetLastError();
}

// One token: the row kernel (the whole down projection and combine in one
// launch, its 10 slots in one round of its 16 lane groups).  More tokens: the
// per-slot kernel and the combine (measured per layer, same box: 2 tokens
// 28.7 -> 28.3 us, 4 tokens 40.4 -> 37.1, 8 tokens 66.2 -> 55.7, 16 tokens
// 122.0 -> 95.9; 1 token 20.1 against 21.9 us).
static hipError_t launch_w2(const ExpertArgs &a, const Dims &d, const Workspace &ws, const int32_t *ids,
                            const float *wts, hipStream_t st)
{
    return d.T == 1 ? launch_w2_rows(a, d, ws, ids, wts, st) : launch_w2_slots(a, d, ws, ids, wts, st);
}

hipError_t launch_decode_forward(const uint16_t *x, const uint16_t *router_w, const ExpertArgs &a,
                                 const Dims &d, const Workspace &ws, hipEvent_t ev_route,
                                 hipEvent_t ev_mid, hipStream_t st)
{
    RouteOut ro{ws.ids, ws.weights, ws.counts, ws.offsets, ws.sorted_slots};
    hipError_t e = launch_router(RouterArgs{x, router_w, a.sh_gate, d.E, d, ws, ro, kTailTopk}, st);
    if (e != hipSuccess) return e;
    if (ev_route && (e = hipEventRecord(ev_route, st)) != hipSuccess) return e;
    if ((e = launch_w13_slots(a, d, ws, ws.ids, st)) != hipSuccess) return e;
    if (ev_mid && (e = hipEventRecord(ev_mid, st)) != hipSuccess) return e;
    return launch_w2(a, d, ws, ws.ids, ws.weights, st);
}

hipError_t launch_decode_experts(const ExpertArgs &a, const int32_t *ids, const float *wts,
                                 const Dims &d, const Workspace &ws, hipStream_t st)
{
    hipError_t e;
    RouteOut none{};
    // x in pair order (and the shared-expert gate logit, if any)
    e = launch_router(RouterArgs{a.x, nullptr, a.sh_gate, 0, d, ws, none, kTailNone}, st);
    if (e != hipSuccess) return e;
    if ((e = launch_w13_slots(a, d, ws, ids, st)) != hipSuccess) return e;
    return launch_w2(a, d, ws, ids, wts, st);
}

}  // namespace moe
