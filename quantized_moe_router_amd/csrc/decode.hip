// Decode path (few tokens): three kernels.
//
//   1. router_kernel        logits[t][e] = x_t . router_w[e]  (bf16, fp32 sum),
//                           plus the shared-expert gate logit as one more row;
//                           its last workgroup selects every token's experts
//                           (and builds the permutation for the routing-only
//                           entry point)
//   2. w13_slot_kernel      per (slot, 16-output tile): the INT4 gate/up GEMV
//                           and a = silu(g) * u -> fp16 (w13_shared_kernel:
//                           the INT6 shared expert's gate/up per token)
//   3. w2_rows_kernel       each workgroup owns 16 output rows and sums, in a
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
// 1. Router GEMV with the routing tail in its last workgroup.
//    One router row per wave (8 per workgroup; row E is the shared-expert gate
//    when present), activations of four tokens in flight at a time.  Each
//    workgroup stores its 8 logits of a token with one 32-byte coherent store,
//    waits for its stores and takes a ticket; the workgroup that takes the
//    last ticket selects every token's experts (one wave per token) and, for
//    the routing-only entry point, builds the expert permutation.  ("MoE block
//    (decode-05)": the CTA that finishes last does the top-k, the
//    renormalisation and the block alignment, with no separate kernel.)
//    The ticket needs no cache write-back: the logits are written and read
//    with agent-scope coherent accesses.
// ---------------------------------------------------------------------------
constexpr int kRtWaves = 8;
enum RouteTail { kTailNone = 0, kTailTopk = 1, kTailPermute = 2 };

struct RouterArgs {
    const uint16_t *x, *router_w, *gate_w;
    int nrouted;     // router rows: E, or 0 when only the gate logit is wanted
    Dims d;
    Workspace ws;
    RouteOut ro;     // tail outputs: ids, weights (+ counts, offsets, sorted_slots)
    int tail;        // RouteTail
};

template <int CPL>
__global__ __launch_bounds__(kRtWaves *kWave) void router_kernel(RouterArgs r)
{
    __shared__ float s_lg[kDecodeMaxTokens][kRtWaves];
    __shared__ uint32_t s_topk[kRtWaves][kTopkLds];
    __shared__ int32_t s_ids[kDecodeMaxTokens * kMaxTopK];
    __shared__ int32_t s_run[kMaxExperts];
    __shared__ uint32_t s_last;
    const Dims &d = r.d;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
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
        for (int t0 = 0; t0 < d.T; t0 += 4) {
            uint4 xv[4][CPL];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = min(t0 + u, d.T - 1);
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const int idx = lane + kWave * c;
                    xv[u][c] = reinterpret_cast<const uint4 *>(r.x + (size_t)t * d.H)[idx < nck ? idx : 0];
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
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
    // x in nibble-pair order with its 32-value chunk sums, for the gate/up kernel
    {
        const int nchunk = d.T * (d.H / 32);
        for (int ci = blockIdx.x * blockDim.x + tid; ci < nchunk; ci += gridDim.x * blockDim.x) {
            const uint4 *src = reinterpret_cast<const uint4 *>(r.x) + (size_t)ci * 4;
            uint4 *dst = reinterpret_cast<uint4 *>(r.ws.xp) + (size_t)ci * 4;
            float sum = 0.f;
#pragma unroll
            for (int o = 0; o < 4; ++o) {
                const uint4 v = src[o];
                const uint32_t in[4] = {v.x, v.y, v.z, v.w};
                uint32_t pr[4];
                octet_to_pair_order(in, pr);
                sum = dot2(in[0], 0x3F803F80u, sum);  // bf16 (1.0, 1.0)
                sum = dot2(in[1], 0x3F803F80u, sum);
                sum = dot2(in[2], 0x3F803F80u, sum);
                sum = dot2(in[3], 0x3F803F80u, sum);
                dst[o] = make_uint4(pr[0], pr[1], pr[2], pr[3]);
            }
            r.ws.xs[ci] = sum;
        }
    }
    if (r.tail == kTailNone) return;

    __syncthreads();
    // the workgroup's logits of token t are 8 consecutive words: one 32-byte store
    if (tid < kRtWaves * d.T) {
        const int t = tid / kRtWaves, j = tid % kRtWaves, rr = blockIdx.x * kRtWaves + j;
        if (rr < r.nrouted)
            store_coherent(reinterpret_cast<uint32_t *>(r.ws.logits) + (size_t)t * d.E + rr,
                           __float_as_uint(s_lg[t][j]));
    }
    wait_memory();
    __syncthreads();
    if (tid == 0) s_last = atomic_add_agent(r.ws.route_ticket, 1u) == gridDim.x - 1 ? 1u : 0u;
    __syncthreads();
    if (!s_last) return;

    // last workgroup: routing of every token
    if (tid == 0) *r.ws.route_ticket = 0;   // ready for the next call
    for (int t = wave; t < d.T; t += kRtWaves) {
        const TopkLane tk = topk_any<true>(r.ws.logits + (size_t)t * d.E, d.E, d.k, lane, s_topk[wave]);
        if (lane < d.k) {
            const int id = clamp_expert(tk.id, d.E);
            r.ro.ids[t * d.k + lane] = id;
            r.ro.weights[t * d.k + lane] = tk.w;
            s_ids[t * d.k + lane] = id;
        }
    }
    if (r.tail == kTailPermute) {
        __syncthreads();
        if (wave == 0)
            wave_permute(s_ids, d.S, d.E, lane, s_run, r.ro.counts, r.ro.offsets, r.ro.sorted_slots,
                         r.ws.slot_pos, r.ws.active);
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
        acc += __shfl_xor(acc, 8, kWave);
        acc += __shfl_xor(acc, 4, kWave);
        acc += __shfl_xor(acc, 2, kWave);
        acc += __shfl_xor(acc, 1, kWave);
        const float up = __shfl(acc, (lane + 32) & (kWave - 1), kWave);
        if (lane == 0 || lane == 16)
            hrow[i0 + 2 * qd + grp] = (uint16_t)f32_to_f16_sat(silu(acc) * up);
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
    __shared__ __align__(16) uint16_t s_x[kMaxHidden];
    __shared__ float s_xs[kMaxHidden / 32];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int s = blockIdx.y;
    const int i0 = blockIdx.x * kTileOut + wave * 4;
    if (blockIdx.x * kTileOut >= d.I) return;
    const int t = s / d.k, e = clamp_expert(ids[s], d.E);
    const int grp = lane >> 4, q = lane & 15;
    const int nck = d.H / 32, words = d.H / 8, nsc = d.H / kGroup;
    // the token's activations first (cache-hot; the LDS store waits only for
    // them, since loads complete in issue order), then the weights
    constexpr int kXPer = kMaxHidden / 8 / 256;
    uint4 xr[kXPer];
    float xsr = 0.f;
    {
        const uint4 *xsrc = reinterpret_cast<const uint4 *>(ws.xp + (size_t)t * d.H);
#pragma unroll
        for (int j = 0; j < kXPer; ++j) {
            const int i = tid + 256 * j;
            xr[j] = xsrc[i < d.H / 8 ? i : 0];
        }
        xsr = ws.xs[(size_t)t * nck + (tid < nck ? tid : 0)];
    }
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
            const float sv = bf16_to_f32(a.w13s[r * nsc + kcl / 4]);
            sc[qd][c] = ok ? sv : 0.f;
        }
    }
#pragma unroll
    for (int j = 0; j < kXPer; ++j) {
        const int i = tid + 256 * j;
        if (i < d.H / 8) reinterpret_cast<uint4 *>(s_x)[i] = xr[j];
    }
    if (tid < nck) s_xs[tid] = xsr;
    __syncthreads();
    uint16_t *hrow = ws.h + (size_t)s * d.I;
#pragma unroll
    for (int qd = 0; qd < 2; ++qd) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int kc = q + 16 * c, kcl = kc < nck ? kc : 0;
            const uint32_t *xv = reinterpret_cast<const uint32_t *>(s_x + kcl * 32);
            acc = fmaf(sc[qd][c], chunk_dot(w[qd][c], xv) - 136.f * s_xs[kcl], acc);
        }
        acc += __shfl_xor(acc, 8, kWave);
        acc += __shfl_xor(acc, 4, kWave);
        acc += __shfl_xor(acc, 2, kWave);
        acc += __shfl_xor(acc, 1, kWave);
        const float up = __shfl(acc, (lane + 32) & (kWave - 1), kWave);
        if (lane == 0 || lane == 16) {
            const int i = i0 + 2 * qd + grp;
            hrow[(i & ~7) | pair_pos(i & 7)] = (uint16_t)f32_to_f16_sat(silu(acc) * up);
        }
    }
}

// ---------------------------------------------------------------------------
// 3. down projection + combine.  Each workgroup owns kDnRows output rows and
//    every slot.  A lane group of 32 lanes takes one slot at a time (4 lanes
//    per row; lane q reads chunks q + 4c of the row), 2 groups per wave, so a
//    workgroup has 16 groups; group g takes the slots g, g + 16, ...  Each
//    group keeps its own partial sum per (token, row), and the partials are
//    added in group order at the end (a fixed order: deterministic).  The
//    weights of a batch of slots are requested before the activations are
//    staged in LDS, so the two latencies overlap.  h arrives in nibble-pair
//    order; each 32-value chunk's sum (for the +8 code bias) is formed once
//    while staging, not once per output row.
// ---------------------------------------------------------------------------
constexpr int kDnWaves = 8;
constexpr int kDnRows = 8;
constexpr int kDnGroups = kDnWaves * 2;    // 32-lane slot groups per workgroup
constexpr int kDnBatch = 1;               // slots per group with weights in flight
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
    const int nck = d.I / 32, words = d.I / 8, nsc = d.I / kGroup;
    const int slots_per_group = kDnHBytes / (2 * d.I);
    int tg = slots_per_group / d.k;
    tg = tg < 1 ? 1 : (tg > kDnMaxGroup ? kDnMaxGroup : tg);

    for (int t0 = 0; t0 < d.T; t0 += tg) {
        const int nt = min(tg, d.T - t0);
        const int s0 = t0 * d.k, ns = nt * d.k;
        for (int i = tid; i < kDnGroups * kDnMaxGroup * kDnRows; i += kDnWaves * kWave)
            (&s_part[0][0][0])[i] = 0.f;
        bool staged = false;
        for (int b0 = grp; b0 < ns || !staged; b0 += kDnGroups * kDnBatch) {
            // this group's next batch of slots: weights first
            uint4 w[kDnBatch][CPL];
            float sc[kDnBatch][CPL];
            int sl[kDnBatch];
            float rw[kDnBatch];
#pragma unroll
            for (int u = 0; u < kDnBatch; ++u) {
                const int sr = b0 + u * kDnGroups;  // slot relative to the token group
                sl[u] = sr;
                const int sg = s0 + (sr < ns ? sr : 0);
                const int e = clamp_expert(ids[sg], d.E);
                rw[u] = sr < ns ? wts[sg] : 0.f;
                const size_t r = (size_t)e * d.H + row;
                const uint4 *wrow = reinterpret_cast<const uint4 *>(a.w2p + r * words);
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const int kc = q + 4 * c, ok = kc < nck, kcl = ok ? kc : 0;
                    w[u][c] = load_stream(wrow + kcl);
                    const float s = bf16_to_f32(a.w2s[r * nsc + kcl / 4]);
                    sc[u][c] = ok ? s : 0.f;
                }
            }
            if (!staged) {
                // the group's activations (ns x I fp16, nibble-pair order) into LDS, once
                const uint4 *src = reinterpret_cast<const uint4 *>(ws.h + (size_t)s0 * d.I);
                uint4 *dst = reinterpret_cast<uint4 *>(s_h);
                const int n16 = ns * d.I / 8;
                for (int i = tid; i < n16; i += kDnWaves * kWave) dst[i] = src[i];
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
                staged = true;
            }
#pragma unroll
            for (int u = 0; u < kDnBatch; ++u) {
                if (sl[u] >= ns) break;
                float acc = 0.f;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const int kc = q + 4 * c, kcl = kc < nck ? kc : 0;
                    const uint4 *hp = reinterpret_cast<const uint4 *>(s_h + (size_t)sl[u] * d.I + kcl * 32);
                    uint32_t hv[16];
#pragma unroll
                    for (int o = 0; o < 4; ++o) {
                        const uint4 v = hp[o];
                        hv[4 * o] = v.x; hv[4 * o + 1] = v.y; hv[4 * o + 2] = v.z; hv[4 * o + 3] = v.w;
                    }
                    const float hs = s_hs[sl[u] * nck + kcl];
                    acc = fmaf(sc[u][c], chunk_dot_h(w[u][c], hv) - 136.f * hs, acc);
                }
                acc += __shfl_xor(acc, 2, kWave);
                acc += __shfl_xor(acc, 1, kWave);
                if (q == 0) s_part[grp][sl[u] / d.k][rl] += rw[u] * acc;
            }
            if (b0 >= ns) break;   // a group with no slots only helped to stage
        }
        // shared expert: one extra slot per token, INT6 rows of the same outputs
        if (d.sh_I > 0) {
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
                acc += __shfl_xor(acc, 2, kWave);
                acc += __shfl_xor(acc, 1, kWave);
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
// launchers
// ---------------------------------------------------------------------------
static int cpl_of(int chunks, int lanes) { return (chunks + lanes - 1) / lanes; }

static hipError_t launch_router(const RouterArgs &r, hipStream_t st)
{
    const int rows = r.nrouted + (r.gate_w ? 1 : 0);
    const int nchunk = r.d.T * (r.d.H / 32);
    const int grid = max((rows + kRtWaves - 1) / kRtWaves, (nchunk + kRtWaves * kWave - 1) / (kRtWaves * kWave));
    switch (cpl_of(r.d.H / 8, kWave)) {
#define MOE_CASE(N) \
    case N: router_kernel<N><<<grid, kRtWaves * kWave, 0, st>>>(r); break;
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
    dim3 grid(d.I / kTileOut, d.S);
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
    const int shcpl = d.sh_I ? cpl_of(d.sh_I / 32, 4) : 1;
#define MOE_CASE(N, M) \
    if (cpl == N && shcpl == M) { w2_rows_kernel<N, M><<<grid, kDnWaves * kWave, 0, st>>>(a, d, ws, ids, wts); return hipGetLastError(); }
#define MOE_ROW(N) MOE_CASE(N, 1) MOE_CASE(N, 2) MOE_CASE(N, 3) MOE_CASE(N, 4) MOE_CASE(N, 5) MOE_CASE(N, 6) MOE_CASE(N, 7) MOE_CASE(N, 8)
    MOE_ROW(1) MOE_ROW(2) MOE_ROW(3) MOE_ROW(4) MOE_ROW(5) MOE_ROW(6) MOE_ROW(7) MOE_ROW(8)
#undef MOE_ROW
#undef MOE_CASE
    return hipErrorInvalidValue;
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
    return launch_w2_rows(a, d, ws, ws.ids, ws.weights, st);
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
    return launch_w2_rows(a, d, ws, ids, wts, st);
}

}  // namespace moe
