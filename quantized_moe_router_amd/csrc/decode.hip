// Decode path (few tokens): three kernels, no cross-workgroup synchronisation
// inside any of them.
//
//   1. router_gemv_kernel   logits[t][e] = x_t . router_w[e]  (bf16, fp32 sum),
//                           plus the shared-expert gate logit as one more row
//   2. w13_slot_kernel      per (slot, 16-output tile): the top-k of the slot's
//                           token (recomputed by one wave of every workgroup,
//                           cheaper than a grid-wide handshake), then the INT4
//                           gate/up GEMV and a = silu(g) * u -> fp16;
//                           extra slots run the INT6 shared expert's gate/up
//   3. w2_rows_kernel       each workgroup owns 16 output rows and sums, in a
//                           fixed order, every slot's down projection weighted
//                           by its routing weight (plus sigmoid(gate) times the
//                           shared expert), then rounds once to bf16
//
// Method ("Running 125B MoE on Three 3090s - vLLM Optimization Edition",
// section 3.3, "MoE block (decode-05)"): router and shared gate as one GEMV;
// top-k with renormalisation; routed experts; shared expert added as
// sigmoid(gate) x shared; down projection fused with the final combine.
// On MI355X a kernel boundary costs about 2 us and a device-scope release/
// acquire handshake several us once many workgroups take part, so the
// dependencies (routing -> experts -> combine) are carried by the two kernel
// boundaries only, and the small top-k is recomputed where it is needed.
#include "int6.h"
#include "permute.h"
#include "topk.h"

namespace moe {

// ---------------------------------------------------------------------------
// 1. router GEMV: one wave per row; rows [0, nrouted) are router rows, row
//    nrouted (if gate_w) is the shared-expert gate.
// ---------------------------------------------------------------------------
template <int CPL>
__global__ __launch_bounds__(256) void router_gemv_kernel(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ router_w,
                                                          const uint16_t *__restrict__ gate_w,
                                                          int nrouted, Dims d, Workspace ws)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const bool gate = gate_w != nullptr && row == nrouted;
    if (row >= nrouted && !gate) return;
    const uint16_t *wrow = gate ? gate_w : router_w + (size_t)row * d.H;
    const int nck = d.H / 8;
    uint4 wr[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        // unconditional loads; a chunk past the row end re-reads chunk 0, zeroed
        const int idx = lane + kWave * c, ok = idx < nck;
        const uint4 v = reinterpret_cast<const uint4 *>(wrow)[ok ? idx : 0];
        wr[c] = ok ? v : make_uint4(0, 0, 0, 0);
    }
    for (int t = 0; t < d.T; ++t) {
        uint4 xv[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int idx = lane + kWave * c;
            xv[c] = reinterpret_cast<const uint4 *>(x + (size_t)t * d.H)[idx < nck ? idx : 0];
        }
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            acc = dot2(wr[c].x, xv[c].x, acc);
            acc = dot2(wr[c].y, xv[c].y, acc);
            acc = dot2(wr[c].z, xv[c].z, acc);
            acc = dot2(wr[c].w, xv[c].w, acc);
        }
        acc = wave_sum(acc);
        if (lane == 0) {
            if (gate) ws.shared_gate[t] = acc;
            else ws.logits[(size_t)t * d.E + row] = acc;
        }
    }
}

// ---------------------------------------------------------------------------
// 1b. routing only (moe_int4_route for few tokens): one workgroup selects every
//     token's experts (one wave per token) and builds the permutation.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_tail_kernel(Dims d, Workspace ws, RouteOut ro)
{
    __shared__ int32_t s_ids[kDecodeMaxTokens * kMaxTopK];
    __shared__ int32_t s_run[kMaxExperts];
    __shared__ uint32_t s_topk[4][128];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
    for (int t = wave; t < d.T; t += 4) {
        TopkLane r = topk_any(ws.logits + (size_t)t * d.E, d.E, d.k, lane, s_topk[wave]);
        if (lane < d.k) {
            ro.ids[t * d.k + lane] = r.id;
            ro.weights[t * d.k + lane] = r.w;
            s_ids[t * d.k + lane] = r.id;
        }
    }
    __syncthreads();
    if (wave == 0)
        wave_permute(s_ids, d.S, d.E, lane, s_run, ro.counts, ro.offsets, ro.sorted_slots,
                     ws.slot_pos, ws.active);
}

// ---------------------------------------------------------------------------
// 2. gate/up projection per slot.  Lane groups of 16 handle the rows gate i,
//    gate i+1, up i, up i+1; lane q reads 16-byte chunks q + 16c of its row,
//    so each load instruction reads 256 contiguous bytes of four rows and a
//    lane's activation chunks are fixed (kept in registers).
// ---------------------------------------------------------------------------
constexpr int kTileOut = 16;  // outputs of a per workgroup (4 waves x 2 quads x 2)

__device__ __forceinline__ int clamp_expert(int id, int E)
{
    return id < 0 ? 0 : (id >= E ? E - 1 : id);
}

template <int CPL>
__device__ __forceinline__ void w13_int4_tile(const ExpertArgs &a, const Dims &d, int e, int t,
                                              uint16_t *hrow, int i0, int lane)
{
    const int grp = lane >> 4, q = lane & 15;
    const int nck = d.H / 32, words = d.H / 8, nsc = d.H / kGroup;
    ActRaw raw[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int kc = q + 16 * c, kcl = kc < nck ? kc : 0;
        raw[c] = load_act_raw(a.x + (size_t)t * d.H + kcl * 32);
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
            const float s = bf16_to_f32(a.w13s[r * nsc + kcl / 4]);
            sc[qd][c] = ok ? s : 0.f;
        }
    }
    uint32_t xv[CPL][16];
    float xs[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) xs[c] = act_pairs(raw[c], xv[c]);
#pragma unroll
    for (int qd = 0; qd < 2; ++qd) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            acc = fmaf(sc[qd][c], chunk_dot(w[qd][c], xv[c]) - 136.f * xs[c], acc);
        acc += __shfl_xor(acc, 8, kWave);
        acc += __shfl_xor(acc, 4, kWave);
        acc += __shfl_xor(acc, 2, kWave);
        acc += __shfl_xor(acc, 1, kWave);
        const float up = __shfl(acc, (lane + 32) & (kWave - 1), kWave);
        if (lane == 0 || lane == 16)
            hrow[i0 + 2 * qd + grp] = (uint16_t)f32_to_f16_sat(silu(acc) * up);
    }
}

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

// grid (max(I, sh_I) / 16, S + (shared ? T : 0)).  TOPK: routing from the
// logits (forward); otherwise from ids_in / w_in (caller routing).
template <int CPL, bool TOPK>
__global__ __launch_bounds__(256) void w13_slot_kernel(ExpertArgs a, Dims d, Workspace ws,
                                                       const int32_t *__restrict__ ids_in)
{
    __shared__ int s_e;
    __shared__ uint32_t s_topk[128];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
    const int s = blockIdx.y;
    const int i0 = blockIdx.x * kTileOut + wave * 4;
    if (s >= d.S) {  // shared expert of token s - S
        if (blockIdx.x * kTileOut >= d.sh_I) return;
        const int t = s - d.S;
        w13_int6_tile<CPL>(a, d, t, ws.sh_h + (size_t)t * d.sh_I, i0, lane);
        return;
    }
    if (blockIdx.x * kTileOut >= d.I) return;
    const int t = s / d.k, j = s - t * d.k;
    int e;
    if constexpr (TOPK) {
        if (wave == 0) {
            const TopkLane r = topk_any(ws.logits + (size_t)t * d.E, d.E, d.k, lane, s_topk);
            if (lane == j) s_e = r.id;
            if (blockIdx.x == 0 && j == 0 && lane < d.k) {
                ws.ids[t * d.k + lane] = r.id;
                ws.weights[t * d.k + lane] = r.w;
            }
        }
        __syncthreads();
        e = s_e;
    } else {
        e = clamp_expert(ids_in[s], d.E);
    }
    w13_int4_tile<CPL>(a, d, e, t, ws.h + (size_t)s * d.I, i0, lane);
}

// ---------------------------------------------------------------------------
// 3. down projection + combine: each workgroup owns 16 output rows (4 lanes
//    per row, lane q reads chunks q + 4c) and all slots; waves take slots
//    round-robin and their partial sums are added in wave order.
// ---------------------------------------------------------------------------
constexpr int kDnWaves = 8;
constexpr int kDnRows = 16;
constexpr int kDnBatch = 4;               // slots whose weights are in flight together
constexpr int kDnHBytes = 64 * 1024;      // LDS for staged activations
constexpr int kDnMaxGroup = 16;           // tokens per LDS group

template <int CPL, int SHCPL>
__global__ __launch_bounds__(kDnWaves *kWave) void w2_rows_kernel(ExpertArgs a, Dims d,
                                                                 Workspace ws,
                                                                 const int32_t *__restrict__ ids,
                                                                 const float *__restrict__ wts)
{
    __shared__ __align__(16) uint16_t s_h[kDnHBytes / 2];
    __shared__ float s_part[kDnWaves][kDnMaxGroup][kDnRows];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
    const int q = lane & 3, rl = lane >> 2;
    const int row = blockIdx.x * kDnRows + rl;
    const int nck = d.I / 32, words = d.I / 8, nsc = d.I / kGroup;
    const int slots_per_group = kDnHBytes / (2 * d.I);
    int tg = slots_per_group / d.k;
    tg = tg < 1 ? 1 : (tg > kDnMaxGroup ? kDnMaxGroup : tg);

    for (int t0 = 0; t0 < d.T; t0 += tg) {
        const int nt = min(tg, d.T - t0);
        const int s0 = t0 * d.k, ns = nt * d.k;
        // stage the group's activations (ns x I fp16) into LDS
        {
            const uint4 *src = reinterpret_cast<const uint4 *>(ws.h + (size_t)s0 * d.I);
            uint4 *dst = reinterpret_cast<uint4 *>(s_h);
            const int n16 = ns * d.I / 8;
            for (int i = threadIdx.x; i < n16; i += kDnWaves * kWave) dst[i] = src[i];
        }
        for (int i = threadIdx.x; i < kDnWaves * kDnMaxGroup * kDnRows; i += kDnWaves * kWave)
            (&s_part[0][0][0])[i] = 0.f;
        __syncthreads();

        for (int b0 = wave; b0 < ns; b0 += kDnWaves * kDnBatch) {
            uint4 w[kDnBatch][CPL];
            float sc[kDnBatch][CPL];
            int sl[kDnBatch];
            float rw[kDnBatch];
#pragma unroll
            for (int u = 0; u < kDnBatch; ++u) {
                const int sr = b0 + u * kDnWaves;  // slot relative to the group
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
#pragma unroll
            for (int u = 0; u < kDnBatch; ++u) {
                if (sl[u] >= ns) break;
                float acc = 0.f;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const int kc = q + 4 * c, kcl = kc < nck ? kc : 0;
                    const ActRaw raw = *reinterpret_cast<const ActRaw *>(s_h + (size_t)sl[u] * d.I + kcl * 32);
                    uint32_t hv[16];
                    const float hs = act_pairs_h(raw, hv);
                    acc = fmaf(sc[u][c], chunk_dot_h(w[u][c], hv) - 136.f * hs, acc);
                }
                acc += __shfl_xor(acc, 2, kWave);
                acc += __shfl_xor(acc, 1, kWave);
                if (q == 0) s_part[wave][sl[u] / d.k][rl] += rw[u] * acc;
            }
        }
        // shared expert: one extra slot per token, INT6 rows of the same 16 outputs
        if (d.sh_I > 0) {
            const int snck = d.sh_I / 32, swords = d.sh_I / 32 * 6, snsc = d.sh_I / kShGroup;
            for (int tl = wave; tl < nt; tl += kDnWaves) {
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
                if (q == 0) s_part[wave][tl][rl] += g * acc;
            }
        }
        __syncthreads();
        for (int i = threadIdx.x; i < nt * kDnRows; i += kDnWaves * kWave) {
            const int tl = i / kDnRows, r = i % kDnRows;
            float acc = 0.f;
#pragma unroll
            for (int w = 0; w < kDnWaves; ++w) acc += s_part[w][tl][r];
            a.out[(size_t)(t0 + tl) * d.H + blockIdx.x * kDnRows + r] = (uint16_t)f32_to_bf16(acc);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static int cpl_of(int chunks, int lanes) { return (chunks + lanes - 1) / lanes; }

hipError_t launch_router_gemv(const uint16_t *x, const uint16_t *router_w, const uint16_t *gate_w,
                              int nrouted, const Dims &d, const Workspace &ws, hipStream_t st)
{
    const int rows = nrouted + (gate_w ? 1 : 0);
    const int grid = (rows + 3) / 4;
    switch (cpl_of(d.H / 8, kWave)) {
#define MOE_CASE(N) \
    case N: router_gemv_kernel<N><<<grid, 256, 0, st>>>(x, router_w, gate_w, nrouted, d, ws); break;
        MOE_CASE(1) MOE_CASE(2) MOE_CASE(3) MOE_CASE(4) MOE_CASE(5) MOE_CASE(6) MOE_CASE(7) MOE_CASE(8)
#undef MOE_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode_route(const uint16_t *x, const uint16_t *router_w, const Dims &d,
                               const Workspace &ws, const RouteOut &ro, hipStream_t st)
{
    hipError_t e = launch_router_gemv(x, router_w, nullptr, d.E, d, ws, st);
    if (e != hipSuccess) return e;
    route_tail_kernel<<<1, 256, 0, st>>>(d, ws, ro);
    return hipGetLastError();
}

template <bool TOPK>
static hipError_t launch_w13_slots(const ExpertArgs &a, const Dims &d, const Workspace &ws,
                                   const int32_t *ids, hipStream_t st)
{
    const int outs = d.I > d.sh_I ? d.I : d.sh_I;
    dim3 grid(outs / kTileOut, d.S + (d.sh_I ? d.T : 0));
    switch (cpl_of(d.H / 32, 16)) {
#define MOE_CASE(N) \
    case N: w13_slot_kernel<N, TOPK><<<grid, 256, 0, st>>>(a, d, ws, ids); break;
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
    hipError_t e = launch_router_gemv(x, router_w, a.sh_gate, d.E, d, ws, st);
    if (e != hipSuccess) return e;
    if (ev_route && (e = hipEventRecord(ev_route, st)) != hipSuccess) return e;
    if ((e = launch_w13_slots<true>(a, d, ws, nullptr, st)) != hipSuccess) return e;
    if (ev_mid && (e = hipEventRecord(ev_mid, st)) != hipSuccess) return e;
    return launch_w2_rows(a, d, ws, ws.ids, ws.weights, st);
}

hipError_t launch_decode_experts(const ExpertArgs &a, const int32_t *ids, const float *wts,
                                 const Dims &d, const Workspace &ws, hipStream_t st)
{
    hipError_t e;
    if (d.sh_I > 0 && (e = launch_router_gemv(a.x, nullptr, a.sh_gate, 0, d, ws, st)) != hipSuccess)
        return e;
    if ((e = launch_w13_slots<false>(a, d, ws, ids, st)) != hipSuccess) return e;
    return launch_w2_rows(a, d, ws, ids, wts, st);
}

}  // namespace moe
