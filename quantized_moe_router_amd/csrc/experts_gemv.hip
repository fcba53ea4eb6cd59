// Expert kernels for few tokens per expert (decode): in-register INT4
// dequant GEMV, no matrix cores.
//
// Method ("Running 125B MoE on Three 3090s - vLLM Optimization Edition",
// section 3.3, "MoE block (decode-05)"; INT4 group-128 symmetric experts from
// the model card's "What is quantized" table):
//   a = silu(W1 x) * (W3 x)  with W1/W3 the gate/up halves of the fused W13,
//   out[t] = sum_j w[t][j] * W2_{e_j} a_{t,j}.
// x is bf16 (dot products on bf16 pairs); a is kept in fp16 (fp16 pairs).
// Like the page's down + final-combine fusion, the combine runs inside the
// down-projection kernel: the last workgroup to finish a tile of output rows
// (acquire-release ticket) sums that tile's k expert outputs per token in a
// fixed order, so the result does not depend on scheduling.
//
// Layout on the chip: each weight row is read as 16-byte chunks (32 codes),
// LPR lanes per row, chunk kc = q + LPR*c for lane q, so every load
// instruction reads LPR*16 contiguous bytes of each row and a lane's
// activation chunks are the same for every row (kept in registers).
#include "common.h"

namespace moe {

constexpr int kW13Waves = 4;
constexpr int kW13QuadsPerWave = 2;                                // 4 rows per quad
constexpr int kW13HPerBlock = kW13Waves * kW13QuadsPerWave * 2;    // 16 outputs of a
constexpr int kW2Waves = 4;
constexpr int kW2RowsPerBlock = kW2Waves * 16;                     // 64 output rows

// W13 for one workgroup: 16 outputs of a (32 weight rows) of one expert, for
// every token routed to it.  Lane groups of 16: gate i, gate i+1, up i, up i+1.
template <int CPL>
__global__ __launch_bounds__(kW13Waves *kWave) void w13_gemv_kernel(ExpertArgs a, Dims d,
                                                                    Workspace ws, RouteOut ro)
{
    const int n_active = ws.active[0];
    if ((int)blockIdx.y >= n_active) return;
    const int e = ws.active[1 + blockIdx.y];
    const int beg = ro.offsets[e], ne = ro.counts[e];

    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
    const int grp = lane >> 4, q = lane & 15;
    const int nck = d.H / 32;                 // 16-byte chunks per row
    const int words = d.H / 8, nsc = d.H / kGroup;

    uint4 w[kW13QuadsPerWave][CPL];
    float sc[kW13QuadsPerWave][CPL];
    int hidx[kW13QuadsPerWave];
#pragma unroll
    for (int qd = 0; qd < kW13QuadsPerWave; ++qd) {
        int i = blockIdx.x * kW13HPerBlock + (wave * kW13QuadsPerWave + qd) * 2;
        hidx[qd] = i;
        int row = (grp < 2) ? i + grp : d.I + i + (grp - 2);
        size_t r = (size_t)e * 2 * d.I + row;
        const uint4 *wrow = reinterpret_cast<const uint4 *>(a.w13p + r * words);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            // unconditional loads (a guard here makes the compiler wait on each
            // load in turn); chunks past the row end read chunk 0 with scale 0
            const int kc = q + 16 * c, ok = kc < nck, kcl = ok ? kc : 0;
            w[qd][c] = load_stream(wrow + kcl);
            const float s = bf16_to_f32(a.w13s[r * nsc + kcl / 4]);
            sc[qd][c] = ok ? s : 0.f;
        }
    }

    for (int tok = 0; tok < ne; ++tok) {
        const int p = beg + tok;
        const int t = ro.sorted_slots[p] / d.k;
        ActRaw raw[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int kc = q + 16 * c, kcl = kc < nck ? kc : 0;
            raw[c] = load_act_raw(a.x + (size_t)t * d.H + kcl * 32);
        }
        uint32_t xv[CPL][16];
        float xs[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) xs[c] = act_pairs(raw[c], xv[c]);
#pragma unroll
        for (int qd = 0; qd < kW13QuadsPerWave; ++qd) {
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                acc = fmaf(sc[qd][c], chunk_dot(w[qd][c], xv[c]) - 136.f * xs[c], acc);
            acc += __shfl_xor(acc, 8, kWave);
            acc += __shfl_xor(acc, 4, kWave);
            acc += __shfl_xor(acc, 2, kWave);
            acc += __shfl_xor(acc, 1, kWave);
            float up = __shfl(acc, (lane + 32) & (kWave - 1), kWave);
            if (lane == 0 || lane == 16) {
                float hv = silu(acc) * up;
                ws.h[(size_t)p * d.I + hidx[qd] + grp] = (uint16_t)f32_to_f16_sat(hv);
            }
        }
    }
}

// W2 for one workgroup: 64 output rows of one expert for every token routed to
// it, written to ypart; the last expert to finish the row tile combines.
template <int CPL>
__global__ __launch_bounds__(kW2Waves *kWave) void w2_gemv_kernel(ExpertArgs a, Dims d,
                                                                 Workspace ws, RouteOut ro)
{
    __shared__ int s_last;
    const int n_active = ws.active[0];
    if ((int)blockIdx.y >= n_active) return;
    const int e = ws.active[1 + blockIdx.y];
    const int beg = ro.offsets[e], ne = ro.counts[e];

    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
    const int q = lane & 3;
    const int row = blockIdx.x * kW2RowsPerBlock + wave * 16 + (lane >> 2);
    const int nck = d.I / 32, words = d.I / 8, nsc = d.I / kGroup;

    uint4 w[CPL];
    float sc[CPL];
    {
        size_t r = (size_t)e * d.H + row;
        const uint4 *wrow = reinterpret_cast<const uint4 *>(a.w2p + r * words);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int kc = q + 4 * c, ok = kc < nck, kcl = ok ? kc : 0;
            w[c] = load_stream(wrow + kcl);
            const float s = bf16_to_f32(a.w2s[r * nsc + kcl / 4]);
            sc[c] = ok ? s : 0.f;
        }
    }
    for (int tok = 0; tok < ne; ++tok) {
        const int p = beg + tok;
        ActRaw raw[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int kc = q + 4 * c, kcl = kc < nck ? kc : 0;
            raw[c] = load_act_raw(ws.h + (size_t)p * d.I + kcl * 32);
        }
        uint32_t hv[CPL][16];
        float hs[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) hs[c] = act_pairs_h(raw[c], hv[c]);
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            acc = fmaf(sc[c], chunk_dot_h(w[c], hv[c]) - 136.f * hs[c], acc);
        acc += __shfl_xor(acc, 2, kWave);
        acc += __shfl_xor(acc, 1, kWave);
        if (q == 0) ws.ypart[(size_t)p * d.H + row] = acc;
    }

    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t ticket = atomicAdd(ws.tile_ticket + blockIdx.x, 1u);
        s_last = (ticket == (uint32_t)n_active - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    const int r0 = blockIdx.x * kW2RowsPerBlock;
    for (int idx = threadIdx.x; idx < d.T * kW2RowsPerBlock; idx += kW2Waves * kWave) {
        const int t = idx / kW2RowsPerBlock, r = r0 + idx % kW2RowsPerBlock;
        float acc = 0.f;
        for (int j = 0; j < d.k; ++j) {
            const int s = t * d.k + j;
            acc = fmaf(a.weights[s], ws.ypart[(size_t)ws.slot_pos[s] * d.H + r], acc);
        }
        if (d.sh_I > 0) {
            float g = ws.shared_gate[t];
            acc = fmaf(1.f / (1.f + expf(-g)), ws.ypart[((size_t)d.S + t) * d.H + r], acc);
        }
        a.out[(size_t)t * d.H + r] = (uint16_t)f32_to_bf16(acc);
    }
    if (threadIdx.x == 0) ws.tile_ticket[blockIdx.x] = 0;
}

hipError_t launch_w13_gemv(const ExpertArgs &a, const Dims &d, const Workspace &ws,
                           const RouteOut &ro, hipStream_t st)
{
    const int max_active = d.E < d.S ? d.E : d.S;
    {
        dim3 grid(d.I / kW13HPerBlock, max_active);
        int cpl = (d.H / 32 + 15) / 16;
#define MOE_W13_CASE(N) \
    case N: w13_gemv_kernel<N><<<grid, kW13Waves * kWave, 0, st>>>(a, d, ws, ro); break;
        switch (cpl) {
            MOE_W13_CASE(1) MOE_W13_CASE(2) MOE_W13_CASE(3) MOE_W13_CASE(4)
            MOE_W13_CASE(5) MOE_W13_CASE(6) MOE_W13_CASE(7) MOE_W13_CASE(8)
            default: return hipErrorInvalidValue;
        }
#undef MOE_W13_CASE
    }
    return hipGetLastError();
}

hipError_t launch_w2_gemv(const ExpertArgs &a, const Dims &d, const Workspace &ws,
                          const RouteOut &ro, hipStream_t st)
{
    const int max_active = d.E < d.S ? d.E : d.S;
    {
        dim3 grid(d.H / kW2RowsPerBlock, max_active);
        int cpl = (d.I / 32 + 3) / 4;
#define MOE_W2_CASE(N) \
    case N: w2_gemv_kernel<N><<<grid, kW2Waves * kWave, 0, st>>>(a, d, ws, ro); break;
        switch (cpl) {
            MOE_W2_CASE(1) MOE_W2_CASE(2) MOE_W2_CASE(3) MOE_W2_CASE(4)
            MOE_W2_CASE(5) MOE_W2_CASE(6) MOE_W2_CASE(7) MOE_W2_CASE(8)
            default: return hipErrorInvalidValue;
        }
#undef MOE_W2_CASE
    }
    return hipGetLastError();
}

}  // namespace moe
