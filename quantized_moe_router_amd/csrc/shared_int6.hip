// Always-on shared expert with INT6 group-64 weights.
//
// Method ("Running 125B MoE on Three 3090s - vLLM Optimization Edition",
// section 3.3, "MoE block (decode-05)"; model card "What is quantized",
// group B): the shared expert is a SwiGLU MLP applied to every token, and
// its output is added as sigmoid(gate logit) * shared output, the gate logit
// being one more bf16 router row.  The INT6 layout packs 32 codes into six
// 32-bit words; code i (stored code+32) is bits 6i..6i+5 of the
// little-endian 192-bit block.  The page repacks this into bit planes at
// load time; here the tight layout is read directly, two codes per pair via a
// funnel shift (v_alignbit) and the same exponent trick as the INT4 path:
// bf16 0x4300 | v (against bf16 x) and fp16 (v << 3) | 0x5800 (against the
// fp16 activation) are exactly 128 + v for v < 128.
#include "int6.h"

namespace moe {

constexpr int kShTok = 8;  // tokens per workgroup

// Gate logit of every token: one wave per token.
__global__ __launch_bounds__(256) void shared_gate_kernel(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ gate_w,
                                                          Dims d, float *__restrict__ out)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= d.T) return;
    float acc = 0.f;
    for (int c = lane; c < d.H / 8; c += kWave) {
        uint4 xv = reinterpret_cast<const uint4 *>(x + (size_t)t * d.H)[c];
        uint4 gv = reinterpret_cast<const uint4 *>(gate_w)[c];
        acc = dot2(gv.x, xv.x, acc);
        acc = dot2(gv.y, xv.y, acc);
        acc = dot2(gv.z, xv.z, acc);
        acc = dot2(gv.w, xv.w, acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) out[t] = acc;
}

// Shared W13: 16 outputs of a per workgroup (lane groups: gate i, gate i+1,
// up i, up i+1; 16 lanes per row), kShTok tokens per workgroup.
template <int CPL>
__global__ __launch_bounds__(256) void sh_w13_kernel(ExpertArgs a, Dims d, Workspace ws)
{
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
    const int grp = lane >> 4, q = lane & 15;
    const int nck = d.H / 32, words = d.H / 32 * 6, nsc = d.H / kShGroup;
    const int SI = d.sh_I;
    const int i = blockIdx.x * 16 + (wave * 2 + 0) * 2;  // first pair of this wave
    uint32_t w[2][CPL][7];
    float sc[2][CPL];
#pragma unroll
    for (int qd = 0; qd < 2; ++qd) {
        int ii = i + qd * 2;
        int row = (grp < 2) ? ii + grp : SI + ii + (grp - 2);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int kc = q + 16 * c, ok = kc < nck, kcl = ok ? kc : 0;
            load_block6(a.sh_w13p + (size_t)row * words + kcl * 6, w[qd][c]);
            const float s = bf16_to_f32(a.sh_w13s[(size_t)row * nsc + kcl / 2]);
            sc[qd][c] = ok ? s : 0.f;
        }
    }
    const int t_end = min(d.T, (int)(blockIdx.y + 1) * kShTok);
    for (int t = blockIdx.y * kShTok; t < t_end; ++t) {
        uint32_t xv[CPL][16];
        float xs[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int kc = q + 16 * c, kcl = kc < nck ? kc : 0;
            xs[c] = load_act_natural<false>(a.x + (size_t)t * d.H + kcl * 32, xv[c]);
        }
#pragma unroll
        for (int qd = 0; qd < 2; ++qd) {
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                acc = fmaf(sc[qd][c], chunk_dot6<false>(w[qd][c], xv[c]) - 160.f * xs[c], acc);
            acc += __shfl_xor(acc, 8, kWave);
            acc += __shfl_xor(acc, 4, kWave);
            acc += __shfl_xor(acc, 2, kWave);
            acc += __shfl_xor(acc, 1, kWave);
            float up = __shfl(acc, (lane + 32) & (kWave - 1), kWave);
            if (lane == 0 || lane == 16)
                ws.sh_h[(size_t)t * SI + i + qd * 2 + grp] = (uint16_t)f32_to_f16_sat(silu(acc) * up);
        }
    }
}

// Shared W2: 64 output rows per workgroup (4 lanes per row), kShTok tokens;
// writes the shared output into ypart rows S + t.
template <int CPL>
__global__ __launch_bounds__(256) void sh_w2_kernel(ExpertArgs a, Dims d, Workspace ws)
{
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
    const int q = lane & 3;
    const int row = blockIdx.x * 64 + wave * 16 + (lane >> 2);
    const int SI = d.sh_I, nck = SI / 32, words = SI / 32 * 6, nsc = SI / kShGroup;
    uint32_t w[CPL][7];
    float sc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int kc = q + 4 * c, ok = kc < nck, kcl = ok ? kc : 0;
        load_block6(a.sh_w2p + (size_t)row * words + kcl * 6, w[c]);
        const float s = bf16_to_f32(a.sh_w2s[(size_t)row * nsc + kcl / 2]);
        sc[c] = ok ? s : 0.f;
    }
    const int t_end = min(d.T, (int)(blockIdx.y + 1) * kShTok);
    for (int t = blockIdx.y * kShTok; t < t_end; ++t) {
        uint32_t hv[CPL][16];
        float hs[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int kc = q + 4 * c, kcl = kc < nck ? kc : 0;
            hs[c] = load_act_natural<true>(ws.sh_h + (size_t)t * SI + kcl * 32, hv[c]);
        }
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            acc = fmaf(sc[c], chunk_dot6<true>(w[c], hv[c]) - 160.f * hs[c], acc);
        acc += __shfl_xor(acc, 2, kWave);
        acc += __shfl_xor(acc, 1, kWave);
        if (q == 0) ws.ypart[((size_t)d.S + t) * d.H + row] = acc;
    }
}

hipError_t launch_shared(const ExpertArgs &a, const Dims &d, const Workspace &ws, hipStream_t st)
{
    shared_gate_kernel<<<(d.T + 3) / 4, 256, 0, st>>>(a.x, a.sh_gate, d, ws.shared_gate);
    const int ttiles = (d.T + kShTok - 1) / kShTok;
    {
        dim3 grid(d.sh_I / 16, ttiles);
        int cpl = (d.H / 32 + 15) / 16;
#define MOE_SH13_CASE(N) case N: sh_w13_kernel<N><<<grid, 256, 0, st>>>(a, d, ws); break;
        switch (cpl) {
            MOE_SH13_CASE(1) MOE_SH13_CASE(2) MOE_SH13_CASE(3) MOE_SH13_CASE(4)
            MOE_SH13_CASE(5) MOE_SH13_CASE(6) MOE_SH13_CASE(7) MOE_SH13_CASE(8)
            default: return hipErrorInvalidValue;
        }
#undef MOE_SH13_CASE
    }
    {
        dim3 grid(d.H / 64, ttiles);
        int cpl = (d.sh_I / 32 + 3) / 4;
#define MOE_SH2_CASE(N) case N: sh_w2_kernel<N><<<grid, 256, 0, st>>>(a, d, ws); break;
        switch (cpl) {
            MOE_SH2_CASE(1) MOE_SH2_CASE(2) MOE_SH2_CASE(3) MOE_SH2_CASE(4)
            MOE_SH2_CASE(5) MOE_SH2_CASE(6) MOE_SH2_CASE(7) MOE_SH2_CASE(8)
            default: return hipErrorInvalidValue;
        }
#undef MOE_SH2_CASE
    }
    return hipGetLastError();
}

}  // namespace moe
