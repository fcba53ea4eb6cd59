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
#include "common.h"

namespace moe {

// 6-bit field i (0..31) of a 192-bit block held in w[0..5] (w[6] == 0).
template <int I>
__device__ __forceinline__ uint32_t field6(const uint32_t w[7])
{
    constexpr int lo = (6 * I) / 32, sh = (6 * I) % 32;
    if constexpr (sh <= 26)
        return (w[lo] >> sh) & 63u;
    else
        return __builtin_amdgcn_alignbit(w[lo + 1], w[lo], sh) & 63u;
}

// One pair (fields 2J, 2J+1) as 128 + v: bf16 (0x4300 | v) when F16 is
// false, fp16 ((v << 3) | 0x5800) when true.
template <int J, bool F16>
__device__ __forceinline__ float pair6_dot(const uint32_t w[7], const uint32_t x[16], float acc)
{
    if constexpr (F16) {
        uint32_t p = (field6<2 * J>(w) << 3) | (field6<2 * J + 1>(w) << 19) | 0x58005800u;
        return dot2h(p, x[J], acc);
    } else {
        uint32_t p = field6<2 * J>(w) | (field6<2 * J + 1>(w) << 16) | 0x43004300u;
        return dot2(p, x[J], acc);
    }
}

// sum over 32 (code + 32 + 128) * x for one block; x in natural pairs
// (bf16 when F16 is false, fp16 when true).
template <bool F16>
__device__ __forceinline__ float chunk_dot6(const uint32_t w[7], const uint32_t x[16])
{
    float acc = 0.f;
    acc = pair6_dot<0, F16>(w, x, acc);  acc = pair6_dot<1, F16>(w, x, acc);
    acc = pair6_dot<2, F16>(w, x, acc);  acc = pair6_dot<3, F16>(w, x, acc);
    acc = pair6_dot<4, F16>(w, x, acc);  acc = pair6_dot<5, F16>(w, x, acc);
    acc = pair6_dot<6, F16>(w, x, acc);  acc = pair6_dot<7, F16>(w, x, acc);
    acc = pair6_dot<8, F16>(w, x, acc);  acc = pair6_dot<9, F16>(w, x, acc);
    acc = pair6_dot<10, F16>(w, x, acc); acc = pair6_dot<11, F16>(w, x, acc);
    acc = pair6_dot<12, F16>(w, x, acc); acc = pair6_dot<13, F16>(w, x, acc);
    acc = pair6_dot<14, F16>(w, x, acc); acc = pair6_dot<15, F16>(w, x, acc);
    return acc;
}

__device__ __forceinline__ void load_block6(const int32_t *p, uint32_t w[7])
{
    const uint2 *q = reinterpret_cast<const uint2 *>(p);
    uint2 a = q[0], b = q[1], c = q[2];
    w[0] = a.x; w[1] = a.y; w[2] = b.x; w[3] = b.y; w[4] = c.x; w[5] = c.y; w[6] = 0;
}

// 32 natural-order activations (bf16, or fp16 when F16) and their sum.
template <bool F16>
__device__ __forceinline__ float load_act_natural(const uint16_t *p, uint32_t x[16])
{
    const uint4 *q = reinterpret_cast<const uint4 *>(p);
    float s = 0.f;
#pragma unroll
    for (int o = 0; o < 4; ++o) {
        uint4 v = q[o];
        x[4 * o] = v.x; x[4 * o + 1] = v.y; x[4 * o + 2] = v.z; x[4 * o + 3] = v.w;
        if constexpr (F16) {
            s = dot2h(v.x, 0x3C003C00u, s); s = dot2h(v.y, 0x3C003C00u, s);
            s = dot2h(v.z, 0x3C003C00u, s); s = dot2h(v.w, 0x3C003C00u, s);
        } else {
            s = dot2(v.x, 0x3F803F80u, s); s = dot2(v.y, 0x3F803F80u, s);
            s = dot2(v.z, 0x3F803F80u, s); s = dot2(v.w, 0x3F803F80u, s);
        }
    }
    return s;
}

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
            int kc = q + 16 * c;
            if (kc < nck) {
                load_block6(a.sh_w13p + (size_t)row * words + kc * 6, w[qd][c]);
                sc[qd][c] = bf16_to_f32(a.sh_w13s[(size_t)row * nsc + kc / 2]);
            }
        }
    }
    const int t_end = min(d.T, (int)(blockIdx.y + 1) * kShTok);
    for (int t = blockIdx.y * kShTok; t < t_end; ++t) {
        uint32_t xv[CPL][16];
        float xs[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            int kc = q + 16 * c;
            if (kc < nck) xs[c] = load_act_natural<false>(a.x + (size_t)t * d.H + kc * 32, xv[c]);
        }
#pragma unroll
        for (int qd = 0; qd < 2; ++qd) {
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                int kc = q + 16 * c;
                if (kc < nck) acc = fmaf(sc[qd][c], chunk_dot6<false>(w[qd][c], xv[c]) - 160.f * xs[c], acc);
            }
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
        int kc = q + 4 * c;
        if (kc < nck) {
            load_block6(a.sh_w2p + (size_t)row * words + kc * 6, w[c]);
            sc[c] = bf16_to_f32(a.sh_w2s[(size_t)row * nsc + kc / 2]);
        }
    }
    const int t_end = min(d.T, (int)(blockIdx.y + 1) * kShTok);
    for (int t = blockIdx.y * kShTok; t < t_end; ++t) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            int kc = q + 4 * c;
            if (kc < nck) {
                uint32_t hv[16];
                float hs = load_act_natural<true>(ws.sh_h + (size_t)t * SI + kc * 32, hv);
                acc = fmaf(sc[c], chunk_dot6<true>(w[c], hv) - 160.f * hs, acc);
            }
        }
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
