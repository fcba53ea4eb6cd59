// INT6 (shared expert) helpers: 32 codes per six int32 words, code i (stored
// code + 32) in bits 6i..6i+5 of the little-endian 192-bit block ("Running
// 125B MoE on Three 3090s - vLLM Optimization Edition", section 3.3, "MoE
// block (decode-05)"; model card "What is quantized", group B).  Codes are
// turned into 128 + v operands of v_dot2 with the same exponent trick as the
// INT4 path: bf16 0x4300 | v (against bf16 activations) or fp16
// (v << 3) | 0x5800 (against fp16 activations), exact for v < 128.
#pragma once

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

}  // namespace moe
