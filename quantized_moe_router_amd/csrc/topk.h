// Wave-level top-k with renormalised softmax (one wave per token).
//
// Method ("Running 125B MoE on Three 3090s - vLLM Optimization Edition",
// section 3.3, "MoE block (decode-05)"): each logit becomes an
// order-preserving integer with the inverted expert id packed below it, so a
// single max yields value and id and equal logits resolve to the lower id;
// with renormalisation the full softmax denominator cancels, so the weights
// are a softmax over the k selected logits.  Logits stay fp32 here (the page
// keys bf16 logits), packed into 64-bit keys.
//
// The selection is latency-bound (one wave, a few microseconds if done as k
// dependent wave-wide max reductions), so it is done with ballots instead.
#pragma once

#include "common.h"

namespace moe {

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

struct TopkLane {
    int id;    // valid on lanes < k
    float w;
};

__device__ __forceinline__ int popc(uint64_t m) { return __popcll(m); }

// Top-k of one token's E logits (lrow) by one wave; KPL = ceil(E / 64).
// `lds` is 128 words of wave-private LDS scratch.
//
// Selection without a chain of k wave reductions:
//   1. V = the k-th largest order-preserving logit image, by a 32-step binary
//      search whose counts are popcounts of v_cmp masks (no lane shuffles);
//   2. chosen = every key above V, plus the (k - #above) lowest ids equal to V
//      (equal logits resolve to the lower id);
//   3. the k chosen (id, value) pairs are compacted into LDS, ranked by
//      (value descending, id ascending) against each other, and re-read in
//      rank order, so lane j holds the j-th selection.
template <int KPL>
__device__ TopkLane wave_topk(const float *lrow, int E, int k, int lane, uint32_t *lds)
{
    uint32_t val[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const int e = lane + kWave * i;
        const float l = lrow[e < E ? e : 0];
        val[i] = e < E ? float_order(l) : 0u;  // finite logits map above 0
    }
    uint32_t V = 0;
    for (int b = 31; b >= 0; --b) {
        const uint32_t cand = V | (1u << b);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < KPL; ++i) cnt += popc(__ballot(val[i] >= cand));
        if (cnt >= k) V = cand;
    }
    int gt = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) gt += popc(__ballot(val[i] > V));
    const int need = k - gt;
    const uint64_t lt = (1ull << lane) - 1;
    int eq_before = 0, sel_before = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        const uint64_t eqm = __ballot(val[i] == V);
        const bool sel = val[i] > V || (val[i] == V && eq_before + popc(eqm & lt) < need);
        const uint64_t selm = __ballot(sel);
        if (sel) {
            const int pos = sel_before + popc(selm & lt);
            lds[2 * pos] = val[i];
            lds[2 * pos + 1] = (uint32_t)(lane + kWave * i);
        }
        eq_before += popc(eqm);
        sel_before += popc(selm);
    }
    __builtin_amdgcn_wave_barrier();
    uint32_t my_v = 0, my_e = 0;
    if (lane < k) {
        my_v = lds[2 * lane];
        my_e = lds[2 * lane + 1];
    }
    // rank among the chosen: larger value first, then lower id
    int rank = 0;
    for (int j = 0; j < k; ++j) {
        const uint32_t vj = (uint32_t)__builtin_amdgcn_readlane((int)my_v, j);
        const uint32_t ej = (uint32_t)__builtin_amdgcn_readlane((int)my_e, j);
        rank += (vj > my_v || (vj == my_v && ej < my_e)) ? 1 : 0;
    }
    __builtin_amdgcn_wave_barrier();
    if (lane < k) {
        lds[64 + 2 * rank] = my_v;
        lds[64 + 2 * rank + 1] = my_e;
    }
    __builtin_amdgcn_wave_barrier();
    TopkLane out{0, 0.f};
    float l = 0.f;
    if (lane < k) {
        l = order_float(lds[64 + 2 * lane]);
        out.id = (int)lds[64 + 2 * lane + 1];
    }
    const float first = order_float(lds[64]);
    const float ex = lane < k ? expf(l - first) : 0.f;
    out.w = ex / wave_sum(ex);
    return out;
}

__device__ __forceinline__ TopkLane topk_any(const float *lrow, int E, int k, int lane,
                                             uint32_t *lds)
{
    if (E <= 64) return wave_topk<1>(lrow, E, k, lane, lds);
    if (E <= 128) return wave_topk<2>(lrow, E, k, lane, lds);
    if (E <= 256) return wave_topk<4>(lrow, E, k, lane, lds);
    if (E <= 512) return wave_topk<8>(lrow, E, k, lane, lds);
    return wave_topk<16>(lrow, E, k, lane, lds);
}

}  // namespace moe
