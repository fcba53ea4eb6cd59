// Wave-level top-k with renormalised softmax (one wave per token).
//
// Method ("Running 125B MoE on Three 3090s - vLLM Optimization Edition",
// section 3.3, "MoE block (decode-05)"): each logit becomes an
// order-preserving integer, the k largest are taken with equal logits
// resolving to the lower expert id, and with renormalisation the full softmax
// denominator cancels, so the weights are a softmax over the k selected
// logits.  Logits stay fp32 here (the page keys bf16 logits).
//
// The selection is latency-bound (one wave, E = 512 logits, k = 10), so it
// avoids k dependent wave-wide reductions:
//   1. P = the k-th largest of the 64 per-lane maxima with its low 16 bits
//      cleared (a 16-step binary search on one value per lane, counting with
//      ballots).  At least k logits are >= P, so every selected logit is >= P,
//      and for continuous logits only a few more than k are.
//   2. The candidates (logits >= P) are compacted into LDS as 64-bit
//      composites (key << 32 | ~id), which order as the selection does:
//      larger key first, then lower id.  Each candidate's rank is the number
//      of composites above its own, from broadcast LDS reads of all of them;
//      rank < k is selected, at that position.
//   3. If more than 64 logits are >= P (heavy ties), an exact fallback finds
//      the k-th value itself by a binary search over all logits and keeps
//      exactly k candidates.
#pragma once

#include "common.h"

namespace moe {

constexpr int kTopkLds = 192;  // words of wave-private LDS scratch per call

// Order-preserving map of a finite float onto uint32 (-0 and +0 coincide).
// Finite floats map above 0, so 0 can mark "no logit".
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

// Population count of a ballot as a 32-bit value (two 32-bit counts: a 64-bit
// count would be compared on the vector unit, the scalar unit has no 64-bit
// ordered compare).
__device__ __forceinline__ int popc(uint64_t m)
{
    return __builtin_popcount((uint32_t)m) + __builtin_popcount((uint32_t)(m >> 32));
}

// Largest V with #{keys >= V} >= k, by a binary search over the 32 key bits.
// k must be wave-uniform; it is read into a scalar register so that the count
// and the choice of each bit stay on the scalar unit (a vector compare there
// would bounce every step between the vector and scalar units).
template <int KPL>
__device__ __forceinline__ uint32_t kth_key(const uint32_t (&val)[KPL], int k)
{
    const uint32_t ku = (uint32_t)__builtin_amdgcn_readfirstlane(k);
    uint32_t V = 0;
#pragma unroll
    for (int b = 31; b >= 0; --b) {
        const uint32_t cand = V | (1u << b);
        uint32_t cnt = 0;
#pragma unroll
        for (int i = 0; i < KPL; ++i) cnt += (uint32_t)popc(__ballot(val[i] >= cand));
        V = cnt >= ku ? cand : V;
    }
    return V;
}

// Writes the keys with val >= thr (val > thr, plus the lowest-id `eq_take`
// keys equal to thr if eq_take >= 0) to LDS as composites (~id, key) =
// 64-bit (key << 32 | ~id), at positions 0..n-1 in ascending id order;
// returns n.  The caller guarantees n <= 64.
template <int KPL>
__device__ __forceinline__ int compact_keys(const uint32_t (&val)[KPL], uint32_t thr, int eq_take,
                                            int lane, uint32_t *lds)
{
    const uint64_t lt = (1ull << lane) - 1;
    int eq_before = 0, n = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        bool sel;
        if (eq_take < 0) {
            sel = val[i] >= thr && val[i] != 0u;
        } else {
            const uint64_t eqm = __ballot(val[i] == thr);
            sel = val[i] > thr || (val[i] == thr && eq_before + popc(eqm & lt) < eq_take);
            eq_before += popc(eqm);
        }
        const uint64_t selm = __ballot(sel);
        if (sel) {
            const int pos = n + popc(selm & lt);
            reinterpret_cast<uint2 *>(lds)[pos] = make_uint2(~(uint32_t)(lane + kWave * i), val[i]);
        }
        n += popc(selm);
    }
    return n;
}

__device__ __forceinline__ uint64_t as_u64(uint2 v) { return ((uint64_t)v.y << 32) | v.x; }

// Top-k of one token from its order-preserving keys val[i] = key of expert
// lane + 64 i (0 where the expert does not exist).  Requires 1 <= k <= 32 and
// at least k existing experts.  Lane j < k returns the j-th selection.
template <int KPL>
__device__ TopkLane wave_topk_keys(const uint32_t (&val)[KPL], int k_in, int lane, uint32_t *lds)
{
    const int k = __builtin_amdgcn_readfirstlane(k_in);   // uniform: scalar compares
    uint32_t m = val[0];
#pragma unroll
    for (int i = 1; i < KPL; ++i) m = max(m, val[i]);
    // 1. P: largest V with 16 low zero bits and #{lane maxima >= V} >= k
    uint32_t P = 0;
#pragma unroll
    for (int b = 31; b >= 16; --b) {
        const uint32_t cand = P | (1u << b);
        P = popc(__ballot(m >= cand)) >= k ? cand : P;
    }
    int n = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) n += popc(__ballot(val[i] >= P && val[i] != 0u));

    // 2. candidates as composites; slots 0..15 start as zero (never above a candidate)
    uint2 *slot = reinterpret_cast<uint2 *>(lds);
    if (lane < 16) slot[lane] = make_uint2(0u, 0u);
    int ncand;
    if (n <= kWave) {
        ncand = compact_keys<KPL>(val, P, -1, lane, lds);
    } else {
        // heavy ties: the exact k-th key, then exactly k candidates
        const uint32_t V = kth_key<KPL>(val, k);
        int gt = 0;
#pragma unroll
        for (int i = 0; i < KPL; ++i) gt += popc(__ballot(val[i] > V));
        ncand = compact_keys<KPL>(val, V, k - gt, lane, lds);
    }
    __builtin_amdgcn_wave_barrier();
    const uint64_t mine = as_u64(slot[lane]);   // meaningful on lanes < ncand
    int rank = 0;
    if (ncand <= 16) {
        // all 16 slots, read unconditionally (a branch per slot would serialise the reads)
        uint4 c[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = reinterpret_cast<const uint4 *>(lds)[j];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            rank += as_u64(make_uint2(c[j].x, c[j].y)) > mine ? 1 : 0;
            rank += as_u64(make_uint2(c[j].z, c[j].w)) > mine ? 1 : 0;
        }
    } else {
        for (int j = 0; j < ncand; ++j) rank += as_u64(slot[j]) > mine ? 1 : 0;
    }
    __builtin_amdgcn_wave_barrier();
    if (lane < ncand && rank < k) slot[64 + rank] = make_uint2((uint32_t)mine, (uint32_t)(mine >> 32));
    __builtin_amdgcn_wave_barrier();
    // 3. softmax over the k selected logits (the full denominator cancels)
    TopkLane out{0, 0.f};
    float l = 0.f;
    if (lane < k) {
        const uint2 c = slot[64 + lane];
        l = order_float(c.y);
        out.id = (int)~c.x;
    }
    const float first = order_float(slot[64].y);
    const float ex = lane < k ? expf(l - first) : 0.f;
    out.w = ex / wave_sum(ex);
    __builtin_amdgcn_wave_barrier();
    return out;
}

// One token's E fp32 logits, given as nsplit partial rows (lrow, lrow +
// split_stride, ...) added in split order, as order-preserving keys: val[i] =
// key of expert lane + 64 i (0 where the expert does not exist); KPL =
// ceil(E / 64).  NB splits' loads are in flight per pass (clamped addresses,
// no branch around a load); NB matches the split count up to 4, so no
// register holds a repeated load.
template <int KPL, int NB>
__device__ __forceinline__ void logit_keys(const float *lrow, int nsplit, size_t split_stride, int E, int lane,
                                           uint32_t (&val)[KPL])
{
    float l[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) l[i] = 0.f;
    for (int z0 = 0; z0 < nsplit; z0 += NB) {
        float v[KPL][NB];
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
            const int e = lane + kWave * i, ec = e < E ? e : 0;
#pragma unroll
            for (int u = 0; u < NB; ++u) v[i][u] = lrow[(size_t)min(z0 + u, nsplit - 1) * split_stride + ec];
        }
#pragma unroll
        for (int i = 0; i < KPL; ++i)
#pragma unroll
            for (int u = 0; u < NB; ++u) l[i] += z0 + u < nsplit ? v[i][u] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < KPL; ++i) val[i] = lane + kWave * i < E ? float_order(l[i]) : 0u;
}

}  // namespace moe
