// Stable grouping of token slots by expert, computed by one wave with
// ballots ("Running 125B MoE on Three 3090s - vLLM Optimization Edition",
// section 3.3, "MoE block (decode-05)": the block-alignment step groups the
// token slots by expert).  slot s = t*k + j; within an expert, slots keep
// increasing order, so the result is unique and integer-exact.
#pragma once

#include "common.h"

namespace moe {

__device__ __forceinline__ int wave_incl_scan(int v, int lane)
{
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int o = __shfl_up(v, off, kWave);
        if (lane >= off) v += o;
    }
    return v;
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

// The ids of slots [beg, end), end - beg <= kPermChunk, loaded all at once
// (lane l holds slots beg + l + 64 j; clamped addresses, no branch around a
// load, so no iteration waits on its own load).
constexpr int kPermPer = kPermChunk / kWave;

__device__ __forceinline__ void load_chunk_ids(const int32_t *ids, int beg, int end, int E, int lane,
                                               int (&idv)[kPermPer])
{
#pragma unroll
    for (int j = 0; j < kPermPer; ++j) idv[j] = clamp_id(ids[min(beg + lane + kWave * j, end - 1)], E);
}

// Count slots per expert over slots [beg, end) into run[] (LDS, E ints, must
// be zero on entry).  One wave; end - beg <= kPermChunk.
__device__ inline void wave_count(const int32_t *ids, int beg, int end, int E, int lane, int32_t *run)
{
    if (end <= beg) return;
    const int nbits = id_bits(E);
    int idv[kPermPer];
    load_chunk_ids(ids, beg, end, E, lane, idv);
#pragma unroll
    for (int j = 0; j < kPermPer; ++j) {
        const int base = beg + kWave * j;
        if (base >= end) break;   // uniform
        const bool valid = base + lane < end;
        const int id = valid ? idv[j] : 0;
        const uint64_t m = match_id(id, valid, nbits);
        const bool leader = valid && ((m & ((1ull << lane) - 1)) == 0);
        if (leader) run[id] += __popcll(m);
    }
}

// Place slots [beg, end) at run[id] + (rank among equal ids), advancing run[].
// One wave; end - beg <= kPermChunk; idv as loaded by load_chunk_ids.
__device__ inline void wave_scatter_ids(const int (&idv)[kPermPer], int beg, int end, int E, int lane,
                                        int32_t *run, int32_t *sorted_slots, int32_t *slot_pos)
{
    if (end <= beg) return;
    const int nbits = id_bits(E);
#pragma unroll
    for (int j = 0; j < kPermPer; ++j) {
        const int base = beg + kWave * j;
        if (base >= end) break;   // uniform
        const int s = base + lane;
        const bool valid = s < end;
        const int id = valid ? idv[j] : 0;
        const uint64_t m = match_id(id, valid, nbits);
        const uint64_t below = m & ((1ull << lane) - 1);
        const int pos = valid ? run[id] + __popcll(below) : 0;
        if (valid) {
            sorted_slots[pos] = s;
            slot_pos[s] = pos;
        }
        if (valid && below == 0) run[id] += __popcll(m);
    }
}

__device__ inline void wave_scatter(const int32_t *ids, int beg, int end, int E, int lane, int32_t *run,
                             int32_t *sorted_slots, int32_t *slot_pos)
{
    if (end <= beg) return;
    int idv[kPermPer];
    load_chunk_ids(ids, beg, end, E, lane, idv);
    wave_scatter_ids(idv, beg, end, E, lane, run, sorted_slots, slot_pos);
}

// counts -> offsets (exclusive) and the active-expert list; turns run[] into
// the per-expert write cursor.  One wave; run[] holds the counts on entry.
__device__ inline void wave_offsets(int E, int S, int lane, int32_t *run, int32_t *counts,
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
__device__ inline void wave_permute(const int32_t *ids, int S, int E, int lane, int32_t *run,
                             int32_t *counts, int32_t *offsets, int32_t *sorted_slots,
                             int32_t *slot_pos, int32_t *active)
{
    for (int e = lane; e < E; e += kWave) run[e] = 0;
    // the ids are loaded once, counted with one LDS atomic each (a count
    // needs no ranking) and kept in registers for the scatter
    int idv[kPermPer];
    if (S > 0) {
        load_chunk_ids(ids, 0, S, E, lane, idv);
#pragma unroll
        for (int j = 0; j < kPermPer; ++j) {
            if (kWave * j >= S) break;   // uniform
            if (kWave * j + lane < S) atomicAdd(&run[idv[j]], 1);
        }
    }
    wave_offsets(E, S, lane, run, counts, offsets, active);
    if (S > 0) wave_scatter_ids(idv, 0, S, E, lane, run, sorted_slots, slot_pos);
}

}  // namespace moe
