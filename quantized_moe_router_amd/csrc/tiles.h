// Tile list of the grouped GEMMs, shared by the tile-list kernel and the
// one-workgroup permutation (which builds the list right after the counts).
#pragma once

#include "common.h"

namespace moe {

// Tile list of the grouped GEMMs.  Expert e has ceil(count_e / 128) row
// tiles (e | mblock << 16).  The list is a sequence of pairs of tiles: first
// the experts with two or more tiles, each rounded up to whole pairs (an odd
// count leaves one empty slot, -1), then the one-tile experts, two to a pair.
// Pair q goes to XCD q % 8 as list slots (2 (q / 8) + j) * 8 + q % 8, j = 0, 1.
// The GEMM gives list slot t to workgroups on XCD t % 8, in order, so the row
// tiles of a pair run on one XCD at about the same time and share that
// expert's weights through its L2; a large expert still spreads over the
// XCDs two tiles at a time.  One workgroup of 1024 threads (thread e: expert e).
__device__ __forceinline__ int tile_slot(int pos)   // list slot of tile position pos
{
    const int q = pos >> 1;
    return (2 * (q >> 3) + (pos & 1)) * 8 + (q & 7);
}

__device__ __forceinline__ int block_excl_sum(int v, int *s_sum, int &total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    __syncthreads();
    if (lane == 63) s_sum[wave] = incl;
    __syncthreads();
    int base = 0;
    total = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
        base += w < wave ? s_sum[w] : 0;
        total += s_sum[w];
    }
    return base + incl - v;
}

// Chunk list of the whole-expert GEMM (mt == kBigRows): expert e's count_e
// rows are split into ceil(count_e / kBigRows) chunks of nearly equal size
// (consecutive sorted rows), listed densely in expert order; list slot p goes
// to XCD p % 8, and every weight block of a chunk runs on that XCD, so the
// chunk's activation rows are read into one L2.  Slots past the last chunk
// are empty (-1).
__device__ inline void build_chunk_list(int cnt, int off, int nslots, int4 *__restrict__ tiles, int *s_sum)
{
    const int e = threadIdx.x;
    const int nc = (cnt + kBigRows - 1) / kBigRows;
    int total;
    const int p0 = block_excl_sum(nc, s_sum, total);
    for (int i = 0; i < nc; ++i) {
        const int b = (int)((long)cnt * i / nc), en = (int)((long)cnt * (i + 1) / nc);
        tiles[p0 + i] = make_int4(e, off + b, en - b, 0);
    }
    for (int pos = total + (int)threadIdx.x; pos < nslots; pos += blockDim.x) tiles[pos] = make_int4(-1, 0, 0, 0);
}

// The list from the expert counts and offsets; called by all 1024 threads
// of one workgroup, thread e passing expert e's count and offset (count 0
// for e >= E).
__device__ inline void build_tile_list(int cnt, int off, int nslots, int mt, int4 *__restrict__ tiles,
                                       int *s_sum)
{
    if (mt == kBigRows) {
        build_chunk_list(cnt, off, nslots, tiles, s_sum);
        return;
    }
    const int e = threadIdx.x;
    const int nt = (cnt + mt - 1) / mt;
    const int multi = nt >= 2 ? (nt + 1) & ~1 : 0;   // positions of a multi-tile expert
    int nmulti, nsingle;
    const int pm = block_excl_sum(multi, s_sum, nmulti);
    const int ps = block_excl_sum(nt == 1 ? 1 : 0, s_sum, nsingle);
    auto entry = [&](int i) { return make_int4(e | (i << 16), off + i * mt, min(mt, cnt - i * mt), 0); };
    if (nt >= 2) {
        for (int i = 0; i < multi; ++i) tiles[tile_slot(pm + i)] = i < nt ? entry(i) : make_int4(-1, 0, 0, 0);
    } else if (nt == 1) {
        tiles[tile_slot(nmulti + ps)] = entry(0);
    }
    // every other slot the GEMM grid covers is empty
    const int used = nmulti + nsingle;
    for (int pos = used + (int)threadIdx.x; pos < nslots; pos += blockDim.x) tiles[tile_slot(pos)] = make_int4(-1, 0, 0, 0);
}

}  // namespace moe
