// Many-token path: matrix-core (MFMA) kernels for the router GEMM and the
// expert grouped GEMMs.
//
// Method ("Running 125B MoE on Three 3090s - vLLM Optimization Edition",
// section 3.3: the routed experts are a W4A16 grouped GEMM over the token
// slots grouped by expert, gate_up followed by SiLU-and-multiply, then down
// and the weighted sum of the k expert outputs per token; the INT6 shared
// expert is added as sigmoid(gate) x shared).  The page's lesson that decode
// and prefill need different kernels holds here too: this path is a dense
// contraction, so it runs on matrix cores.
//
// gfx950 design
//   * tile 128 rows (64 when the slots per expert are few) x 256 weight rows
//     per workgroup, 4 waves each owning all rows x 64 weight rows
//     (v_mfma_f32_32x32x16_f16), K stages of 64; activations through
//     double-buffered LDS, read as whole 128-byte lines; INT4 weights through
//     LDS one 128-wide group at a time, read as whole 64-byte sectors;
//   * weights are dequantized once per workgroup, in registers, as
//     fp16 values (code * scale * 2^10): a 4-bit code times a bf16 scale has
//     at most 11 significant bits, so the value is exact in fp16 (the 2^10
//     keeps small scales out of the subnormal range and is removed from the
//     fp32 accumulator);
//   * activations are fp16: bf16 inputs are converted once per forward
//     (exact in fp16's normal range) into nibble-pair order, and the SwiGLU
//     activation is produced in fp16;
//   * nibble pairs (n_j, n_j+4) are formed with one mask, so the 8 K values a
//     lane holds are in the order 0,4,1,5,2,6,3,7 on both operands (the dot
//     product does not care);
//   * the down projection's per-row factors and output rows are placed in
//     LDS during the K loop, so the epilogue waits on no global load;
//   * gate and up rows of the same outputs sit in the same wave, so
//     silu(gate) * up is formed in registers;
//   * the down projection writes each slot's weighted output (fp16) and a
//     combine kernel sums a token's slots in a fixed order (deterministic; the
//     fp32-atomic alternative measured about 2x slower on this layer);
//   * workgroup -> tile order is XCD-aware: the weight-row blocks of one token
//     tile go to the same XCD back to back, so the gathered activations are
//     re-read from that XCD's L2, and an expert's token tiles are dealt to
//     the XCDs in pairs.
#include <type_traits>

#include "int6.h"
#include "tiles.h"

namespace moe {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

constexpr int kMT = 128;          // tokens (sorted rows) per tile
constexpr int kNT = 256;          // weight rows per tile (4 waves x 64)
constexpr int kKS = 64;           // K per stage
constexpr int kLdsRow = kKS + 8;  // padded LDS row (fp16 elements)
constexpr int kGemmThreads = 256;
constexpr int kRouterThreads = 512;
constexpr float kScaleUp = 1024.f;
constexpr float kScaleDown = 1.f / 1024.f;

enum GemmMode { kRoutedW13 = 0, kRoutedW2 = 1, kSharedW13 = 2, kSharedW2 = 3 };

struct GemmArgs {
    const uint16_t *x;         // fp16 [T][H] in nibble-pair order (gate/up modes)
    const uint16_t *a16;       // fp16 activation rows (down modes), pair order
    const int32_t *bp;         // packed weights (expert 0)
    const uint16_t *bs;        // bf16 scales (expert 0)
    const int4 *tiles;         // routed: {(mblock << 16) | expert or -1, first row, rows, 0}
    const int32_t *offsets;
    const int32_t *counts;
    const int32_t *sorted_slots;
    int small_rows;            // routed: tiles of at most this many rows are left to the small-tile launch
    const float *weights;      // routing weights per slot
    const float *gate;         // shared-expert gate logits [T]
    uint16_t *h_out;           // fp16 activation out (gate/up modes)
    uint16_t *y_out;           // fp16 weighted down-projection rows [T][k+1][H], columns interleaved
                               // (column n at 64 (n / 64) + 2 (n % 32) + (n % 64) / 32)
    int T, H, I, k;            // I: intermediate of this expert kind
    int K;                     // reduction length
    size_t b_words;            // words of packed weights per expert
    size_t b_scales;           // scales per expert
};

// INT4 word -> one MFMA operand: 8 fp16 values (n - 8) * s in pair order
// (0,4)(1,5)(2,6)(3,7); s2 = fp16 pair (s, s).  fp16 0x6400 is 1024 with
// mantissa step 1, so a nibble OR-ed into mantissa bits 0-3 gives 1024 + n and
// into bits 4-7 gives 1024 + 16 n, both exact, as are (1024 + n) - 1032 and
// (1024 + 16 n) / 16 - 72, i.e. n - 8.  One mask picks nibbles j and j + 4 of
// the word at once: a word takes one shift, four AND-ORs and two packed fp16
// operations per pair.
__device__ __forceinline__ f16x8_t dequant_int4_f16(uint32_t w, h2_t s2)
{
    const uint32_t m0 = vconst(0x000F000Fu), m1 = vconst(0x00F000F0u), b = vconst(0x64006400u);
    const h2_t c0 = {(_Float16)-1032.f, (_Float16)-1032.f};
    const h2_t k16 = {(_Float16)0.0625f, (_Float16)0.0625f}, c1 = {(_Float16)-72.f, (_Float16)-72.f};
    const uint32_t w2 = w >> 8;
    const uint32_t p[4] = {(w & m0) | b, (w & m1) | b, (w2 & m0) | b, (w2 & m1) | b};
    f16x8_t out;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        h2_t v = __builtin_bit_cast(h2_t, p[j]);
        v = (j & 1) ? v * k16 + c1 : v + c0;   // n - 8, exact
        v = v * s2;                            // (n - 8) * s, exact
        out[2 * j] = v[0];
        out[2 * j + 1] = v[1];
    }
    return out;
}

// 8 INT6 codes (octet o of a 32-code block) -> one MFMA operand in pair order.
template <int O>
__device__ __forceinline__ f16x8_t dequant_int6_octet(const uint32_t w[7], h2_t s2)
{
    const h2_t bias = {(_Float16)-160.f, (_Float16)-160.f};
    f16x8_t out;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t a, b;
        switch (j) {  // fields 8O + j and 8O + j + 4 (compile-time)
        case 0: a = field6<8 * O + 0>(w); b = field6<8 * O + 4>(w); break;
        case 1: a = field6<8 * O + 1>(w); b = field6<8 * O + 5>(w); break;
        case 2: a = field6<8 * O + 2>(w); b = field6<8 * O + 6>(w); break;
        default: a = field6<8 * O + 3>(w); b = field6<8 * O + 7>(w); break;
        }
        const uint32_t p = (a << 3) | (b << 19) | 0x58005800u;  // 128 + v
        h2_t v = __builtin_bit_cast(h2_t, p);
        v = (v + bias) * s2;  // (v - 32) * s
        out[2 * j] = v[0];
        out[2 * j + 1] = v[1];
    }
    return out;
}

// xh[t][:] = x[t][:] as fp16 in nibble-pair order, once per forward: the
// gate/up GEMMs read each token row once per weight block, so converting here
// saves that many conversions.
__global__ __launch_bounds__(256) void convert_x_kernel(const uint16_t *__restrict__ x,
                                                        uint16_t *__restrict__ xh, size_t n8)
{
    const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    if (i >= n8) return;
    reinterpret_cast<uint4 *>(xh)[i] = bf16_octet_to_f16_pairs(reinterpret_cast<const uint4 *>(x)[i]);
}

__device__ __forceinline__ h2_t scale_pair(uint16_t bf)
{
    const _Float16 s = (_Float16)(bf16_to_f32(bf) * kScaleUp);
    return h2_t{s, s};
}

// Grouped / dense GEMM.  Workgroup tile: 128 rows (tokens or sorted slots) x
// 256 weight rows; wave w owns all 128 rows and weight rows [64 w, +64) as two
// 32-wide MFMA tiles.  Activations go through double-buffered LDS.  INT4
// weights go through LDS a 128-wide K group at a time (below); INT6 weights
// are loaded by each lane straight from global memory.  Either way every
// weight byte is read and converted once per workgroup.  Within a 64-wide K
// stage, MFMA step j uses, on lanes 0-31, octet j and, on lanes 32-63,
// octet 4 + j.
//
// MAXMA is the most 32-row tiles a workgroup takes: 4 (the 128-row tile, two
// workgroups per CU), or 2 for routed tiles of at most 64 rows, which then
// fit three workgroups per CU (fewer accumulators, half the activation LDS):
// with few slots per expert the tiles are small and the extra workgroup per
// CU hides more of the weights' memory latency.  QG is the number of INT4
// scale groups per 128 inputs: 1 (group 128) or 2 (group 64, one scale per
// 64-wide K stage).
template <int MODE, int MAXMA = 4, int QG = 1>
__global__ __launch_bounds__(kGemmThreads, MAXMA <= 2 ? 3 : 2) void moe_gemm_kernel(GemmArgs g, int nblocks)
{
    constexpr bool kW13 = (MODE == kRoutedW13 || MODE == kSharedW13);
    constexpr bool kRouted = (MODE == kRoutedW13 || MODE == kRoutedW2);
    constexpr bool kInt6 = !kRouted;
    static_assert(MAXMA == 4 || (MAXMA == 2 && kRouted), "small tiles are a routed-GEMM variant");
    static_assert(QG == 1 || (QG == 2 && kRouted), "group 64 is an INT4 (routed) variant");
    __shared__ __align__(16) _Float16 s_a[2][32 * MAXMA * kLdsRow];
    __shared__ int s_tok[kMT];     // token of each tile row (-1: none)
    __shared__ int s_yrow[kMT];    // down modes: row of y that each tile row writes
    __shared__ float s_wgt[kMT];   // down modes: output factor of each tile row

    // ---- tile assignment (XCD-aware: the n-blocks of one tile share an XCD) ----
    const int wid = blockIdx.x;
    const int xcd = wid & 7, r = wid >> 3;
    const int nb = r % nblocks, tile = (r / nblocks) * 8 + xcd;
    int e = 0, m0 = 0, rows = 0, pbase = 0;
    if constexpr (kRouted) {
        // one load gives the expert, the tile's first sorted row and its rows
        const int4 tv = g.tiles[tile];
        if (tv.x < 0) return;   // empty slot
        e = tv.x & 0xFFFF;
        pbase = tv.y;
        rows = tv.z;
        // with a small-tile launch beside it, each launch takes its own tiles
        if (MAXMA == 2 ? rows > 64 : rows <= g.small_rows) return;
    } else {
        m0 = tile * kMT;
        if (m0 >= g.T) return;
        rows = min(kMT, g.T - m0);
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // down modes: the factor of each row (routing weight, or the shared
    // expert's gate logit) is loaded here and only written to LDS after the K
    // loop, so its latency is hidden; rows past the tile load row 0's
    float wraw = 0.f;
    if (tid < kMT) {
        const int i = tid < rows ? tid : 0;
        int tok, slot = 0;
        if constexpr (kRouted) {
            slot = g.sorted_slots[pbase + i];
            tok = slot / g.k;
        } else {
            tok = m0 + i;
        }
        if constexpr (!kW13) {
            wraw = kRouted ? g.weights[slot] : g.gate[tok];
            s_yrow[tid] = tok * (g.k + 1) + (kRouted ? slot - tok * g.k : g.k);
        }
        s_tok[tid] = tid < rows ? tok : -1;
    }
    __syncthreads();

    const int K = g.K, nsteps = K / kKS;
    // ---- activation staging: thread -> 16-byte chunk c8 of rows r8 + 32 o,
    // o < 4 (row tile o): eight lanes read one row's 128 bytes of a stage, so
    // each load instruction reads eight whole cache lines ----
    const int c8 = tid & 7, r8 = tid >> 3;
    // rows past the tile read a valid row (row 0), so no load sits behind a
    // branch (a guarded load makes the compiler wait for every outstanding
    // load at the next use); what such a row accumulates is never stored
    const uint16_t *asrc[4];
#pragma unroll
    for (int o = 0; o < 4; ++o) {
        const int row = r8 + 32 * o, arow = s_tok[row] >= 0 ? row : 0;
        if constexpr (kW13) asrc[o] = g.x + (size_t)s_tok[arow] * g.H + 8 * c8;
        else asrc[o] = g.a16 + (size_t)(kRouted ? pbase + arow : s_tok[arow]) * K + 8 * c8;
    }
    // two register sets: stage s's activations are loaded two stages before
    // they are used (set s % 2) and stored to LDS one stage before
    u32x4_t ra[2][4];   // vector type: copied to LDS by value, never through memory

    // ---- weight fragments: lane -> (row n = base + lane % 32, octets 4 * half ..) ----
    const int half = lane >> 5;
    int brow[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int c = 64 * wave + 32 * nt + (lane & 31);  // weight row within the tile
        if constexpr (kW13) brow[nt] = nt == 0 ? 128 * nb + 32 * wave + (lane & 31)
                                               : g.I + 128 * nb + 32 * wave + (lane & 31);
        else brow[nt] = kNT * nb + c;
    }
    const int32_t *bp = g.bp + (size_t)e * g.b_words;
    const uint16_t *bs = g.bs + (size_t)e * g.b_scales;
    const size_t bstride = kInt6 ? (size_t)K / 32 * 6 : (size_t)K / 8;
    const int sgroup = kInt6 ? kShGroup : kGroup;
    // INT6 (shared expert): each lane loads its own weight fragments, two
    // stages ahead, set q holding stage s with s % 2 == q
    uint32_t rb6[2][2][7];
    uint16_t rsc[2][2];
    auto load_b6 = [&](int s, int q) {
        const int k0 = s * kKS + 32 * half;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            load_block6(bp + brow[nt] * bstride + k0 / 32 * 6, rb6[q][nt]);
            rsc[q][nt] = bs[(size_t)brow[nt] * (K / sgroup) + k0 / sgroup];
        }
    };
    // INT4 (routed experts): weights go through LDS one 128-wide K group (two
    // stages, one scale) at a time.  Thread t loads 16-byte chunk t % 4 of the
    // group's 64 bytes for tile rows t / 4 + 64 i (i < 4), so a load
    // instruction reads sixteen whole 64-byte sectors, and the scale of tile
    // row t.  A group is stored to LDS one group ahead of its use while the
    // next is in flight.  In LDS, chunk c of tile row r sits at position
    // c ^ ((r >> 1) & 3), so the fragment reads of eight consecutive rows hit
    // distinct banks.  Tile row r = 64 w + 32 nt + l is the row wave w uses as
    // MFMA column l of its weight tile nt.
    constexpr int QB = kInt6 ? 1 : 2;
    __shared__ u32x4_t s_bq[QB][kInt6 ? 1 : kNT * 4];
    __shared__ uint16_t s_bqs[QB][kInt6 ? 1 : QG * kNT];
    auto tile_row = [&](int r) {
        const int w = r >> 6, nt = (r >> 5) & 1, l = r & 31;
        if constexpr (kW13) return nt == 0 ? 128 * nb + 32 * w + l : g.I + 128 * nb + 32 * w + l;
        else return kNT * nb + r;
    };
    const int c4 = tid & 3;
    const uint8_t *bq = reinterpret_cast<const uint8_t *>(bp) + 16 * c4;
    uint32_t qoff[4];      // byte offsets of this thread's four rows
#pragma unroll
    for (int i = 0; i < 4; ++i) qoff[i] = (uint32_t)(tile_row((tid >> 2) + 64 * i) * bstride * 4);
    const uint16_t *qs = bs + (size_t)tile_row(tid) * (K / kGroup * QG);
    u32x4_t rq[4];         // vector type: stored to LDS by value
    uint16_t rqs[QG];
    auto load_q = [&](int grp) {
#pragma unroll
        for (int i = 0; i < 4; ++i) rq[i] = *reinterpret_cast<const u32x4_t *>(bq + qoff[i] + 64 * grp);
#pragma unroll
        for (int j = 0; j < QG; ++j) rqs[j] = qs[QG * grp + j];
    };
    auto store_q = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = (tid >> 2) + 64 * i;
            s_bq[buf][r * 4 + (c4 ^ ((r >> 1) & 3))] = rq[i];
        }
#pragma unroll
        for (int j = 0; j < QG; ++j) s_bqs[buf][j * kNT + tid] = rqs[j];
    };

    f32x16_t acc[MAXMA][2];
#pragma unroll
    for (int i = 0; i < MAXMA; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
    const int mtiles = (rows + 31) / 32;

    // The K loop, compiled once per number of active 32-row tiles (MA) and
    // chosen once per workgroup: with the count known at compile time there
    // is no branch between the matrix instructions, so the activation reads of
    // the next MFMA step can be issued ahead of them (a branch per tile left
    // each read waiting on its own).
    auto kloop = [&](auto ma_c) {
        constexpr int MA = decltype(ma_c)::value;
        h2_t s2[2];                           // fp16 scale pairs of the current stage
        // only the active row tiles are staged
        auto load_a = [&](int s, int p) {
#pragma unroll
            for (int o = 0; o < MA; ++o) ra[p][o] = *reinterpret_cast<const u32x4_t *>(asrc[o] + s * kKS);
        };
        auto store_a = [&](int buf, int p) {
#pragma unroll
            for (int o = 0; o < MA; ++o)
                *reinterpret_cast<u32x4_t *>(s_a[buf] + (r8 + 32 * o) * kLdsRow + 8 * c8) = ra[p][o];
        };

        // one K stage: stage s's weights (set q = s % 2) against LDS buffer q,
        // while stage s+1's activations (set 1-q, loaded two stages ago) are
        // stored and the loads of stages s+3 (activations) and s+2 (weights)
        // are issued
        auto stage = [&](int s, int q) {
            const int grp = s >> 1, ngrp = nsteps >> 1;
            if (s + 1 < nsteps) store_a(q ^ 1, q ^ 1);
            if constexpr (!kInt6) {
                if (q == 0) store_q((grp + 1) & 1);
            }
            // keep this stage's raw weights; the set is reloaded below
            uint4 w4[2];
            uint32_t w6[2][7];
            if constexpr (kInt6) {
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    s2[nt] = scale_pair(rsc[q][nt]);
#pragma unroll
                    for (int u = 0; u < 7; ++u) w6[nt][u] = rb6[q][nt][u];
                }
            }
            {   // the last stages re-load the last one (no branch around loads)
                load_a(min(s + 3, nsteps - 1), q ^ 1);
                if constexpr (kInt6) load_b6(min(s + 2, nsteps - 1), q);
                else if (q == 0) load_q(min(grp + 2, ngrp - 1));
            }
            if constexpr (!kInt6) {
                // this stage's fragments: chunk 2 q + half of tile rows
                // 64 wave + 32 nt + lane % 32, stored a group ago
                const int buf = grp & 1;
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const int r = 64 * wave + 32 * nt + (lane & 31);
                    const u32x4_t v = s_bq[buf][r * 4 + ((2 * q + half) ^ ((r >> 1) & 3))];
                    w4[nt] = make_uint4(v[0], v[1], v[2], v[3]);
                    if (QG == 2 || q == 0) s2[nt] = scale_pair(s_bqs[buf][(QG == 2 ? q : 0) * kNT + r]);
                }
            }
            // activation fragments of the active row tiles are read one MFMA
            // step ahead; weight operands are converted per step, between the
            // matrix instructions
            const _Float16 *A = s_a[s & 1] + (lane & 31) * kLdsRow + 32 * half;
            f16x8_t af[2][MA];
#pragma unroll
            for (int mt = 0; mt < MA; ++mt)
                af[0][mt] = *reinterpret_cast<const f16x8_t *>(A + 32 * mt * kLdsRow);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (j < 3) {
#pragma unroll
                    for (int mt = 0; mt < MA; ++mt)
                        af[(j + 1) & 1][mt] = *reinterpret_cast<const f16x8_t *>(A + 32 * mt * kLdsRow + 8 * (j + 1));
                }
                f16x8_t bf[2];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    if constexpr (!kInt6) {
                        const uint32_t wj = j == 0 ? w4[nt].x : j == 1 ? w4[nt].y : j == 2 ? w4[nt].z : w4[nt].w;
                        bf[nt] = dequant_int4_f16(wj, s2[nt]);
                    } else {
                        bf[nt] = j == 0 ? dequant_int6_octet<0>(w6[nt], s2[nt])
                               : j == 1 ? dequant_int6_octet<1>(w6[nt], s2[nt])
                               : j == 2 ? dequant_int6_octet<2>(w6[nt], s2[nt])
                                        : dequant_int6_octet<3>(w6[nt], s2[nt]);
                    }
                }
#pragma unroll
                for (int mt = 0; mt < MA; ++mt) {
                    acc[mt][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[j & 1][mt], bf[0], acc[mt][0], 0, 0, 0);
                    acc[mt][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[j & 1][mt], bf[1], acc[mt][1], 0, 0, 0);
                }
            }
            __syncthreads();
        };

        // prologue: stage 0's activations and (INT4) weight group 0 in LDS;
        // stages 1 and 2 activations, weights of stages 0 and 1 (INT6) or
        // group 1 (INT4) in flight
        load_a(0, 0);
        if constexpr (kInt6) {
            load_b6(0, 0);
            load_b6(min(1, nsteps - 1), 1);
        } else {
            load_q(0);
        }
        load_a(min(1, nsteps - 1), 1);
        store_a(0, 0);
        if constexpr (!kInt6) {
            store_q(0);
            load_q(min(1, (nsteps >> 1) - 1));
        }
        load_a(min(2, nsteps - 1), 0);
        __syncthreads();
        int s = 0;
        for (; s + 1 < nsteps; s += 2) {
            stage(s, 0);
            stage(s + 1, 1);
        }
        if (s < nsteps) stage(s, 0);
    };
    if constexpr (MAXMA == 2) {
        if (mtiles == 1) kloop(std::integral_constant<int, 1>{});
        else kloop(std::integral_constant<int, 2>{});
    } else {
        switch (mtiles) {
        case 1: kloop(std::integral_constant<int, 1>{}); break;
        case 2: kloop(std::integral_constant<int, 2>{}); break;
        case 3: kloop(std::integral_constant<int, 3>{}); break;
        default: kloop(std::integral_constant<int, 4>{}); break;
        }
    }

    // ---- epilogue ----
    if constexpr (!kW13) {
        // weighted row of slot (t, j) -> y[t][j][:]; the shared expert is slot k
        // with factor sigmoid(gate); the 2^-10 of the weight scale is folded in
        if (tid < kMT) s_wgt[tid] = (kRouted ? wraw : 1.f / (1.f + expf(-wraw))) * kScaleDown;
        __syncthreads();
    }
    const int col = lane & 31;
#pragma unroll
    for (int mt = 0; mt < MAXMA; ++mt) {
        if (mt >= mtiles) continue;
        // output rows (and factors) of the lane's 16 rows of this tile, read
        // from LDS before the first store
        int rowv[16];
        float wv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int m = 32 * mt + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
            if constexpr (kW13) {
                rowv[j] = kRouted ? pbase + m : s_tok[m];
            } else {
                rowv[j] = s_yrow[m];
                wv[j] = s_wgt[m];
            }
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int m = 32 * mt + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
            if (m >= rows) continue;
            if constexpr (kW13) {
                const float gv = acc[mt][0][j] * kScaleDown, uv = acc[mt][1][j] * kScaleDown;
                const int i = 128 * nb + 32 * wave + col;
                const int ip = (i & ~7) | pair_pos(i & 7);
                g.h_out[(size_t)rowv[j] * g.I + ip] = (uint16_t)f32_to_f16_sat(silu(gv) * uv);
            } else {
                // the lane's columns of both column tiles as one word (interleaved columns)
                uint32_t *yr = reinterpret_cast<uint32_t *>(g.y_out + (size_t)rowv[j] * g.H + kNT * nb + 64 * wave) + col;
                *yr = f32_to_f16_sat(wv[j] * acc[mt][0][j]) | (f32_to_f16_sat(wv[j] * acc[mt][1][j]) << 16);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Whole-expert grouped GEMM (many slots per expert).  A workgroup takes one
// chunk of up to 192 sorted rows of one expert (all of an expert's rows for
// balanced routing) and one block of 256 weight rows, so every weight is
// fetched from memory once per chunk.  Wave c of column group c takes the
// weight rows [64 c, 64 c + 64) of the block (two 32-wide column tiles), as
// v_mfma_f32_32x32x16_f16 tiles:
//   * gate/up: four waves, one per SIMD, each with all T 32-row tiles of the
//     chunk, so every weight is converted once (with two row groups each
//     weight was converted by both, and the conversions outweighed the
//     matrix work of a step; one wave per SIMD with up to 6 x 2 accumulator
//     tiles: 8192 tokens 659 -> 590 us);
//   * routed down: eight waves, two per SIMD: row group g takes the first
//     ceil(T / 2) row tiles for g = 0, the rest for g = 1 (its block loop
//     does not fit the registers of one wave per SIMD);
//   * the shared expert's gate/up (INT6, group 64; every token a row,
//     chunk c the tokens [192 c, 192 c + 192)): four waves.  Its down
//     projection stays with moe_gemm_kernel (K = 640 is short: here it took
//     66 us against 54 at 8192 tokens).
//   * K advances one 128-wide weight group (one scale per row) per stage, with
//     one barrier per stage.  The chunk's scales are copied to LDS once.
//   * Weights: each wave loads its own rows straight into registers, two
//     groups ahead: per row the two lane halves read the 16-byte pieces at
//     bytes 16h and 32 + 16h of the group's 64 bytes.  Piece p of half h,
//     word w, holds K = 64 p + 32 h + 8 w .. + 7, and MFMA step j = 4 p + w
//     consumes it; the activation tile is read in the same K order.
//   * Activations: gathered rows (256 bytes per row and stage) are loaded
//     into registers a stage ahead and written to the other half of a
//     double-buffered LDS tile during the stage before their use, spread
//     over its MFMA steps.
//   * Software pipeline: while the MFMAs of step j run, the activation
//     fragments and weight operands of step j + 1 are prepared; scheduling
//     barriers keep that preparation in the shadow of the step's MFMAs.
// ---------------------------------------------------------------------------
constexpr int kBigMA = kBigRows / 32;   // row tiles per chunk
constexpr int kBigKS = 128;             // K per stage (one weight group)
constexpr int kBigLdsRow = kBigKS + 8;  // padded LDS row (fp16 elements)
constexpr int kBigMaxGroups = kMaxHidden / kGroup;   // scales per weight row
// waves per workgroup: 4 for the gate/up projections (one per SIMD, each with
// every row tile of the chunk, so each weight is converted once), 8 for the
// down projections (two row groups: the block loop needs the registers)
__host__ __device__ constexpr int big_waves(int mode) { return mode == kRoutedW2 ? 8 : 4; }
constexpr int kBigMaxGroups6 = kMaxHidden / kShGroup;   // INT6 scales per weight row

// QG: INT4 scale groups per 128-input stage (1: group 128, 2: group 64).
template <int MODE, int QG>
__global__ __launch_bounds__(big_waves(MODE) * kWave, 8 / big_waves(MODE)) void moe_gemm_big_kernel(GemmArgs g, int nblocks, int nbg)
{
    static_assert(kBigKS == kGroup, "one INT4 weight group per stage");
    static_assert(MODE != kSharedW2, "the shared down projection (K = its inter) runs in moe_gemm_kernel");
    constexpr bool kW13 = MODE == kRoutedW13 || MODE == kSharedW13;
    // the shared expert: INT6 codes in groups of 64 (two scale groups per
    // stage), every token a row (chunk c = tokens [192 c, 192 c + 192))
    constexpr bool kInt6 = MODE == kSharedW13 || MODE == kSharedW2;
    static_assert(QG == 1 || (QG == 2 && !kInt6), "INT6 groups are set by the lane half");
    constexpr int kScPerStage = kInt6 ? 2 : QG;
    constexpr int kScRows = kInt6 ? kBigMaxGroups6 : kBigMaxGroups * QG;
    constexpr int kBigWaves = big_waves(MODE);
    constexpr int kBigThreads = kBigWaves * kWave;
    constexpr int kRowGroups = kBigWaves / 4;
    constexpr int kBigStageRows = kBigThreads / 8;   // rows one staging pass covers (8 threads per row)
    // several weight blocks per workgroup only for the routed down projection
    // (its K is short, so a block's set-up costs as much as a good part of its
    // loop; the gate/up projection's 20 groups of scales fill the LDS for one
    // block); the other modes take nbg = 1
    constexpr bool kBlockLoop = MODE == kRoutedW2;
    __shared__ __align__(16) _Float16 s_a[2][kBigRows * kBigLdsRow];
    __shared__ uint16_t s_sc[kScRows][kNT];   // [block * groups + group][tile weight row] bf16 scales
    __shared__ int s_tok[kBigRows];     // token of each chunk row (-1: none)
    __shared__ int s_yrow[kBigRows];    // down mode: row of y that each chunk row writes
    __shared__ float s_wgt[kBigRows];   // down mode: output factor of each chunk row

    // ---- chunk and first weight block (XCD-aware: the blocks of one chunk
    // share an XCD); the workgroup runs weight blocks b0 .. b0 + nbg - 1 ----
    const int wid = blockIdx.x;
    const int xcd = wid & 7, r = wid >> 3;
    const int ngroups_b = nblocks / nbg;
    const int b0 = (r % ngroups_b) * nbg, chunk = (r / ngroups_b) * 8 + xcd;
    int e = 0, pbase, rows;
    if constexpr (kInt6) {
        pbase = chunk * kBigRows;
        if (pbase >= g.T) return;   // past the last token
        rows = min(kBigRows, g.T - pbase);
    } else {
        const int4 tv = g.tiles[chunk];
        if (tv.x < 0) return;   // empty slot
        e = tv.x & 0xFFFF;
        pbase = tv.y;
        rows = tv.z;
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
    const int cg = wave & 3, rg = wave >> 2;   // column group, row group (0 with 4 waves)
    const int K = g.K, nstages = K / kBigKS;
    // weight row of tile column c (0..255) of weight block nb: column group
    // c / 64, column tile (c / 32) & 1; block nb + 1 is kBlockRows rows on
    constexpr int kBlockRows = kW13 ? 128 : kNT;
    auto tile_row = [&](int nb, int c) __attribute__((always_inline)) {
        const int w = c >> 6, nt = (c >> 5) & 1, l = c & 31;
        if constexpr (kW13) return nt == 0 ? 128 * nb + 32 * w + l : g.I + 128 * nb + 32 * w + l;
        else return kNT * nb + c;
    };
    const int32_t *bpe = g.bp + (size_t)e * g.b_words;
    const uint16_t *bse = g.bs + (size_t)e * g.b_scales;
    static_assert(kBigThreads >= kNT && kBigThreads >= kBigRows, "one thread per tile column and chunk row");
    if (tid < kNT) {
        // this thread's tile column's scales, every block of the workgroup -> LDS
        const int spr = nstages * kScPerStage;   // scale groups per weight row
        for (int bi = 0; bi < nbg; ++bi) {
            const uint16_t *sr = bse + (size_t)tile_row(b0 + bi, tid) * spr;
            for (int q = 0; q < spr; ++q) s_sc[bi * spr + q][tid] = sr[q];
        }
    }
    if (tid < kBigRows) {
        const int i = tid < rows ? tid : 0;
        if constexpr (kInt6) {
            s_tok[tid] = tid < rows ? pbase + i : -1;
        } else {
            const int slot = g.sorted_slots[pbase + i];
            const int tok = slot / g.k;
            if constexpr (!kW13) {
                s_wgt[tid] = g.weights[slot] * kScaleDown;   // routing weight times the 2^-10 of the scales
                s_yrow[tid] = tok * (g.k + 1) + (slot - tok * g.k);
            }
            s_tok[tid] = tid < rows ? tok : -1;
        }
    }
    __syncthreads();

    // activation staging: thread -> 16-byte chunks c8 and c8 + 8 of rows r8 + 64 o
    const int c8 = tid & 7, r8 = tid >> 3;
    constexpr int kNO = kBigRows / kBigStageRows;   // staging passes for a full chunk
    uint32_t aoff[kNO];   // element offsets of this thread's rows (row 0 of the chunk past its end)
    const uint16_t *abase = kW13 ? g.x : g.a16;
#pragma unroll
    for (int o = 0; o < kNO; ++o) {
        const int row = r8 + kBigStageRows * o, arow = row < rows ? row : 0;
        aoff[o] = kW13 ? (uint32_t)s_tok[arow] * (uint32_t)g.H + 8 * c8
                       : (uint32_t)(pbase + arow) * (uint32_t)K + 8 * c8;
    }
    const int col = lane & 31;
    // a weight row's stage (128 inputs) is 64 bytes of INT4 or 96 of INT6;
    // lane half h takes 16-byte pieces h and 2 + h of an INT4 stage, pieces
    // 3 h .. 3 h + 2 (32-code blocks 2 h and 2 h + 1) of an INT6 one
    constexpr int kU4Stage = kInt6 ? 6 : 4, kU4Lane = kInt6 ? 3 : 2;
    const size_t bstride = kInt6 ? (size_t)K / 32 * 6 : (size_t)K / 8;   // words per weight row
    const size_t bblock = (size_t)kBlockRows * bstride / 4;   // 16-byte units from one block to the next
    const u32x4_t *bq[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
        bq[nt] = reinterpret_cast<const u32x4_t *>(bpe + (size_t)tile_row(b0, 64 * cg + 32 * nt + col) * bstride) +
                 (kInt6 ? 3 * half : half);
    const int mtiles = (rows + 31) / 32;
    const int t0 = rg == 0 ? 0 : (mtiles + 1) / 2;   // first row tile of this wave's row group
    constexpr int kMaxMA = kBigMA / kRowGroups;       // most row tiles of one wave
    const int nst_all = nbg * nstages;                // stages over all the workgroup's blocks

    f32x16_t acc[kMaxMA][2];
    auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kMaxMA; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
    };
    zero_acc();

    // MA: this wave's row tiles; NO: staging passes of the chunk (every wave
    // takes part in staging)
    auto kloop = [&](auto ma_c, auto no_c) __attribute__((always_inline)) {
        constexpr int MA = decltype(ma_c)::value;
        constexpr int NO = decltype(no_c)::value;
        u32x4_t ra[NO][2];          // the next stage's activations
        u32x4_t rb[3][2][kU4Lane];  // weight stages in flight: [set][nt][piece]
        // global stage gs: block gs / nstages of the workgroup, K stage gs % nstages
        auto load_a_pass = [&](int gs, int o) __attribute__((always_inline)) {
            const uint16_t *src = abase + aoff[o] + (gs % nstages) * kBigKS;
            ra[o][0] = *reinterpret_cast<const u32x4_t *>(src);
            ra[o][1] = *reinterpret_cast<const u32x4_t *>(src + 64);
        };
        auto store_a_pass = [&](int buf, int o) __attribute__((always_inline)) {
            _Float16 *dst = s_a[buf] + (r8 + kBigStageRows * o) * kBigLdsRow + 8 * c8;
            *reinterpret_cast<u32x4_t *>(dst) = ra[o][0];
            *reinterpret_cast<u32x4_t *>(dst + 64) = ra[o][1];
        };
        auto load_b_piece = [&](int gs, int set, int nt) __attribute__((always_inline)) {
            const int bi = gs / nstages, grp = gs - bi * nstages;
            const u32x4_t *q = bq[nt] + bi * bblock + kU4Stage * grp;   // the lane half's offset applied
            if constexpr (kInt6) {
                rb[set][nt][0] = q[0];
                rb[set][nt][1] = q[1];
                rb[set][nt][2] = q[2];
            } else {
                rb[set][nt][0] = q[0];
                rb[set][nt][1] = q[2];
            }
        };
        // fp16 scale pairs of global stage gs for this lane's two rows:
        // [inputs 0-63 / 64-127 of the stage][nt].  INT6: the lane half's group
        // of 64 (both entries); INT4 group 64: groups 2 gs and 2 gs + 1 (MFMA
        // step j reads group j / 4); INT4 group 128: the stage's one group.
        auto scales_of = [&](int gs, h2_t (&s2)[2][2]) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int c = 64 * cg + 32 * nt + col;
                if constexpr (kInt6) {
                    s2[0][nt] = s2[1][nt] = scale_pair(s_sc[2 * gs + half][c]);
                } else if constexpr (QG == 2) {
                    s2[0][nt] = scale_pair(s_sc[2 * gs][c]);
                    s2[1][nt] = scale_pair(s_sc[2 * gs + 1][c]);
                } else {
                    s2[0][nt] = s2[1][nt] = scale_pair(s_sc[gs][c]);
                }
            }
        };
        // weight operands of MFMA step j (0..7) of the weight group in `set`
        auto dequant_step = [&](int set, const h2_t (&s2g)[2][2], int j, f16x8_t (&out)[2]) {
            const h2_t (&s2)[2] = s2g[j >> 2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                if constexpr (kInt6) {
                    // octet j & 3 of the lane's 32-code block j >> 2
                    uint32_t w7[7];
#pragma unroll
                    for (int q = 0; q < 6; ++q) {
                        const int dw = 6 * (j >> 2) + q;
                        w7[q] = rb[set][nt][dw >> 2][dw & 3];
                    }
                    w7[6] = 0;
                    switch (j & 3) {
                    case 0: out[nt] = dequant_int6_octet<0>(w7, s2[nt]); break;
                    case 1: out[nt] = dequant_int6_octet<1>(w7, s2[nt]); break;
                    case 2: out[nt] = dequant_int6_octet<2>(w7, s2[nt]); break;
                    default: out[nt] = dequant_int6_octet<3>(w7, s2[nt]); break;
                    }
                } else {
                    const u32x4_t v = rb[set][nt][j >> 2];
                    out[nt] = dequant_int4_f16(v[j & 3], s2[nt]);
                }
            }
        };
        // outputs of weight block b from the accumulators
        auto store_block = [&](int b) __attribute__((always_inline)) {
            if constexpr (kW13) {
                // h rows of the chunk through a buffer resource that covers
                // exactly its rows: the stores of rows past the chunk fall
                // outside it and are dropped, so no row test and no 64-bit
                // address per value; the lane's column is the same for all
                const __amdgpu_buffer_rsrc_t hrs = __builtin_amdgcn_make_buffer_rsrc(
                    g.h_out + (size_t)pbase * g.I, (short)0, rows * g.I * 2, kBufferWord3);
                const int i = 128 * b + 32 * cg + col;
                const int lane_off = ((32 * t0 + 4 * half) * g.I + ((i & ~7) | pair_pos(i & 7))) * 2;
#pragma unroll
                for (int mt = 0; mt < MA; ++mt) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int mrow = 32 * mt + 8 * (j >> 2) + (j & 3);   // the same for the wave
                        const float gv = acc[mt][0][j] * kScaleDown, uv = acc[mt][1][j] * kScaleDown;
                        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_f16_sat(silu(gv) * uv), hrs,
                                                              lane_off + mrow * g.I * 2, 0, 0);
                    }
                }
                return;
            }
#pragma unroll
            for (int mt = 0; mt < MA; ++mt) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int m = 32 * (t0 + mt) + 8 * (j >> 2) + 4 * half + (j & 3);
                    if (m >= rows) continue;
                    const float wv = s_wgt[m];
                    // the lane's columns of both column tiles side by side (interleaved
                    // columns; two 16-bit stores: a packed word costs this kernel spills;
                    // a buffer resource over y, as for h above, measured slower here)
                    uint16_t *yr = g.y_out + (size_t)s_yrow[m] * g.H + kNT * b + 64 * cg + 2 * col;
                    yr[0] = (uint16_t)f32_to_f16_sat(wv * acc[mt][0][j]);
                    yr[1] = (uint16_t)f32_to_f16_sat(wv * acc[mt][1][j]);
                }
            }
        };
        f16x8_t bcur[2];   // weight operands of the step about to run
        // global stage gs: its weight group in `set` (the next stage's in
        // nset), activations in LDS buffer gs & 1; during it the next stage's
        // activations go to the other buffer (unconditionally: the last stage
        // writes a buffer no stage reads any more and reloads the last stage,
        // so no branch leaves the compiler guessing how many loads are in
        // flight), the stage after next's are loaded, and the weights of stage
        // gs + 2 are loaded into (set + 2) % 3.  The next block's first stages
        // are loaded during the previous block's last ones.
        auto stage = [&](int gs, int set, int nset) __attribute__((always_inline)) {
            const int ngs = min(gs + 2, nst_all - 1);
            h2_t s2c[2][2];
            scales_of(gs, s2c);
            // the activations in the weights' K order: step j of half h is
            // K = 64 (j / 4) + 32 h + 8 (j % 4) for INT4, 64 h + 32 (j / 4) +
            // 8 (j % 4) for INT6
            const _Float16 *A = s_a[gs & 1] + (32 * t0 + col) * kBigLdsRow + (kInt6 ? 64 : 32) * half;
            f16x8_t af[2][MA > 0 ? MA : 1];
#pragma unroll
            for (int mt = 0; mt < MA; ++mt)
                af[0][mt] = *reinterpret_cast<const f16x8_t *>(A + 32 * mt * kBigLdsRow);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                __builtin_amdgcn_sched_barrier(0);
                if (j < NO) {
                    store_a_pass((gs + 1) & 1, j);
                    load_a_pass(ngs, j);
                }
                if (j == 3) load_b_piece(ngs, (set + 2) % 3, 0);
                if (j == 5) load_b_piece(ngs, (set + 2) % 3, 1);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (MA > 0) {
                    f16x8_t bnext[2];
                    if (j < 7) {
                        const int ko = (kInt6 ? 32 : 64) * ((j + 1) >> 2) + 8 * ((j + 1) & 3);
#pragma unroll
                        for (int mt = 0; mt < MA; ++mt)
                            af[(j + 1) & 1][mt] = *reinterpret_cast<const f16x8_t *>(A + 32 * mt * kBigLdsRow + ko);
                        dequant_step(set, s2c, j + 1, bnext);
                    } else {
                        h2_t s2n[2][2];
                        scales_of(min(gs + 1, nst_all - 1), s2n);
                        dequant_step(nset, s2n, 0, bnext);   // the next stage's first step
                    }
#pragma unroll
                    for (int mt = 0; mt < MA; ++mt) {
                        acc[mt][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[j & 1][mt], bcur[0], acc[mt][0], 0, 0, 0);
                        acc[mt][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[j & 1][mt], bcur[1], acc[mt][1], 0, 0, 0);
                    }
                    // interleave: one MFMA, then a share of the step's
                    // preparation (LDS reads first, then conversions)
#pragma unroll
                    for (int i = 0; i < 2 * MA; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                        if (j < 7 && i < MA) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
                        __builtin_amdgcn_sched_group_barrier(0x002, (30 + 2 * MA - 1) / (2 * MA), 0);   // VALU
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    bcur[0] = bnext[0];
                    bcur[1] = bnext[1];
                }
            }
            __syncthreads();
            if constexpr (kBlockLoop) {
                // the end of a weight block: its outputs, then fresh accumulators
                const int bi = gs / nstages;
                if (gs - bi * nstages == nstages - 1) {
                    store_block(b0 + bi);
                    zero_acc();
                }
            }
        };
        // prologue: the first two stages' weights, stage 0's activations in
        // LDS and stage 1's in flight
        load_b_piece(0, 0, 0);
        load_b_piece(0, 0, 1);
        load_b_piece(min(1, nst_all - 1), 1, 0);
        load_b_piece(min(1, nst_all - 1), 1, 1);
#pragma unroll
        for (int o = 0; o < NO; ++o) load_a_pass(0, o);
#pragma unroll
        for (int o = 0; o < NO; ++o) store_a_pass(0, o);
#pragma unroll
        for (int o = 0; o < NO; ++o) load_a_pass(min(1, nst_all - 1), o);
        if constexpr (MA > 0) {
            h2_t s20[2][2];
            scales_of(0, s20);
            dequant_step(0, s20, 0, bcur);
        }
        __syncthreads();
        int gs = 0;
        for (; gs + 3 <= nst_all; gs += 3) {
            stage(gs, 0, 1);
            stage(gs + 1, 1, 2);
            stage(gs + 2, 2, 0);
        }
        if (gs < nst_all) stage(gs, 0, 1);
        if (gs + 1 < nst_all) stage(gs + 1, 1, 2);
        if constexpr (!kBlockLoop) store_block(b0);
    };
    static_assert(kBigMA == 6 && kNO == 6 / kRowGroups, "K loop variants below");
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    if constexpr (kRowGroups == 1) {
        // every wave takes all T row tiles; the staging passes cover T * 32 rows
        using I4 = std::integral_constant<int, 4>;
        using I5 = std::integral_constant<int, 5>;
        using I6 = std::integral_constant<int, 6>;
        switch (mtiles) {
        case 1: kloop(I1{}, I1{}); break;
        case 2: kloop(I2{}, I2{}); break;
        case 3: kloop(I3{}, I3{}); break;
        case 4: kloop(I4{}, I4{}); break;
        case 5: kloop(I5{}, I5{}); break;
        default: kloop(I6{}, I6{}); break;
        }
        return;
    }
    // row tiles: row group 0 takes ceil(T / 2), row group 1 the rest; the
    // staging passes cover ceil(T / 2) * 64 rows
    switch (mtiles * 2 + rg) {
    case 2: kloop(I1{}, I1{}); break;   // 1 tile: group 0 has it
    case 3: kloop(I0{}, I1{}); break;
    case 4: kloop(I1{}, I1{}); break;   // 2 tiles
    case 5: kloop(I1{}, I1{}); break;
    case 6: kloop(I2{}, I2{}); break;   // 3 tiles
    case 7: kloop(I1{}, I2{}); break;
    case 8: kloop(I2{}, I2{}); break;   // 4 tiles
    case 9: kloop(I2{}, I2{}); break;
    case 10: kloop(I3{}, I3{}); break;  // 5 tiles
    case 11: kloop(I2{}, I3{}); break;
    default: kloop(I3{}, I3{}); break;  // 6 tiles
    }
}

// ---------------------------------------------------------------------------
// Routed down projection with the activation rows resident in LDS.
//
// Its K (the intermediate size) is short, so half a chunk's h rows (at most
// three 32-row tiles) fit in LDS for the whole K.  A workgroup loads them
// once and its 8 waves (two per SIMD) then run independently, with no
// barrier: wave w takes the 64-column output groups w, w + 8, ...; for each
// it streams that group's 64 weight rows over K (INT4 codes and scales two
// K stages ahead in registers, dequantised exactly to fp16 as in the other
// GEMMs), accumulates 3 x 2 MFMA tiles and stores its weighted y values.
// The two halves of a chunk are dispatched next to each other on one XCD,
// so they read each weight from HBM once between them.  Against a kernel
// that stages the rows per weight block this reads h from L2 once instead
// of once per block, and no wave waits on another.
// ---------------------------------------------------------------------------
constexpr int kDnWaves = 8;
constexpr int kDnThreads = kDnWaves * kWave;
constexpr int kDnMaxTiles = 3;                 // row tiles of a workgroup (half of a kBigRows chunk)
constexpr int kDnRows = 32 * kDnMaxTiles;
constexpr int kDnMaxK = 768;                   // longest K held in LDS
constexpr int kDnLdsRow = kDnMaxK + 8;         // padded row, fp16 elements
static_assert(2 * kDnRows == kBigRows, "two halves per chunk");

template <int QG>
__global__ __launch_bounds__(kDnThreads, 1) void moe_down_resident_kernel(GemmArgs g)
{
    __shared__ __align__(16) _Float16 s_h[kDnRows * kDnLdsRow];
    __shared__ float s_wgt[kDnRows];   // routing weight x 2^-10 per row
    __shared__ int s_yrow[kDnRows];    // row of y per row
    __shared__ uint32_t s_yoff[kDnRows];   // its byte offset in y (2^31 past the rows; y under 2^31 bytes)

    const int wid = blockIdx.x, xcd = wid & 7, r = wid >> 3;
    const int chunk = (r >> 1) * 8 + xcd, part = r & 1;
    const int4 tv = g.tiles[chunk];
    if (tv.x < 0) return;   // empty slot
    const int ctiles = (tv.z + 31) / 32;
    const int tfirst = part == 0 ? 0 : (ctiles + 1) / 2;
    const int ntiles = part == 0 ? (ctiles + 1) / 2 : ctiles / 2;
    if (ntiles == 0) return;   // a one-tile chunk has no second half
    const int e = tv.x & 0xFFFF;
    const int pbase = tv.y + 32 * tfirst, rows = min(32 * ntiles, tv.z - 32 * tfirst);
    const int K = g.K, ldsrow = K + 8, nst = K / kBigKS;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5, col = lane & 31;

    // while y is under 2^31 bytes its stores go through one buffer resource
    // over y, and a row past the workgroup's has offset 2^31, outside it, so
    // the hardware drops those stores (no row test, no 64-bit addresses)
    const long ybytes = (long)g.T * (g.k + 1) * g.H * 2;
    const bool ybuf = ybytes < 0x80000000L;
    if (tid < 32 * ntiles) {
        s_yoff[tid] = 0x80000000u;
        if (tid < rows) {
            const int slot = g.sorted_slots[pbase + tid];
            const int tok = slot / g.k;
            const int yrow = tok * (g.k + 1) + (slot - tok * g.k);
            s_wgt[tid] = g.weights[slot] * kScaleDown;
            s_yrow[tid] = yrow;
            if (ybuf) s_yoff[tid] = (uint32_t)yrow * (uint32_t)g.H * 2u;
        }
    }
    // the rows' h (K fp16 each) -> LDS, 16-byte pieces, eight loads in flight per thread
    {
        const uint32_t pr = (uint32_t)K / 8, npieces = (uint32_t)rows * pr;
        const uint32_t inv = (uint32_t)((0x100000000ull + pr - 1) / pr);   // exact p / pr for p < 2^16
        const uint16_t *src = g.a16 + (size_t)pbase * K;
        for (uint32_t p0 = 0; p0 < npieces; p0 += 8 * kDnThreads) {
            u32x4_t v[8];
            int dst[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t p = p0 + u * kDnThreads + tid, pc = p < npieces ? p : 0;
                const uint32_t rr = __umulhi(pc, inv), c = pc - rr * pr;
                v[u] = *reinterpret_cast<const u32x4_t *>(src + rr * (uint32_t)K + 8 * c);
                dst[u] = p < npieces ? (int)(rr * (uint32_t)ldsrow + 8 * c) : -1;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (dst[u] >= 0) *reinterpret_cast<u32x4_t *>(s_h + dst[u]) = v[u];
        }
    }
    __syncthreads();

    const int ngroups = g.H / 64;   // 64-column output groups
    const int npass = ngroups > wave ? (ngroups - wave + kDnWaves - 1) / kDnWaves : 0;
    if (npass == 0) return;
    const int nst_all = npass * nst;
    const size_t bstride = (size_t)K / 8;   // words per weight row
    const int32_t *bpe = g.bp + (size_t)e * g.b_words;
    const uint16_t *bse = g.bs + (size_t)e * g.b_scales;

    auto kloop = [&](auto ma_c) __attribute__((always_inline)) {
        constexpr int MA = decltype(ma_c)::value;
        f32x16_t acc[MA][2];
        auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < MA; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
        };
        zero_acc();
        u32x4_t rb[3][2][2];   // weight stages in flight: [set][nt][piece]
        uint32_t rs[3][2];     // their bf16 scales: the stage's first and second 64 inputs
        // global stage gs: pass gs / nst (output group wave + 8 pass), K stage gs % nst
        auto load_b = [&](int gs, int set) __attribute__((always_inline)) {
            const int ps = gs / nst, s = gs - ps * nst;
            const int n0 = 64 * (wave + kDnWaves * ps) + col;
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int n = n0 + 32 * nt;
                const u32x4_t *q = reinterpret_cast<const u32x4_t *>(bpe + (size_t)n * bstride) + 4 * s + half;
                rb[set][nt][0] = q[0];
                rb[set][nt][1] = q[2];
                if constexpr (QG == 2) {
                    // groups 2 s and 2 s + 1 of the row: one aligned word (a row holds 2 nst scales)
                    rs[set][nt] = reinterpret_cast<const uint32_t *>(bse)[(size_t)n * nst + s];
                } else {
                    rs[set][nt] = bse[(size_t)n * nst + s];
                }
            }
        };
        // the stage's fp16 scale pairs: [inputs 0-63 / 64-127][nt] (the same scale at group 128)
        auto stage_scales = [&](int set, h2_t (&s2)[2][2]) __attribute__((always_inline)) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                s2[0][nt] = scale_pair((uint16_t)rs[set][nt]);
                s2[1][nt] = QG == 2 ? scale_pair((uint16_t)(rs[set][nt] >> 16)) : s2[0][nt];
            }
        };
        // step j reads inputs 64 (j / 4) + 32 h + 8 (j % 4) of the stage: group j / 4 of 64
        auto dequant_step = [&](int set, const h2_t (&s2)[2][2], int j, f16x8_t (&out)[2]) __attribute__((always_inline)) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) out[nt] = dequant_int4_f16(rb[set][nt][j >> 2][j & 3], s2[j >> 2][nt]);
        };
        auto store_pass = [&](int ps) __attribute__((always_inline)) {
            const int n0 = 64 * (wave + kDnWaves * ps);
            if (ybuf) {
                const __amdgpu_buffer_rsrc_t yrs =
                    __builtin_amdgcn_make_buffer_rsrc(g.y_out, (short)0, (int)ybytes, kBufferWord3);
                const uint32_t lane_off = (uint32_t)(n0 + 2 * col) * 2u;
#pragma unroll
                for (int mt = 0; mt < MA; ++mt) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int m = 32 * mt + 8 * (j >> 2) + 4 * half + (j & 3);
                        const float wv = s_wgt[m];
                        // the lane's columns of both tiles side by side: one word
                        const uint32_t pk = f32_to_f16_sat(wv * acc[mt][0][j]) | f32_to_f16_sat(wv * acc[mt][1][j]) << 16;
                        __builtin_amdgcn_raw_buffer_store_b32(pk, yrs, (int)(s_yoff[m] + lane_off), 0, 0);
                    }
                }
                return;
            }
#pragma unroll
            for (int mt = 0; mt < MA; ++mt) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int m = 32 * mt + 8 * (j >> 2) + 4 * half + (j & 3);
                    if (m >= rows) continue;
                    const float wv = s_wgt[m];
                    // interleaved columns: the lane's columns of both tiles side by side
                    uint16_t *yr = g.y_out + (size_t)s_yrow[m] * g.H + n0 + 2 * col;
                    yr[0] = (uint16_t)f32_to_f16_sat(wv * acc[mt][0][j]);
                    yr[1] = (uint16_t)f32_to_f16_sat(wv * acc[mt][1][j]);
                }
            }
        };
        f16x8_t bcur[2];
        auto stage = [&](int gs, int set, int nset) __attribute__((always_inline)) {
            load_b(min(gs + 2, nst_all - 1), (set + 2) % 3);
            const int ps = gs / nst, s = gs - ps * nst;
            h2_t s2c[2][2];
            stage_scales(set, s2c);
            // step j of lane half h reads K = 64 (j / 4) + 32 h + 8 (j % 4) of the stage
            const _Float16 *A = s_h + col * ldsrow + kBigKS * s + 32 * half;
            f16x8_t af[2][MA];
#pragma unroll
            for (int mt = 0; mt < MA; ++mt) af[0][mt] = *reinterpret_cast<const f16x8_t *>(A + 32 * mt * ldsrow);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                __builtin_amdgcn_sched_barrier(0);
                f16x8_t bnext[2];
                if (j < 7) {
                    const int ko = 64 * ((j + 1) >> 2) + 8 * ((j + 1) & 3);
#pragma unroll
                    for (int mt = 0; mt < MA; ++mt)
                        af[(j + 1) & 1][mt] = *reinterpret_cast<const f16x8_t *>(A + 32 * mt * ldsrow + ko);
                    dequant_step(set, s2c, j + 1, bnext);
                } else {
                    h2_t s2n[2][2];
                    stage_scales(nset, s2n);
                    dequant_step(nset, s2n, 0, bnext);   // the next stage's first step
                }
#pragma unroll
                for (int mt = 0; mt < MA; ++mt) {
                    acc[mt][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[j & 1][mt], bcur[0], acc[mt][0], 0, 0, 0);
                    acc[mt][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[j & 1][mt], bcur[1], acc[mt][1], 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 2 * MA; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                    if (j < 7 && i < MA) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
                    __builtin_amdgcn_sched_group_barrier(0x002, (30 + 2 * MA - 1) / (2 * MA), 0);   // VALU
                }
                __builtin_amdgcn_sched_barrier(0);
                bcur[0] = bnext[0];
                bcur[1] = bnext[1];
            }
            if (s == nst - 1) {
                store_pass(ps);
                zero_acc();
            }
        };
        load_b(0, 0);
        load_b(min(1, nst_all - 1), 1);
        {
            h2_t s20[2][2];
            stage_scales(0, s20);
            dequant_step(0, s20, 0, bcur);
        }
        int gs = 0;
        for (; gs + 3 <= nst_all; gs += 3) {
            stage(gs, 0, 1);
            stage(gs + 1, 1, 2);
            stage(gs + 2, 2, 0);
        }
        if (gs < nst_all) stage(gs, 0, 1);
        if (gs + 1 < nst_all) stage(gs + 1, 1, 2);
    };
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    switch (ntiles) {
    case 1: kloop(I1{}); break;
    case 2: kloop(I2{}); break;
    default: kloop(I3{}); break;
    }
}

// Weight blocks per workgroup of the whole-expert GEMM: the most that divide
// the block count, keep every block's scales in LDS (kBigMaxGroups) and leave
// at least kBigMinWgs workgroups for the given chunk count, so the block loop
// shares one set-up among several blocks where K is short.
constexpr long kBigMinWgs = 512;
constexpr int kBigSharedMinTokens = 6144;   // the shared expert's whole-chunk gate/up GEMM from this many tokens (32 chunks)
static int big_blocks_per_wg(int nblocks, int groups_per_block, int chunks)
{
    int best = 1;
    for (int n = 1; n <= nblocks; ++n) {
        if (nblocks % n || n * groups_per_block > kBigMaxGroups) continue;
        if ((long)chunks * (nblocks / n) < kBigMinWgs) break;
        best = n;
    }
    return best;
}

// out[t][n] = bf16( sum_j y[t][j][n] (+ y[t][k][n] for the shared expert) ),
// fixed order.  The down GEMMs store a lane's columns of its two 32-wide
// column tiles as one word, so a y row holds column n at position
// 64 (n / 64) + 2 (n % 32) + (n % 64) / 32: one thread takes 16 positions,
// i.e. columns c .. c + 7 and c + 32 .. c + 39 of a 64-column group.  The
// slot rows are loaded four at a time, all in flight together (clamped,
// unconditional loads; a clamped duplicate adds +0), instead of one load
// waited for per slot.
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t *__restrict__ y, int T, int H,
                                                      int k, int nslots, uint16_t *__restrict__ out)
{
    const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    const size_t n16 = (size_t)T * H / 16;
    if (i >= n16) return;
    const size_t t = i / (H / 16), c = i % (H / 16);
    const uint4 *src = reinterpret_cast<const uint4 *>(y + t * (k + 1) * H) + 2 * c;
    const size_t stride = H / 8;   // 16-byte pieces per slot row
    float acc[16];                 // position p of the 16: column 8 (c % 4) + p / 2 of tile p % 2
#pragma unroll
    for (int p = 0; p < 16; ++p) acc[p] = 0.f;
    for (int j0 = 0; j0 < nslots; j0 += 4) {
        uint4 v[4][2];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int h = 0; h < 2; ++h) v[u][h] = src[(size_t)min(j0 + u, nslots - 1) * stride + h];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            // a duplicate adds +0 (a select, not a branch, so the loads stay
            // ahead of the first use)
            const bool dup = j0 + u >= nslots;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t w[4] = {dup ? 0u : v[u][h].x, dup ? 0u : v[u][h].y, dup ? 0u : v[u][h].z,
                                       dup ? 0u : v[u][h].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const h2_t hv = __builtin_bit_cast(h2_t, w[q]);
                    acc[8 * h + 2 * q] += (float)hv[0];
                    acc[8 * h + 2 * q + 1] += (float)hv[1];
                }
            }
        }
    }
    uint32_t o0[4], o1[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        o0[r] = f32x2_to_bf16x2(acc[4 * r], acc[4 * r + 2]);
        o1[r] = f32x2_to_bf16x2(acc[4 * r + 1], acc[4 * r + 3]);
    }
    uint16_t *orow = out + t * H + 64 * (c / 4) + 8 * (c % 4);
    *reinterpret_cast<uint4 *>(orow) = make_uint4(o0[0], o0[1], o0[2], o0[3]);
    *reinterpret_cast<uint4 *>(orow + 32) = make_uint4(o1[0], o1[1], o1[2], o1[3]);
}

// ---------------------------------------------------------------------------
// Router GEMM on matrix cores: logits[t][e] = x_t . router_w[e] with bf16
// operands (exact products) and fp32 accumulation.  Tile 128 tokens x 128
// experts, 8 waves (2 x 4), each 64 x 32.
// ---------------------------------------------------------------------------
constexpr int kRT_N = 128;

__global__ __launch_bounds__(kRouterThreads, 4) void router_mfma_kernel(const uint16_t *__restrict__ x,
                                                                   const uint16_t *__restrict__ rw,
                                                                   int T, int H, int E,
                                                                   float *__restrict__ logits)
{
    __shared__ __align__(16) uint16_t s_a[2][kMT * kLdsRow];
    __shared__ __align__(16) uint16_t s_b[2][kRT_N * kLdsRow];
    const int m0 = blockIdx.x * kMT, e0 = blockIdx.y * kRT_N;
    // this split's share of the reduction over H, and its partial-logit plane
    const int nsteps = H / kKS / gridDim.z, s0 = blockIdx.z * nsteps;
    logits += (size_t)blockIdx.z * T * E;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int mh = wave & 1, nq = wave >> 1;
    // staging: A 128 x 64 bf16 (2 octets per thread), B 128 x 64 (2 octets per
    // thread: rows br and br + 64)
    const int ar = tid >> 2, apart = tid & 3;
    const int br = tid >> 3, bpart = tid & 7;
    // rows past T or E load the last valid row (their sums are not stored), so
    // every load is unconditional and the compiler counts them exactly
    const uint16_t *arow = x + (size_t)min(m0 + ar, T - 1) * H + 16 * apart;
    const uint16_t *brow0 = rw + (size_t)min(e0 + br, E - 1) * H + 8 * bpart;
    const uint16_t *brow1 = rw + (size_t)min(e0 + br + 64, E - 1) * H + 8 * bpart;
    // kRtDepth stages in flight in registers: a stage's MFMAs (8 per wave)
    // take far less than a memory round trip
    constexpr int kRtDepth = 3;
    u32x4_t ra[kRtDepth][2], rb[kRtDepth][2];
    auto load_stage = [&](int s, int slot) __attribute__((always_inline)) {
        const int k0 = (s0 + min(s, nsteps - 1)) * kKS;   // past the last stage: reload it (unused)
        ra[slot][0] = *reinterpret_cast<const u32x4_t *>(arow + k0);
        ra[slot][1] = *reinterpret_cast<const u32x4_t *>(arow + k0 + 8);
        rb[slot][0] = *reinterpret_cast<const u32x4_t *>(brow0 + k0);
        rb[slot][1] = *reinterpret_cast<const u32x4_t *>(brow1 + k0);
    };
    auto store_stage = [&](int slot, int buf) __attribute__((always_inline)) {
        *reinterpret_cast<u32x4_t *>(s_a[buf] + ar * kLdsRow + 16 * apart) = ra[slot][0];
        *reinterpret_cast<u32x4_t *>(s_a[buf] + ar * kLdsRow + 16 * apart + 8) = ra[slot][1];
        *reinterpret_cast<u32x4_t *>(s_b[buf] + br * kLdsRow + 8 * bpart) = rb[slot][0];
        *reinterpret_cast<u32x4_t *>(s_b[buf] + (br + 64) * kLdsRow + 8 * bpart) = rb[slot][1];
    };
    f32x16_t acc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][q] = 0.f;
    // stage j lives in register slot j % kRtDepth until it is stored to LDS
    // buffer j & 1 (at the end of step j - 1), which frees the slot for stage
    // j + kRtDepth
#pragma unroll
    for (int j = 0; j < kRtDepth; ++j) load_stage(j, j);
    store_stage(0, 0);
    load_stage(kRtDepth, 0);
    __syncthreads();
    auto step = [&](int s, auto slot_c) __attribute__((always_inline)) {
        constexpr int nslot = (decltype(slot_c)::value + 1) % kRtDepth;   // slot of stage s + 1
        const int buf = s & 1;
#pragma unroll
        for (int ks = 0; ks < kKS / 16; ++ks) {
            const int kk = 16 * ks + 8 * (lane >> 5);
            bf16x8_t af[2], bfr;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                af[mt] = *reinterpret_cast<const bf16x8_t *>(s_a[buf] + (64 * mh + 32 * mt + (lane & 31)) * kLdsRow + kk);
            bfr = *reinterpret_cast<const bf16x8_t *>(s_b[buf] + (32 * nq + (lane & 31)) * kLdsRow + kk);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mt], bfr, acc[mt], 0, 0, 0);
        }
        store_stage(nslot, buf ^ 1);   // stage s + 1 (past the end: a reload nobody reads)
        load_stage(s + 1 + kRtDepth, nslot);
        __syncthreads();
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    static_assert(kRtDepth == 3, "the step loop below rotates three slots");
    int s = 0;
    for (; s + 3 <= nsteps; s += 3) {
        step(s, C0{});
        step(s + 1, C1{});
        step(s + 2, C2{});
    }
    if (s < nsteps) step(s, C0{});
    if (s + 1 < nsteps) step(s + 1, C1{});
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int m = m0 + 64 * mh + 32 * mt + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
            const int n = e0 + 32 * nq + (lane & 31);
            if (m < T && n < E) logits[(size_t)m * E + n] = acc[mt][j];
        }
}

__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t *__restrict__ counts,
                                                           const int32_t *__restrict__ offsets, int E,
                                                           int nslots, int mt, int4 *__restrict__ tiles)
{
    __shared__ int s_sum[16];
    const int e = threadIdx.x;
    build_tile_list(e < E ? counts[e] : 0, e < E ? offsets[e] : 0, nslots, mt, tiles, s_sum);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_shared_gate(const uint16_t *x, const uint16_t *gate_w, const Dims &d, float *out,
                              hipStream_t st);

hipError_t launch_router_mfma(const uint16_t *x, const uint16_t *router_w, const Dims &d,
                              float *logits, hipStream_t st)
{
    dim3 grid((d.T + kMT - 1) / kMT, (d.E + kRT_N - 1) / kRT_N, router_ksplit(d));
    router_mfma_kernel<<<grid, kRouterThreads, 0, st>>>(x, router_w, d.T, d.H, d.E, logits);
    return hipGetLastError();
}


template <int MODE>
static hipError_t launch_gemm(const GemmArgs &g, int ntiles_max, int nblocks, hipStream_t st, bool g64 = false,
                              bool big = false)
{
    const int groups = (ntiles_max + 7) / 8;
    if constexpr (MODE == kRoutedW13 || MODE == kRoutedW2) {
        const unsigned grid = groups * 8 * nblocks;
        if (MODE == kRoutedW2 && big && g.K <= kDnMaxK) {
            // two workgroups per chunk slot, one per half of its row tiles
            if (g64) moe_down_resident_kernel<2><<<groups * 8 * 2, kDnThreads, 0, st>>>(g);
            else moe_down_resident_kernel<1><<<groups * 8 * 2, kDnThreads, 0, st>>>(g);
            return hipGetLastError();
        }
        if (big) {
            // chunks: about one per expert for balanced routing (the list has
            // room for at most S / kBigRows + E, about twice that)
            const int nbg = MODE == kRoutedW2 ? big_blocks_per_wg(nblocks, g.K / kBigKS, ntiles_max / 2) : 1;
            const unsigned bgrid = groups * 8 * (nblocks / nbg);
            if (g64) moe_gemm_big_kernel<MODE, 2><<<bgrid, big_waves(MODE) * kWave, 0, st>>>(g, nblocks, nbg);
            else moe_gemm_big_kernel<MODE, 1><<<bgrid, big_waves(MODE) * kWave, 0, st>>>(g, nblocks, nbg);
            return hipGetLastError();
        }
        if (g.small_rows > 0) {
            if (g64) moe_gemm_kernel<MODE, 2, 2><<<grid, kGemmThreads, 0, st>>>(g, nblocks);
            else moe_gemm_kernel<MODE, 2><<<grid, kGemmThreads, 0, st>>>(g, nblocks);
            return hipGetLastError();
        }
        if (g64) {
            moe_gemm_kernel<MODE, 4, 2><<<grid, kGemmThreads, 0, st>>>(g, nblocks);
            return hipGetLastError();
        }
    }
    moe_gemm_kernel<MODE><<<groups * 8 * nblocks, kGemmThreads, 0, st>>>(g, nblocks);
    return hipGetLastError();
}

hipError_t launch_shared_expert(const ExpertArgs &a, const Dims &d, const Workspace &ws, hipStream_t st,
                                bool x_converted)
{
    // gate logits, gate/up -> sh_h, down -> y[t][k] = sigmoid(g) * ys
    hipError_t e;
    if (!x_converted && (e = launch_shared_gate(a.x, a.sh_gate, d, ws.shared_gate, st)) != hipSuccess) return e;
    GemmArgs gs{};
    gs.x = ws.xh; gs.bp = a.sh_w13p; gs.bs = a.sh_w13s; gs.h_out = ws.sh_h;
    gs.T = d.T; gs.H = d.H; gs.I = d.sh_I; gs.k = d.k; gs.K = d.H;
    GemmArgs gs2{};
    gs2.a16 = ws.sh_h; gs2.bp = a.sh_w2p; gs2.bs = a.sh_w2s; gs2.gate = ws.shared_gate; gs2.y_out = ws.y;
    gs2.T = d.T; gs2.H = d.H; gs2.I = d.sh_I; gs2.k = d.k; gs2.K = d.sh_I;
    if (d.T >= kBigSharedMinTokens) {
        // whole-chunk gate/up GEMM: 192 tokens per workgroup and weight block
        const int groups = (d.T + 8 * kBigRows - 1) / (8 * kBigRows);
        const int nb13 = d.sh_I / 128;
        moe_gemm_big_kernel<kSharedW13, 1><<<groups * 8 * nb13, big_waves(kSharedW13) * kWave, 0, st>>>(gs, nb13, 1);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else if ((e = launch_gemm<kSharedW13>(gs, (d.T + kMT - 1) / kMT, d.sh_I / 128, st)) != hipSuccess) {
        return e;
    }
    return launch_gemm<kSharedW2>(gs2, (d.T + kMT - 1) / kMT, d.H / kNT, st);
}

hipError_t launch_prefill_experts(const ExpertArgs &a, const Dims &d, const Workspace &ws,
                                  const RouteOut &ro, hipStream_t st, hipEvent_t ev_mid, bool x_converted,
                                  hipEvent_t ev_shared)
{
    hipError_t e;
    const size_t xn8 = (size_t)d.T * d.H / 8;
    if (!x_converted) convert_x_kernel<<<(unsigned)((xn8 + 255) / 256), 256, 0, st>>>(a.x, ws.xh, xn8);
    const bool small = routed_tile_rows(d) < kMT;
    // the one-workgroup permutation builds the list itself
    if (!permute_builds_tiles(d)) {
        build_tiles_kernel<<<1, 1024, 0, st>>>(ro.counts, ro.offsets, d.E, (int)routed_tile_slots(d),
                                               routed_tile_rows(d), ws.tiles);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    uint16_t *y = ws.y;
    // routed gate/up -> h (sorted slot order)
    const int tmax = (int)routed_tile_slots(d);
    GemmArgs g{};
    g.x = ws.xh; g.bp = a.w13p; g.bs = a.w13s; g.tiles = ws.tiles;
    g.offsets = ro.offsets; g.counts = ro.counts; g.sorted_slots = ro.sorted_slots;
    g.h_out = ws.h; g.T = d.T; g.H = d.H; g.I = d.I; g.k = d.k; g.K = d.H;
    // fewer than 32 slots per expert on average: 64-row tiles and the
    // three-workgroups-per-CU kernel, so the few busy experts of a skewed
    // routing are spread over twice as many workgroups
    g.small_rows = small ? 64 : 0;
    g.b_words = (size_t)2 * d.I * d.H / 8; g.b_scales = (size_t)2 * d.I * (d.H >> (d.gsh + 5));
    const bool big = routed_big(d);
    if ((e = launch_gemm<kRoutedW13>(g, tmax, d.I / 128, st, d.gsh == 1, big)) != hipSuccess) return e;
    if (ev_mid && (e = hipEventRecord(ev_mid, st)) != hipSuccess) return e;
    // routed down -> y[t][j] = w * (W2 h)
    GemmArgs g2 = g;
    g2.a16 = ws.h; g2.bp = a.w2p; g2.bs = a.w2s; g2.weights = a.weights; g2.y_out = y;
    g2.K = d.I;
    g2.b_words = (size_t)d.H * d.I / 8; g2.b_scales = (size_t)d.H * (d.I >> (d.gsh + 5));
    if ((e = launch_gemm<kRoutedW2>(g2, tmax, d.H / kNT, st, d.gsh == 1, big)) != hipSuccess) return e;
    if (d.sh_I > 0) {
        if (ev_shared) {
            if ((e = hipStreamWaitEvent(st, ev_shared, 0)) != hipSuccess) return e;
        } else if ((e = launch_shared_expert(a, d, ws, st, x_converted)) != hipSuccess) {
            return e;
        }
    }
    const size_t n16 = (size_t)d.T * d.H / 16;
    combine_kernel<<<(unsigned)((n16 + 255) / 256), 256, 0, st>>>(y, d.T, d.H, d.k,
                                                                 d.k + (d.sh_I > 0 ? 1 : 0), a.out);
    return hipGetLastError();
}

}  // namespace moe
