// INT8 W8A16 linear layer:
//   y[t][n] = bf16( sum_k x[t][k] * (q[n][k] - 128) * s[n][k / G] ),
// fp32 accumulation, one bf16 rounding (round to nearest even) per output.
//
// Method ("Running 125B MoE on Three 3090s - vLLM Optimization Edition",
// section 3.3, "Hyper-connection (decode-04)": an INT8 pack-quantized weight
// holds four codes per 32-bit word, least significant byte first, each stored
// as code + 128, so the word array viewed as bytes already is the stored code
// matrix and is read in place, with no repack; a GEMV serves a few tokens and
// a W8A16 GEMM serves more.  Model card "What is quantized", groups C and D:
// symmetric groups of 64 (hyper-connection low-rank mixers) and 128 (lm_head,
// embeddings).)
//
// gfx950 design
//   * codes become exact fp16 values with one byte permute per pair: fp16
//     0x6400 is 1024 with mantissa step 1, so the stored byte placed in the
//     low mantissa byte reads 1024 + q, and one packed fp16 add of -1152
//     leaves q - 128 (every integer of magnitude <= 2048 is exact in fp16);
//   * activations are fp16 (bf16 inputs convert exactly in fp16's normal
//     range; the conversion saturates outside it, as in the expert GEMMs);
//   * the scale is applied in fp32 to a partial sum that covers one group
//     only, so code * x products are exact and nothing is rounded before the
//     fp32 accumulator: no dequantized weight is ever formed;
//   * the dot-product GEMV skips the bias removal per code pair: it sums the
//     exact products (1024 + q) x of a 16-input chunk and subtracts 1152
//     times the chunk's activation sum (staged in LDS with x) once per row
//     and token;
//   * few tokens (GEMV): x sits in LDS; a wave streams four weight rows at a
//     time, every lane on the same 16-byte column chunk of the four rows, so
//     one LDS read of x serves four rows; rows are spread over the waves of
//     a persistent grid; per-lane sums are reduced across the wave by
//     halving exchanges that leave one (row, token) result per lane group;
//   * many tokens (GEMM): 128 tokens x 128 weight rows per workgroup, each
//     wave all tokens x 32 weight rows (v_mfma_f32_32x32x16_f16); a group's
//     MFMA sums start from zero and are folded into the accumulator with the
//     group's scale (one FMA per output and group); K is split over
//     workgroups when the output tiles alone would leave the chip idle, with
//     fp32 partials summed in a fixed order (deterministic).
#include <type_traits>

#include "common.h"

namespace moe {

namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Stored bytes 2i and 2i+1 of a word -> fp16 pair (q - 128), exact.  The
// permute takes result bytes from {0x64646464 (bytes 4-7), w (bytes 0-3)}.
template <int I>
__device__ __forceinline__ h2_t code_pair(uint32_t w)
{
    constexpr uint32_t sel = I == 0 ? 0x04010400u : 0x04030402u;
    const uint32_t p = __builtin_amdgcn_perm(0x64646464u, w, sel);
    return __builtin_bit_cast(h2_t, p) + h2_t{(_Float16)-1152.f, (_Float16)-1152.f};
}

// Stored bytes 2i and 2i+1 -> fp16 pair (1024 + q), exact; the caller
// removes the bias (1152 per unit of the activation sum) once per chunk.
template <int I>
__device__ __forceinline__ h2_t code_pair_biased(uint32_t w)
{
    constexpr uint32_t sel = I == 0 ? 0x04010400u : 0x04030402u;
    return __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, w, sel));
}

// 8 bf16 (natural order) -> 8 fp16 (natural order); exact in fp16's normal
// range, toward zero outside it (saturating at 65504).
__device__ __forceinline__ u32x4_t bf16x8_to_f16x8(u32x4_t v)
{
    u32x4_t o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        o[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(bf16_lo(v[j]), bf16_hi(v[j])));
    return o;
}

__device__ __forceinline__ float xor_shfl(float v, int m) { return __shfl_xor(v, m, 64); }

// ---------------------------------------------------------------------------
// GEMV (T <= kInt8GemvMaxTokens)
// ---------------------------------------------------------------------------
constexpr int kGvThreads = 256;
constexpr int kGvRows = 4;   // weight rows per wave block

// Sum v[0..M) over the 64 lanes of a wave.  Each halving step sends the half
// of the values this lane gives up to its partner and keeps the other half,
// so after log2(M) steps lane l holds one value, index l >> (6 - log2 M),
// summed over the lanes that share those bits; plain exchanges over the
// remaining bits finish the sum.
template <int M>
__device__ __forceinline__ float wave_transpose_sum(float (&v)[M], int lane)
{
    static_assert(M >= 1 && M <= 64 && (M & (M - 1)) == 0, "power of two");
    constexpr int kSteps = M == 1 ? 0 : M == 2 ? 1 : M == 4 ? 2 : M == 8 ? 3 : M == 16 ? 4 : M == 32 ? 5 : 6;
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
        const int h = (M >> st) / 2, bit = 32 >> st;
        // the choice is made on the values' bits (a select of two array
        // elements would otherwise become a select of their addresses, which
        // moves the array to scratch memory)
        const uint32_t m = (lane & bit) ? 0xFFFFFFFFu : 0u;
#pragma unroll
        for (int j = 0; j < M / 2; ++j) {
            if (j < h) {
                const uint32_t lo = __float_as_uint(v[j]), hi = __float_as_uint(v[j + h]);
                const float give = __uint_as_float((lo & m) | (hi & ~m));
                const float keep = __uint_as_float((hi & m) | (lo & ~m));
                v[j] = keep + xor_shfl(give, bit);
            }
        }
    }
    float s = v[0];
#pragma unroll
    for (int bit = 32 / M; bit >= 1; bit >>= 1) s += xor_shfl(s, bit);
    return s;
}

template <int T>
__global__ __launch_bounds__(kGvThreads) void int8_gemv_kernel(const uint16_t *__restrict__ x,
                                                               const int32_t *__restrict__ wq,
                                                               const uint16_t *__restrict__ wscale,
                                                               int N, int K, int gshift,
                                                               uint16_t *__restrict__ out)
{
    // x as fp16 in LDS: chunk c (16 inputs) of token t is split into two
    // planes of 8 inputs, [t][p][c], so the 16-byte reads of consecutive
    // lanes are consecutive (no bank conflicts)
    extern __shared__ u32x4_t s_x[];
    const int CPR = K >> 4;   // 16-input chunks per row
    // after the T x 2 x CPR units of x: the fp32 sum of each chunk's 16 fp16
    // activations, [T][CPR]
    float *s_xsum = reinterpret_cast<float *>(s_x + T * 2 * CPR);
    for (int i = threadIdx.x; i < T * CPR; i += kGvThreads) {
        const int t = i / CPR, c = i - t * CPR;
        const u32x4_t *src = reinterpret_cast<const u32x4_t *>(x + (size_t)t * K + 16 * c);
        const h2_t one = {(_Float16)1.f, (_Float16)1.f};
        float sum = 0.f;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const u32x4_t v = bf16x8_to_f16x8(src[p]);
            s_x[(t * 2 + p) * CPR + c] = v;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t e = v[q];
                sum = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, e), one, sum, false);
            }
        }
        s_xsum[t * CPR + c] = sum;
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * (kGvThreads / 64) + (threadIdx.x >> 6);
    const int W = gridDim.x * (kGvThreads / 64);
    const int nrb = (N + kGvRows - 1) / kGvRows;
    if (gw >= nrb) return;
    const int NI = (CPR + 63) >> 6;                   // column passes per row block
    const int my_blocks = (nrb - gw + W - 1) / W;
    const int U = my_blocks * NI;                     // (row block, pass) units of this wave
    const size_t rstride = (size_t)K / 4;             // words per row
    const int nsc = K >> gshift;                      // scales per row

    // one unit's raw weights and scales
    struct Raw {
        u32x4_t w[kGvRows];
        uint16_t s[kGvRows];
    };
    auto load = [&](int u, Raw &r) {
        const int b = u / NI, i = u - b * NI;
        const int rb = gw + b * W;
        const int c = min(i * 64 + lane, CPR - 1);   // a lane past the row re-reads a valid chunk
#pragma unroll
        for (int j = 0; j < kGvRows; ++j) {
            const int row = min(rb * kGvRows + j, N - 1);
            r.w[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(wq + row * rstride) + c);
            r.s[j] = wscale[(size_t)row * nsc + ((16 * c) >> gshift)];
        }
    };

    constexpr int M = T == 1 ? 4 : T == 2 ? 8 : 16;   // kGvRows * T, padded to a power of two
    float acc[M];
#pragma unroll
    for (int j = 0; j < M; ++j) acc[j] = 0.f;

    auto compute = [&](int u, const Raw &r) {
        const int b = u / NI, i = u - b * NI;
        const int c0 = i * 64 + lane, c = min(c0, CPR - 1);
        const bool valid = c0 < CPR;
        h2_t xv[T][8];
        float xsum[T];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            xsum[t] = s_xsum[t * CPR + c];
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const u32x4_t v = s_x[(t * 2 + p) * CPR + c];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    // element copied out first: a bit cast of a vector
                    // element itself reads the vector's first element
                    const uint32_t e = v[q];
                    xv[t][4 * p + q] = __builtin_bit_cast(h2_t, e);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kGvRows; ++j) {
            h2_t cp[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                cp[2 * q] = code_pair_biased<0>(r.w[j][q]);
                cp[2 * q + 1] = code_pair_biased<1>(r.w[j][q]);
            }
            const float sf = valid ? bf16_to_f32(r.s[j]) : 0.f;
#pragma unroll
            for (int t = 0; t < T; ++t) {
                float p = 0.f;
#pragma unroll
                for (int q = 0; q < 8; ++q) p = __builtin_amdgcn_fdot2(cp[q], xv[t][q], p, false);
                // sum (1024 + q) x - 1152 sum x = sum (q - 128) x
                acc[j * T + t] = fmaf(sf, fmaf(-1152.f, xsum[t], p), acc[j * T + t]);
            }
        }
        if (i == NI - 1) {
            // row block done: reduce over the wave and store
            const float s = wave_transpose_sum<M>(acc, lane);
            constexpr int shift = M == 4 ? 4 : M == 8 ? 3 : 2;   // 6 - log2 M
            const int idx = lane >> shift;
            const int j = idx / T, t = idx - j * T;
            const int row = (gw + b * W) * kGvRows + j;
            if ((lane & ((1 << shift) - 1)) == 0 && idx < kGvRows * T && row < N)
                out[(size_t)t * N + row] = (uint16_t)f32_to_bf16(s);
#pragma unroll
            for (int q = 0; q < M; ++q) acc[q] = 0.f;
        }
    };

    // two explicit register sets, the next unit's loads in flight while the
    // current one is computed
    Raw r0, r1;
    load(0, r0);
    int u = 0;
    for (; u + 1 < U; u += 2) {
        load(u + 1, r1);
        compute(u, r0);
        if (u + 2 < U) load(u + 2, r0);
        compute(u + 1, r1);
    }
    if (u < U) compute(u, r0);
}

// Narrow matrices (few rows, long rows: the hyper-connection down projection
// [320, 10240]): four row blocks per wave would leave most of the chip idle,
// so a workgroup takes one row and its four waves split the row's chunks.
// Activations come straight from global memory (a few KB, read by every
// workgroup, so L2 hits) with the weights, converted in registers: no LDS
// staging and no barrier before the first product.  The four wave sums
// meet in LDS (added in wave order).
template <int T>
__global__ __launch_bounds__(kGvThreads) void int8_gemv_rowsplit_kernel(const uint16_t *__restrict__ x,
                                                                        const int32_t *__restrict__ wq,
                                                                        const uint16_t *__restrict__ wscale,
                                                                        int N, int K, int gshift,
                                                                        uint16_t *__restrict__ out)
{
    __shared__ float s_red[kGvThreads / 64][4];
    const int CPR = K >> 4;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = blockIdx.x;
    const int CPW = (CPR + 3) / 4;                  // chunks per wave
    const int cbeg = wave * CPW, cend = min(CPR, cbeg + CPW);
    const int NI = (CPW + 63) >> 6;
    const u32x4_t *wrow = reinterpret_cast<const u32x4_t *>(wq + (size_t)row * (K / 4));
    const uint16_t *srow = wscale + (size_t)row * (K >> gshift);
    auto chunk = [&](int i) { return min(cbeg + i * 64 + lane, CPR - 1); };
    struct Raw {
        u32x4_t w;
        u32x4_t xb[T][2];   // bf16 activations of the chunk
        uint16_t s;
    };
    auto load = [&](int i, Raw &r) {
        const int c = chunk(i);
        r.w = __builtin_nontemporal_load(wrow + c);
        r.s = srow[(16 * c) >> gshift];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const u32x4_t *xp = reinterpret_cast<const u32x4_t *>(x + (size_t)t * K) + 2 * c;
            r.xb[t][0] = xp[0];
            r.xb[t][1] = xp[1];
        }
    };

    constexpr int M = T == 1 ? 1 : T == 2 ? 2 : 4;   // T, padded to a power of two
    float acc[M];
#pragma unroll
    for (int t = 0; t < M; ++t) acc[t] = 0.f;
    auto compute = [&](int i, const Raw &r) {
        const bool valid = cbeg + i * 64 + lane < cend;
        h2_t cp[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            cp[2 * q] = code_pair<0>(r.w[q]);
            cp[2 * q + 1] = code_pair<1>(r.w[q]);
        }
        const float sf = valid ? bf16_to_f32(r.s) : 0.f;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            float p = 0.f;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const u32x4_t v = bf16x8_to_f16x8(r.xb[t][h]);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t e = v[q];   // element copied out before the bit cast
                    p = __builtin_amdgcn_fdot2(cp[4 * h + q], __builtin_bit_cast(h2_t, e), p, false);
                }
            }
            acc[t] = fmaf(sf, p, acc[t]);
        }
    };
    Raw r0, r1;
    load(0, r0);
    int i = 0;
    for (; i + 1 < NI; i += 2) {
        load(i + 1, r1);
        compute(i, r0);
        if (i + 2 < NI) load(i + 2, r0);
        compute(i + 1, r1);
    }
    if (i < NI) compute(i, r0);

    const float sum = wave_transpose_sum<M>(acc, lane);
    constexpr int shift = M == 1 ? 6 : M == 2 ? 5 : 4;
    const int t = lane >> shift;
    if ((lane & ((1 << shift) - 1)) == 0 && t < T) s_red[wave][t] = sum;
    __syncthreads();
    if (threadIdx.x < T) {
        const float v = ((s_red[0][threadIdx.x] + s_red[1][threadIdx.x]) + s_red[2][threadIdx.x]) +
                        s_red[3][threadIdx.x];
        out[(size_t)threadIdx.x * N + row] = (uint16_t)f32_to_bf16(v);
    }
}

// 5..16 tokens on wide matrices: the dot products go to the matrix cores,
// so the vector ALU work per weight byte (one permute and one packed add per
// two codes) no longer grows with the token count.  (Up to 4 tokens the
// dot-product GEMV is faster: its 1 KB-per-row loads keep DRAM pages open,
// while the matrix-core operand layout spreads a load over 16 rows.)  A wave owns 16 weight
// rows; per 64-input step each lane loads 16 codes (16 bytes) of row
// lane % 16 at offset 16 (lane / 16), and two v_mfma_f32_16x16x32_f16 take
// them as the B operand (column = weight row) against fp16 activations from
// LDS as the A operand (row = token, lane % 16; rows past T repeat the last
// token and are never stored).  Each lane's output column is its own weight
// row, so the group scale is applied per lane: a group's MFMA sums start
// from zero and are folded in with one FMA per output.  Weight loads run
// in two batches of four steps (named register sets), each batch's loads
// issued back to back so a row's 256 consecutive bytes are requested
// together.
constexpr int kMfRows = 16;

typedef float f32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kGvThreads) void int8_gemv_mfma_kernel(const uint16_t *__restrict__ x,
                                                                   const int32_t *__restrict__ wq,
                                                                   const uint16_t *__restrict__ wscale,
                                                                   int T, int N, int K, int gshift,
                                                                   uint16_t *__restrict__ out)
{
    // x as fp16 [T][K / 8 + 1] 16-byte units (one unit of padding per row so
    // the 16 token rows of a read fall in different banks)
    extern __shared__ u32x4_t s_x[];
    const int K8 = K >> 3, xs = K8 + 1;
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * (kGvThreads / 64) + (threadIdx.x >> 6);
    const int W = gridDim.x * (kGvThreads / 64);
    const int nrb = (N + kMfRows - 1) / kMfRows;
    const int steps = K >> 6;
    const int my_blocks = gw < nrb ? (nrb - gw + W - 1) / W : 0;
    const int U = my_blocks * steps;
    const int n = lane & 15, kq = lane >> 4;
    const size_t rstride = (size_t)K / 4;
    const int nsc = K >> gshift;

    // wave-uniform cursors (block b, step st) for the loads, which run up to
    // eight units ahead of the compute; past the last unit the loads repeat
    // it (a cache hit, never used)
    int lb = 0, lst = 0;
    auto lrow_of = [&](int b) { return min((gw + b * W) * kMfRows + n, N - 1); };
    int lrow = lrow_of(0);
    struct Raw {
        u32x4_t w;
        uint16_t s;
    };
    auto load_next = [&](Raw &r) {
        r.w = *(reinterpret_cast<const u32x4_t *>(wq + lrow * rstride) + 4 * lst + kq);
        r.s = wscale[(size_t)lrow * nsc + ((lst << 6) >> gshift)];
        if (lst + 1 < steps) {
            ++lst;
        } else if (lb + 1 < my_blocks) {
            lst = 0;
            lrow = lrow_of(++lb);
        }
    };
    Raw a0, a1, a2, a3, b0, b1, b2, b3;
    if (U > 0) {
        load_next(a0);
        load_next(a1);
        load_next(a2);
        load_next(a3);
        load_next(b0);
        load_next(b1);
        load_next(b2);
        load_next(b3);
    }
    for (int i = threadIdx.x; i < T * K8; i += kGvThreads) {
        const int t = i / K8, c = i - t * K8;
        s_x[t * xs + c] = bf16x8_to_f16x8(*reinterpret_cast<const u32x4_t *>(x + (size_t)t * K + 8 * c));
    }
    __syncthreads();
    if (U == 0) return;

    const int tr = min(n, T - 1);
    const u32x4_t *xrow = s_x + tr * xs + 2 * kq;
    const int gmask = (1 << (gshift - 6)) - 1;   // steps per scale group, minus one
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, tmp = {0.f, 0.f, 0.f, 0.f};
    int cb = 0, cst = 0;   // compute cursor

    auto compute = [&](const Raw &r) {
        f16x8_t bq[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const h2_t p0 = code_pair<0>(r.w[2 * h]), p1 = code_pair<1>(r.w[2 * h]);
            const h2_t p2 = code_pair<0>(r.w[2 * h + 1]), p3 = code_pair<1>(r.w[2 * h + 1]);
            bq[h] = f16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        }
        const f16x8_t a0f = __builtin_bit_cast(f16x8_t, xrow[8 * cst]);
        const f16x8_t a1f = __builtin_bit_cast(f16x8_t, xrow[8 * cst + 1]);
        if ((cst & gmask) == 0) {
            const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
            tmp = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0f, bq[0], z, 0, 0, 0);
        } else {
            tmp = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0f, bq[0], tmp, 0, 0, 0);
        }
        tmp = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1f, bq[1], tmp, 0, 0, 0);
        if ((cst & gmask) == gmask) {
            const float sf = bf16_to_f32(r.s);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = fmaf(sf, tmp[j], acc[j]);
        }
        if (cst + 1 < steps) {
            ++cst;
        } else {
            // row block done: lane holds tokens 4 (lane / 16) + j of row n
            const int row = (gw + cb * W) * kMfRows + n;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 4 * kq + j;
                if (t < T && row < N) out[(size_t)t * N + row] = (uint16_t)f32_to_bf16(acc[j]);
                acc[j] = 0.f;
            }
            cst = 0;
            ++cb;
        }
    };

    // two batches of four units: a batch is computed while the other is in
    // flight, and its refill issues four consecutive steps of the same rows
    // back to back (256 contiguous bytes per row)
    for (int u = 0; u < U; u += 8) {
        compute(a0);
        if (u + 1 < U) compute(a1);
        if (u + 2 < U) compute(a2);
        if (u + 3 < U) compute(a3);
        load_next(a0);
        load_next(a1);
        load_next(a2);
        load_next(a3);
        if (u + 4 < U) compute(b0);
        if (u + 5 < U) compute(b1);
        if (u + 6 < U) compute(b2);
        if (u + 7 < U) compute(b3);
        load_next(b0);
        load_next(b1);
        load_next(b2);
        load_next(b3);
    }
}

// ---------------------------------------------------------------------------
// GEMM (MFMA)
// ---------------------------------------------------------------------------
constexpr int kGmM = 128;           // tokens per tile
constexpr int kGmN = 128;           // weight rows per tile (4 waves x 32)
constexpr int kGmKS = 64;           // K per stage
constexpr int kGmLds = kGmKS + 8;   // padded LDS row (fp16 elements)
constexpr int kGmThreads = 256;
constexpr int kGmCs = kGmN + 8;     // padded LDS row of the epilogue (fp32 words)
constexpr int kGmScGroups = 64;     // scale groups of the tile's rows staged in LDS at a time
constexpr int kGmScRegs = 8;        // of those, per thread, loaded with the prologue's loads
constexpr int kSumThreads = 64;     // split-K sum: four outputs per thread

struct Int8GemmArgs {
    const uint16_t *x;        // bf16 [T][K]
    const int32_t *wq;        // [N][K/4]
    const uint16_t *ws;       // bf16 [N][K/G]
    uint16_t *out;            // bf16 [T][N] (one K split)
    float *part;              // fp32 [ksplit][pstride] (several K splits)
    size_t pstride;           // T * N rounded up to a multiple of 4
    int T, N, K, gshift;
    int mtiles, ntiles, ksplit, kslice;
};

// Tile: 128 tokens x 128 weight rows, K range [k0, k0 + len).  Wave w owns
// all tokens x weight rows [32 w, +32) of the tile as up to four 32 x 32
// MFMA tiles.  Within a 64-wide K stage, MFMA step j uses on lanes 0-31
// inputs 8 j .. 8 j + 7 and on lanes 32-63 inputs 32 + 8 j .., for both
// operands, so each lane reads 32 contiguous bytes of its weight row per
// stage.  GS = G / 64 stages make up one scale group.
template <int GS>
__global__ __launch_bounds__(kGmThreads, 2) void int8_gemm_kernel(Int8GemmArgs g)
{
    constexpr int D = 2;   // register sets of loads in flight
    __shared__ __align__(16) _Float16 s_a[2][kGmM * kGmLds];

    // ---- tile (XCD-aware: each XCD takes a contiguous range of tiles, the
    // weight-row tiles of one token tile and K split back to back, so the
    // token tile is re-read from that XCD's L2) ----
    const int per = gridDim.x >> 3;
    const int tile = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (tile >= g.mtiles * g.ntiles * g.ksplit) return;
    const int nt_i = tile % g.ntiles, rest = tile / g.ntiles;
    const int mt_i = rest % g.mtiles, split = rest / g.mtiles;
    const int m0 = mt_i * kGmM, n0 = nt_i * kGmN;
    const int rows = min(kGmM, g.T - m0);
    const int k0 = split * g.kslice, len = min(g.kslice, g.K - k0);
    const int nsteps = len / kGmKS;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;

    // ---- activation staging: thread -> 16-byte chunk c8 of rows r8 + 32 o;
    // rows past T read row 0 of the tile (never stored) ----
    const int c8 = tid & 7, r8 = tid >> 3;
    const uint16_t *asrc[4];
#pragma unroll
    for (int o = 0; o < 4; ++o) {
        const int row = r8 + 32 * o;
        asrc[o] = g.x + (size_t)(m0 + (row < rows ? row : 0)) * g.K + k0 + 8 * c8;
    }
    u32x4_t ra[D][4];

    // ---- weights: lane -> row n0 + 32 wave + lane % 32 (clamped to N - 1),
    // bytes [32 half, +32) of each stage ----
    const int n = n0 + 32 * wave + (lane & 31);
    const int nrow = min(n, g.N - 1);
    const u32x4_t *bsrc = reinterpret_cast<const u32x4_t *>(g.wq + (size_t)nrow * (g.K / 4) + k0 / 4) + 2 * half;
    u32x4_t rb[D][2];

    // ---- scales: the tile's rows x up to kGmScGroups groups in LDS, [group]
    // [row], so that no scale value is carried in registers from one stage
    // to the next (a loop-carried load result ends up copied at the loop's
    // back edge, which waits for every load in flight) ----
    __shared__ uint16_t s_sc[kGmScGroups * kGmN];
    const int ngroups = len >> g.gshift;
    const uint16_t *sbase = g.ws + (k0 >> g.gshift);
    const size_t spitch = (size_t)(g.K >> g.gshift);
    auto scale_src = [&](int i, int g0) {   // element i = row + kGmN * group of the chunk at g0
        return sbase + (size_t)min(n0 + (i & (kGmN - 1)), g.N - 1) * spitch + g0 + i / kGmN;
    };
    auto load_scales_sync = [&](int g0) {
        const int cnt = min(kGmScGroups, ngroups - g0) * kGmN;
        for (int i = tid; i < cnt; i += kGmThreads) s_sc[i] = *scale_src(i, g0);
    };

    f32x16_t acc[4], tmp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][q] = 0.f;
    const int mtiles = (rows + 31) / 32;

    auto kloop = [&](auto ma_c) {
        constexpr int MA = decltype(ma_c)::value;
        auto load_a = [&](int s, int p) {
#pragma unroll
            for (int o = 0; o < MA; ++o) ra[p][o] = *reinterpret_cast<const u32x4_t *>(asrc[o] + s * kGmKS);
        };
        auto store_a = [&](int buf, int p) {
#pragma unroll
            for (int o = 0; o < MA; ++o)
                *reinterpret_cast<u32x4_t *>(s_a[buf] + (r8 + 32 * o) * kGmLds + 8 * c8) = bf16x8_to_f16x8(ra[p][o]);
        };
        auto load_b = [&](int s, int p) {
            rb[p][0] = bsrc[4 * s];
            rb[p][1] = bsrc[4 * s + 1];
        };

        // stage s (register set q = s % D, LDS buffer s % 2): stage s+1's
        // activations are stored, stages s+1+D (activations) and s+D
        // (weights) are loaded
        auto stage = [&](int s, auto qc) {
            constexpr int q = decltype(qc)::value, q1 = (q + 1) % D;
            const int grp = (s * kGmKS) >> g.gshift;   // scale group within the K range
            if (s > 0 && (s * kGmKS) % (kGmScGroups << g.gshift) == 0) {
                // the next chunk of scales (every wave is past the previous
                // stage's barrier, so none still reads the old chunk)
                load_scales_sync(grp);
                __syncthreads();
            }
            if (s + 1 < nsteps) store_a((q + 1) & 1, q1);
            const u32x4_t w0 = rb[q][0], w1 = rb[q][1];
            load_a(min(s + 1 + D, nsteps - 1), q1);
            load_b(min(s + D, nsteps - 1), q);
            const bool gfirst = (q % GS) == 0, glast = (q % GS) == GS - 1;
            const _Float16 *A = s_a[q & 1] + (lane & 31) * kGmLds + 32 * half;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t wa = j < 2 ? w0[2 * j] : w1[2 * j - 4];
                const uint32_t wb = j < 2 ? w0[2 * j + 1] : w1[2 * j - 3];
                const h2_t p0 = code_pair<0>(wa), p1 = code_pair<1>(wa);
                const h2_t p2 = code_pair<0>(wb), p3 = code_pair<1>(wb);
                const f16x8_t bf = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
                for (int mt = 0; mt < MA; ++mt) {
                    const f16x8_t af = *reinterpret_cast<const f16x8_t *>(A + 32 * mt * kGmLds + 8 * j);
                    if (gfirst && j == 0) {
                        const f32x16_t z = {};
                        tmp[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bf, z, 0, 0, 0);
                    } else {
                        tmp[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bf, tmp[mt], 0, 0, 0);
                    }
                }
            }
            if (glast) {
                const float sf = bf16_to_f32(s_sc[(grp % kGmScGroups) * kGmN + 32 * wave + (lane & 31)]);
#pragma unroll
                for (int mt = 0; mt < MA; ++mt)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[mt][v] = fmaf(sf, tmp[mt][v], acc[mt][v]);
            }
            __syncthreads();
        };

        // prologue: stage 0's activations in LDS, stages 1 .. D in
        // registers, weights of stages 0 .. D-1 in flight, the first chunk of
        // scales in LDS (its first kGmScRegs * kGmThreads values loaded
        // alongside, the rest, if any, after)
        const int sc0 = min(kGmScGroups, ngroups) * kGmN;
        uint32_t sv[kGmScRegs];
        load_a(0, 0);
        load_b(0, 0);
#pragma unroll
        for (int u = 0; u < kGmScRegs; ++u) {
            const int i = tid + kGmThreads * u;
            sv[u] = i < sc0 ? *scale_src(i, 0) : 0u;
        }
#pragma unroll
        for (int j = 1; j < D; ++j) load_b(min(j, nsteps - 1), j);
#pragma unroll
        for (int j = 1; j < D; ++j) load_a(min(j, nsteps - 1), j);
        store_a(0, 0);
        load_a(min(D, nsteps - 1), 0);
#pragma unroll
        for (int u = 0; u < kGmScRegs; ++u) {
            const int i = tid + kGmThreads * u;
            if (i < sc0) s_sc[i] = (uint16_t)sv[u];
        }
        for (int i = tid + kGmThreads * kGmScRegs; i < sc0; i += kGmThreads) s_sc[i] = *scale_src(i, 0);
        __syncthreads();
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        int s = 0;
        for (; s + 1 < nsteps; s += 2) {
            stage(s, I0{});
            stage(s + 1, I1{});
        }
        if (s < nsteps) stage(s, I0{});
    };
    switch (mtiles) {
    case 1: kloop(std::integral_constant<int, 1>{}); break;
    case 2: kloop(std::integral_constant<int, 2>{}); break;
    case 3: kloop(std::integral_constant<int, 3>{}); break;
    default: kloop(std::integral_constant<int, 4>{}); break;
    }

    // ---- epilogue: the accumulators pass through LDS, 64 tokens at a time
    // in fp32 (rows padded to kGmCs words, so the two half-waves' rows fall
    // in different banks); then each thread writes four consecutive outputs
    // of one token: a 16-byte partial store or an 8-byte bf16 store, whole
    // rows of the tile coalesced ----
    float *s_c = reinterpret_cast<float *>(&s_a[0][0]);
    static_assert(64 * kGmCs * sizeof(float) <= sizeof(s_a), "64 fp32 token rows fit the activation buffers");
    const bool vec = (g.N & 3) == 0;   // every 4-column group starts 8-byte aligned (bf16) / 16-byte (fp32)
    float *part = g.part + (size_t)split * g.pstride;
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
        if (64 * hp >= rows) break;   // uniform over the workgroup
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (2 * hp + u >= mtiles) continue;
#pragma unroll
            for (int j = 0; j < 16; ++j)
                s_c[(32 * u + 8 * (j >> 2) + 4 * half + (j & 3)) * kGmCs + 32 * wave + (lane & 31)] =
                    acc[2 * hp + u][j];
        }
        __syncthreads();
        for (int it = tid; it < 64 * (kGmN / 4); it += kGmThreads) {
            const int r = it / (kGmN / 4), c4 = 4 * (it % (kGmN / 4));
            const int m = 64 * hp + r, nn = n0 + c4;
            if (m >= rows || nn >= g.N) continue;
            const float4 v = *reinterpret_cast<const float4 *>(s_c + r * kGmCs + c4);
            const size_t o = (size_t)(m0 + m) * g.N + nn;
            if (vec) {
                if (g.ksplit == 1)
                    *reinterpret_cast<uint2 *>(g.out + o) =
                        make_uint2(f32x2_to_bf16x2(v.x, v.y), f32x2_to_bf16x2(v.z, v.w));
                else
                    *reinterpret_cast<float4 *>(part + o) = v;
            } else {
                const float e4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (nn + e >= g.N) break;
                    if (g.ksplit == 1) g.out[o + e] = (uint16_t)f32_to_bf16(e4[e]);
                    else part[o + e] = e4[e];
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// GEMM over a short K range (NS <= kGoMaxSteps stages of 64 inputs): every
// load of the tile is issued at the start (weights into registers, the
// activation tile into registers and then, as fp16, into LDS), so a
// workgroup waits for memory once instead of once per stage, and the stage
// loop is unrolled with no value carried from one iteration to the next.
// Tile: 128 tokens x 256 weight rows, wave w all tokens x rows [32 w, +32),
// the same MFMA step layout and per-group fold as int8_gemm_kernel.
// ---------------------------------------------------------------------------
constexpr int kGoWaves = 8;
constexpr int kGoThreads = kGoWaves * 64;
constexpr int kGoN = 32 * kGoWaves;    // weight rows per tile
constexpr int kGoMaxSteps = 5;         // K <= 320
constexpr int kGoCs = kGoN + 8;        // padded epilogue row (fp32 words)

template <int NS>
constexpr size_t go_lds_bytes()
{
    const size_t x = (size_t)kGmM * (NS * kGmKS + 8) * 2, c = (size_t)64 * kGoCs * 4;
    return x > c ? x : c;
}

template <int NS, int GS>
__global__ __launch_bounds__(kGoThreads, 1) void int8_gemm_short_kernel(Int8GemmArgs g)
{
    constexpr int LR = NS * kGmKS + 8;    // padded activation row (fp16)
    constexpr int CH = NS * 8;            // 16-byte chunks per activation row
    constexpr int XPER = (kGmM * CH + kGoThreads - 1) / kGoThreads;
    constexpr int NG = NS / GS;           // scale groups
    constexpr int SPER = (NG * kGoN + kGoThreads - 1) / kGoThreads;
    static_assert(NS % GS == 0, "whole groups");
    __shared__ __align__(16) unsigned char s_raw[go_lds_bytes<NS>()];
    __shared__ uint16_t s_sc[NG * kGoN];   // [group][row]
    _Float16 *s_x = reinterpret_cast<_Float16 *>(s_raw);

    // ---- tile (XCD-aware as in int8_gemm_kernel) ----
    const int per = gridDim.x >> 3;
    const int tile = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (tile >= g.mtiles * g.ntiles) return;
    const int nt_i = tile % g.ntiles, mt_i = tile / g.ntiles;
    const int m0 = mt_i * kGmM, n0 = nt_i * kGoN;
    const int rows = min(kGmM, g.T - m0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;

    // ---- every load at once: weights (lane -> row n0 + 32 wave + lane % 32,
    // clamped to N - 1; bytes [32 half, +32) of each stage), the activation
    // chunks (rows past T read row 0 of the tile, never stored), the scales ----
    const int n = n0 + 32 * wave + (lane & 31);
    const u32x4_t *bsrc = reinterpret_cast<const u32x4_t *>(g.wq + (size_t)min(n, g.N - 1) * (g.K / 4)) + 2 * half;
    u32x4_t rb[NS][2];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        rb[s][0] = bsrc[4 * s];
        rb[s][1] = bsrc[4 * s + 1];
    }
    u32x4_t rx[XPER];
#pragma unroll
    for (int u = 0; u < XPER; ++u) {
        const int c = min(tid + kGoThreads * u, kGmM * CH - 1), r = c / CH, col = c % CH;
        rx[u] = *reinterpret_cast<const u32x4_t *>(g.x + (size_t)(m0 + (r < rows ? r : 0)) * g.K + 8 * col);
    }
    const int gpr = g.K >> g.gshift;   // groups per weight row
    uint32_t rsc[SPER];
#pragma unroll
    for (int u = 0; u < SPER; ++u) {
        const int i = min(tid + kGoThreads * u, NG * kGoN - 1);
        rsc[u] = g.ws[(size_t)min(n0 + i % kGoN, g.N - 1) * gpr + i / kGoN];
    }
#pragma unroll
    for (int u = 0; u < XPER; ++u) {
        const int c = tid + kGoThreads * u;
        if (c < kGmM * CH)
            *reinterpret_cast<u32x4_t *>(s_x + (c / CH) * LR + 8 * (c % CH)) = bf16x8_to_f16x8(rx[u]);
    }
#pragma unroll
    for (int u = 0; u < SPER; ++u) {
        const int i = tid + kGoThreads * u;
        if (i < NG * kGoN) s_sc[i] = (uint16_t)rsc[u];
    }
    __syncthreads();

    f32x16_t acc[4], tmp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][q] = 0.f;
    const int mtiles = (rows + 31) / 32;

    auto compute = [&](auto ma_c) {
        constexpr int MA = decltype(ma_c)::value;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const bool gfirst = s % GS == 0, glast = s % GS == GS - 1;
            const u32x4_t w0 = rb[s][0], w1 = rb[s][1];
            const _Float16 *A = s_x + (lane & 31) * LR + kGmKS * s + 32 * half;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t wa = j < 2 ? w0[2 * j] : w1[2 * j - 4];
                const uint32_t wb = j < 2 ? w0[2 * j + 1] : w1[2 * j - 3];
                const h2_t p0 = code_pair<0>(wa), p1 = code_pair<1>(wa);
                const h2_t p2 = code_pair<0>(wb), p3 = code_pair<1>(wb);
                const f16x8_t bf = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
                for (int mt = 0; mt < MA; ++mt) {
                    const f16x8_t af = *reinterpret_cast<const f16x8_t *>(A + 32 * mt * LR + 8 * j);
                    if (gfirst && j == 0) {
                        const f32x16_t z = {};
                        tmp[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bf, z, 0, 0, 0);
                    } else {
                        tmp[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bf, tmp[mt], 0, 0, 0);
                    }
                }
            }
            if (glast) {
                const float sf = bf16_to_f32(s_sc[(s / GS) * kGoN + 32 * wave + (lane & 31)]);
#pragma unroll
                for (int mt = 0; mt < MA; ++mt)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[mt][v] = fmaf(sf, tmp[mt][v], acc[mt][v]);
            }
        }
    };
    switch (mtiles) {
    case 1: compute(std::integral_constant<int, 1>{}); break;
    case 2: compute(std::integral_constant<int, 2>{}); break;
    case 3: compute(std::integral_constant<int, 3>{}); break;
    default: compute(std::integral_constant<int, 4>{}); break;
    }

    // ---- epilogue through LDS, 64 tokens at a time (as in int8_gemm_kernel) ----
    __syncthreads();   // every wave is done reading the activations
    float *s_c = reinterpret_cast<float *>(s_raw);
    const bool vec = (g.N & 3) == 0;
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
        if (64 * hp >= rows) break;   // uniform over the workgroup
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (2 * hp + u >= mtiles) continue;
#pragma unroll
            for (int j = 0; j < 16; ++j)
                s_c[(32 * u + 8 * (j >> 2) + 4 * half + (j & 3)) * kGoCs + 32 * wave + (lane & 31)] =
                    acc[2 * hp + u][j];
        }
        __syncthreads();
        for (int it = tid; it < 64 * (kGoN / 4); it += kGoThreads) {
            const int r = it / (kGoN / 4), c4 = 4 * (it % (kGoN / 4));
            const int m = 64 * hp + r, nn = n0 + c4;
            if (m >= rows || nn >= g.N) continue;
            const float4 v = *reinterpret_cast<const float4 *>(s_c + r * kGoCs + c4);
            const size_t o = (size_t)(m0 + m) * g.N + nn;
            if (vec) {
                *reinterpret_cast<uint2 *>(g.out + o) =
                    make_uint2(f32x2_to_bf16x2(v.x, v.y), f32x2_to_bf16x2(v.z, v.w));
            } else {
                const float e4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (nn + e >= g.N) break;
                    g.out[o + e] = (uint16_t)f32_to_bf16(e4[e]);
                }
            }
        }
        __syncthreads();
    }
}

// out[i] = bf16( sum_s part[s][i] ), splits in order; 4 outputs per thread,
// every split's load issued before the first add (pstride is a multiple of
// 4, so every 16-byte load is aligned).
__global__ __launch_bounds__(kSumThreads) void int8_splitk_sum_kernel(const float *__restrict__ part, size_t count,
                                                                      size_t pstride, int ksplit,
                                                                      uint16_t *__restrict__ out)
{
    const size_t i = (blockIdx.x * (size_t)blockDim.x + threadIdx.x) * 4;
    if (i >= count) return;
    if (i + 4 <= count) {
        float4 v[kInt8MaxSplitK];
#pragma unroll
        for (int s = 0; s < kInt8MaxSplitK; ++s)
            if (s < ksplit) v[s] = *reinterpret_cast<const float4 *>(part + (size_t)s * pstride + i);
        float4 a = v[0];
#pragma unroll
        for (int s = 1; s < kInt8MaxSplitK; ++s)
            if (s < ksplit) {
                a.x += v[s].x;
                a.y += v[s].y;
                a.z += v[s].z;
                a.w += v[s].w;
            }
        const uint32_t lo = f32x2_to_bf16x2(a.x, a.y);
        const uint32_t hi = f32x2_to_bf16x2(a.z, a.w);
        if ((reinterpret_cast<uintptr_t>(out + i) & 7) == 0) {
            *reinterpret_cast<uint2 *>(out + i) = make_uint2(lo, hi);
        } else {
            out[i] = (uint16_t)lo;
            out[i + 1] = (uint16_t)(lo >> 16);
            out[i + 2] = (uint16_t)hi;
            out[i + 3] = (uint16_t)(hi >> 16);
        }
        return;
    }
    for (size_t e = i; e < count; ++e) {
        float a = part[e];
        for (int s = 1; s < ksplit; ++s) a += part[(size_t)s * pstride + e];
        out[e] = (uint16_t)f32_to_bf16(a);
    }
}

}  // namespace

// Launch plan of one call (shared by the workspace query and the launch).
Int8Plan int8_plan(int T, int N, int K, int G)
{
    Int8Plan p{};
    // narrow: fewer row blocks of four than waves of the persistent grid
    const bool narrow = (N + 3) / 4 < kInt8GemvMaxBlocks && K >= 1024;
    if (T >= 1 && T <= kInt8GemvMaxTokens && narrow) {
        p.gemv = p.rowsplit = true;   // one row per workgroup, K split over its waves
    } else if (T >= 1 && T <= kInt8GemvMaxTokens &&
               (size_t)T * K * 2 + (size_t)T * (K / 16) * 4 <= kInt8GemvMaxLds) {
        p.gemv = true;                // dot-product GEMV, four rows per wave
    } else if (T > kInt8GemvMaxTokens && T <= kInt8MfmaGemvMaxTokens && !narrow &&
               (size_t)T * (K / 8 + 1) * 16 <= kInt8GemvMaxLds) {
        p.gemv = p.mfma = true;       // matrix-core GEMV, 16 rows per wave
    }
    if (p.gemv || T == 0) return p;
    p.mtiles = (T + kGmM - 1) / kGmM;
    if (K <= kGoMaxSteps * kGmKS) {   // the whole K range at once, no split
        p.short_k = true;
        p.ntiles = (N + kGoN - 1) / kGoN;
        p.ksplit = 1;
        p.kslice = K;
        p.pstride = ((size_t)T * N + 3) / 4 * 4;
        p.part_bytes = 0;
        return p;
    }
    p.ntiles = (N + kGmN - 1) / kGmN;
    const int unit = G > kGmKS ? G : kGmKS;   // a K split is whole groups and whole stages
    const int units = K / unit;
    const long tiles = (long)p.mtiles * p.ntiles;
    int ks = 1;
    if (tiles < kInt8GemmTargetTiles) {
        ks = (int)((kInt8GemmTargetTiles + tiles - 1) / tiles);
        const int max_split = units / (kInt8MinSplitK / unit > 0 ? kInt8MinSplitK / unit : 1);
        ks = ks < max_split ? ks : max_split;
        ks = ks < kInt8MaxSplitK ? ks : kInt8MaxSplitK;
        ks = ks > 1 ? ks : 1;
    }
    const int per = (units + ks - 1) / ks;
    p.kslice = per * unit;
    p.ksplit = (K + p.kslice - 1) / p.kslice;
    p.pstride = ((size_t)T * N + 3) / 4 * 4;
    p.part_bytes = p.ksplit > 1 ? (size_t)p.ksplit * p.pstride * 4 : 0;
    return p;
}

hipError_t launch_int8_linear(const uint16_t *x, const int32_t *wq, const uint16_t *ws, int T, int N,
                              int K, int G, uint16_t *out, void *workspace, hipStream_t st)
{
    const Int8Plan p = int8_plan(T, N, K, G);
    const int gshift = G == 64 ? 6 : 7;
    if (p.gemv && p.rowsplit) {
        switch (T) {
        case 1: int8_gemv_rowsplit_kernel<1><<<N, kGvThreads, 0, st>>>(x, wq, ws, N, K, gshift, out); break;
        case 2: int8_gemv_rowsplit_kernel<2><<<N, kGvThreads, 0, st>>>(x, wq, ws, N, K, gshift, out); break;
        case 3: int8_gemv_rowsplit_kernel<3><<<N, kGvThreads, 0, st>>>(x, wq, ws, N, K, gshift, out); break;
        default: int8_gemv_rowsplit_kernel<4><<<N, kGvThreads, 0, st>>>(x, wq, ws, N, K, gshift, out); break;
        }
        return hipGetLastError();
    }
    if (p.gemv && p.mfma) {
        const int nrb = (N + kMfRows - 1) / kMfRows;
        const int wpb = kGvThreads / 64;
        int grid = (nrb + wpb - 1) / wpb;
        grid = grid < kInt8GemvMaxBlocks ? grid : kInt8GemvMaxBlocks;
        const size_t lds = (size_t)T * (K / 8 + 1) * 16;
        int8_gemv_mfma_kernel<<<grid, kGvThreads, lds, st>>>(x, wq, ws, T, N, K, gshift, out);
        return hipGetLastError();
    }
    if (p.gemv) {
        const int nrb = (N + kGvRows - 1) / kGvRows;
        const int wpb = kGvThreads / 64;
        int grid = (nrb + wpb - 1) / wpb;
        grid = grid < kInt8GemvMaxBlocks ? grid : kInt8GemvMaxBlocks;
        const size_t lds = (size_t)T * K * 2 + (size_t)T * (K / 16) * 4;
        switch (T) {
        case 1: int8_gemv_kernel<1><<<grid, kGvThreads, lds, st>>>(x, wq, ws, N, K, gshift, out); break;
        case 2: int8_gemv_kernel<2><<<grid, kGvThreads, lds, st>>>(x, wq, ws, N, K, gshift, out); break;
        case 3: int8_gemv_kernel<3><<<grid, kGvThreads, lds, st>>>(x, wq, ws, N, K, gshift, out); break;
        default: int8_gemv_kernel<4><<<grid, kGvThreads, lds, st>>>(x, wq, ws, N, K, gshift, out); break;
        }
        return hipGetLastError();
    }
    Int8GemmArgs a{};
    a.x = x;
    a.wq = wq;
    a.ws = ws;
    a.out = out;
    a.part = static_cast<float *>(workspace);
    a.T = T;
    a.N = N;
    a.K = K;
    a.gshift = gshift;
    a.mtiles = p.mtiles;
    a.ntiles = p.ntiles;
    a.ksplit = p.ksplit;
    a.kslice = p.kslice;
    a.pstride = p.pstride;
    const long tiles = (long)p.mtiles * p.ntiles * p.ksplit;
    const int grid = (int)((tiles + 7) / 8 * 8);
    if (p.short_k) {
        const int ns = K / kGmKS;
        if (G == 64) {
            switch (ns) {
            case 1: int8_gemm_short_kernel<1, 1><<<grid, kGoThreads, 0, st>>>(a); break;
            case 2: int8_gemm_short_kernel<2, 1><<<grid, kGoThreads, 0, st>>>(a); break;
            case 3: int8_gemm_short_kernel<3, 1><<<grid, kGoThreads, 0, st>>>(a); break;
            case 4: int8_gemm_short_kernel<4, 1><<<grid, kGoThreads, 0, st>>>(a); break;
            default: int8_gemm_short_kernel<5, 1><<<grid, kGoThreads, 0, st>>>(a); break;
            }
        } else {
            if (ns == 2) int8_gemm_short_kernel<2, 2><<<grid, kGoThreads, 0, st>>>(a);
            else int8_gemm_short_kernel<4, 2><<<grid, kGoThreads, 0, st>>>(a);
        }
        return hipGetLastError();
    }
    if (G == 64) int8_gemm_kernel<1><<<grid, kGmThreads, 0, st>>>(a);
    else int8_gemm_kernel<2><<<grid, kGmThreads, 0, st>>>(a);
    if (p.ksplit > 1) {
        const size_t count = (size_t)T * N;
        const size_t threads = (count + 3) / 4;
        int8_splitk_sum_kernel<<<(unsigned)((threads + kSumThreads - 1) / kSumThreads), kSumThreads, 0, st>>>(
            a.part, count, p.pstride, p.ksplit, out);
    }
    return hipGetLastError();
}

}  // namespace moe
