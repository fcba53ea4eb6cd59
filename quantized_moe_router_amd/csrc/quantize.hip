// Load-time INT4 quantizer: bf16 weights -> the path's packed INT4 codes and
// bf16 scales.  Method ("Running 125B MoE on Three 3090s - vLLM Optimization
// Edition", section 7): round to nearest, group 128, symmetric, with a
// per-group search for the clip that gives the smallest squared error.
//
// Per group of G inputs of one row (G = 128, the pages' choice, or 64 for the
// group-64 variant of the experts):
//   amax = max |w|;  for j = 0..19: c_j = 1 - j/40 (1 down to 0.525),
//   s_j = bf16(fp32(amax * fp32(c_j / 7))) (the clipped magnitude maps to the
//   largest positive code 7), q = nearest integer to w / s_j with ties to
//   even, clamped to [-8, 7], err_j = sum (w - q s_j)^2 in fp32 in index
//   order; the first smallest err_j wins.  Scales below 2^-126 are not
//   candidates; a group with none (all zeros) gets scale 0 and codes 0.
//
// gfx950 design: one thread per group (the 20 x 128 candidate evaluations
// are compute-bound, so the group's 256 bytes are read once into registers
// and every candidate runs from them; the error sums keep the fixed index
// order).  The nearest code comes from w * (1/s): for bf16 w and s a quotient
// that is not an exact half-integer lies at least 1/512 from one, far beyond
// the reciprocal's error, and an exact tie is recognised exactly as
// |w - q s| == s / 2 (w - q s is exact in fp32) and moved to the even code
// when the codes are written.
#include "common.h"

namespace moe {

constexpr int kQClips = 20;
constexpr int kQThreads = 256;

__device__ __forceinline__ float bf16_bits_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Nearest code in [-8, 7] to x / s, ties to even.  In the candidate search
// the tie direction does not matter (either neighbour of an exact tie leaves
// a residual of +-s/2, the same square), so only the written codes take the
// exact tie test.
__device__ __forceinline__ float code_even(float x, float s, float rs)
{
    float q = rintf(x * rs);
    const float d = fmaf(-q, s, x);          // exact
    const float h = q * 0.5f;
    if (fabsf(d) == 0.5f * s && h != rintf(h)) q += d > 0.f ? 1.f : -1.f;
    return __builtin_amdgcn_fmed3f(q, -8.f, 7.f);
}

template <int kQGroup>
__global__ __launch_bounds__(kQThreads, 2) void quantize_int4_kernel(const uint16_t *__restrict__ w,
                                                                  int rows, int K,
                                                                  int32_t *__restrict__ packed,
                                                                  uint16_t *__restrict__ scales)
{
    const int ng = K / kQGroup;
    const long gid = (long)blockIdx.x * kQThreads + threadIdx.x;
    if (gid >= (long)rows * ng) return;
    const long r = gid / ng, g = gid % ng;
    const uint4 *src = reinterpret_cast<const uint4 *>(w + r * K + g * kQGroup);
    uint32_t v[kQGroup / 2];   // bf16 pairs, element 2i in the low half
#pragma unroll
    for (int c = 0; c < kQGroup / 8; ++c) {
        const uint4 x = src[c];
        v[4 * c] = x.x; v[4 * c + 1] = x.y; v[4 * c + 2] = x.z; v[4 * c + 3] = x.w;
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < kQGroup / 2; ++i) {
        amax = fmaxf(amax, fabsf(bf16_bits_f32(v[i] & 0xFFFFu)));
        amax = fmaxf(amax, fabsf(bf16_bits_f32(v[i] >> 16)));
    }
    float best_err = __builtin_inff();
    uint32_t best_s = 0;
#pragma unroll 1
    for (int j = 0; j < kQClips; ++j) {
        const float kj = (float)((1.0 - j / 40.0) / 7.0);
        const uint32_t sb = f32_to_bf16(amax * kj);
        const float s = bf16_bits_f32(sb);
        if (!(s >= 1.17549435e-38f)) continue;
        const float rs = 1.f / s;
        float err = 0.f;
#pragma unroll
        for (int i = 0; i < kQGroup; ++i) {
            const float x = bf16_bits_f32((i & 1) ? (v[i >> 1] >> 16) : (v[i >> 1] & 0xFFFFu));
            const float q = __builtin_amdgcn_fmed3f(rintf(x * rs), -8.f, 7.f);
            const float d = fmaf(-q, s, x);          // exact
            err = __fadd_rn(err, __fmul_rn(d, d));   // fixed order, no contraction
        }
        if (err < best_err) {
            best_err = err;
            best_s = sb;
        }
    }
    uint32_t words[kQGroup / 8];
    if (best_err == __builtin_inff()) {
#pragma unroll
        for (int c = 0; c < kQGroup / 8; ++c) words[c] = 0x88888888u;   // codes 0
        best_s = 0;
    } else {
        const float s = bf16_bits_f32(best_s), rs = 1.f / s;
#pragma unroll
        for (int c = 0; c < kQGroup / 8; ++c) {
            uint32_t wd = 0;
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const int i = 8 * c + b;
                const float x = bf16_bits_f32((i & 1) ? (v[i >> 1] >> 16) : (v[i >> 1] & 0xFFFFu));
                const int q = (int)code_even(x, s, rs);
                wd |= (uint32_t)(q + 8) << (4 * b);
            }
            words[c] = wd;
        }
    }
    uint4 *dst = reinterpret_cast<uint4 *>(packed + r * (K / 8) + g * (kQGroup / 8));
#pragma unroll
    for (int c = 0; c < kQGroup / 32; ++c)
        dst[c] = make_uint4(words[4 * c], words[4 * c + 1], words[4 * c + 2], words[4 * c + 3]);
    scales[gid] = (uint16_t)best_s;
}

hipError_t launch_quantize_int4(const uint16_t *w, int rows, int K, int group, int32_t *packed,
                                uint16_t *scales, hipStream_t st)
{
    const long groups = (long)rows * (K / group);
    if (groups == 0) return hipSuccess;
    const unsigned grid = (unsigned)((groups + kQThreads - 1) / kQThreads);
    if (group == 64) quantize_int4_kernel<64><<<grid, kQThreads, 0, st>>>(w, rows, K, packed, scales);
    else quantize_int4_kernel<128><<<grid, kQThreads, 0, st>>>(w, rows, K, packed, scales);
    return hipGetLastError();
}

}  // namespace moe
