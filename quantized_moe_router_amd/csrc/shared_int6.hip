// Shared-expert gate logit for the many-token path (one wave per token); the
// shared expert's gate/up and down projections run on the grouped-GEMM
// kernels (dense over all tokens), and in decode it rides in the decode
// kernels.  Always-on shared expert with INT6 group-64 weights.
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

hipError_t launch_shared_gate(const uint16_t *x, const uint16_t *gate_w, const Dims &d, float *out,
                              hipStream_t st)
{
    shared_gate_kernel<<<(d.T + 3) / 4, 256, 0, st>>>(x, gate_w, d, out);
    return hipGetLastError();
}

}  // namespace moe
