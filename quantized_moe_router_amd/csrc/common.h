// Internal declarations of libmoe_int4: device helpers, the workspace map and
// the kernel launchers.  Not part of the public ABI (see include/moe_int4.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kMaxHidden = 4096;
constexpr int kGroup = 128;      // INT4 group along the input dimension (64 also accepted)
constexpr int kShGroup = 64;     // INT6 group (shared expert)
// Decode (GEMV) path for T <= kDecodeMaxTokens, grouped-GEMM path above.
constexpr int kDecodeMaxTokens = 16;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load of data read exactly once (weights): non-temporal hint.
__device__ __forceinline__ uint4 load_stream(const uint4 *p)
{
    u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------------------
// bf16 helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (inputs are finite).
// fp32 -> bf16 with round to nearest even, by the packed hardware convert
// (v_cvt_pk_bf16_f32): the same bits as adding 0x7FFF plus the kept lsb and
// truncating, for every non-NaN input; a NaN stays a NaN.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi)
{
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    return f32x2_to_bf16x2(f, 0.f) & 0xFFFFu;
}

// c + a.lo*b.lo + a.hi*b.hi on bf16 pairs (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---------------------------------------------------------------------------
// INT4 nibbles -> bf16 without a conversion instruction.
//
// bf16 0x4300 is 128.0 with a zero 7-bit mantissa, so OR-ing a nibble n into
// the mantissa gives exactly 128 + n.  Masking a word with 0x000F000F keeps
// nibble 0 in the low half and nibble 4 in the high half, i.e. a bf16 pair
// (128+n0, 128+n4); shifting by 4, 8, 12 first gives (n1,n5), (n2,n6),
// (n3,n7).  A dot product over these pairs against activations arranged the
// same way gives sum (128 + n) x; the stored nibble is code + 8, so the true
// sum of code * x is that minus 136 * sum x.
// ---------------------------------------------------------------------------
// A constant in a vector register, opaque to constant folding.  gfx9 VOP3
// instructions (v_and_or_b32 and its like) take no literal and read at most
// one scalar register, so (x & mask) | pattern with both constants as
// literals is emitted as two instructions; with both in vector registers it
// is one v_and_or_b32.
__device__ __forceinline__ uint32_t vconst(uint32_t c)
{
    uint32_t v;
    asm("; vconst" : "=v"(v) : "0"(c));
    return v;
}

__device__ __forceinline__ void nib_pairs(uint32_t w, uint32_t p[4])
{
    const uint32_t m = vconst(0x000F000Fu), b = vconst(0x43004300u);
    p[0] = (w & m) | b;
    p[1] = ((w >> 4) & m) | b;
    p[2] = ((w >> 8) & m) | b;
    p[3] = ((w >> 12) & m) | b;
}

// Natural-order bf16 octet (4 dwords: (e0,e1)(e2,e3)(e4,e5)(e6,e7)) ->
// nibble-pair order (e0,e4)(e1,e5)(e2,e6)(e3,e7).
__device__ __forceinline__ void octet_to_pair_order(const uint32_t in[4], uint32_t out[4])
{
    out[0] = __builtin_amdgcn_perm(in[2], in[0], 0x05040100u);
    out[1] = __builtin_amdgcn_perm(in[2], in[0], 0x07060302u);
    out[2] = __builtin_amdgcn_perm(in[3], in[1], 0x05040100u);
    out[3] = __builtin_amdgcn_perm(in[3], in[1], 0x07060302u);
}

// Position of element i (0..7) of an 8-block in nibble-pair order.
__device__ __forceinline__ int pair_pos(int i) { return (i < 4) ? 2 * i : 2 * (i - 4) + 1; }

// sum over 32 (code+8+128) * x of one 16-byte chunk of 4 INT4 words, with x
// given as 16 dwords in nibble-pair order.
__device__ __forceinline__ float chunk_dot(const uint4 w, const uint32_t x[16])
{
    uint32_t p[4];
    float acc = 0.f;
    nib_pairs(w.x, p);
    acc = dot2(p[0], x[0], acc); acc = dot2(p[1], x[1], acc);
    acc = dot2(p[2], x[2], acc); acc = dot2(p[3], x[3], acc);
    nib_pairs(w.y, p);
    acc = dot2(p[0], x[4], acc); acc = dot2(p[1], x[5], acc);
    acc = dot2(p[2], x[6], acc); acc = dot2(p[3], x[7], acc);
    nib_pairs(w.z, p);
    acc = dot2(p[0], x[8], acc); acc = dot2(p[1], x[9], acc);
    acc = dot2(p[2], x[10], acc); acc = dot2(p[3], x[11], acc);
    nib_pairs(w.w, p);
    acc = dot2(p[0], x[12], acc); acc = dot2(p[1], x[13], acc);
    acc = dot2(p[2], x[14], acc); acc = dot2(p[3], x[15], acc);
    return acc;
}

// 32 activations (64 bytes) as four 16-byte loads.  Loading every chunk
// first and transforming afterwards keeps all loads in flight together.
struct ActRaw {
    uint4 v[4];
};

__device__ __forceinline__ ActRaw load_act_raw(const uint16_t *p)
{
    const uint4 *q = reinterpret_cast<const uint4 *>(p);
    return ActRaw{{q[0], q[1], q[2], q[3]}};
}

// Natural-order bf16 activations -> nibble-pair order, plus their sum.
__device__ __forceinline__ float act_pairs(const ActRaw &r, uint32_t x[16])
{
    float s = 0.f;
#pragma unroll
    for (int o = 0; o < 4; ++o) {
        uint32_t in[4] = {r.v[o].x, r.v[o].y, r.v[o].z, r.v[o].w};
        octet_to_pair_order(in, x + 4 * o);
        s = dot2(in[0], 0x3F803F80u, s);  // bf16 (1.0, 1.0)
        s = dot2(in[1], 0x3F803F80u, s);
        s = dot2(in[2], 0x3F803F80u, s);
        s = dot2(in[3], 0x3F803F80u, s);
    }
    return s;
}

// ---------------------------------------------------------------------------
// fp16 variant for the SwiGLU activation a = silu(g) * u, which the kernels
// keep in fp16 (11 significant bits; bf16's 8 were too coarse for a's heavy
// tail).  fp16 0x5800 is 128.0 with mantissa step 1/8, so (n << 3) | 0x5800 is
// exactly 128 + n for n < 128: the same exponent trick as above.
// ---------------------------------------------------------------------------
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2h(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c,
                                  false);
}

// fp32 -> fp16 bits, round to nearest even, saturating at +-65504.
__device__ __forceinline__ uint32_t f32_to_f16_sat(float f)
{
    f = __builtin_amdgcn_fmed3f(f, -65504.f, 65504.f);
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// INT4 word -> fp16 pairs (128+n0,128+n4) (128+n1,128+n5) (128+n2,128+n6)
// (128+n3,128+n7).
__device__ __forceinline__ void nib_pairs_h(uint32_t w, uint32_t p[4])
{
    const uint32_t m = vconst(0x00780078u), b = vconst(0x58005800u);
    p[0] = ((w << 3) & m) | b;
    p[1] = ((w >> 1) & m) | b;
    p[2] = ((w >> 5) & m) | b;
    p[3] = ((w >> 9) & m) | b;
}

__device__ __forceinline__ float chunk_dot_h(const uint4 w, const uint32_t x[16])
{
    uint32_t p[4];
    float acc = 0.f;
    nib_pairs_h(w.x, p);
    acc = dot2h(p[0], x[0], acc); acc = dot2h(p[1], x[1], acc);
    acc = dot2h(p[2], x[2], acc); acc = dot2h(p[3], x[3], acc);
    nib_pairs_h(w.y, p);
    acc = dot2h(p[0], x[4], acc); acc = dot2h(p[1], x[5], acc);
    acc = dot2h(p[2], x[6], acc); acc = dot2h(p[3], x[7], acc);
    nib_pairs_h(w.z, p);
    acc = dot2h(p[0], x[8], acc); acc = dot2h(p[1], x[9], acc);
    acc = dot2h(p[2], x[10], acc); acc = dot2h(p[3], x[11], acc);
    nib_pairs_h(w.w, p);
    acc = dot2h(p[0], x[12], acc); acc = dot2h(p[1], x[13], acc);
    acc = dot2h(p[2], x[14], acc); acc = dot2h(p[3], x[15], acc);
    return acc;
}

// Natural-order fp16 activations -> nibble-pair order, plus their sum.
__device__ __forceinline__ float act_pairs_h(const ActRaw &r, uint32_t x[16])
{
    float s = 0.f;
#pragma unroll
    for (int o = 0; o < 4; ++o) {
        uint32_t in[4] = {r.v[o].x, r.v[o].y, r.v[o].z, r.v[o].w};
        octet_to_pair_order(in, x + 4 * o);
        s = dot2h(in[0], 0x3C003C00u, s);  // fp16 (1.0, 1.0)
        s = dot2h(in[1], 0x3C003C00u, s);
        s = dot2h(in[2], 0x3C003C00u, s);
        s = dot2h(in[3], 0x3C003C00u, s);
    }
    return s;
}

// silu(g) = g / (1 + e^-g) with the hardware exp2 and reciprocal (each within
// about 1 ulp of fp32); every caller rounds the product to fp16 (2^-11)
// right after, so the shortcut is far below the result's own rounding.  For
// g << 0, e^-g overflows to inf and the reciprocal gives 0.
__device__ __forceinline__ float silu(float g)
{
    return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.44269504088896341f));
}

// ---------------------------------------------------------------------------
// Hand-over between workgroups of one launch.  Agent-scope relaxed atomic
// loads and stores are coherent across the XCDs' separate L2 caches (they
// compile to sc1 accesses), so data written this way and read this way needs
// no cache write-back or invalidate: the writer only waits until its stores
// have completed (vmcnt counts stores on this architecture) before it
// publishes a counter, and the reader reads the data after it has seen the
// counter.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store_coherent(uint16_t *p, uint16_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(uint64_t *p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_coherent(const uint64_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_coherent(const uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this wave has issued has completed.
__device__ __forceinline__ void wait_memory()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t *p, uint32_t v)
{
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Record a failed bounded wait in the sticky status word (a vector atomic).
__device__ __forceinline__ void set_status(uint32_t *status, uint32_t bit)
{
    __hip_atomic_fetch_or(status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Cross-lane sums with DPP lane moves (VALU only; a shuffle would go through
// the LDS crossbar with a full wait per step).  Every lane of a quad / row /
// wave gets the same sum: each step adds a value and its mirror image, and
// fp32 addition is commutative.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // lane 7 - i within each 8
constexpr int kDppMirror = 0x140;      // lane 15 - i within each 16

// Word 3 of a CDNA buffer resource for raw (stride 0) accesses, 32-bit data
// format.  The hardware drops a store whose offset lies at or beyond the
// resource's num_records bytes, which bounds a tile's stores without a branch.
constexpr int kBufferWord3 = 0x00020000;

// Sum over the 4 lanes of a quad.
__device__ __forceinline__ float quad_sum(float v)
{
    v += dpp_move<kDppXor1>(v);
    v += dpp_move<kDppXor2>(v);
    return v;
}
// Sum over the 16 lanes of a row.
__device__ __forceinline__ float row_sum(float v)
{
    v = quad_sum(v);
    v += dpp_move<kDppHalfMirror>(v);
    v += dpp_move<kDppMirror>(v);
    return v;
}
__device__ __forceinline__ float read_lane(float v, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// Sum over the wave (uniform result).
__device__ __forceinline__ float wave_sum(float v)
{
    v = row_sum(v);
    return (read_lane(v, 0) + read_lane(v, 16)) + (read_lane(v, 32) + read_lane(v, 48));
}

// ---------------------------------------------------------------------------
// Workspace map.  Every region is 256-byte aligned; counters first so that
// the zero-state contract covers a fixed prefix.
// ---------------------------------------------------------------------------
// The workspace starts with a fixed control prefix, the same for every shape:
// the few-token router's keys (64 KiB), then 256 bytes of control words.
// Control word 0 is the sticky status (kStatus* bits, set when a bounded
// wait gives up; never cleared by the library); the other control words are
// hand-off counters that are zero between calls.
constexpr size_t kKeysBytes = 4 * (size_t)kDecodeMaxTokens * kMaxExperts;   // 65536
constexpr size_t kCtrlBytes = 256;
constexpr uint32_t kStatusKeyWait = 1u;     // a routing wave gave up waiting for router keys
constexpr uint32_t kStatusRouteWait = 2u;   // an expert workgroup gave up waiting for the routing
constexpr uint32_t kStatusHWait = 4u;       // a down-projection workgroup gave up waiting for h

struct Workspace {
    // zero between calls (a fixed prefix of every layout)
    uint32_t *dec_keys;      // [kDecodeMaxTokens * kMaxExperts] decode router keys, 0 = unset
    uint32_t *ctrl;          // [kCtrlBytes / 4] control words: [0] sticky status, then counters
    uint32_t *status;        // where failed bounded waits are recorded (ctrl[0] unless redirected)
    // routing
    float *logits;           // [T][E]
    int32_t *ids;            // [T][k]   (forward: internal copy)
    float *weights;          // [T][k]
    int32_t *counts;         // [E]
    int32_t *offsets;        // [E+1]
    int32_t *sorted_slots;   // [S]
    int32_t *slot_pos;       // [S]   inverse of sorted_slots
    int32_t *active;         // [E+1] active[0] = n_active, then expert ids
    int32_t *chunk_hist;     // [nchunks][E]
    int4 *tiles;             // [routed_tile_slots] grouped-GEMM tiles {expert | block << 16, first row, rows, 0}
    // expert intermediates
    uint16_t *h;             // [S][I] fp16, sorted order
    uint16_t *y;             // [T][k+1][H] fp16 weighted slot outputs (many-token path)
    float *shared_gate;      // [T] shared-expert gate logits
    uint16_t *sh_h;          // [T][I_sh] fp16
    uint16_t *xh;            // [T][H] fp16 copy of x in nibble-pair order (many-token path)
    uint16_t *xp;            // [T][H] bf16 copy of x in nibble-pair order (decode path)
    float *xs;               // [T][H/32] sums of 32-value chunks of x (decode path)
    size_t bytes;
};

struct Dims {
    int T, H, E, I, k, S;
    int sh_I;  // 0 = no shared expert
    int gsh;   // INT4 group = 32 << gsh (2: group 128, 1: group 64)
};

constexpr int kPermChunk = 1024;  // most slots per chunk of the large permutation

// Slots per chunk of the large permutation (S > kPermChunk): about 128 chunks
// (one wave each in the count and scatter passes), a multiple of 64 between 64
// and kPermChunk.
__host__ __device__ inline int perm_chunk(int S)
{
    const int c = ((S + 127) / 128 + 63) / 64 * 64;
    return c < 64 ? 64 : (c > kPermChunk ? kPermChunk : c);
}

// Split of the many-token router GEMM's reduction over H: the smallest divisor
// of its 64-wide stage count that gives at least 512 workgroups of 128 tokens
// x 128 experts, keeping at least two stages per split and at most 8 splits.
// Each split writes its own fp32 partial logits ([split][T][E]); the top-k
// adds them in split order.
inline int router_ksplit(const Dims &d)
{
    const int nsteps = d.H / 64;
    const long tiles = (long)((d.T + 127) / 128) * ((d.E + 127) / 128);
    int best = 1;
    for (int ks = 1; 2 * ks <= nsteps && ks <= 8; ++ks) {
        if (nsteps % ks) continue;
        best = ks;
        if (tiles * ks >= 512) break;
    }
    return best;
}

// Slots of the grouped-GEMM tile list: row tiles (128 rows, or 64 when the
// slots per expert are few) in pairs, pairs dealt round-robin to the 8 XCDs,
// 16 slots per round.  At most S / 64 + 2 E tile positions are used (each
// expert's tiles rounded up to a pair), which this bound covers.
// Routed grouped GEMMs.  With many slots per expert (at least
// kBigMinRowsPerExpert on average) one workgroup takes a whole chunk of up to
// kBigRows rows of one expert (every row of it, for balanced routing), so the
// expert's weights are fetched and dequantised once per weight block
// (moe_gemm_big_kernel); otherwise row tiles of 128 rows, or 64 when the
// slots per expert are few (moe_gemm_kernel).
constexpr int kBigRows = 192;
constexpr int kBigMinRowsPerExpert = 64;
inline bool routed_big(const Dims &d)
{
    return (long)d.S >= (long)kBigMinRowsPerExpert * d.E;   // group 128 or 64
}
// Rows per routed tile list entry.
inline int routed_tile_rows(const Dims &d)
{
    return routed_big(d) ? kBigRows : ((long)d.S < 32L * d.E ? 64 : 128);
}

// Permutations of kPermChunk < S <= kPermMidWaves * kPermChunk run in one
// workgroup of kPermMidWaves waves; larger ones scan in one workgroup.  Both
// of those workgroups also build the GEMM tile list.
constexpr int kPermMidWaves = 16;
inline bool permute_builds_tiles(const Dims &d) { return d.S > kPermChunk; }

inline size_t routed_tile_slots(const Dims &d)
{
    if (routed_big(d)) {
        // chunks: at most ceil(S / kBigRows) + E, a multiple of 8
        const size_t chunks = ((size_t)d.S + kBigRows - 1) / kBigRows + (size_t)d.E;
        return 8 * ((chunks + 7) / 8);
    }
    const size_t pairs = ((size_t)d.S + 63) / 64 / 2 + (size_t)d.E + 1;
    return 16 * ((pairs + 7) / 8);
}

Workspace carve_workspace(void *base, const Dims &d);
size_t workspace_size(const Dims &d);

// ---------------------------------------------------------------------------
// Launchers (return hipError_t of the launch)
// ---------------------------------------------------------------------------
struct RouteOut {
    int32_t *ids;
    float *weights;
    int32_t *counts;
    int32_t *offsets;
    int32_t *sorted_slots;
};

// convert_x (many-token routing only): the top-k kernel also writes x in the
// gate/up GEMMs' fp16 pair order to ws.xh and, given gate_w, the shared
// expert's gate logits to ws.shared_gate.  ev_topk (may be null) is recorded
// on st right after the top-k kernel, ahead of the permutation.
hipError_t launch_route(const uint16_t *x, const uint16_t *router_w, const Dims &d,
                        const Workspace &ws, const RouteOut &ro, hipStream_t st, bool convert_x = false,
                        const uint16_t *gate_w = nullptr, hipEvent_t ev_topk = nullptr);
hipError_t launch_permute(const Dims &d, const Workspace &ws, const RouteOut &ro,
                          hipStream_t st);

struct ExpertArgs {
    const uint16_t *x;
    const int32_t *w13p;
    const uint16_t *w13s;
    const int32_t *w2p;
    const uint16_t *w2s;
    const float *weights;  // [T][k] routing weights (slot order)
    uint16_t *out;
    // shared expert (nullptr when absent)
    const uint16_t *sh_gate;
    const int32_t *sh_w13p;
    const uint16_t *sh_w13s;
    const int32_t *sh_w2p;
    const uint16_t *sh_w2s;
};

// Many-token experts: grouped GEMMs (gate/up, then down + combine), with the
// shared expert when present.  `ev_mid` (may be null) is recorded between the
// gate/up and down projections.
// x_converted: ws.xh already holds x in fp16 pair order (from the routing),
// and ws.shared_gate the shared expert's gate logits when it has one.
// ev_shared: null, or the shared expert was enqueued on another stream by
// launch_shared_expert and ev_shared recorded there after it; the combine
// then waits on it instead of running the shared expert on st.
hipError_t launch_prefill_experts(const ExpertArgs &a, const Dims &d, const Workspace &ws,
                                  const RouteOut &ro, hipStream_t st, hipEvent_t ev_mid,
                                  bool x_converted = false, hipEvent_t ev_shared = nullptr);
// The shared expert of a many-token forward (gate logits unless x_converted,
// gate/up -> ws.sh_h, down -> its y rows); it needs ws.xh in pair order.
hipError_t launch_shared_expert(const ExpertArgs &a, const Dims &d, const Workspace &ws, hipStream_t st,
                                bool x_converted);

// bf16 octet (natural order) -> fp16 octet in pair order.
__device__ __forceinline__ uint4 bf16_octet_to_f16_pairs(uint4 v)
{
    const uint32_t in[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // element j is in dword j/2, element j+4 in dword 2 + j/2
        const uint32_t a = in[j >> 1], b = in[2 + (j >> 1)];
        const float fa = __uint_as_float((j & 1) ? (a & 0xFFFF0000u) : (a << 16));
        const float fb = __uint_as_float((j & 1) ? (b & 0xFFFF0000u) : (b << 16));
        out[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(fa, fb));
    }
    return make_uint4(out[0], out[1], out[2], out[3]);
}

// ---------------------------------------------------------------------------
// INT8 W8A16 linear layer (int8_linear.hip)
// ---------------------------------------------------------------------------
constexpr int kInt8GemvMaxTokens = 4;          // dot-product GEMV up to this many tokens
constexpr int kInt8MfmaGemvMaxTokens = 16;     // matrix-core GEMV (wide matrices) up to this many
constexpr size_t kInt8GemvMaxLds = 65536;      // GEMV keeps T x K fp16 activations in LDS
constexpr int kInt8GemvMaxBlocks = 2048;       // persistent GEMV grid (8 per CU)
constexpr long kInt8GemmTargetTiles = 256;     // K is split until about this many workgroups
constexpr int kInt8MinSplitK = 256;            // shortest K range of one split
constexpr int kInt8MaxSplitK = 16;

struct Int8Plan {
    bool gemv;
    bool rowsplit;       // GEMV with one row per workgroup (narrow matrices)
    bool mfma;           // matrix-core GEMV (5..16 tokens, wide matrices)
    bool short_k;        // GEMM whose whole K range is loaded at once (K <= 320)
    int mtiles, ntiles, ksplit, kslice;
    size_t pstride;      // floats per split in the partials (T * N rounded up to 4)
    size_t part_bytes;   // fp32 split-K partials (workspace)
};
Int8Plan int8_plan(int T, int N, int K, int G);
hipError_t launch_int8_linear(const uint16_t *x, const int32_t *wq, const uint16_t *ws, int T, int N,
                              int K, int G, uint16_t *out, void *workspace, hipStream_t st);

}  // namespace moe
