// qkrope_kernel_impl.h -- the fused QK-RMSNorm + RoPE (+ V) kernel family for gfx950.
// Included by the qkrope_kernels_*.hip translation units, each of which instantiates a subset.
//
// What is computed follows two API pages:
//   vLLM-Omni "vllm_omni.diffusion.layers.fused_qk_norm_rope" (module contract): per-head Q/K
//     RMSNorm with [head_dim] weights, then RoPE from a [tokens, rotary_dim] table of
//     [cos | sin], half-split pairs (d, d + R/2) or interleaved pairs (2i, 2i+1); the fused path
//     keeps normalised and rotated values in registers (no intermediates in memory).
//   FlashInfer "flashinfer.norm.fused_qk_rmsnorm_rope" (description, parameters): across-heads
//     RMSNorm, frame/height/width RoPE with YaRN and an attention factor on cos/sin, V copied
//     out of packed QKV, optional FP8 E4M3 outputs.
//
// Work decomposition (MI355X-first; the pages give no kernel design for this hardware):
//   * The operation is HBM-bound (a few flops per byte), so the design goal is 16-byte coalesced
//     loads and stores with many bytes in flight, and little ALU work per byte.
//   * One workgroup per token (two when a token fills only half a wave's multiple, see TPW; one
//     per region of a token in the 3D form without norm, see RS). On MI355X the hardware's own
//     workgroup scheduling hides memory latency better than a software-pipelined walk over
//     several tokens per workgroup, which measured slower at every depth tried. Large grids
//     deal runs of 16 consecutive token blocks (64 with the region split) to each XCD
//     (KernelArgs::xcd_group); a call whose grid would exceed one dispatch runs as several
//     launches over token ranges (host).
//   * A token's Q, K (and V) rows are cut into units of one 16-byte chunk (8 bf16), so every
//     load and store instruction of a wave covers whole contiguous cache lines. Interleaved
//     pairs never leave a chunk. Half-split/NeoX pairs (d, d + R/2) join chunk c with chunk
//     c + R/16 of the same head: each lane normalises its own chunk, then fetches its partner
//     lane's normalised values with a cross-lane permute and writes only its own chunk.
//     Each head gets L = 2^k >= D/8 consecutive lanes; lane `tid` owns chunk tid mod L of
//     several heads (its slots). Because the workgroup size is a multiple of L, every slot of a
//     lane covers the same dims, so angles and per-head weights are fetched once per lane.
//   * Two slot layouts. Region-major (SU): each region (Q, K, V) has NS slots per lane, slot i
//     covering heads (tid + i*nth)/L of that region; region, base pointers and weights of every
//     slot are compile-time/scalar. Mixed: the regions' units are concatenated and lane-slot j
//     covers unit tid + j*nth of the token, whichever region it falls in (fills the lanes when
//     a region's unit count does not divide the workgroup, e.g. 20 heads of 64).
//   * Sum of squares: per-head norm reduces inside the L lanes of the head with DPP/permlane
//     butterflies; across-heads norm reduces each wave, then combines the waves through LDS.
//   * 3D angles: lanes k < head_dim/2 compute (cos, sin) of pair k once per token (angle in
//     revolutions, fract, hardware sin/cos), scaled by the attention factor, into LDS; the
//     barrier that publishes them is the one the across-heads reduction needs anyway.
//   * Phases per token: all loads, reductions and the barrier, all outputs computed into
//     registers, then all stores, so no data wait ever sits behind an outstanding store.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qkrope_internal.h"

namespace qkrope {
namespace dev {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ---- number formats ---------------------------------------------------------------------------

// bf16 -> fp32 is exact: the bf16 bits are the upper half of the fp32 pattern.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// IEEE binary16 -> fp32 is exact (subnormals included).
__device__ __forceinline__ f32x2 f16x2_to_f32(uint32_t u)
{
    return __builtin_convertvector(__builtin_bit_cast(f16x2, u), f32x2);
}

// Eight 16-bit activations of a chunk (bf16 or binary16, per ACT) -> fp32, exactly.
template <int ACT>
__device__ __forceinline__ void unpack8(const uint4 v, float x[8])
{
    if (ACT == kActBF16) {
        x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
        x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
        x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
        x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
    } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x2 f = f16x2_to_f32(w[i]);
            x[2 * i] = f.x;
            x[2 * i + 1] = f.y;
        }
    }
}

// Two fp32 -> two 16-bit values with round-to-nearest-even (one packed conversion on gfx950
// for bf16; binary16 overflows to +-inf as IEEE rounding does).
template <int ACT>
__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    f32x2 v = {a, b};
    if (ACT == kActBF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

template <int ACT>
__device__ __forceinline__ uint4 pack8(const float y[8])
{
    return make_uint4(pack2<ACT>(y[0], y[1]), pack2<ACT>(y[2], y[3]),
                      pack2<ACT>(y[4], y[5]), pack2<ACT>(y[6], y[7]));
}

// OCP E4M3 (gfx950's fp8 conversions produce the OCP encoding): finite values beyond the largest
// finite magnitude 448 saturate to +-448, NaN stays NaN (the comparison is false for NaN), and
// the hardware conversion rounds to nearest even.
__device__ __forceinline__ float sat_e4m3(float y)
{
    return __builtin_fabsf(y) > 448.0f ? __builtin_copysignf(448.0f, y) : y;
}

// Each conversion writes one 16-bit half of its destination and keeps the other; the first of
// each pair starts from the register of its own first input, which dies there (the other half is
// written by the second conversion), so no copy is needed.
// The conversion itself maps NaN to the NaN code, so saturation is only needed where some
// |y| > 448; that is rare, so lanes test the chunk's largest magnitude (v_max3 ignores NaN)
// and only those above 448 take the saturating path.
__device__ __forceinline__ uint2 pack8_e4m3(const float yin[8])
{
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = yin[i];
    // a chain of three-operand maxima with |.| operand modifiers: four v_max3_f32
    float m = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(y[0]), __builtin_fabsf(y[1])),
                              __builtin_fabsf(y[2]));
    m = __builtin_fmaxf(__builtin_fmaxf(m, __builtin_fabsf(y[3])), __builtin_fabsf(y[4]));
    m = __builtin_fmaxf(__builtin_fmaxf(m, __builtin_fabsf(y[5])), __builtin_fabsf(y[6]));
    m = __builtin_fmaxf(m, __builtin_fabsf(y[7]));
    if (m > 448.0f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = sat_e4m3(y[i]);
    }
    const float a0 = y[0], a1 = y[1], a2 = y[2], a3 = y[3];
    const float b0 = y[4], b1 = y[5], b2 = y[6], b3 = y[7];
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, __float_as_int(a0), false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(b0, b1, __float_as_int(b0), false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(b2, b3, hi, true);
    return make_uint2((uint32_t)lo, (uint32_t)hi);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2v __attribute__((ext_vector_type(2)));

// Magnitudes of two packed 16-bit floats as unsigned integers (order-preserving for non-NaN).
__device__ __forceinline__ u16x2 mag16(uint32_t w) { return __builtin_bit_cast(u16x2, w & 0x7fff7fffu); }

// E4M3 codes of four bf16 values (two packed pairs) divided by a power of two `inv` (the
// conversion uses the scale's exponent only): v_cvt_scalef32_pk_fp8_bf16, round to nearest even,
// no saturation. Each conversion writes one 16-bit half of its destination; the first starts from
// its own input's register, whose other half the second conversion overwrites.
__device__ __forceinline__ uint32_t pack4_e4m3_pow2(uint32_t lo, uint32_t hi, float inv)
{
    s16x2v r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(__builtin_bit_cast(s16x2v, lo),
                                                         __builtin_bit_cast(bf16x2, lo), inv, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2, hi), inv, true);
    return __builtin_bit_cast(uint32_t, r);
}

// ---- memory -----------------------------------------------------------------------------------

// Cache policy of the streamed activations: every input byte is read once and every output
// byte written once, so both carry the non-temporal hint (measured on MI355X: plain stores are
// 3-5% slower). Weights and tables, which every workgroup re-reads, use normal loads.

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16-byte load at a (usually uniform) base plus a 32-bit unsigned byte offset, the form the
// global_load saddr+voffset encoding takes: one VGPR per address.
__device__ __forceinline__ uint4 ld16(const void *base, uint32_t byte_off)
{
    return *reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(base) + byte_off);
}

// The same for streamed (read-once) activations; NT selects the non-temporal hint.
template <bool NT>
__device__ __forceinline__ uint4 ld16_stream(const void *base, uint32_t byte_off)
{
    const u32x4 *p = reinterpret_cast<const u32x4 *>(static_cast<const uint8_t *>(base) + byte_off);
    const u32x4 v = NT ? __builtin_nontemporal_load(p) : *p;
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Streamed 16- and 8-byte stores at a base plus a 32-bit byte offset, like the loads: no 64-bit
// address arithmetic per lane; all carry the non-temporal hint. Large launches (DEV, a uniform
// flag the host sets from the bytes a launch writes) with a uniform base (UNI) store through a
// buffer resource spanning the 4 GiB above the base instead, whose instruction also takes
// device scope (sc1), so each XCD's L2 passes the written lines on to memory at once instead of
// holding them dirty. Measured on MI355X: a plain 16-byte copy of 3 GB runs at 79-81% of
// 8 TB/s with device scope against 77% without; the 122880-token YaRN workload went from 955 to
// 934 us per launch and the 32768-token tables gained 0.4-1%, but launches writing under 100 MB
// lost (the 4-way head-sharded rank's apply kernel 31.1 -> 32.4 us, the 4096-token table
// 19.55 -> 19.9 us): there the lines a write-back L2 would hold past the kernel's end are
// written inside it. A per-lane base (the mixed slot layout) always takes the global form.
constexpr int kStoreNTDevice = 2 | 16;      // nt | sc1 in the buffer instruction's aux field
constexpr int kBufferFlags = 0x00020000;    // raw (untyped) buffer: word 3 of the resource

__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(void *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, -1, kBufferFlags);
}

template <bool UNI>
__device__ __forceinline__ void st16_stream(void *base, uint32_t byte_off, uint4 v, bool dev)
{
    const u32x4 w = {v.x, v.y, v.z, v.w};
    if (UNI && dev)
        __builtin_amdgcn_raw_buffer_store_b128(w, stream_rsrc(base), (int)byte_off, 0, kStoreNTDevice);
    else
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(static_cast<uint8_t *>(base) + byte_off));
}

template <bool UNI>
__device__ __forceinline__ void st8_stream(void *base, uint32_t byte_off, uint2 v, bool dev)
{
    const u32x2 w = {v.x, v.y};
    if (UNI && dev)
        __builtin_amdgcn_raw_buffer_store_b64(w, stream_rsrc(base), (int)byte_off, 0, kStoreNTDevice);
    else
        __builtin_nontemporal_store(w, reinterpret_cast<u32x2 *>(static_cast<uint8_t *>(base) + byte_off));
}

// n / d for n < 2^31 with a host-computed magic pair (m, l): q = (mulhi(n, m) + n) >> l.
__device__ __forceinline__ uint32_t fast_div(uint32_t n, uint32_t m, uint32_t l)
{
    return (__umulhi(n, m) + n) >> l;
}

template <typename T>
__device__ __forceinline__ T sel3(int r, T a, T b, T c) { return r == 0 ? a : (r == 1 ? b : c); }

// ---- reductions -------------------------------------------------------------------------------
//
// All on the VALU: DPP quad permutations and row mirrors inside each 16-lane row, then the gfx950
// row-swap permutes across rows. Each step adds a lane's value to its partner's, and IEEE
// addition is commutative, so every lane of a group ends with a bitwise identical sum.

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v)
{
    return v + __builtin_amdgcn_update_dpp(0.0f, v, CTRL, 0xF, 0xF, false);
}

constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7-i inside each 8 lanes
constexpr int kDppRowMirror = 0x140;    // lane i <-> 15-i inside each 16 lanes

__device__ __forceinline__ float swap16_add(float v)   // rows 0+1 and 2+3
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ __forceinline__ float swap32_add(float v)   // lanes 0-31 + 32-63
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Sum over aligned groups of `width` lanes (1, 2, 4, ..., 64); `width` is uniform.
__device__ __forceinline__ float group_sum(float v, int width)
{
    if (width >= 2) v = dpp_add<kDppQuadXor1>(v);
    if (width >= 4) v = dpp_add<kDppQuadXor2>(v);
    if (width >= 8) v = dpp_add<kDppHalfMirror>(v);
    if (width >= 16) v = dpp_add<kDppRowMirror>(v);
    if (width >= 32) v = swap16_add(v);
    if (width >= 64) v = swap32_add(v);
    return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum(v, 64); }

// Two sums through one tree. v_permlane16_swap exchanges the second 16-lane row of its first
// operand with the first row of its second (and rows 3 and 2 likewise), so with (a, b) the first
// row of each 32-lane group ends with a of lanes i and i + 16, the second with b of lanes i - 16
// and i: the first row then carries a's pair sums, the second b's, for a 16-lane tree to finish.
__device__ __forceinline__ float pair_rows_add(float a, float b)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// The same swap with v in both operands gives every lane of a 32-lane group its first row's
// value (.x) and its second row's (.y).
__device__ __forceinline__ f32x2 rows_to_all(float v)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return f32x2{__uint_as_float(p[0]), __uint_as_float(p[1])};
}

// Sum of squares of the 8 activations of a chunk, from the packed pairs (v_dot2c_f32_bf16 or
// v_dot2_f32_f16: products of 16-bit values are exact in fp32, the sums are fp32).
template <int ACT>
__device__ __forceinline__ float sumsq_packed(const uint4 v, float acc)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (ACT == kActBF16) {
            const bf16x2 b = __builtin_bit_cast(bf16x2, w[i]);
            acc = __builtin_amdgcn_fdot2_f32_bf16(b, b, acc, false);
        } else {
            const f16x2 h = __builtin_bit_cast(f16x2, w[i]);
            acc = __builtin_amdgcn_fdot2(h, h, acc, false);
        }
    }
    return acc;
}

// ---- the kernel -------------------------------------------------------------------------------

// DT: head_dim as a compile-time constant (64/128/256), or 0 to read it from the arguments.
// PAIR: kPairInterleaved, kPairHalf (half-split, R/2 a multiple of 8) or kPairHalfAny
// (half-split, any even R; partners exchanged through LDS). NORM: kNormNone/PerHead/Across/
// AcrossExt. SRC: cos/sin from a fp32, bf16 or binary16 table, or computed (3D).
// ACT: 16-bit activation format (bf16 or binary16). FP8: E4M3 outputs.
// SU: region-major slots (NS per region); otherwise mixed slots (NS in all).
// TPW: tokens per workgroup, 1, or 2 (region-major, one slot per region) when a token needs a
// multiple of 32 but not of 64 lanes, so that two tokens fill whole waves.
// RS: one region (Q, K or V) of one token per workgroup, NS slots; workgroup b takes region
// b mod NREG of token b / NREG (in XCD order). Launched for the 3D form without norm and with
// 16-bit outputs (either pairing), where every workgroup only streams.
template <int DT, int PAIR, int NORM, int SRC, int ACT, bool FP8, int NS, bool SU, int TPW, bool RS>
__global__ void __launch_bounds__(1024) qkrope_kernel(const KernelArgs a)
{
    static_assert(TPW == 1 || (TPW == 2 && SU && NS == 1), "two tokens per workgroup: region-major, one slot");
    static_assert(!RS || (SU && TPW == 1), "one region per workgroup: region-major, one token");
    constexpr bool HALF = PAIR != kPairInterleaved;
    constexpr bool XCH = PAIR == kPairHalfAny;  // partners through LDS, per element
    constexpr bool IS3D = (SRC == kSrc3D);
    constexpr bool ACROSS = NORM == kNormAcross || NORM == kNormAcrossExt;
    constexpr int NREG = IS3D ? 3 : 2;          // regions: Q, K (, V)
    constexpr int NSLOT = SU && !RS ? NREG * NS : NS;
    constexpr int NPAIR = HALF ? 8 : 4;         // rotation pairs a chunk takes part in
    constexpr bool NEED_BARRIER = IS3D || NORM == kNormAcross;
    static_assert(!(SRC == kSrcTableBF16 && ACT == kActF16) && !(SRC == kSrcTableF16 && ACT == kActBF16),
                  "a 16-bit table has the activation format");
    constexpr int ESIZE = FP8 ? 1 : 2;          // output bytes per element

    // 3D angles of the token, in two planes: (cos, -sin) and (cos, sin) per pair, so a
    // half-split lane reads its signed pair directly (first half: y = n cos - n' sin, second
    // half: y = n cos + n' sin). A lane reads the NPAIR consecutive pairs from pair0 =
    // NPAIR * g0; pair g * NPAIR + e sits at row e, column g of a plane (rows padded to an odd
    // stride CSR), so for each e the lanes of a wave read consecutive 8-byte words (no bank
    // conflicts; a pair-major table put the lanes 64-128 bytes apart, 8- to 16-way conflicts),
    // and the writing lanes (pair tl) spread over the banks too.
    constexpr int CSR = kMaxPairs / NPAIR + 1;  // row stride of a plane, f32x2
    constexpr int CSP = NPAIR * CSR;            // one plane
    __shared__ f32x2 s_cs[IS3D ? TPW * 2 * CSP : 1];
    __shared__ f32x2 s_red[32];                 // across-heads partials (Q, K) per wave or group
    float *const s_redf = reinterpret_cast<float *>(s_red);
    // kPairHalfAny: one area of 64 lanes x 8 floats per wave (launched with threads * 32 bytes)
    extern __shared__ float s_xch[];

    const int D = DT > 0 ? DT : a.head_dim;
    // a table kernel with a compile-time head_dim is launched only for rotary_dim == head_dim
    const int R = (IS3D || DT > 0) ? D : a.rotary_dim;
    const int units = D / 8;                    // chunks per head
    const int L = DT > 0 ? units : a.lanes_per_head;
    const int lgL = __builtin_ctz(L);
    const int tid = threadIdx.x;
    const int nth = blockDim.x;
    // Token of this lane: with two tokens per workgroup, lanes [0, LT) take the first and
    // [LT, 2 LT) the second; LT is a multiple of 32 and of L, so neither a head nor a 32-lane
    // group straddles the two.
    const int LT = nth / TPW;
    const int ts = (TPW == 2 && tid >= LT) ? 1 : 0;
    const int tl = tid - ts * LT;               // lane index within its token
    const int u = tid & (L - 1);                // this lane's chunk inside every head it covers
    const bool unit_ok = u < units;
    const uint32_t off0 = 8 * u;                // element offset of the chunk inside a head

    // Rotation geometry of the chunk.
    //   interleaved: pairs (2i, 2i+1) inside the chunk, angles 4u .. 4u+3 (those < R/2 rotate)
    //   half-split:  chunk u < P pairs with chunk u + P (P = R/16), angles 8u .. 8u+7; the
    //                partner lane is tid +- P; chunks >= 2P pass through.
    const int P = HALF ? R / 16 : 0;
    bool rotated;
    int pair0, partner;
    float half_sign = 1.0f;                     // first half: y = n c - n' s; second: n c + n' s
    if (XCH) {
        // element 8u + e of a head is rotated when below R; its pair and sign are per element
        rotated = 8 * u < R;
        pair0 = 0;
        partner = tid & 63;
    } else if (HALF) {
        rotated = u < 2 * P;
        const bool first = u < P;
        pair0 = 8 * (first ? u : u - P);
        partner = rotated ? ((tid & 63) + (first ? P : -P)) : (tid & 63);
        half_sign = first ? -1.0f : 1.0f;
    } else {
        rotated = 8 * u < R;
        pair0 = 4 * u;
        partner = tid & 63;
    }

    // Workgroups are dealt to the 8 XCDs round-robin (block b to XCD b % 8). With xcd_group G
    // (a power of two), XCD x takes runs of G consecutive blocks instead of every 8th block, so a
    // page of the streams is touched by one XCD's translation caches, not all eight; blocks past
    // the last whole run of 8G (xcd_full, 0 when off) keep their own index. Uniform, so scalar
    // shifts and masks, and branch-free, so the scalar loads of every argument the first data
    // loads need issue together at the start instead of one round trip after another.
    // Every argument the first data loads depend on, taken by an empty asm statement at the
    // start: the compiler then fetches them in one batch of scalar loads, one round trip, where
    // it otherwise spread them over two or three dependent ones between the block renumbering
    // and the first data load.
    // 3D form, one token per workgroup under the across-heads norm (16-bit outputs): the wave
    // raises its issue priority until its data loads are out, so a newly started workgroup's
    // loads go ahead of the arithmetic of workgroups past their barrier. Measured on MI355X: the
    // 15360-token across-heads workload 122.1 -> 120.5 us per launch; the same in the FP8 NeoX
    // (two tokens per workgroup), YaRN (region split) and E4M3 table kernels cost 2%, 1.8% and
    // 8%, and in the table form with the across-heads norm (32768 tokens) 0.5%.
    constexpr bool PRIO = IS3D && NORM == kNormAcross && TPW == 1 && !FP8 && !RS;
    if (PRIO) __builtin_amdgcn_s_setprio(3);
    asm volatile("" ::"s"(a.xcd_lg), "s"(a.xcd_full), "s"(a.heads[0]), "s"(a.heads[1]),
                 "s"(a.heads[2]), "s"(a.in[0]), "s"(a.in[1]), "s"(a.in[2]), "s"(a.in_stride[0]),
                 "s"(a.in_stride[1]), "s"(a.in_stride[2]), "s"(a.weight[0]), "s"(a.weight[1]),
                 "s"(a.num_tokens));
    uint32_t blk = blockIdx.x;
    {
        const uint32_t lg = a.xcd_lg, j = blk >> 3, x = blk & 7u;
        const uint32_t r = ((j >> lg) << (lg + 3)) + (x << lg) + (j & ((1u << lg) - 1u));
        blk = blk < a.xcd_full ? r : blk;
    }
    // RS: this workgroup's region (uniform); blk becomes its token
    const int rs = RS ? (int)(blk % (uint32_t)NREG) : 0;
    if (RS) blk /= (uint32_t)NREG;
    const bool v_wg = RS && NREG == 3 && rs == kV;   // V only: no norm, no angles, no barrier

    // Slot -> region (3 = idle) and the element offset of the slot's head inside its region row.
    const int Hq = a.heads[kQ], Hk = a.heads[kK], Hv = NREG == 3 ? a.heads[kV] : 0;
    int reg[NSLOT];
    uint32_t hoff[NSLOT];
    bool ok[NSLOT];
#pragma unroll
    for (int j = 0; j < NSLOT; ++j) {
        if (RS) {
            const int hh = (tl + j * LT) >> lgL;
            reg[j] = rs;
            ok[j] = unit_ok && hh < sel3(rs, Hq, Hk, Hv);
            hoff[j] = (uint32_t)(hh * D);
        } else if (SU) {
            const int r = j / NS;                       // compile-time after unrolling
            const int hh = (tl + (j % NS) * LT) >> lgL;
            reg[j] = r;
            ok[j] = unit_ok && hh < sel3(r, Hq, Hk, Hv);
            hoff[j] = (uint32_t)(hh * D);
        } else {
            const int hh = (tid + j * nth) >> lgL;
            const int r = hh < Hq ? 0 : (hh < Hq + Hk ? 1 : (hh < Hq + Hk + Hv ? 2 : 3));
            const int hstart = r == 0 ? 0 : (r == 1 ? Hq : Hq + Hk);
            reg[j] = r;
            ok[j] = unit_ok && r < 3;
            hoff[j] = (uint32_t)((hh - hstart) * D);
        }
    }

    // Per-head norm weights ([head_dim], shared by every head) stay packed in registers. Under
    // this norm both pointers are valid (a region without heads borrows the other's weights),
    // so both loads are issued unconditionally, lanes past the head's chunks reading chunk 0:
    // a load under a branch has the compiler wait for it before the data loads are issued.
    uint4 wq = make_uint4(0, 0, 0, 0), wk = wq;
    if (NORM == kNormPerHead) {
        const uint32_t wo = unit_ok ? 2 * off0 : 0u;
        wq = ld16(a.weight[0], wo);
        wk = ld16(a.weight[1], wo);
    }

    // 3D: this lane's pair (tl < D/2) frequency in revolutions and its position axis. Vector
    // loads complete in order, so read before the data loads the angle lanes start their sin/cos
    // while the data is still on its way; read after them, the angles wait for every data load.
    // Measured on MI355X: before is better where a lane loads several chunks (the 4-way
    // head-sharded rank's apply kernel 1% slower the other way), after is better for the region
    // split, one chunk a lane and a third of its workgroups without angles (the 122880-token
    // YaRN workload 0.7% faster).
    float omega_rev = 0.0f;
    int axis = 0;
    if (!RS && IS3D && tl < D / 2 && !v_wg) {
        omega_rev = a.omega_rev[tl];
        axis = a.axis[tl];
    }

    // The workgroup's first token, and this lane's: a missing second token (odd token count)
    // re-reads the first token's row and stores nothing.
    const int64_t t0 = (int64_t)blk * TPW;
    const bool tok_ok = TPW == 1 || t0 + ts < a.num_tokens;
    const int ts_eff = tok_ok ? ts : 0;
    const int64_t t = t0 + ts_eff;
    // The second token's rows are one stride further: offset = ts * stride_bytes + in-row
    // offset, one 24-bit multiply-add per access (the host picks two tokens per workgroup only
    // for strides below 2^24 bytes). The empty asm hides that ts is 0 or 1, which would
    // otherwise turn the multiply into a select, a copy and an add.
    uint32_t ts_ld = (uint32_t)ts_eff, ts_st = (uint32_t)ts;
    if (TPW == 2) {
        asm("" : "+v"(ts_ld));
        asm("" : "+v"(ts_st));
    }
    {
        // -- loads: every chunk of every slot, and the across-heads weights. Issued
        // unconditionally from one basic block so all are in flight together; an idle slot
        // reads its row's first chunk (in bounds, and read by another lane anyway).
        uint4 x[NSLOT], wa[NSLOT];
        (void)wa;
        {
            // rows of the workgroup's first token (uniform); a second token's row is one token
            // stride further, added to the lane's 32-bit byte offset
            const uint16_t *in_q = a.in[kQ] + t0 * a.in_stride[kQ];
            const uint16_t *in_k = a.in[kK] + t0 * a.in_stride[kK];
            const uint16_t *in_v = NREG == 3 ? a.in[kV] + t0 * a.in_stride[kV] : in_k;
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) {
                const int r = reg[j] < 3 ? reg[j] : 0;
                const uint32_t oh = ok[j] ? 2 * (hoff[j] + off0) : 0u;
                const uint32_t off = TPW == 2 ? __umul24(ts_ld, (uint32_t)(2 * a.in_stride[r])) + oh : oh;
                x[j] = ld16_stream<true>(sel3(r, in_q, in_k, in_v), off);
                if (ACROSS && (SU ? r < 2 : true)) {
                    const uint16_t *w = r == 1 ? a.weight[1] : a.weight[0];
                    wa[j] = ld16(w, (ok[j] && r < 2) ? oh : 0u);
                }
            }
        }
        if (PRIO) __builtin_amdgcn_s_setprio(0);

        if (RS && IS3D && tl < D / 2 && !v_wg) {   // the region split: after the data loads
            omega_rev = a.omega_rev[tl];
            axis = a.axis[tl];
        }

        // -- cos/sin: the table row, or the 3D angle of pair `tid` into LDS
        float cs_c[NPAIR], cs_s[NPAIR];
        if (IS3D) {
            if (!v_wg) {    // a V-only workgroup rotates nothing
                // grid positions of the workgroup's tokens (uniform; t < 2^31); the lane picks
                // its pair's axis below
                uint32_t pf, ph, pw;
                {
                    const uint32_t tt = (uint32_t)t0 + a.token_offset;
                    const uint32_t s = tt - fast_div(tt, a.div_seq.m, a.div_seq.l) * a.seq_len;
                    pf = fast_div(s, a.div_hw.m, a.div_hw.l);
                    const uint32_t rem = s - pf * a.hw;
                    ph = fast_div(rem, a.div_w.m, a.div_w.l);
                    pw = rem - ph * a.ppw;
                }
                if (TPW == 2) {
                    const uint32_t tt = (uint32_t)t0 + 1u + a.token_offset;
                    const uint32_t s = tt - fast_div(tt, a.div_seq.m, a.div_seq.l) * a.seq_len;
                    const uint32_t pf1 = fast_div(s, a.div_hw.m, a.div_hw.l);
                    const uint32_t rem = s - pf1 * a.hw;
                    const uint32_t ph1 = fast_div(rem, a.div_w.m, a.div_w.l);
                    const uint32_t pw1 = rem - ph1 * a.ppw;
                    pf = ts ? pf1 : pf;
                    ph = ts ? ph1 : ph;
                    pw = ts ? pw1 : pw;
                }
                if (tl < D / 2) {               // the host gives every token >= D/2 lanes
                    const uint32_t pos = axis == 0 ? pf : (axis == 1 ? ph : pw);
                    // angle in revolutions, reduced to [0, 1): sin/cos(2*pi*rev) in hardware
                    const float rev = __builtin_amdgcn_fractf((float)pos * omega_rev);
                    const float c = __builtin_amdgcn_cosf(rev) * a.attention_factor;
                    const float sn = __builtin_amdgcn_sinf(rev) * a.attention_factor;
                    f32x2 *cs_tok = s_cs + ts * 2 * CSP;
                    const int slot = (tl % NPAIR) * CSR + tl / NPAIR;
                    cs_tok[CSP + slot] = f32x2{c, sn};
                    if (HALF) cs_tok[slot] = f32x2{c, -sn};
                }
            }
        } else if (XCH) {
            // per element g = 8u + e: angle index g (first half, sign -) or g - R/2 (second
            // half, sign +); elements at or beyond R keep (1, 0). R >= 2 here, so the loads are
            // issued unconditionally (index 0 where the element is not rotated).
            const int half = R / 2;
#pragma unroll
            for (int e = 0; e < NPAIR; ++e) {
                const int g = 8 * u + e;
                const bool on = unit_ok && g < R;
                const int i = on ? (g < half ? g : g - half) : 0;
                float c, sn;
                {
                    if (SRC == kSrcTableF32) {
                        c = (static_cast<const float *>(a.table_cos) + t * a.cos_stride)[i];
                        sn = (static_cast<const float *>(a.table_sin) + t * a.sin_stride)[i];
                    } else {
                        const uint16_t cb = (static_cast<const uint16_t *>(a.table_cos) + t * a.cos_stride)[i];
                        const uint16_t sb = (static_cast<const uint16_t *>(a.table_sin) + t * a.sin_stride)[i];
                        if (SRC == kSrcTableBF16) {
                            c = __uint_as_float((uint32_t)cb << 16);
                            sn = __uint_as_float((uint32_t)sb << 16);
                        } else {
                            c = (float)__builtin_bit_cast(_Float16, cb);
                            sn = (float)__builtin_bit_cast(_Float16, sb);
                        }
                    }
                }
                cs_c[e] = on ? c : 1.0f;
                cs_s[e] = on ? (g < half ? -sn : sn) : 0.0f;
            }
        } else if (!XCH && a.table_vec) {
            // A lane's NPAIR pairs lie all below R/2 or all at/above it (NPAIR divides R/2), and
            // the rows are aligned: one or two vector loads per table, issued unconditionally
            // (a lane without rotated pairs reads pair 0 and discards it).
            const bool on = unit_ok && rotated;
            const int64_t i0 = on ? pair0 : 0;
            if (SRC == kSrcTableF32) {
                const f32x4 *cp = reinterpret_cast<const f32x4 *>(
                    static_cast<const float *>(a.table_cos) + t * a.cos_stride + i0);
                const f32x4 *sp = reinterpret_cast<const f32x4 *>(
                    static_cast<const float *>(a.table_sin) + t * a.sin_stride + i0);
#pragma unroll
                for (int v = 0; v < NPAIR / 4; ++v) {
                    const f32x4 c = cp[v], sn = sp[v];
                    cs_c[4 * v + 0] = c.x; cs_c[4 * v + 1] = c.y;
                    cs_c[4 * v + 2] = c.z; cs_c[4 * v + 3] = c.w;
                    cs_s[4 * v + 0] = sn.x; cs_s[4 * v + 1] = sn.y;
                    cs_s[4 * v + 2] = sn.z; cs_s[4 * v + 3] = sn.w;
                }
            } else {
                const uint16_t *cp = static_cast<const uint16_t *>(a.table_cos) + t * a.cos_stride + i0;
                const uint16_t *sp = static_cast<const uint16_t *>(a.table_sin) + t * a.sin_stride + i0;
                uint32_t cw[NPAIR / 2], sw[NPAIR / 2];
                if (NPAIR == 8) {
                    const u32x4 c = *reinterpret_cast<const u32x4 *>(cp);
                    const u32x4 sn = *reinterpret_cast<const u32x4 *>(sp);
                    cw[0] = c.x; cw[1] = c.y; cw[NPAIR / 2 - 2] = c.z; cw[NPAIR / 2 - 1] = c.w;
                    sw[0] = sn.x; sw[1] = sn.y; sw[NPAIR / 2 - 2] = sn.z; sw[NPAIR / 2 - 1] = sn.w;
                } else {
                    const u32x2 c = *reinterpret_cast<const u32x2 *>(cp);
                    const u32x2 sn = *reinterpret_cast<const u32x2 *>(sp);
                    cw[0] = c.x; cw[1] = c.y;
                    sw[0] = sn.x; sw[1] = sn.y;
                }
#pragma unroll
                for (int v = 0; v < NPAIR / 2; ++v) {
                    if (SRC == kSrcTableBF16) {
                        cs_c[2 * v] = bf16_lo(cw[v]); cs_c[2 * v + 1] = bf16_hi(cw[v]);
                        cs_s[2 * v] = bf16_lo(sw[v]); cs_s[2 * v + 1] = bf16_hi(sw[v]);
                    } else {
                        const f32x2 c = f16x2_to_f32(cw[v]), sn = f16x2_to_f32(sw[v]);
                        cs_c[2 * v] = c.x; cs_c[2 * v + 1] = c.y;
                        cs_s[2 * v] = sn.x; cs_s[2 * v + 1] = sn.y;
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < NPAIR; ++e) {
                cs_c[e] = on ? cs_c[e] : 1.0f;
                cs_s[e] = on ? (HALF ? cs_s[e] * half_sign : cs_s[e]) : 0.0f;
            }
        } else if (unit_ok && rotated) {
            const int half = R / 2;
#pragma unroll
            for (int e = 0; e < NPAIR; ++e) {
                const int i = pair0 + e;
                float c = 1.0f, sn = 0.0f;
                if (HALF || i < half) {
                    if (SRC == kSrcTableF32) {
                        c = (static_cast<const float *>(a.table_cos) + t * a.cos_stride)[i];
                        sn = (static_cast<const float *>(a.table_sin) + t * a.sin_stride)[i];
                    } else {
                        const uint16_t cb = (static_cast<const uint16_t *>(a.table_cos) + t * a.cos_stride)[i];
                        const uint16_t sb = (static_cast<const uint16_t *>(a.table_sin) + t * a.sin_stride)[i];
                        if (SRC == kSrcTableBF16) {
                            c = __uint_as_float((uint32_t)cb << 16);
                            sn = __uint_as_float((uint32_t)sb << 16);
                        } else {
                            c = (float)__builtin_bit_cast(_Float16, cb);
                            sn = (float)__builtin_bit_cast(_Float16, sb);
                        }
                    }
                }
                cs_c[e] = c;
                cs_s[e] = HALF ? sn * half_sign : sn;
            }
        }

        // -- sums of squares (Q and K slots only)
        float ss[NSLOT];
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) {
            ss[j] = 0.0f;
            if ((NORM == kNormPerHead || NORM == kNormAcross) && !v_wg) {
                const float v = sumsq_packed<ACT>(x[j], 0.0f);
                ss[j] = (ok[j] && reg[j] < 2) ? v : 0.0f;
            }
        }
        if (NORM == kNormPerHead) {
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) ss[j] = group_sum(ss[j], L);
        } else if (NORM == kNormAcross && !v_wg) {
            float sq = -0.0f, sk = -0.0f;           // x + -0 == x for every x: folds away
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) {
                sq += reg[j] == kQ ? ss[j] : 0.0f;
                sk += reg[j] == kK ? ss[j] : 0.0f;
            }
            // Q's and K's sums through one tree: after the row pairing the first row of each
            // 32-lane group carries Q, the second K. Per 32-lane group with two tokens (each
            // group belongs to one), per wave with one.
            float v = group_sum(pair_rows_add(sq, sk), 16);
            if (TPW == 1) v = swap32_add(v);
            // lane 0 of the group (or wave) holds Q's sum, lane 16 K's: s_red[g] = (Q, K)
            if ((tid & 15) == 0 && (TPW == 2 || (tid & 32) == 0))
                s_redf[2 * (tid >> (TPW == 1 ? 6 : 5)) + ((tid >> 4) & 1)] = v;
        }

        if (NEED_BARRIER && !v_wg) __syncthreads();   // v_wg is uniform

        float rq = 1.0f, rk = 1.0f;
        if (v_wg) {
            // V only: neither scale is used
        } else if (NORM == kNormAcrossExt) {
            // sums over every head of the token, reduced by the caller (uniform scalar load)
            const f32x2 p = reinterpret_cast<const f32x2 *>(a.sumsq_in)[t];   // per lane's token
            rq = __builtin_amdgcn_rsqf(p.x * a.inv_count[0] + a.eps);
            rk = __builtin_amdgcn_rsqf(p.y * a.inv_count[1] + a.eps);
        } else if (NORM == kNormAcross) {
            // every wave sums its token's partials (its waves', or its 32-lane groups' with two
            // tokens; at most 16 either way): lane w of a group's first row reads partial w's Q
            // sum, of its second row the K sum; one 16-lane tree, then both to every lane
            const int np = TPW == 1 ? (nth >> 6) : (LT >> 5);
            const int g0 = TPW == 1 ? 0 : ts * np;
            const int w = tid & 15;
            const float p = w < np ? s_redf[2 * (g0 + w) + ((tid >> 4) & 1)] : 0.0f;
            const f32x2 s = rows_to_all(group_sum(p, 16));
            rq = __builtin_amdgcn_rsqf(s.x * a.inv_count[0] + a.eps);
            rk = __builtin_amdgcn_rsqf(s.y * a.inv_count[1] + a.eps);
        }
        if (IS3D && unit_ok && !v_wg) {
            // interleaved and second-half lanes read (cos, sin), first-half lanes (cos, -sin);
            // pair0 is a multiple of NPAIR here
            const f32x2 *tab = s_cs + ts * 2 * CSP + (HALF && half_sign < 0.0f ? 0 : CSP) +
                               pair0 / NPAIR;
#pragma unroll
            for (int e = 0; e < NPAIR; ++e) {
                const f32x2 cs = tab[e * CSR];
                cs_c[e] = cs.x;
                cs_s[e] = cs.y;
            }
        }

        // -- every slot's outputs, computed unconditionally (idle slots compute on the chunk
        // they loaded and are not stored): normalise, rotate, round once. V is a bit copy or
        // an E4M3 quantisation.
        uint4 pk[NSLOT];                    // bf16 results (FP8: .xy hold the 8 codes)
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) {
            const bool isv = NREG == 3 && reg[j] == kV;   // compile-time in the region-major layout
            const bool isq = reg[j] == 0;
            if (RS && !FP8 && v_wg) {
                pk[j] = x[j];                           // V: bit copy (uniform branch)
                continue;
            }
            if (FP8 && ACT == kActBF16 && isv && a.v_inv_pow2 != 0.0f) {   // uniform
                // V with a power-of-two scale: v * v_scale is exact, so its code is the scaled
                // packed conversion of the bf16 pairs as they are (it divides by the scale's power
                // of two and rounds to nearest even, but does not saturate). A chunk with a
                // magnitude past 448 / v_scale (an infinity or a NaN included) takes the general
                // path below, which saturates; NaN gets the same code 0xFF on either path.
                const uint4 xv = x[j];
                const u16x2 m = __builtin_elementwise_max(
                    __builtin_elementwise_max(mag16(xv.x), mag16(xv.y)),
                    __builtin_elementwise_max(mag16(xv.z), mag16(xv.w)));
                if ((uint32_t)__builtin_elementwise_max(m.x, m.y) <= a.v_limit_bits) {
                    pk[j] = make_uint4(pack4_e4m3_pow2(xv.x, xv.y, a.v_inv_pow2),
                                       pack4_e4m3_pow2(xv.z, xv.w, a.v_inv_pow2), 0, 0);
                    continue;
                }
            }
            float n[8];
            unpack8<ACT>(x[j], n);
            float scale = FP8 ? (isv ? a.v_scale : a.qk_scale) : 1.0f;
            if (ACROSS && !isv) scale *= isq ? rq : rk;
            if (NORM == kNormPerHead)
                scale *= __builtin_amdgcn_rsqf(ss[j] * (isq ? a.inv_count[0] : a.inv_count[1]) + a.eps);
            if (NORM != kNormNone && !isv) {
                float w[8];
                unpack8<ACT>(ACROSS ? wa[j] : (isq ? wq : wk), w);
#pragma unroll
                for (int i = 0; i < 8; ++i) n[i] *= w[i];
            }
            if (FP8 || !isv) {
#pragma unroll
                for (int i = 0; i < 8; ++i) n[i] *= scale;
            }
            float y[8];
            if (XCH) {
                // every lane stages its normalised chunk in its wave's LDS area, where a head's
                // D values sit contiguously, then reads element g +- R/2 of its own head. Only
                // lanes of one wave touch an area, and LDS executes a wave's accesses in order,
                // so keeping the compiler from moving the accesses (signal fence, wave barrier)
                // suffices.
                float *wx = s_xch + (tid >> 6) * 512;
                const int lane = tid & 63;
#pragma unroll
                for (int i = 0; i < 8; ++i) wx[lane * 8 + i] = n[i];
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                __builtin_amdgcn_wave_barrier();
                const int hb = (lane & ~(L - 1)) * 8;
                const int half = R / 2;
                float np[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int g = 8 * u + e;
                    const int src = g < R ? (g < half ? g + half : g - half) : g;
                    np[e] = wx[hb + src];
                }
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = n[e] * cs_c[e] + np[e] * cs_s[e];
            } else if (HALF) {
                // partner chunk's normalised values (all lanes take part in the permute)
                float np[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) np[i] = __shfl(n[i], partner, 64);
                const bool rot = rotated && !isv;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    y[e] = rot ? n[e] * cs_c[e] + np[e] * cs_s[e] : n[e];
            } else if (!rotated || isv) {
#pragma unroll
                for (int i = 0; i < 8; ++i) y[i] = n[i];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float xa = n[2 * e], xb = n[2 * e + 1];
                    const bool on = IS3D || pair0 + e < R / 2;
                    y[2 * e] = on ? xa * cs_c[e] - xb * cs_s[e] : xa;
                    y[2 * e + 1] = on ? xb * cs_c[e] + xa * cs_s[e] : xb;
                }
            }
            if (FP8) {
                const uint2 c = pack8_e4m3(y);
                pk[j] = make_uint4(c.x, c.y, 0, 0);
            } else if (isv) {
                pk[j] = x[j];                           // V: bit copy
            } else {
                pk[j] = pack8<ACT>(y);
            }
        }

        // -- all stores last
        uint8_t *out_q = static_cast<uint8_t *>(a.out[kQ]) + t0 * a.out_stride[kQ] * ESIZE;
        uint8_t *out_k = static_cast<uint8_t *>(a.out[kK]) + t0 * a.out_stride[kK] * ESIZE;
        uint8_t *out_v = NREG == 3 ? static_cast<uint8_t *>(a.out[kV]) + t0 * a.out_stride[kV] * ESIZE
                                   : out_k;
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) {
            if (!ok[j] || !tok_ok) continue;
            const int r = reg[j] < 3 ? reg[j] : 0;
            const uint32_t in_row = (hoff[j] + off0) * ESIZE;
            const uint32_t off = TPW == 2 ? __umul24(ts_st, (uint32_t)(a.out_stride[r] * ESIZE)) + in_row : in_row;
            // region-major slots: the region, so the base, is compile-time; mixed: per lane
            if (FP8) st8_stream<SU>(sel3(reg[j], out_q, out_k, out_v), off, make_uint2(pk[j].x, pk[j].y), a.store_device);
            else st16_stream<SU>(sel3(reg[j], out_q, out_k, out_v), off, pk[j], a.store_device);
        }
    }
}

// ---- per-token sums of squares (first phase of a head-sharded across-heads norm) -----------
//
// One workgroup per token; lane tid covers chunks tid + i*nth (i < NI) of the token's
// contiguous Q|K span. Loads are issued unconditionally (clamped to chunk 0, then discarded),
// then the Q and K partial sums are reduced per wave with DPP/permlane and across waves in LDS.
template <int NI>
__global__ void __launch_bounds__(1024) qkrope_sumsq_kernel(const SumsqArgs a)
{
    __shared__ f32x2 s_red[16];
    const int tid = threadIdx.x;
    const int nth = blockDim.x;
    const int64_t t = blockIdx.x;           // plain order (measured faster here than XCD runs)
    const uint16_t *row = a.qkv + t * a.row;
    const int nq = a.q_chunks, nall = a.q_chunks + a.k_chunks;
    float sq = 0.0f, sk = 0.0f;
    if (nall > 0) {                 // uniform; with no Q or K heads the row may hold nothing
        uint4 x[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int c = tid + i * nth;
            x[i] = ld16_stream<true>(row, c < nall ? 16u * (uint32_t)c : 0u);
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int c = tid + i * nth;
            const float v = sumsq_packed<kActBF16>(x[i], 0.0f);
            sq += c < nq ? v : 0.0f;
            sk += (c >= nq && c < nall) ? v : 0.0f;
        }
    }
    sq = wave_sum(sq);
    sk = wave_sum(sk);
    if ((tid & 63) == 0) s_red[tid >> 6] = f32x2{sq, sk};
    __syncthreads();
    if (tid < 64) {
        const int w = tid & 15;
        const f32x2 p = w < (nth >> 6) ? s_red[w] : f32x2{0.0f, 0.0f};
        const float q = group_sum(p.x, 16), k = group_sum(p.y, 16);
        if (tid == 0) reinterpret_cast<f32x2 *>(a.out)[t] = f32x2{q, k};
    }
}

// ---- launch helpers ---------------------------------------------------------------------------

template <int DT, int PAIR, int NORM, int SRC, int ACT, bool FP8, int NS, bool SU, int TPW, bool RS>
hipError_t go(const LaunchShape &s, const KernelArgs &a, hipStream_t st)
{
    hipLaunchKernelGGL((qkrope_kernel<DT, PAIR, NORM, SRC, ACT, FP8, NS, SU, TPW, RS>), dim3((unsigned)s.blocks),
                       dim3(s.threads), s.lds_bytes, st, a);
    return hipGetLastError();
}

template <int DT, int PAIR, int NORM, int SRC, int ACT, bool FP8, int NS, bool SU>
hipError_t go_if(const LaunchShape &s, const KernelArgs &a, hipStream_t st)
{
    if constexpr (slots_compiled(SRC == kSrc3D ? 3 : 2, SU, NS)) {
        if (s.split) {
            if constexpr (SU && NS == 1 && SRC == kSrc3D && NORM == kNormNone && !FP8) {
                if (s.tpw != 1) return hipErrorInvalidValue;
                return go<DT, PAIR, NORM, SRC, ACT, FP8, NS, SU, 1, true>(s, a, st);
            } else {
                return hipErrorInvalidValue;
            }
        }
        if constexpr (SU && NS == 1) {
            if (s.tpw == 2) return go<DT, PAIR, NORM, SRC, ACT, FP8, NS, SU, 2, false>(s, a, st);
        }
        if (s.tpw != 1) return hipErrorInvalidValue;
        return go<DT, PAIR, NORM, SRC, ACT, FP8, NS, SU, 1, false>(s, a, st);
    } else {
        return hipErrorInvalidValue;
    }
}

template <int DT, int PAIR, int NORM, int SRC, int ACT, bool FP8>
hipError_t by_slots(const KernelKey &k, const LaunchShape &s, const KernelArgs &a, hipStream_t st)
{
    if (k.slot_uniform) {
        switch (k.slots) {
        case 1: return go_if<DT, PAIR, NORM, SRC, ACT, FP8, 1, true>(s, a, st);
        case 2: return go_if<DT, PAIR, NORM, SRC, ACT, FP8, 2, true>(s, a, st);
        case 3: return go_if<DT, PAIR, NORM, SRC, ACT, FP8, 3, true>(s, a, st);
        case 4: return go_if<DT, PAIR, NORM, SRC, ACT, FP8, 4, true>(s, a, st);
        default: return hipErrorInvalidValue;
        }
    }
    switch (k.slots) {
    case 1: return go_if<DT, PAIR, NORM, SRC, ACT, FP8, 1, false>(s, a, st);
    case 2: return go_if<DT, PAIR, NORM, SRC, ACT, FP8, 2, false>(s, a, st);
    case 4: return go_if<DT, PAIR, NORM, SRC, ACT, FP8, 4, false>(s, a, st);
    default: return hipErrorInvalidValue;
    }
}

template <int DT, int PAIR, int NORM, int SRC, int ACT>
hipError_t by_fp8(const KernelKey &k, const LaunchShape &s, const KernelArgs &a, hipStream_t st)
{
    return k.fp8 ? by_slots<DT, PAIR, NORM, SRC, ACT, true>(k, s, a, st)
                 : by_slots<DT, PAIR, NORM, SRC, ACT, false>(k, s, a, st);
}

// 3D form for one compile-time head_dim: pairing x norm (none / across heads / across heads
// from given sums) x output format. Activations are bf16.
template <int DT, int PAIR>
hipError_t launch_3d_pairing(const KernelKey &k, const LaunchShape &s, const KernelArgs &a, hipStream_t st)
{
    switch (k.norm) {
    case kNormNone: return by_fp8<DT, PAIR, kNormNone, kSrc3D, kActBF16>(k, s, a, st);
    case kNormAcross: return by_fp8<DT, PAIR, kNormAcross, kSrc3D, kActBF16>(k, s, a, st);
    case kNormAcrossExt: return by_fp8<DT, PAIR, kNormAcrossExt, kSrc3D, kActBF16>(k, s, a, st);
    default: return hipErrorInvalidValue;
    }
}

template <int DT>
hipError_t launch_3d(const KernelKey &k, const LaunchShape &s, const KernelArgs &a, hipStream_t st)
{
    if (k.src != kSrc3D || k.head_dim_tpl != DT || k.act != kActBF16) return hipErrorInvalidValue;
    if (k.pairing == kPairHalf) return launch_3d_pairing<DT, kPairHalf>(k, s, a, st);
    if (k.pairing == kPairInterleaved) return launch_3d_pairing<DT, kPairInterleaved>(k, s, a, st);
    return hipErrorInvalidValue;
}

template <int PAIR, int ACT, int NORM>
hipError_t launch_table_src(const KernelKey &k, const LaunchShape &s, const KernelArgs &a, hipStream_t st)
{
    constexpr int SRC16 = ACT == kActBF16 ? kSrcTableBF16 : kSrcTableF16;
    if (k.head_dim_tpl == 128) {
        // E4M3 outputs, head_dim == rotary_dim == 128, one slot per region (see the host)
        if constexpr (PAIR == kPairHalfAny) {
            return hipErrorInvalidValue;
        } else {
            if (!k.fp8 || !k.slot_uniform || k.slots != 1) return hipErrorInvalidValue;
            if (k.src == kSrcTableF32) return go_if<128, PAIR, NORM, kSrcTableF32, ACT, true, 1, true>(s, a, st);
            if (k.src == SRC16) return go_if<128, PAIR, NORM, SRC16, ACT, true, 1, true>(s, a, st);
            return hipErrorInvalidValue;
        }
    }
    if (k.src == kSrcTableF32) return by_fp8<0, PAIR, NORM, kSrcTableF32, ACT>(k, s, a, st);
    if (k.src == SRC16) return by_fp8<0, PAIR, NORM, SRC16, ACT>(k, s, a, st);
    return hipErrorInvalidValue;
}

// Table form (runtime head_dim) for one pairing and activation format: norm mode x table
// dtype (fp32 or the activation format) x output format (activation format or E4M3).
template <int PAIR, int ACT>
hipError_t launch_table(const KernelKey &k, const LaunchShape &s, const KernelArgs &a, hipStream_t st)
{
    if ((k.head_dim_tpl != 0 && k.head_dim_tpl != 128) || k.act != ACT || k.pairing != PAIR)
        return hipErrorInvalidValue;
    switch (k.norm) {
    case kNormNone: return launch_table_src<PAIR, ACT, kNormNone>(k, s, a, st);
    case kNormPerHead: return launch_table_src<PAIR, ACT, kNormPerHead>(k, s, a, st);
    case kNormAcross: return launch_table_src<PAIR, ACT, kNormAcross>(k, s, a, st);
    default: return hipErrorInvalidValue;
    }
}

inline hipError_t launch_sumsq_impl(const SumsqArgs &a, int64_t tokens, int threads, hipStream_t st)
{
    const int n = a.q_chunks + a.k_chunks;
    const int ni = n > 0 ? (n + threads - 1) / threads : 1;   // no Q/K heads: one pass writing 0
    const dim3 grid((unsigned)tokens), block(threads);
    switch (ni) {
    case 1: hipLaunchKernelGGL(qkrope_sumsq_kernel<1>, grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL(qkrope_sumsq_kernel<2>, grid, block, 0, st, a); break;
    case 3:
    case 4: hipLaunchKernelGGL(qkrope_sumsq_kernel<4>, grid, block, 0, st, a); break;
    case 5: case 6: case 7:
    case 8: hipLaunchKernelGGL(qkrope_sumsq_kernel<8>, grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dev
}  // namespace qkrope
