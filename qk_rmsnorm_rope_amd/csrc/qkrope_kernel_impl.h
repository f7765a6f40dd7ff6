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
//   * A workgroup owns whole tokens and walks `tokens_per_block` consecutive ones.
//   * A token's Q, K (and V) rows are cut into units: one 16-byte chunk of 8 bf16 (interleaved
//     pairs never leave a chunk) or, for half-split/NeoX pairing, the two chunks at dims 8m and
//     8m + R/2 that hold both halves of 8 rotation pairs, so no lane needs a neighbour's data.
//     Each head gets L = 2^k >= units-per-head consecutive lanes; lane `tid` owns unit
//     tid mod L of several heads (its slots). Because the workgroup size is a multiple of L,
//     every slot of a lane covers the same dims, so angles and per-head weights are fetched
//     once per lane.
//   * Two slot layouts. Region-major (SU): each region (Q, K, V) has NS slots per lane, slot i
//     covering heads (tid + i*nth)/L of that region; region, base pointers and weights of every
//     slot are compile-time/scalar. Mixed: the regions' units are concatenated and lane-slot j
//     covers unit tid + j*nth of the token, whichever region it falls in (fills the lanes when
//     a region's unit count does not divide the workgroup, e.g. 20 heads of 64).
//   * Sum of squares: per-head norm reduces inside the L lanes of the head with xor shuffles;
//     across-heads norm reduces each wave, then combines the waves through LDS.
//   * 3D angles: lanes k < head_dim/2 compute (cos, sin) of pair k once per token (angle in
//     revolutions, fract, hardware sin/cos), scaled by the attention factor, into LDS; the
//     barrier that publishes them is the one the across-heads reduction needs anyway. LDS is
//     double-buffered by token parity, so one barrier per token suffices.
//   * V units are copied (or E4M3-quantised) and stored before the barrier.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qkrope_internal.h"

namespace qkrope {
namespace dev {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---- number formats ---------------------------------------------------------------------------

// bf16 -> fp32 is exact: the bf16 bits are the upper half of the fp32 pattern.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ void unpack8(const uint4 v, float x[8])
{
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
    x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
    x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}

// Two fp32 -> two bf16 with round-to-nearest-even (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b)
{
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint4 pack8_bf16(const float y[8])
{
    return make_uint4(pack2_bf16(y[0], y[1]), pack2_bf16(y[2], y[3]),
                      pack2_bf16(y[4], y[5]), pack2_bf16(y[6], y[7]));
}

// OCP E4M3 (gfx950's fp8 conversions produce the OCP encoding): finite values beyond the largest
// finite magnitude 448 saturate to +-448, NaN stays NaN (the comparison is false for NaN), and
// the hardware conversion rounds to nearest even.
__device__ __forceinline__ float sat_e4m3(float y)
{
    return __builtin_fabsf(y) > 448.0f ? __builtin_copysignf(448.0f, y) : y;
}

__device__ __forceinline__ uint2 pack8_e4m3(const float y[8])
{
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(y[0]), sat_e4m3(y[1]), 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(y[2]), sat_e4m3(y[3]), lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(y[4]), sat_e4m3(y[5]), 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(y[6]), sat_e4m3(y[7]), hi, true);
    return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// ---- memory -----------------------------------------------------------------------------------

// 16-byte load at a (usually uniform) base plus a 32-bit unsigned byte offset, the form the
// global_load saddr+voffset encoding takes: one VGPR per address.
__device__ __forceinline__ uint4 ld16(const void *base, uint32_t byte_off)
{
    return *reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(base) + byte_off);
}

// Store 8 outputs (16 bytes of bf16 or 8 bytes of E4M3) at element `elem` of a row.
template <bool FP8>
__device__ __forceinline__ void store8(uint8_t *row, uint32_t elem, const float y[8])
{
    if (FP8) {
        *reinterpret_cast<uint2 *>(row + elem) = pack8_e4m3(y);
    } else {
        *reinterpret_cast<uint4 *>(row + 2 * elem) = pack8_bf16(y);
    }
}

// n / d for n < 2^31 with a host-computed magic pair (m, l): q = (mulhi(n, m) + n) >> l.
__device__ __forceinline__ uint32_t fast_div(uint32_t n, uint32_t m, uint32_t l)
{
    return (__umulhi(n, m) + n) >> l;
}

template <typename T>
__device__ __forceinline__ T sel3(int r, T a, T b, T c) { return r == 0 ? a : (r == 1 ? b : c); }

// ---- reductions -------------------------------------------------------------------------------

// Sum over aligned groups of `width` lanes (a power of two <= 64) with xor butterflies.
__device__ __forceinline__ float group_sum(float v, int width)
{
    for (int off = width >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ float sumsq8(const float x[8])
{
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s = __builtin_fmaf(x[i], x[i], s);
    return s;
}

// ---- the kernel -------------------------------------------------------------------------------

// DT: head_dim as a compile-time constant (64/128/256), or 0 to read it from the arguments.
// HALF: half-split (NeoX) pairing; otherwise interleaved. NORM: kNormNone/PerHead/Across.
// SRC: cos/sin from a fp32 or bf16 table, or computed (3D). FP8: E4M3 outputs.
// SU: region-major slots (NS per region); otherwise mixed slots (NS in all).
template <int DT, bool HALF, int NORM, int SRC, bool FP8, int NS, bool SU>
__global__ void __launch_bounds__(1024) qkrope_kernel(const KernelArgs a)
{
    constexpr bool IS3D = (SRC == kSrc3D);
    constexpr int NREG = IS3D ? 3 : 2;          // regions: Q, K (, V)
    constexpr int NSLOT = SU ? NREG * NS : NS;
    constexpr int NPAIR = HALF ? 8 : 4;         // rotation pairs per unit
    constexpr bool NEED_BARRIER = IS3D || NORM == kNormAcross;
    constexpr int ESIZE = FP8 ? 1 : 2;          // output bytes per element

    __shared__ f32x2 s_cs[IS3D ? 2 : 1][IS3D ? kMaxPairs : 1];
    __shared__ f32x2 s_red[NORM == kNormAcross ? 2 : 1][16];

    const int D = DT > 0 ? DT : a.head_dim;
    const int R = IS3D ? D : a.rotary_dim;
    const int units = HALF ? D / 16 : D / 8;
    const int L = DT > 0 ? units : a.lanes_per_head;
    const int lgL = __builtin_ctz(L);
    const int P = HALF ? R / 16 : 0;            // rotated chunk pairs per head (half-split)
    const int tid = threadIdx.x;
    const int nth = blockDim.x;
    const int u = tid & (L - 1);
    const bool unit_ok = u < units;

    // Element offsets of this lane's unit inside a head, and whether it is rotated.
    uint32_t off0, off1;
    bool rotated;
    if (HALF) {
        rotated = u < P;
        off0 = rotated ? 8 * u : 16 * u;        // pass-through units take chunk pairs 2u, 2u+1
        off1 = rotated ? 8 * (u + P) : 16 * u + 8;
    } else {
        rotated = 8 * u < R;
        off0 = 8 * u;
        off1 = 0;
    }
    const int pair0 = HALF ? 8 * u : 4 * u;     // first rotation pair (angle index) of the unit

    // Slot -> region (3 = idle) and the element offset of the slot's head inside its region row.
    const int Hq = a.heads[kQ], Hk = a.heads[kK], Hv = NREG == 3 ? a.heads[kV] : 0;
    int reg[NSLOT];
    uint32_t hoff[NSLOT];
    bool ok[NSLOT];
#pragma unroll
    for (int j = 0; j < NSLOT; ++j) {
        if (SU) {
            const int r = j / NS;                       // compile-time after unrolling
            const int hh = (tid + (j % NS) * nth) >> lgL;
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

    // Per-head norm weights ([head_dim], shared by every head) stay packed in registers.
    uint4 wq0 = make_uint4(0, 0, 0, 0), wq1 = wq0, wk0 = wq0, wk1 = wq0;
    if (NORM == kNormPerHead && unit_ok) {
        if (Hq > 0) {
            wq0 = ld16(a.weight[0], 2 * off0);
            if (HALF) wq1 = ld16(a.weight[0], 2 * off1);
        }
        if (Hk > 0) {
            wk0 = ld16(a.weight[1], 2 * off0);
            if (HALF) wk1 = ld16(a.weight[1], 2 * off1);
        }
    }

    // 3D: this lane's pair (tid < D/2) frequency in revolutions and its position axis.
    float omega_rev = 0.0f;
    int axis = 0;
    if (IS3D && tid < D / 2) {
        omega_rev = a.omega_rev[tid];
        axis = a.axis[tid];
    }

    const int64_t t_begin = (int64_t)blockIdx.x * a.tokens_per_block;
    int64_t t_end = t_begin + a.tokens_per_block;
    if (t_end > a.num_tokens) t_end = a.num_tokens;

    int buf = 0;
    for (int64_t t = t_begin; t < t_end; ++t, buf ^= 1) {
        // Row bases of this token (scalar).
        const uint16_t *in_q = a.in[kQ] + t * a.in_stride[kQ];
        const uint16_t *in_k = a.in[kK] + t * a.in_stride[kK];
        const uint16_t *in_v = NREG == 3 ? a.in[kV] + t * a.in_stride[kV] : in_k;
        uint8_t *out_q = static_cast<uint8_t *>(a.out[kQ]) + t * a.out_stride[kQ] * ESIZE;
        uint8_t *out_k = static_cast<uint8_t *>(a.out[kK]) + t * a.out_stride[kK] * ESIZE;
        uint8_t *out_v = NREG == 3 ? static_cast<uint8_t *>(a.out[kV]) + t * a.out_stride[kV] * ESIZE
                                   : out_k;

        // -- load every unit of the token, and across-heads weights (all in flight before use)
        uint4 x0[NSLOT], x1[NSLOT], wa0[NSLOT], wa1[NSLOT];
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) {
            if (ok[j]) {
                const int r = reg[j];
                const uint16_t *row = sel3(r, in_q, in_k, in_v);
                x0[j] = ld16(row, 2 * (hoff[j] + off0));
                if (HALF) x1[j] = ld16(row, 2 * (hoff[j] + off1));
                if (NORM == kNormAcross && r < 2) {
                    const uint16_t *w = r == 0 ? a.weight[0] : a.weight[1];
                    wa0[j] = ld16(w, 2 * (hoff[j] + off0));
                    if (HALF) wa1[j] = ld16(w, 2 * (hoff[j] + off1));
                }
            }
        }

        // -- cos/sin: the table row, or the 3D angle of pair `tid` into LDS
        float cs_c[NPAIR], cs_s[NPAIR];
        if (IS3D) {
            // grid position of the token (uniform across the workgroup; t < 2^31)
            const uint32_t tt = (uint32_t)t;
            const uint32_t s = tt - fast_div(tt, a.div_seq.m, a.div_seq.l) * a.seq_len;
            const uint32_t pf = fast_div(s, a.div_hw.m, a.div_hw.l);
            const uint32_t rem = s - pf * a.hw;
            const uint32_t ph = fast_div(rem, a.div_w.m, a.div_w.l);
            const uint32_t pw = rem - ph * a.ppw;
            if (tid < D / 2) {
                const uint32_t pos = axis == 0 ? pf : (axis == 1 ? ph : pw);
                // angle in revolutions, reduced to [0, 1): sin/cos(2*pi*rev) in hardware
                const float rev = __builtin_amdgcn_fractf((float)pos * omega_rev);
                s_cs[buf][tid] = f32x2{__builtin_amdgcn_cosf(rev) * a.attention_factor,
                                       __builtin_amdgcn_sinf(rev) * a.attention_factor};
            }
        } else if (unit_ok && rotated) {
            const int half = R / 2;
            const int64_t trow = t * a.table_stride;
#pragma unroll
            for (int e = 0; e < NPAIR; ++e) {
                const int i = pair0 + e;
                float c = 1.0f, s = 0.0f;
                if (HALF || i < half) {
                    if (SRC == kSrcTableF32) {
                        const float *tab = static_cast<const float *>(a.table) + trow;
                        c = tab[i];
                        s = tab[half + i];
                    } else {
                        const uint16_t *tab = static_cast<const uint16_t *>(a.table) + trow;
                        c = __uint_as_float((uint32_t)tab[i] << 16);
                        s = __uint_as_float((uint32_t)tab[half + i] << 16);
                    }
                }
                cs_c[e] = c;
                cs_s[e] = s;
            }
        }

        // -- sum of squares
        float ss[NSLOT];
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) {
            ss[j] = 0.0f;
            if (NORM != kNormNone && ok[j] && reg[j] < 2) {
                float x[8];
                unpack8(x0[j], x);
                ss[j] = sumsq8(x);
                if (HALF) {
                    unpack8(x1[j], x);
                    ss[j] += sumsq8(x);
                }
            }
        }
        if (NORM == kNormPerHead) {
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) ss[j] = group_sum(ss[j], L);
        } else if (NORM == kNormAcross) {
            float sq = 0.0f, sk = 0.0f;
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) {
                sq += reg[j] == kQ ? ss[j] : 0.0f;
                sk += reg[j] == kK ? ss[j] : 0.0f;
            }
            sq = group_sum(sq, 64);
            sk = group_sum(sk, 64);
            if ((tid & 63) == 0) s_red[buf][tid >> 6] = f32x2{sq, sk};
        }

        // -- V: copy or quantise, no dependence on the reductions
        if (NREG == 3) {
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) {
                if (!(ok[j] && reg[j] == kV)) continue;
                uint8_t *vrow = out_v;
                if (FP8) {
                    float x[8];
                    unpack8(x0[j], x);
#pragma unroll
                    for (int i = 0; i < 8; ++i) x[i] *= a.v_scale;
                    store8<true>(vrow, hoff[j] + off0, x);
                    if (HALF) {
                        unpack8(x1[j], x);
#pragma unroll
                        for (int i = 0; i < 8; ++i) x[i] *= a.v_scale;
                        store8<true>(vrow, hoff[j] + off1, x);
                    }
                } else {
                    *reinterpret_cast<uint4 *>(vrow + 2 * (hoff[j] + off0)) = x0[j];
                    if (HALF) *reinterpret_cast<uint4 *>(vrow + 2 * (hoff[j] + off1)) = x1[j];
                }
            }
        }

        if (NEED_BARRIER) __syncthreads();

        float rq = 1.0f, rk = 1.0f;
        if (NORM == kNormAcross) {
            float sq = 0.0f, sk = 0.0f;
            const int nw = nth >> 6;
            for (int w = 0; w < nw; ++w) {
                const f32x2 p = s_red[buf][w];
                sq += p.x;
                sk += p.y;
            }
            rq = __builtin_amdgcn_rsqf(sq * a.inv_count[0] + a.eps);
            rk = __builtin_amdgcn_rsqf(sk * a.inv_count[1] + a.eps);
        }
        if (IS3D && unit_ok) {
#pragma unroll
            for (int e = 0; e < NPAIR; ++e) {
                const f32x2 cs = s_cs[buf][pair0 + e];
                cs_c[e] = cs.x;
                cs_s[e] = cs.y;
            }
        }

        // -- Q and K: normalise, rotate, round once, store
#pragma unroll
        for (int j = 0; j < NSLOT; ++j) {
            if (!ok[j] || reg[j] >= 2) continue;
            const bool isq = reg[j] == 0;
            float scale = FP8 ? a.qk_scale : 1.0f;
            if (NORM == kNormAcross) scale *= isq ? rq : rk;
            if (NORM == kNormPerHead)
                scale *= __builtin_amdgcn_rsqf(ss[j] * (isq ? a.inv_count[0] : a.inv_count[1]) + a.eps);

            float n0[8], n1[8];
            unpack8(x0[j], n0);
            if (HALF) unpack8(x1[j], n1);
            if (NORM != kNormNone) {
                float w[8];
                unpack8(NORM == kNormAcross ? wa0[j] : (isq ? wq0 : wk0), w);
#pragma unroll
                for (int i = 0; i < 8; ++i) n0[i] *= w[i];
                if (HALF) {
                    unpack8(NORM == kNormAcross ? wa1[j] : (isq ? wq1 : wk1), w);
#pragma unroll
                    for (int i = 0; i < 8; ++i) n1[i] *= w[i];
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                n0[i] *= scale;
                if (HALF) n1[i] *= scale;
            }

            float y0[8], y1[8];
            if (!rotated) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    y0[i] = n0[i];
                    if (HALF) y1[i] = n1[i];
                }
            } else if (HALF) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    y0[e] = n0[e] * cs_c[e] - n1[e] * cs_s[e];
                    y1[e] = n1[e] * cs_c[e] + n0[e] * cs_s[e];
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float xa = n0[2 * e], xb = n0[2 * e + 1];
                    const bool on = IS3D || pair0 + e < R / 2;
                    y0[2 * e] = on ? xa * cs_c[e] - xb * cs_s[e] : xa;
                    y0[2 * e + 1] = on ? xb * cs_c[e] + xa * cs_s[e] : xb;
                }
            }

            uint8_t *orow = isq ? out_q : out_k;
            store8<FP8>(orow, hoff[j] + off0, y0);
            if (HALF) store8<FP8>(orow, hoff[j] + off1, y1);
        }
    }
}

// ---- launch helpers ---------------------------------------------------------------------------

template <int DT, bool HALF, int NORM, int SRC, bool FP8, int NS, bool SU>
hipError_t go(const LaunchShape &s, const KernelArgs &a, hipStream_t st)
{
    hipLaunchKernelGGL((qkrope_kernel<DT, HALF, NORM, SRC, FP8, NS, SU>), dim3((unsigned)s.blocks),
                       dim3(s.threads), 0, st, a);
    return hipGetLastError();
}

template <int DT, bool HALF, int NORM, int SRC, bool FP8, int NS, bool SU>
hipError_t go_if(const LaunchShape &s, const KernelArgs &a, hipStream_t st)
{
    if constexpr (slots_compiled(SRC == kSrc3D ? 3 : 2, HALF, SU, NS))
        return go<DT, HALF, NORM, SRC, FP8, NS, SU>(s, a, st);
    else
        return hipErrorInvalidValue;
}

template <int DT, bool HALF, int NORM, int SRC, bool FP8>
hipError_t by_slots(const KernelKey &k, const LaunchShape &s, const KernelArgs &a, hipStream_t st)
{
    if (k.slot_uniform) {
        switch (k.slots) {
        case 1: return go_if<DT, HALF, NORM, SRC, FP8, 1, true>(s, a, st);
        case 2: return go_if<DT, HALF, NORM, SRC, FP8, 2, true>(s, a, st);
        case 3: return go_if<DT, HALF, NORM, SRC, FP8, 3, true>(s, a, st);
        case 4: return go_if<DT, HALF, NORM, SRC, FP8, 4, true>(s, a, st);
        default: return hipErrorInvalidValue;
        }
    }
    switch (k.slots) {
    case 1: return go_if<DT, HALF, NORM, SRC, FP8, 1, false>(s, a, st);
    case 2: return go_if<DT, HALF, NORM, SRC, FP8, 2, false>(s, a, st);
    case 4: return go_if<DT, HALF, NORM, SRC, FP8, 4, false>(s, a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace dev
}  // namespace qkrope

namespace qkrope {
namespace dev {

// 3D form for one compile-time head_dim: pairing x norm (none / across heads) x output dtype.
template <int DT>
hipError_t launch_3d(const KernelKey &k, const LaunchShape &s, const KernelArgs &a, hipStream_t st)
{
    if (k.src != kSrc3D || k.head_dim_tpl != DT) return hipErrorInvalidValue;
    if (k.norm == kNormAcross) {
        if (k.half_split)
            return k.fp8 ? by_slots<DT, true, kNormAcross, kSrc3D, true>(k, s, a, st)
                         : by_slots<DT, true, kNormAcross, kSrc3D, false>(k, s, a, st);
        return k.fp8 ? by_slots<DT, false, kNormAcross, kSrc3D, true>(k, s, a, st)
                     : by_slots<DT, false, kNormAcross, kSrc3D, false>(k, s, a, st);
    }
    if (k.norm == kNormNone) {
        if (k.half_split)
            return k.fp8 ? by_slots<DT, true, kNormNone, kSrc3D, true>(k, s, a, st)
                         : by_slots<DT, true, kNormNone, kSrc3D, false>(k, s, a, st);
        return k.fp8 ? by_slots<DT, false, kNormNone, kSrc3D, true>(k, s, a, st)
                     : by_slots<DT, false, kNormNone, kSrc3D, false>(k, s, a, st);
    }
    return hipErrorInvalidValue;
}

template <bool HALF, int NORM>
hipError_t launch_table_src(const KernelKey &k, const LaunchShape &s, const KernelArgs &a, hipStream_t st)
{
    if (k.src == kSrcTableF32) return by_slots<0, HALF, NORM, kSrcTableF32, false>(k, s, a, st);
    if (k.src == kSrcTableBF16) return by_slots<0, HALF, NORM, kSrcTableBF16, false>(k, s, a, st);
    return hipErrorInvalidValue;
}

// Table form (runtime head_dim, bf16 outputs): pairing x norm mode x table dtype.
template <bool HALF>
hipError_t launch_table(const KernelKey &k, const LaunchShape &s, const KernelArgs &a, hipStream_t st)
{
    if (k.head_dim_tpl != 0 || k.fp8) return hipErrorInvalidValue;
    switch (k.norm) {
    case kNormNone: return launch_table_src<HALF, kNormNone>(k, s, a, st);
    case kNormPerHead: return launch_table_src<HALF, kNormPerHead>(k, s, a, st);
    case kNormAcross: return launch_table_src<HALF, kNormAcross>(k, s, a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace dev
}  // namespace qkrope
