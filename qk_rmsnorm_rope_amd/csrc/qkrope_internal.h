// Internal interface between the C-ABI host code (qkrope_api.cpp) and the kernel family
// (qkrope_kernel_impl.h, instantiated by the qkrope_kernels_*.hip translation units). Not
// installed; the public interface is include/qkrope.h.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace qkrope {

constexpr int kMaxPairs = 128;      // head_dim/2 for head_dim <= 256

enum Region { kQ = 0, kK = 1, kV = 2 };
// kNormAcrossExt: across-heads norm whose per-token sums of squares are read from memory
// (sums over every head of a head-sharded problem, reduced by the caller).
enum Norm { kNormNone = 0, kNormPerHead = 1, kNormAcross = 2, kNormAcrossExt = 3 };
enum RopeSrc { kSrcTableF32 = 0, kSrcTableBF16 = 1, kSrcTableF16 = 2, kSrc3D = 3 };
enum Act { kActBF16 = 0, kActF16 = 1 };   // 16-bit activation (and weight) format
// Rotation pairing: interleaved (2i, 2i+1); half-split (d, d + R/2) with R/2 a multiple of 8, so
// partners are whole 16-byte chunks; half-split with any even R, partners exchanged through LDS.
enum Pairing { kPairInterleaved = 0, kPairHalf = 1, kPairHalfAny = 2 };

// Magic pair for n / d with n < 2^31: q = (mulhi(n, m) + n) >> l.
struct FastDiv {
    uint32_t m, l;
};

// Everything one launch needs. Passed by value as the kernel argument; host code fills it.
struct KernelArgs {
    // Regions Q, K, V: token t of region r starts at in[r] + t*in_stride[r] (16-bit activation
    // elements) and its output at out[r] + t*out_stride[r] (output elements: 16-bit, or e4m3
    // bytes).
    const uint16_t *in[3];
    void *out[3];
    int64_t in_stride[3];
    int64_t out_stride[3];
    int heads[3];              // Hq, Hk, Hv (Hv = 0: no V region)
    const uint16_t *weight[2]; // q, k norm weights (activation format) or null
    const void *table_cos;     // table form: row t holds cos(theta_t,i), i < R/2 (table dtype)
    const void *table_sin;     // table form: row t holds sin(theta_t,i)
    int64_t cos_stride;        // token strides of the two tables, elements
    int64_t sin_stride;
    int table_vec;             // rows aligned for whole-vector reads of a lane's pairs (uniform)
    const float *sumsq_in;     // kNormAcrossExt: [T, 2] sums of squares of Q and K rows

    int64_t num_tokens;        // tokens; the grid has one workgroup per token (per 2 with TPW 2)
    uint32_t xcd_group;        // 0: block b takes token block b; G > 0 (a power of two): XCD runs
    uint32_t xcd_lg;           // log2 G (0 when off)
    uint32_t xcd_full;         // blocks below this (whole runs of 8G) are renumbered; 0 when off
    uint32_t store_device;     // 1: streamed stores at device scope (large launches), 0: nt only
    int head_dim;              // D
    int rotary_dim;            // R (== D for the 3D form)
    int lanes_per_head;        // L: power of two >= head_dim / 8 (16-byte chunks per head)
    float eps;
    float inv_count[2];        // 1 / (elements the Q, K norm averages over)
    float qk_scale;            // FP8 scale for Q/K outputs (1 for bf16)
    float v_scale;             // FP8 scale for V (1 for bf16)
    // E4M3 V with v_scale = 2^k, |k| <= 20 (bf16 activations): 1 / v_scale for the scaled packed
    // conversion, and the bf16 pattern of 448 / v_scale, the largest magnitude it takes without
    // saturating; 0 and 0 send V through the general path
    float v_inv_pow2;
    uint32_t v_limit_bits;

    // 3D positions of token t: s = (token_offset + t) mod seq_len; f = s / hw;
    // h = (s / ppw) mod pph; w = s mod ppw.
    uint32_t token_offset;
    uint32_t seq_len, hw, ppw, pph;
    FastDiv div_seq, div_hw, div_w;   // for n / seq_len, n / hw, n / ppw
    float attention_factor;
    float omega_rev[kMaxPairs];    // per pair k: omega'_k / (2*pi), revolutions per position
    uint8_t axis[kMaxPairs];       // per pair k: 0 frame, 1 height, 2 width
};

// Launch shape chosen by the host for one call.
struct LaunchShape {
    int threads;        // workgroup size, multiple of 64, <= 1024
    int slots;          // slots per region (region-major) or per lane (mixed)
    bool slot_uniform;  // region-major slot layout
    int64_t blocks;     // grid size (set per launch by the host's launch loop)
    int lds_bytes;      // dynamic LDS per workgroup (kPairHalfAny: threads * 32)
    int tpw;            // tokens per workgroup: 1, or 2 (region-major, one slot per region)
    bool split;         // one region of one token per workgroup (region-major, tpw 1)
};

// Kernel selection keys.
struct KernelKey {
    int head_dim_tpl;   // 64/128/256 for the 3D kernels; table form: 0 = run-time head_dim, 128 =
                        // E4M3 outputs with head_dim == rotary_dim == 128, one slot per region
    int pairing;        // Pairing
    int norm;           // Norm
    int src;            // RopeSrc
    int act;            // Act
    bool fp8;
    int slots;          // slots per region (region-major) or per lane (mixed)
    bool slot_uniform;  // region-major slot layout
};

// Per-translation-unit launchers. Each returns hipSuccess or the launch error, and
// hipErrorInvalidValue if no compiled kernel matches `key`.
hipError_t launch_3d_d64(const KernelKey &key, const LaunchShape &shape, const KernelArgs &args, hipStream_t stream);
hipError_t launch_3d_d128(const KernelKey &key, const LaunchShape &shape, const KernelArgs &args, hipStream_t stream);
hipError_t launch_3d_d256(const KernelKey &key, const LaunchShape &shape, const KernelArgs &args, hipStream_t stream);
hipError_t launch_table_interleaved_bf16(const KernelKey &key, const LaunchShape &shape, const KernelArgs &args, hipStream_t stream);
hipError_t launch_table_halfsplit_bf16(const KernelKey &key, const LaunchShape &shape, const KernelArgs &args, hipStream_t stream);
hipError_t launch_table_interleaved_f16(const KernelKey &key, const LaunchShape &shape, const KernelArgs &args, hipStream_t stream);
hipError_t launch_table_halfsplit_f16(const KernelKey &key, const LaunchShape &shape, const KernelArgs &args, hipStream_t stream);
hipError_t launch_table_halfsplit_any_bf16(const KernelKey &key, const LaunchShape &shape, const KernelArgs &args, hipStream_t stream);
hipError_t launch_table_halfsplit_any_f16(const KernelKey &key, const LaunchShape &shape, const KernelArgs &args, hipStream_t stream);

// Per-token sums of squares of the Q and K rows of packed QKV: out[2t] = sum over the
// token's q_elems Q values of x^2, out[2t+1] the same over its k_elems K values (fp32).
struct SumsqArgs {
    const uint16_t *qkv;
    float *out;
    int64_t row;           // elements per token row of qkv
    int q_chunks, k_chunks; // 16-byte chunks of the Q and K regions (contiguous, Q first)
};
hipError_t launch_sumsq(const SumsqArgs &args, int64_t tokens, int threads, hipStream_t stream);

// Slot counts the kernels are compiled for: region-major 1..4 slots per region, mixed 1, 2, 4
// slots per lane, limited so that a lane holds at most kMaxChunks 16-byte chunks per token.
constexpr int kMaxSlotsRegionMajor = 4;
constexpr int kMixedSlots[] = {1, 2, 4};
constexpr int kMaxChunks = 8;

constexpr bool slots_compiled(int nreg, bool region_major, int ns)
{
    return (region_major ? ns >= 1 && ns <= kMaxSlotsRegionMajor : (ns == 1 || ns == 2 || ns == 4)) &&
           (region_major ? nreg * ns : ns) <= kMaxChunks;
}

}  // namespace qkrope
