// qkrope_api.cpp -- the C ABI declared in include/qkrope.h: handles, argument validation,
// host-side precomputation and kernel launch. Device work is enqueued on the caller's stream;
// nothing here allocates device memory or synchronises.
#include "qkrope.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <cstring>
#include <new>
#include <string>

#include "qkrope_internal.h"
#include "qkrope_host.h"

namespace qkrope {
namespace host {

namespace {
thread_local std::string g_last_error;
}

int fail(int status, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok()
{
    g_last_error.clear();
    return QKROPE_OK;
}

const char *last_error() { return g_last_error.c_str(); }

}  // namespace host
}  // namespace qkrope

namespace {

using namespace qkrope;
using namespace qkrope::host;

// Workgroup size and slot layout for a token whose regions hold n[r] lane-units (16-byte
// chunks) each. Region-major gives every region `slots` slots per lane (compiled 1..4); mixed
// concatenates the regions and gives every lane `slots` slots (compiled 1, 2, 4).
// Measured on MI355X (launch-shape sweeps of the 3D workloads): region-major with the fewest
// slots that fit one workgroup, threads rounded up to whole waves, is best or within 1.5% of
// best whenever it keeps at least 3/4 of the lanes busy (15360 tokens x 3x32 heads x 128,
// 122880 x 3x16 x 256, and 36960 x 3x20 x 64 at 83% busy lanes, where the best mixed layout was
// 10% slower). Otherwise the layout that leaves the fewest lanes idle wins, preferring
// workgroups near 128 lanes.
// A token whose largest region needs a multiple of 32 but not of 64 lanes (one slot per
// region) leaves half a wave idle; two such tokens share a workgroup instead, filling whole
// waves (36960 x 3x20 x 64: 160 lanes per token, 83% -> 100% of lanes busy).
// `min_lanes`: lanes a token needs besides its chunks (3D: one per angle pair, head_dim / 2).
// `allow_two`: two tokens per workgroup are allowed only when every token stride, in bytes, is
// below 2^24: the kernel forms the second token's row offsets with 24-bit multiplies.
bool choose_shape(const int64_t *n, int nreg, int min_lanes, LaunchShape *s, bool allow_two = true)
{
    int64_t total = 0, maxn = 0;
    for (int r = 0; r < nreg; ++r) {
        total += n[r];
        maxn = n[r] > maxn ? n[r] : maxn;
    }
    if (maxn > 0) {
        const int64_t ns = (maxn + 1023) / 1024;
        const int64_t threads = ((maxn + ns - 1) / ns + 63) / 64 * 64;
        const double util = (double)total / ((double)nreg * ns * threads);
        if (ns == 1) {
            const int64_t t32 = (maxn + 31) / 32 * 32;
            const double util2 = (double)total / ((double)nreg * t32);
            if (allow_two && t32 % 64 != 0 && 2 * t32 <= 1024 && t32 >= min_lanes &&
                util2 >= 0.75 && util2 > util + 0.05) {
                *s = LaunchShape{(int)(2 * t32), 1, true, 0, 0, 2};
                return true;
            }
        }
        if (util >= 0.75 && threads >= min_lanes &&
            slots_compiled(nreg, true, (int)std::min<int64_t>(ns, 1 << 20))) {
            *s = LaunchShape{(int)threads, (int)ns, true, 0, 0, 1};
            return true;
        }
    }
    double best = -1.0;
    for (int threads = std::max(64, (min_lanes + 63) / 64 * 64); threads <= 1024; threads += 64) {
        const double dist = std::fabs(std::log2(threads / 128.0));
        const int64_t ns_rm = (maxn + threads - 1) / threads;
        if (slots_compiled(nreg, true, (int)std::min<int64_t>(ns_rm, 1 << 20))) {
            const double util = (double)total / ((double)nreg * ns_rm * threads);
            const double score = util - 0.01 * dist;
            if (score > best) {
                best = score;
                *s = LaunchShape{threads, (int)ns_rm, true, 0, 0, 1};
            }
        }
        const int64_t need = (total + threads - 1) / threads;
        for (int ns : kMixedSlots) {
            if (ns < need || !slots_compiled(nreg, false, ns)) continue;
            const double util = (double)total / ((double)ns * threads);
            const double score = util - 0.01 * dist + 0.001;
            if (score > best) {
                best = score;
                *s = LaunchShape{threads, ns, false, 0, 0, 1};
            }
            break;
        }
    }
    return best > 0.0;
}

// One region (Q, K or V) of one token per workgroup instead of all of a token's regions in one
// workgroup: lanes hold one 16-byte chunk each and a token's three workgroups run side by side.
// Measured on MI355X (graph replay, 512-lane regions), 3D form without norm and with 16-bit
// outputs: 15360 tokens x 3x32 x 128 78.2% -> 81.1% of 8 TB/s, 122880 x 3x16 x 256 77.6% ->
// 78.6%, the same with half-split pairs 76.85% -> 78.65%. With the across-heads norm the gain
// was within noise from a graph (77.2% -> 77.45%) and a loss with per-launch dispatch (76.2% ->
// 74.3%: three times the workgroups); with E4M3 outputs (79.3% -> 75.5%) and in the table form
// (80% -> 68%) one workgroup per token is faster.
bool split_regions(const LaunchShape &s, const KernelKey &k)
{
    return k.src == kSrc3D && k.norm == kNormNone && !k.fp8 && s.slot_uniform && s.tpw == 1 &&
           s.slots == 1 && s.threads >= 512;
}

// Token-block order across XCDs (KernelArgs::xcd_group). Workgroups are dealt to the 8 XCDs
// round-robin, so in block order every page of the streamed tensors is touched by all eight
// XCDs. Runs of 16 consecutive blocks per XCD, measured on MI355X (graph replay, G in
// {0, 1, 4, 16, 32, 64, 256}): 122880 tokens x 3x16 x 256 (6 GB per launch) 73.5% -> 77.3% of
// 8 TB/s, 15360 x 3x32 x 128 76.2% -> 77.2%, the 4096- and 32768-token tables +0.7-1.2 points,
// the FP8 NeoX workload within noise; larger runs lose again. With the stores at device scope
// the region-split launch (8 KB workgroups that only stream) gains from longer runs: 64 blocks
// (512 KB of input per run) took the 122880-token workload from 945 to 934 us per launch, while
// the 32768-token table lost 1% at 64 and 2.4% at 128 and the 15360-token and FP8 NeoX
// workloads stayed within noise. Grids under 128 blocks keep the plain order (the remap leaves
// blocks past the last whole 8G run in place).
uint32_t xcd_group_for(int64_t blocks, bool split)
{
    if (blocks < 128) return 0u;
    return split ? 64u : 16u;    // a power of two (the kernel shifts by its log)
}

// Store scope of a launch (KernelArgs::store_device): device scope once it writes at least
// 128 MiB. Measured on MI355X (graph replay, A/B on one box, against non-temporal stores only):
// the 122880-token YaRN workload (3 GB written) 2% faster, the 32768-token tables (403 MB)
// 0.4-1%, the 15360-token across-heads (377 MB) and FP8 NeoX (142 MB) workloads within noise;
// the 4-way head-sharded rank (94 MB) 4% slower and the 4096-token table (50 MB) 2-3% slower.
constexpr int64_t kStoreDeviceBytes = int64_t(1) << 27;

uint32_t store_device_for(const KernelKey &k, const KernelArgs &a)
{
    const int64_t elems = int64_t(a.heads[0] + a.heads[1] + a.heads[2]) * a.head_dim;
    return a.num_tokens * elems * (k.fp8 ? 1 : 2) >= kStoreDeviceBytes ? 1u : 0u;
}

hipError_t launch(const KernelKey &k, const LaunchShape &s, const KernelArgs &a, hipStream_t st)
{
    if (k.src == kSrc3D) {
        switch (k.head_dim_tpl) {
        case 64: return launch_3d_d64(k, s, a, st);
        case 128: return launch_3d_d128(k, s, a, st);
        case 256: return launch_3d_d256(k, s, a, st);
        default: return hipErrorInvalidValue;
        }
    }
    const bool f16 = k.act == kActF16;
    switch (k.pairing) {
    case kPairInterleaved: return f16 ? launch_table_interleaved_f16(k, s, a, st) : launch_table_interleaved_bf16(k, s, a, st);
    case kPairHalf: return f16 ? launch_table_halfsplit_f16(k, s, a, st) : launch_table_halfsplit_bf16(k, s, a, st);
    case kPairHalfAny: return f16 ? launch_table_halfsplit_any_f16(k, s, a, st) : launch_table_halfsplit_any_bf16(k, s, a, st);
    default: return hipErrorInvalidValue;
    }
}

// Workgroups one launch of `threads` lanes may have: a dispatch's grid holds at most 2^32 - 1
// work-items per dimension, and HIP takes at most 2^31 - 1 workgroups.
int64_t max_grid_blocks(int threads)
{
    return std::min<int64_t>(((int64_t(1) << 32) - 1) / threads, (int64_t(1) << 31) - 1);
}

// The same call restricted to tokens [t0, t0 + n): every per-token pointer moves t0 tokens on,
// and the 3D positions continue from token_offset + t0.
KernelArgs token_range(const KernelArgs &a, const KernelKey &key, int64_t t0, int64_t n)
{
    KernelArgs b = a;
    const int64_t esize = key.fp8 ? 1 : 2;
    const int64_t tsize = key.src == kSrcTableF32 ? 4 : 2;
    for (int r = 0; r < 3; ++r) {
        if (b.in[r]) b.in[r] += t0 * b.in_stride[r];
        if (b.out[r]) b.out[r] = static_cast<uint8_t *>(b.out[r]) + t0 * b.out_stride[r] * esize;
    }
    if (key.src != kSrc3D) {
        if (b.table_cos) b.table_cos = static_cast<const uint8_t *>(b.table_cos) + t0 * b.cos_stride * tsize;
        if (b.table_sin) b.table_sin = static_cast<const uint8_t *>(b.table_sin) + t0 * b.sin_stride * tsize;
    }
    if (b.sumsq_in) b.sumsq_in += 2 * t0;
    b.token_offset += (uint32_t)t0;
    b.num_tokens = n;
    return b;
}

// Launches the call, as several launches over consecutive token ranges where one grid would
// exceed the dispatch limits (e.g. 64-lane workgroups past 2^26 tokens).
int do_launch(qkrope_handle h, const KernelKey &key, const LaunchShape &shape,
              const KernelArgs &args, void *stream)
{
    DeviceGuard g(h->device);
    if (g.err != hipSuccess) return fail(QKROPE_ERR_DEVICE, "hipSetDevice: %s", hipGetErrorString(g.err));
    const int64_t per_block = shape.split ? (key.src == kSrc3D ? 3 : 2) : 1;  // workgroups per token block
    const int64_t T = args.num_tokens;
    const int64_t chunk = max_grid_blocks(shape.threads) / per_block * shape.tpw;   // tokens per launch
    for (int64_t t0 = 0; t0 < T; t0 += chunk) {
        const int64_t n = std::min(chunk, T - t0);
        LaunchShape s = shape;
        KernelArgs a = n == T ? args : token_range(args, key, t0, n);
        s.blocks = (n + s.tpw - 1) / s.tpw * per_block;
        a.xcd_group = xcd_group_for(s.blocks, s.split);
        a.xcd_lg = a.xcd_group ? (uint32_t)__builtin_ctz(a.xcd_group) : 0u;
        a.xcd_full = a.xcd_group ? (uint32_t)(s.blocks >> (a.xcd_lg + 3) << (a.xcd_lg + 3)) : 0u;
        a.store_device = store_device_for(key, a);
        const hipError_t e = launch(key, s, a, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return fail(QKROPE_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    }
    return ok();
}


// Every argument of the table form, extended contract (qkrope_run_table_ex).
struct TableCall {
    const void *q, *k, *q_weight, *k_weight, *cos_table, *sin_table;
    int table_dtype, act_dtype, out_dtype;
    double out_scale, eps;
    int64_t T;
    int Hq, Hk, D, R, interleaved, norm_mode;
    int64_t q_stride, k_stride, cos_stride, sin_stride;
    void *q_out, *k_out;
    int64_t q_out_stride, k_out_stride;
};

int run_table(qkrope_handle h, const TableCall &c, void *stream)
{
    if (!h) return fail(QKROPE_ERR_INVALID, "handle is NULL");
    const int D = c.D, R = c.R, Hq = c.Hq, Hk = c.Hk;
    const int64_t T = c.T;
    if (T < 0 || Hq < 0 || Hk < 0) return fail(QKROPE_ERR_INVALID, "negative size");
    if (D <= 0) return fail(QKROPE_ERR_INVALID, "head_dim must be positive");
    if (R < 0 || R > D || R % 2) return fail(QKROPE_ERR_INVALID, "rotary_dim must be even and in [0, head_dim]");
    if (c.act_dtype != QKROPE_DTYPE_BF16 && c.act_dtype != QKROPE_DTYPE_F16)
        return fail(QKROPE_ERR_INVALID, "act_dtype must be QKROPE_DTYPE_BF16 or QKROPE_DTYPE_F16");
    if (c.table_dtype != QKROPE_DTYPE_F32 && c.table_dtype != c.act_dtype)
        return fail(QKROPE_ERR_INVALID, "table_dtype must be float32 or the activation dtype");
    if (c.out_dtype != c.act_dtype && c.out_dtype != QKROPE_DTYPE_E4M3)
        return fail(QKROPE_ERR_INVALID, "out_dtype must be the activation dtype or QKROPE_DTYPE_E4M3");
    const bool fp8 = c.out_dtype == QKROPE_DTYPE_E4M3;
    if (fp8 && (!(c.out_scale > 0.0) || !std::isfinite(c.out_scale)))
        return fail(QKROPE_ERR_INVALID, "out_scale must be finite and > 0 for E4M3 outputs");
    if (c.norm_mode < QKROPE_NORM_NONE || c.norm_mode > QKROPE_NORM_ACROSS_HEADS)
        return fail(QKROPE_ERR_INVALID, "unknown norm_mode %d", c.norm_mode);
    if (!(c.eps >= 0.0) || !std::isfinite(c.eps)) return fail(QKROPE_ERR_INVALID, "eps must be finite and >= 0");
    if (D % 8 || D > 256) return fail(QKROPE_ERR_UNSUPPORTED, "head_dim must be a multiple of 8 and <= 256");
    const bool half = !c.interleaved;
    // half-split partners are whole 16-byte chunks when R/2 is a multiple of 8; otherwise they
    // are exchanged element by element through LDS
    const int pairing = !half ? kPairInterleaved : (R % 16 == 0 ? kPairHalf : kPairHalfAny);
    if (T >= (int64_t(1) << 31)) return fail(QKROPE_ERR_UNSUPPORTED, "num_tokens must be < 2^31");
    if (T == 0 || Hq + Hk == 0) return ok();

    if (!c.q && Hq) return fail(QKROPE_ERR_INVALID, "q is NULL");
    if (!c.k && Hk) return fail(QKROPE_ERR_INVALID, "k is NULL");
    if (!c.q_out && Hq) return fail(QKROPE_ERR_INVALID, "q_out is NULL");
    if (!c.k_out && Hk) return fail(QKROPE_ERR_INVALID, "k_out is NULL");
    if (R > 0 && (!c.cos_table || !c.sin_table)) return fail(QKROPE_ERR_INVALID, "rope table is NULL");
    if (c.norm_mode != QKROPE_NORM_NONE && ((Hq && !c.q_weight) || (Hk && !c.k_weight)))
        return fail(QKROPE_ERR_INVALID, "norm weights are NULL");
    if (c.q_stride < (int64_t)Hq * D || c.k_stride < (int64_t)Hk * D ||
        c.q_out_stride < (int64_t)Hq * D || c.k_out_stride < (int64_t)Hk * D)
        return fail(QKROPE_ERR_INVALID, "token strides must be >= heads*head_dim");
    if (R > 0 && (c.cos_stride < R / 2 || c.sin_stride < R / 2))
        return fail(QKROPE_ERR_INVALID, "table token strides must be >= rotary_dim/2");
    if (c.q_stride % 8 || c.k_stride % 8 || c.q_out_stride % 8 || c.k_out_stride % 8)
        return fail(QKROPE_ERR_UNSUPPORTED, "token strides must be multiples of 8 elements");
    // a workgroup addresses its tokens' rows with 32-bit byte offsets from the first one's
    const int64_t kMaxStride = int64_t(1) << 28;
    if (c.q_stride >= kMaxStride || c.k_stride >= kMaxStride || c.q_out_stride >= kMaxStride ||
        c.k_out_stride >= kMaxStride)
        return fail(QKROPE_ERR_UNSUPPORTED, "token strides must be < 2^28 elements");
    const uintptr_t oalign = fp8 ? 8 : 16;
    if (!aligned(c.q, 16) || !aligned(c.k, 16) || !aligned(c.q_weight, 16) || !aligned(c.k_weight, 16))
        return fail(QKROPE_ERR_UNSUPPORTED, "q, k and weights must be 16-byte aligned");
    if (!aligned(c.q_out, oalign) || !aligned(c.k_out, oalign))
        return fail(QKROPE_ERR_UNSUPPORTED, "outputs must be %d-byte aligned", (int)oalign);
    const int tsize = c.table_dtype == QKROPE_DTYPE_F32 ? 4 : 2;
    if (!aligned(c.cos_table, tsize) || !aligned(c.sin_table, tsize))
        return fail(QKROPE_ERR_UNSUPPORTED, "rope table is misaligned");

    // Outputs may alias their own input exactly (in place, same format and stride); any other
    // overlap is rejected.
    const int osize = fp8 ? 1 : 2;
    const int64_t wq_len = c.norm_mode == QKROPE_NORM_ACROSS_HEADS ? (int64_t)Hq * D : D;
    const int64_t wk_len = c.norm_mode == QKROPE_NORM_ACROSS_HEADS ? (int64_t)Hk * D : D;
    const Range rq = span_of(c.q, T, c.q_stride, (int64_t)Hq * D, 2);
    const Range rk = span_of(c.k, T, c.k_stride, (int64_t)Hk * D, 2);
    const Range rqo = span_of(c.q_out, T, c.q_out_stride, (int64_t)Hq * D, osize);
    const Range rko = span_of(c.k_out, T, c.k_out_stride, (int64_t)Hk * D, osize);
    const Range rc = span_of(c.cos_table, R > 0 ? T : 0, c.cos_stride, R / 2, tsize);
    const Range rs = span_of(c.sin_table, R > 0 ? T : 0, c.sin_stride, R / 2, tsize);
    const Range none{0, 0, 0, 0};
    const Range rwq = c.norm_mode != QKROPE_NORM_NONE ? span_of(c.q_weight, 1, 0, wq_len, 2) : none;
    const Range rwk = c.norm_mode != QKROPE_NORM_NONE ? span_of(c.k_weight, 1, 0, wk_len, 2) : none;
    const bool q_inplace = !fp8 && c.q_out == c.q && c.q_out_stride == c.q_stride;
    const bool k_inplace = !fp8 && c.k_out == c.k && c.k_out_stride == c.k_stride;
    if ((!q_inplace && overlap(rqo, rq)) || overlap(rqo, rk) || overlap(rqo, rc) || overlap(rqo, rs) ||
        overlap(rqo, rwq) || overlap(rqo, rwk) || overlap(rqo, rko))
        return fail(QKROPE_ERR_INVALID, "q_out overlaps another argument");
    if ((!k_inplace && overlap(rko, rk)) || overlap(rko, rq) || overlap(rko, rc) || overlap(rko, rs) ||
        overlap(rko, rwq) || overlap(rko, rwk))
        return fail(QKROPE_ERR_INVALID, "k_out overlaps another argument");

    const int L = next_pow2(D / 8);           // lanes per head: one 16-byte chunk each
    const int64_t n_units[2] = {(int64_t)Hq * L, (int64_t)Hk * L};
    const int64_t k24 = int64_t(1) << 24;
    const bool small_strides = 2 * std::max(c.q_stride, c.k_stride) < k24 &&
                               osize * std::max(c.q_out_stride, c.k_out_stride) < k24;
    LaunchShape shape;
    if (!choose_shape(n_units, 2, 1, &shape, small_strides))
        return fail(QKROPE_ERR_UNSUPPORTED, "too many heads for one workgroup per token");

    KernelArgs a;
    std::memset(&a, 0, sizeof a);
    a.in[kQ] = static_cast<const uint16_t *>(c.q);
    a.in[kK] = static_cast<const uint16_t *>(c.k);
    a.out[kQ] = c.q_out;
    a.out[kK] = c.k_out;
    a.in_stride[kQ] = c.q_stride;
    a.in_stride[kK] = c.k_stride;
    a.out_stride[kQ] = c.q_out_stride;
    a.out_stride[kK] = c.k_out_stride;
    a.heads[kQ] = Hq;
    a.heads[kK] = Hk;
    a.heads[kV] = 0;
    a.weight[0] = static_cast<const uint16_t *>(c.q_weight);
    a.weight[1] = static_cast<const uint16_t *>(c.k_weight);
    // Idle slots issue their loads unconditionally at the start of their region's token row (and
    // drop the result); a region without heads may have NULL pointers, so it borrows the other
    // region's row, stride and weights. Every address the kernel forms then lies inside a
    // caller's tensor (Hq + Hk > 0 here).
    if (Hq == 0) {
        a.in[kQ] = a.in[kK];
        a.in_stride[kQ] = a.in_stride[kK];
        a.weight[0] = a.weight[1];
    }
    if (Hk == 0) {
        a.in[kK] = a.in[kQ];
        a.in_stride[kK] = a.in_stride[kQ];
        a.weight[1] = a.weight[0];
    }
    a.table_cos = c.cos_table;
    a.table_sin = c.sin_table;
    a.cos_stride = c.cos_stride;
    a.sin_stride = c.sin_stride;
    {
        // whole-vector table reads: a lane's pairs (4 interleaved, 8 half-split) never straddle
        // R/2, and both tables' rows are aligned for loads of min(16, pairs * size) bytes
        const int pairs = half ? 8 : 4;
        const int64_t vb = std::min(16, pairs * tsize);
        a.table_vec = R > 0 && (R / 2) % pairs == 0 && aligned(c.cos_table, vb) &&
                      aligned(c.sin_table, vb) && (c.cos_stride * tsize) % vb == 0 &&
                      (c.sin_stride * tsize) % vb == 0;
    }
    a.num_tokens = T;
    a.head_dim = D;
    a.rotary_dim = R;
    a.lanes_per_head = L;
    a.eps = (float)c.eps;
    const bool across = c.norm_mode == QKROPE_NORM_ACROSS_HEADS;
    a.inv_count[0] = (float)(1.0 / (double)(across ? (int64_t)Hq * D : D));
    a.inv_count[1] = (float)(1.0 / (double)(across ? (int64_t)Hk * D : D));
    a.qk_scale = fp8 ? (float)c.out_scale : 1.0f;
    a.v_scale = 1.0f;
    a.v_inv_pow2 = 0.0f;
    a.v_limit_bits = 0;
    shape.lds_bytes = pairing == kPairHalfAny ? shape.threads * 32 : 0;

    KernelKey key;
    // E4M3 outputs at head_dim == rotary_dim == 128 with one slot per region take a kernel with
    // the head geometry fixed at compile time (fixed lane groups, no per-pair rotation masks).
    // That path is ALU-bound on MI355X, and measured (graph replay, 32768 tokens x 2x24 heads,
    // fp32 table) 102.2 -> 95.9 us, 75.9% -> 80.9% of 8 TB/s. With 16-bit outputs, bound by
    // memory, the run-time kernel was as fast (bf16) or 1.7% faster (float16).
    key.head_dim_tpl = fp8 && D == 128 && R == 128 && pairing != kPairHalfAny &&
                       shape.slot_uniform && shape.slots == 1 ? 128 : 0;
    key.pairing = pairing;
    key.norm = c.norm_mode == QKROPE_NORM_NONE ? kNormNone
             : c.norm_mode == QKROPE_NORM_PER_HEAD ? kNormPerHead : kNormAcross;
    key.src = c.table_dtype == QKROPE_DTYPE_F32 ? kSrcTableF32
            : c.table_dtype == QKROPE_DTYPE_BF16 ? kSrcTableBF16 : kSrcTableF16;
    key.act = c.act_dtype == QKROPE_DTYPE_F16 ? kActF16 : kActBF16;
    key.fp8 = fp8;
    key.slots = shape.slots;
    key.slot_uniform = shape.slot_uniform;
    return do_launch(h, key, shape, a, stream);
}

// Every argument of the 3D form, sharded contract (qkrope_run_3d_sharded).
struct Rope3DCall {
    const void *qkv, *q_weight, *k_weight;
    int64_t T, token_offset;
    const float *sumsq;
    int64_t norm_elems_q, norm_elems_k;
    int ppf, pph, ppw, C[3], Hq, Hk, Hv, D;
    double eps, base;
    int interleave;
    double factor, low, high, attention_factor;
    int is_qk_norm, output_fp8;
    double output_quant_scale, v_quant_scale;
    void *q_out, *k_out, *v_out;
    bool whole_sequences;     // num_tokens must be a multiple of ppf*pph*ppw (unsharded call)
};

int run_3d(qkrope_handle h, const Rope3DCall &c, void *stream)
{
    if (!h) return fail(QKROPE_ERR_INVALID, "handle is NULL");
    const int D = c.D, Hq = c.Hq, Hk = c.Hk, Hv = c.Hv;
    const int *C = c.C;
    const int64_t T = c.T;
    if (T < 0 || Hq < 0 || Hk < 0 || Hv < 0) return fail(QKROPE_ERR_INVALID, "negative size");
    if (D != 64 && D != 128 && D != 256) return fail(QKROPE_ERR_INVALID, "head_dim must be 64, 128 or 256");
    for (int i = 0; i < 3; ++i)
        if (C[i] < 0 || C[i] % 2) return fail(QKROPE_ERR_INVALID, "channel counts must be even and >= 0");
    if (C[0] + C[1] + C[2] != D) return fail(QKROPE_ERR_INVALID, "channel counts must sum to head_dim");
    if (c.ppf <= 0 || c.pph <= 0 || c.ppw <= 0) return fail(QKROPE_ERR_INVALID, "ppf, pph, ppw must be positive");
    // positions are split with 32-bit magic divisors (divisors < 2^31): bound the grid, each
    // partial product checked before the next multiplication so nothing overflows
    const int64_t kMaxSeq = int64_t(1) << 31;
    const int64_t fh = (int64_t)c.ppf * c.pph;       // < 2^62
    if (fh >= kMaxSeq || fh * c.ppw >= kMaxSeq)
        return fail(QKROPE_ERR_UNSUPPORTED, "ppf*pph*ppw must be < 2^31");
    const int64_t S = fh * c.ppw;
    if (c.whole_sequences && T % S) return fail(QKROPE_ERR_INVALID, "num_tokens must be a multiple of ppf*pph*ppw");
    if (c.token_offset < 0) return fail(QKROPE_ERR_INVALID, "token_offset must be >= 0");
    if (!(c.base > 0.0) || !std::isfinite(c.base)) return fail(QKROPE_ERR_INVALID, "base must be finite and > 0");
    if (!(c.eps >= 0.0) || !std::isfinite(c.eps)) return fail(QKROPE_ERR_INVALID, "eps must be finite and >= 0");
    if (!(c.factor > 0.0) || !std::isfinite(c.factor)) return fail(QKROPE_ERR_INVALID, "factor must be finite and > 0");
    if (!std::isfinite(c.attention_factor)) return fail(QKROPE_ERR_INVALID, "attention_factor must be finite");
    if (c.factor == 1.0 && c.attention_factor != 1.0)
        return fail(QKROPE_ERR_INVALID, "attention_factor must be 1.0 when factor is 1.0");
    if (c.factor != 1.0 && !(c.high > c.low))
        return fail(QKROPE_ERR_INVALID, "YaRN needs high > low");
    if (c.factor != 1.0 && (!std::isfinite(c.low) || !std::isfinite(c.high)))
        return fail(QKROPE_ERR_INVALID, "YaRN low/high must be finite");
    if (c.output_fp8 && (!(c.output_quant_scale > 0.0) || !std::isfinite(c.output_quant_scale) ||
                         !(c.v_quant_scale > 0.0) || !std::isfinite(c.v_quant_scale)))
        return fail(QKROPE_ERR_INVALID, "FP8 scales must be finite and > 0");
    const bool ext = c.is_qk_norm && c.sumsq != nullptr;
    if (ext && (c.norm_elems_q < (int64_t)Hq * D || c.norm_elems_k < (int64_t)Hk * D ||
                c.norm_elems_q <= 0 || c.norm_elems_k <= 0))
        return fail(QKROPE_ERR_INVALID, "norm_elems_q/k must be positive and cover the shard's own heads");
    if (T + c.token_offset >= (int64_t(1) << 31))
        return fail(QKROPE_ERR_UNSUPPORTED, "token_offset + num_tokens must be < 2^31");
    if (T == 0 || Hq + Hk + Hv == 0) return ok();

    if (!c.qkv) return fail(QKROPE_ERR_INVALID, "qkv is NULL");
    if ((Hq && !c.q_out) || (Hk && !c.k_out) || (Hv && !c.v_out)) return fail(QKROPE_ERR_INVALID, "output is NULL");
    if (c.is_qk_norm && ((Hq && !c.q_weight) || (Hk && !c.k_weight)))
        return fail(QKROPE_ERR_INVALID, "norm weights are NULL while is_qk_norm is set");
    const int osize = c.output_fp8 ? 1 : 2;
    const uintptr_t oalign = c.output_fp8 ? 8 : 16;
    if (!aligned(c.qkv, 16) || !aligned(c.q_out, oalign) || !aligned(c.k_out, oalign) || !aligned(c.v_out, oalign))
        return fail(QKROPE_ERR_UNSUPPORTED, "qkv must be 16-byte aligned, outputs %d-byte aligned", (int)oalign);
    if (c.is_qk_norm && (!aligned(c.q_weight, 16) || !aligned(c.k_weight, 16)))
        return fail(QKROPE_ERR_UNSUPPORTED, "norm weights must be 16-byte aligned");
    if (ext && !aligned(c.sumsq, 8)) return fail(QKROPE_ERR_UNSUPPORTED, "sumsq must be 8-byte aligned");

    const int64_t row = (int64_t)(Hq + Hk + Hv) * D;
    const Range none{0, 0, 0, 0};
    const Range rin = span_of(c.qkv, T, row, row, 2);
    const Range rq = span_of(c.q_out, T, (int64_t)Hq * D, (int64_t)Hq * D, osize);
    const Range rk = span_of(c.k_out, T, (int64_t)Hk * D, (int64_t)Hk * D, osize);
    const Range rv = span_of(c.v_out, T, (int64_t)Hv * D, (int64_t)Hv * D, osize);
    const Range rwq = c.is_qk_norm ? span_of(c.q_weight, 1, 0, (int64_t)Hq * D, 2) : none;
    const Range rwk = c.is_qk_norm ? span_of(c.k_weight, 1, 0, (int64_t)Hk * D, 2) : none;
    const Range rss = ext ? span_of(c.sumsq, T, 2, 2, 4) : none;
    const Range outs[3] = {rq, rk, rv};
    for (int i = 0; i < 3; ++i) {
        if (overlap(outs[i], rin) || overlap(outs[i], rwq) || overlap(outs[i], rwk) || overlap(outs[i], rss))
            return fail(QKROPE_ERR_INVALID, "an output overlaps qkv, a weight or sumsq");
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outs[j])) return fail(QKROPE_ERR_INVALID, "outputs overlap each other");
    }

    const bool half = !c.interleave;
    const int units = D / 8;                   // 16-byte chunks per head: 8, 16 or 32
    const int64_t n_units[3] = {(int64_t)Hq * units, (int64_t)Hk * units, (int64_t)Hv * units};
    LaunchShape shape;
    if (!choose_shape(n_units, 3, D / 2, &shape))
        return fail(QKROPE_ERR_UNSUPPORTED, "too many heads for one workgroup per token");

    KernelArgs a;
    std::memset(&a, 0, sizeof a);
    const uint16_t *base_in = static_cast<const uint16_t *>(c.qkv);
    // a region without heads points at the row start, so its idle-slot loads stay inside the
    // row (its own offset could be the end of qkv)
    a.in[kQ] = base_in;
    a.in[kK] = Hk ? base_in + (int64_t)Hq * D : base_in;
    a.in[kV] = Hv ? base_in + (int64_t)(Hq + Hk) * D : base_in;
    a.out[kQ] = c.q_out;
    a.out[kK] = c.k_out;
    a.out[kV] = c.v_out;
    for (int r = 0; r < 3; ++r) a.in_stride[r] = row;
    a.out_stride[kQ] = (int64_t)Hq * D;
    a.out_stride[kK] = (int64_t)Hk * D;
    a.out_stride[kV] = (int64_t)Hv * D;
    a.heads[kQ] = Hq;
    a.heads[kK] = Hk;
    a.heads[kV] = Hv;
    a.weight[0] = static_cast<const uint16_t *>(c.q_weight);
    a.weight[1] = static_cast<const uint16_t *>(c.k_weight);
    // as for the table form: an empty Q or K region borrows the other's weights for its idle
    // loads; with neither, there is nothing to normalise (and the weights may be NULL)
    const bool norm = c.is_qk_norm && Hq + Hk > 0;
    if (Hq == 0) a.weight[0] = a.weight[1];
    if (Hk == 0) a.weight[1] = a.weight[0];
    a.sumsq_in = ext ? c.sumsq : nullptr;
    a.num_tokens = T;
    a.head_dim = D;
    a.rotary_dim = D;
    a.lanes_per_head = units;
    a.eps = (float)c.eps;
    const double nq = ext ? (double)c.norm_elems_q : (double)Hq * D;
    const double nk = ext ? (double)c.norm_elems_k : (double)Hk * D;
    a.inv_count[0] = nq > 0 ? (float)(1.0 / nq) : 0.0f;
    a.inv_count[1] = nk > 0 ? (float)(1.0 / nk) : 0.0f;
    a.qk_scale = c.output_fp8 ? (float)c.output_quant_scale : 1.0f;
    a.v_scale = c.output_fp8 ? (float)c.v_quant_scale : 1.0f;
    a.v_inv_pow2 = 0.0f;
    a.v_limit_bits = 0;
    if (c.output_fp8) {
        int e = 0;
        const double m = std::frexp(c.v_quant_scale, &e);     // v_quant_scale = m * 2^e
        if (m == 0.5 && e - 1 >= -20 && e - 1 <= 20) {
            a.v_inv_pow2 = (float)std::ldexp(1.0, 1 - e);
            // 448 / v_scale = 1.75 * 2^(9 - e): bf16 pattern of its exact value
            const float lim = (float)std::ldexp(1.75, 9 - e);
            uint32_t bits;
            std::memcpy(&bits, &lim, 4);
            a.v_limit_bits = bits >> 16;
        }
    }
    a.token_offset = (uint32_t)c.token_offset;
    a.seq_len = (uint32_t)S;
    a.hw = (uint32_t)((int64_t)c.pph * c.ppw);
    a.ppw = (uint32_t)c.ppw;
    a.pph = (uint32_t)c.pph;
    a.div_seq = make_fast_div(a.seq_len);
    a.div_hw = make_fast_div(a.hw);
    a.div_w = make_fast_div(a.ppw);
    a.attention_factor = (float)c.attention_factor;
    // Per pair k of the concatenated [frame | height | width] frequency vector: its axis and the
    // YaRN-blended angular frequency, in fp64, handed to the kernel as revolutions per position.
    const double two_pi = 2.0 * 3.14159265358979323846;
    for (int k = 0, axis = 0, j = 0; k < D / 2; ++k, ++j) {
        while (j >= C[axis] / 2) {
            j -= C[axis] / 2;
            ++axis;
        }
        double omega = std::pow(c.base, -2.0 * j / (double)C[axis]);
        if (c.factor != 1.0) {
            double rho = (j - c.low) / (c.high - c.low);
            rho = rho < 0.0 ? 0.0 : (rho > 1.0 ? 1.0 : rho);
            omega = (omega / c.factor) * rho + omega * (1.0 - rho);
        }
        a.omega_rev[k] = (float)(omega / two_pi);
        a.axis[k] = (uint8_t)axis;
    }
    KernelKey key;
    key.head_dim_tpl = D;
    key.pairing = half ? kPairHalf : kPairInterleaved;     // R/2 = D/2 is a multiple of 8
    key.norm = !norm ? kNormNone : (ext ? kNormAcrossExt : kNormAcross);
    key.src = kSrc3D;
    key.act = kActBF16;
    key.fp8 = c.output_fp8 != 0;
    key.slots = shape.slots;
    key.slot_uniform = shape.slot_uniform;

    shape.split = split_regions(shape, key);
    shape.lds_bytes = 0;
    return do_launch(h, key, shape, a, stream);
}

}  // namespace

extern "C" {

const char *qkrope_status_str(int status)
{
    switch (status) {
    case QKROPE_OK: return "ok";
    case QKROPE_ERR_INVALID: return "invalid argument";
    case QKROPE_ERR_UNSUPPORTED: return "unsupported argument";
    case QKROPE_ERR_DEVICE: return "device error";
    case QKROPE_ERR_ALLOC: return "allocation failed";
    default: return "unknown status";
    }
}

const char *qkrope_last_error(void) { return qkrope::host::last_error(); }

int qkrope_min_tokens(int64_t default_tokens, int64_t *out)
{
    if (!out) return fail(QKROPE_ERR_INVALID, "out is NULL");
    if (default_tokens < 0) return fail(QKROPE_ERR_INVALID, "default_tokens must be >= 0");
    const char *env = std::getenv("QKROPE_FUSED_MIN_TOKENS");
    if (!env) {
        *out = default_tokens;
        return ok();
    }
    const char *p = env;
    while (*p == ' ' || *p == '\t') ++p;
    const char *end = p + std::strlen(p);
    while (end > p && (end[-1] == ' ' || end[-1] == '\t' || end[-1] == '\n')) --end;
    if (p == end) {
        *out = default_tokens;
        return ok();
    }
    int64_t v = 0;
    for (const char *c = p; c < end; ++c) {
        if (*c < '0' || *c > '9' || v > (INT64_MAX - 9) / 10)
            return fail(QKROPE_ERR_INVALID,
                        "QKROPE_FUSED_MIN_TOKENS=\"%s\" is not a non-negative integer", env);
        v = v * 10 + (*c - '0');
    }
    *out = v;
    return ok();
}

int qkrope_create(int device_ordinal, qkrope_handle *out)
{
    if (!out) return fail(QKROPE_ERR_INVALID, "out is NULL");
    *out = nullptr;
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess) return fail(QKROPE_ERR_DEVICE, "hipGetDeviceCount: %s", hipGetErrorString(e));
    if (device_ordinal < 0 || device_ordinal >= count)
        return fail(QKROPE_ERR_INVALID, "device %d out of range (%d devices)", device_ordinal, count);
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, device_ordinal);
    if (e != hipSuccess) return fail(QKROPE_ERR_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(QKROPE_ERR_DEVICE, "device %d is %s; this library is built for gfx950",
                    device_ordinal, prop.gcnArchName);
    qkrope_ctx *c = new (std::nothrow) qkrope_ctx;
    if (!c) return fail(QKROPE_ERR_ALLOC, "out of host memory");
    c->device = device_ordinal;
    c->num_cus = prop.multiProcessorCount;
    std::snprintf(c->arch, sizeof c->arch, "%s", prop.gcnArchName);
    *out = c;
    return ok();
}

int qkrope_destroy(qkrope_handle h)
{
    delete h;
    return ok();
}

int qkrope_run_table(qkrope_handle h, const void *q, const void *k, const void *q_weight,
                     const void *k_weight, const void *rope_table, int table_dtype, double eps,
                     int64_t num_tokens, int num_heads_q, int num_heads_k, int head_dim,
                     int rotary_dim, int interleaved, int norm_mode, int64_t q_token_stride,
                     int64_t k_token_stride, int64_t table_token_stride, void *q_out, void *k_out,
                     int64_t q_out_token_stride, int64_t k_out_token_stride, void *stream)
{
    if (table_dtype != QKROPE_TABLE_BF16 && table_dtype != QKROPE_TABLE_F32)
        return fail(QKROPE_ERR_INVALID, "table_dtype must be QKROPE_TABLE_BF16 or QKROPE_TABLE_F32");
    if (rotary_dim > 0 && table_token_stride < rotary_dim)
        return fail(QKROPE_ERR_INVALID, "table_token_stride must be >= rotary_dim");
    // the packed [cos | sin] row is the split layout with sin starting rotary_dim/2 later
    const int tsize = table_dtype == QKROPE_TABLE_F32 ? 4 : 2;
    const void *sin_table = rope_table && rotary_dim > 0
        ? static_cast<const uint8_t *>(rope_table) + (int64_t)(rotary_dim / 2) * tsize : nullptr;
    const TableCall c{q, k, q_weight, k_weight, rope_table, sin_table, table_dtype,
                      QKROPE_DTYPE_BF16, QKROPE_DTYPE_BF16, 1.0, eps, num_tokens, num_heads_q,
                      num_heads_k, head_dim, rotary_dim, interleaved, norm_mode, q_token_stride,
                      k_token_stride, table_token_stride, table_token_stride, q_out, k_out,
                      q_out_token_stride, k_out_token_stride};
    return run_table(h, c, stream);
}

int qkrope_run_table_ex(qkrope_handle h, const void *q, const void *k, const void *q_weight,
                        const void *k_weight, const void *cos_table, const void *sin_table,
                        int table_dtype, int act_dtype, int out_dtype, double out_scale,
                        double eps, int64_t num_tokens, int num_heads_q, int num_heads_k,
                        int head_dim, int rotary_dim, int interleaved, int norm_mode,
                        int64_t q_token_stride, int64_t k_token_stride, int64_t cos_token_stride,
                        int64_t sin_token_stride, void *q_out, void *k_out,
                        int64_t q_out_token_stride, int64_t k_out_token_stride, void *stream)
{
    const TableCall c{q, k, q_weight, k_weight, cos_table, sin_table, table_dtype, act_dtype,
                      out_dtype, out_scale, eps, num_tokens, num_heads_q, num_heads_k, head_dim,
                      rotary_dim, interleaved, norm_mode, q_token_stride, k_token_stride,
                      cos_token_stride, sin_token_stride, q_out, k_out, q_out_token_stride,
                      k_out_token_stride};
    return run_table(h, c, stream);
}

int qkrope_run_3d(qkrope_handle h, const void *qkv, const void *q_weight, const void *k_weight,
                  int64_t num_tokens, int ppf, int pph, int ppw, int num_frame_channels,
                  int num_height_channels, int num_width_channels, int num_heads_q,
                  int num_heads_k, int num_heads_v, int head_dim, double eps, double base,
                  int interleave, double factor, double low, double high, double attention_factor,
                  int is_qk_norm, int output_fp8, double output_quant_scale, double v_quant_scale,
                  void *q_out, void *k_out, void *v_out, void *stream)
{
    const Rope3DCall c{qkv, q_weight, k_weight, num_tokens, 0, nullptr, 0, 0, ppf, pph, ppw,
                       {num_frame_channels, num_height_channels, num_width_channels},
                       num_heads_q, num_heads_k, num_heads_v, head_dim, eps, base, interleave,
                       factor, low, high, attention_factor, is_qk_norm, output_fp8,
                       output_quant_scale, v_quant_scale, q_out, k_out, v_out, true};
    return run_3d(h, c, stream);
}

int qkrope_run_3d_sharded(qkrope_handle h, const void *qkv, const void *q_weight,
                          const void *k_weight, int64_t num_tokens, int64_t token_offset,
                          const float *sumsq, int64_t norm_elems_q, int64_t norm_elems_k,
                          int ppf, int pph, int ppw, int num_frame_channels,
                          int num_height_channels, int num_width_channels, int num_heads_q,
                          int num_heads_k, int num_heads_v, int head_dim, double eps, double base,
                          int interleave, double factor, double low, double high,
                          double attention_factor, int is_qk_norm, int output_fp8,
                          double output_quant_scale, double v_quant_scale, void *q_out,
                          void *k_out, void *v_out, void *stream)
{
    const Rope3DCall c{qkv, q_weight, k_weight, num_tokens, token_offset, sumsq, norm_elems_q,
                       norm_elems_k, ppf, pph, ppw,
                       {num_frame_channels, num_height_channels, num_width_channels},
                       num_heads_q, num_heads_k, num_heads_v, head_dim, eps, base, interleave,
                       factor, low, high, attention_factor, is_qk_norm, output_fp8,
                       output_quant_scale, v_quant_scale, q_out, k_out, v_out, false};
    return run_3d(h, c, stream);
}

int qkrope_sumsq_3d(qkrope_handle h, const void *qkv, int64_t num_tokens, int num_heads_q,
                    int num_heads_k, int num_heads_v, int head_dim, float *sumsq, void *stream)
{
    if (!h) return fail(QKROPE_ERR_INVALID, "handle is NULL");
    const int64_t T = num_tokens;
    if (T < 0 || num_heads_q < 0 || num_heads_k < 0 || num_heads_v < 0 || head_dim <= 0)
        return fail(QKROPE_ERR_INVALID, "negative size or non-positive head_dim");
    if (head_dim % 8) return fail(QKROPE_ERR_UNSUPPORTED, "head_dim must be a multiple of 8");
    const int64_t chunks = (int64_t)(num_heads_q + num_heads_k) * head_dim / 8;
    if (chunks > 8192) return fail(QKROPE_ERR_UNSUPPORTED, "(num_heads_q + num_heads_k) * head_dim / 8 must be <= 8192");
    if (T >= (int64_t(1) << 31)) return fail(QKROPE_ERR_UNSUPPORTED, "num_tokens must be < 2^31");
    if (T == 0) return ok();
    if (!qkv || !sumsq) return fail(QKROPE_ERR_INVALID, "qkv or sumsq is NULL");
    if (!aligned(qkv, 16)) return fail(QKROPE_ERR_UNSUPPORTED, "qkv must be 16-byte aligned");
    if (!aligned(sumsq, 8)) return fail(QKROPE_ERR_UNSUPPORTED, "sumsq must be 8-byte aligned");
    const int64_t row = (int64_t)(num_heads_q + num_heads_k + num_heads_v) * head_dim;
    if (overlap(span_of(sumsq, T, 2, 2, 4), span_of(qkv, T, row, row, 2)))
        return fail(QKROPE_ERR_INVALID, "sumsq overlaps qkv");
    SumsqArgs a;
    a.qkv = static_cast<const uint16_t *>(qkv);
    a.out = sumsq;
    a.row = row;
    a.q_chunks = num_heads_q * head_dim / 8;
    a.k_chunks = num_heads_k * head_dim / 8;
    // one 16-byte chunk per lane where the row fits one workgroup, whole waves
    const int64_t per = chunks <= 1024 ? chunks : (chunks + (chunks + 1023) / 1024 - 1) / ((chunks + 1023) / 1024);
    const int threads = (int)std::max<int64_t>(64, (per + 63) / 64 * 64);
    DeviceGuard g(h->device);
    if (g.err != hipSuccess) return fail(QKROPE_ERR_DEVICE, "hipSetDevice: %s", hipGetErrorString(g.err));
    const int64_t chunk = max_grid_blocks(threads);        // one workgroup per token
    for (int64_t t0 = 0; t0 < T; t0 += chunk) {
        SumsqArgs b = a;
        b.qkv += t0 * row;
        b.out += 2 * t0;
        const hipError_t e = launch_sumsq(b, std::min(chunk, T - t0), threads, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return fail(QKROPE_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    }
    return ok();
}

}  // extern "C"
