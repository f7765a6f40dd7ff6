// qkrope_api.cpp -- the C ABI declared in include/qkrope.h: handles, argument validation,
// host-side precomputation and kernel launch. Device work is enqueued on the caller's stream;
// nothing here allocates device memory or synchronises.
#include "qkrope.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <new>
#include <string>

#include "qkrope_internal.h"

struct qkrope_ctx {
    int device;
    int num_cus;
    char arch[64];
};

namespace {

using namespace qkrope;

thread_local std::string g_last_error;

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

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Bytes touched by a strided [tokens, span] tensor: rows of `span` elements every `stride`.
struct Range {
    uintptr_t lo, hi;          // bounding interval [lo, hi)
    int64_t stride_b, span_b;  // row stride and row length in bytes
};

Range span_of(const void *p, int64_t tokens, int64_t stride, int64_t span, int64_t esize)
{
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    if (tokens <= 0 || span <= 0) return {lo, lo, 0, 0};
    return {lo, lo + (uintptr_t)(((tokens - 1) * stride + span) * esize), stride * esize,
            span * esize};
}

// Whether two strided tensors share a byte. Exact when both have the same row stride (rows of
// one sit in a gap of the other's period, as for column slices of one packed buffer);
// otherwise the bounding intervals decide.
bool overlap(Range a, Range b)
{
    if (a.lo == a.hi || b.lo == b.hi) return false;
    if (!(a.lo < b.hi && b.lo < a.hi)) return false;
    if (a.stride_b == b.stride_b && a.stride_b > 0 && a.span_b <= a.stride_b &&
        b.span_b <= b.stride_b) {
        const int64_t period = a.stride_b;
        const int64_t diff = (int64_t)(b.lo - a.lo);
        const int64_t d = ((diff % period) + period) % period;  // b's row start in a's period
        if (d >= a.span_b && d + b.span_b <= period) return false;
    }
    return true;
}

int next_pow2(int v)
{
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

// Workgroup size and slot layout for a token whose regions hold n[r] lane-units (16-byte
// chunks) each. Region-major gives every region `slots` slots per lane (compiled 1..4); mixed
// concatenates the regions and gives every lane `slots` slots (compiled 1, 2, 4).
// Measured on MI355X (launch-shape sweeps of the 3D workloads): region-major with the fewest
// slots that fit one workgroup, threads rounded up to whole waves, is best or within 1.5% of
// best whenever it keeps at least 3/4 of the lanes busy (15360 tokens x 3x32 heads x 128,
// 122880 x 3x16 x 256, and 36960 x 3x20 x 64 at 83% busy lanes, where the best mixed layout was
// 10% slower). Otherwise the layout that leaves the fewest lanes idle wins, preferring
// workgroups near 128 lanes.
bool choose_shape(const int64_t *n, int nreg, LaunchShape *s)
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
        if (util >= 0.75 && slots_compiled(nreg, true, (int)std::min<int64_t>(ns, 1 << 20))) {
            *s = LaunchShape{(int)threads, (int)ns, true, 0};
            return true;
        }
    }
    double best = -1.0;
    for (int threads = 64; threads <= 1024; threads += 64) {
        const double dist = std::fabs(std::log2(threads / 128.0));
        const int64_t ns_rm = (maxn + threads - 1) / threads;
        if (slots_compiled(nreg, true, (int)std::min<int64_t>(ns_rm, 1 << 20))) {
            const double util = (double)total / ((double)nreg * ns_rm * threads);
            const double score = util - 0.01 * dist;
            if (score > best) {
                best = score;
                *s = LaunchShape{threads, (int)ns_rm, true, 0};
            }
        }
        const int64_t need = (total + threads - 1) / threads;
        for (int ns : kMixedSlots) {
            if (ns < need || !slots_compiled(nreg, false, ns)) continue;
            const double util = (double)total / ((double)ns * threads);
            const double score = util - 0.01 * dist + 0.001;
            if (score > best) {
                best = score;
                *s = LaunchShape{threads, ns, false, 0};
            }
            break;
        }
    }
    return best > 0.0;
}

// Magic pair for n / d, n < 2^31 (round-up method): with l = ceil(log2 d) and
// m = floor(2^32 * (2^l - d) / d) + 1, n / d = (mulhi(n, m) + n) >> l; the sum cannot
// overflow 32 bits because mulhi(n, m) <= n < 2^31.
FastDiv make_fast_div(uint32_t d)
{
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
    return FastDiv{(uint32_t)m, l};
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
    return k.half_split ? launch_table_halfsplit(k, s, a, st) : launch_table_interleaved(k, s, a, st);
}

// Device guard: make h->device current for the launch and restore the caller's device after.
struct DeviceGuard {
    int prev = -1;
    bool switched = false;
    hipError_t err = hipSuccess;
    explicit DeviceGuard(int dev)
    {
        err = hipGetDevice(&prev);
        if (err == hipSuccess && prev != dev) {
            err = hipSetDevice(dev);
            switched = err == hipSuccess;
        }
    }
    ~DeviceGuard()
    {
        if (switched) (void)hipSetDevice(prev);
    }
};

int do_launch(qkrope_handle h, const KernelKey &key, const LaunchShape &shape,
              const KernelArgs &args, void *stream)
{
    DeviceGuard g(h->device);
    if (g.err != hipSuccess) return fail(QKROPE_ERR_DEVICE, "hipSetDevice: %s", hipGetErrorString(g.err));
    hipError_t e = launch(key, shape, args, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(QKROPE_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
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

const char *qkrope_last_error(void) { return g_last_error.c_str(); }

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
    if (!h) return fail(QKROPE_ERR_INVALID, "handle is NULL");
    const int D = head_dim, R = rotary_dim, Hq = num_heads_q, Hk = num_heads_k;
    const int64_t T = num_tokens;
    if (T < 0 || Hq < 0 || Hk < 0) return fail(QKROPE_ERR_INVALID, "negative size");
    if (D <= 0) return fail(QKROPE_ERR_INVALID, "head_dim must be positive");
    if (R < 0 || R > D || R % 2) return fail(QKROPE_ERR_INVALID, "rotary_dim must be even and in [0, head_dim]");
    if (table_dtype != QKROPE_TABLE_BF16 && table_dtype != QKROPE_TABLE_F32)
        return fail(QKROPE_ERR_INVALID, "table_dtype must be QKROPE_TABLE_BF16 or QKROPE_TABLE_F32");
    if (norm_mode < QKROPE_NORM_NONE || norm_mode > QKROPE_NORM_ACROSS_HEADS)
        return fail(QKROPE_ERR_INVALID, "unknown norm_mode %d", norm_mode);
    if (!(eps >= 0.0) || !std::isfinite(eps)) return fail(QKROPE_ERR_INVALID, "eps must be finite and >= 0");
    if (D % 8 || D > 256) return fail(QKROPE_ERR_UNSUPPORTED, "head_dim must be a multiple of 8 and <= 256");
    const bool half = !interleaved;
    if (half && R % 16)
        return fail(QKROPE_ERR_UNSUPPORTED, "half-split pairing needs rotary_dim to be a multiple of 16");
    if (T >= (int64_t(1) << 31)) return fail(QKROPE_ERR_UNSUPPORTED, "num_tokens must be < 2^31");
    if (T == 0 || Hq + Hk == 0) return ok();

    if (!q && Hq) return fail(QKROPE_ERR_INVALID, "q is NULL");
    if (!k && Hk) return fail(QKROPE_ERR_INVALID, "k is NULL");
    if (!q_out && Hq) return fail(QKROPE_ERR_INVALID, "q_out is NULL");
    if (!k_out && Hk) return fail(QKROPE_ERR_INVALID, "k_out is NULL");
    if (R > 0 && !rope_table) return fail(QKROPE_ERR_INVALID, "rope_table is NULL");
    if (norm_mode != QKROPE_NORM_NONE && ((Hq && !q_weight) || (Hk && !k_weight)))
        return fail(QKROPE_ERR_INVALID, "norm weights are NULL");
    if (q_token_stride < (int64_t)Hq * D || k_token_stride < (int64_t)Hk * D ||
        q_out_token_stride < (int64_t)Hq * D || k_out_token_stride < (int64_t)Hk * D)
        return fail(QKROPE_ERR_INVALID, "token strides must be >= heads*head_dim");
    if (R > 0 && table_token_stride < R) return fail(QKROPE_ERR_INVALID, "table_token_stride must be >= rotary_dim");
    if (q_token_stride % 8 || k_token_stride % 8 || q_out_token_stride % 8 || k_out_token_stride % 8)
        return fail(QKROPE_ERR_UNSUPPORTED, "token strides must be multiples of 8 elements");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(q_out, 16) || !aligned(k_out, 16) ||
        !aligned(q_weight, 16) || !aligned(k_weight, 16))
        return fail(QKROPE_ERR_UNSUPPORTED, "q, k, outputs and weights must be 16-byte aligned");
    const int tsize = table_dtype == QKROPE_TABLE_F32 ? 4 : 2;
    if (!aligned(rope_table, tsize)) return fail(QKROPE_ERR_UNSUPPORTED, "rope_table is misaligned");

    // Outputs may alias their own input exactly (in place); any other overlap is rejected.
    const int64_t wq_len = norm_mode == QKROPE_NORM_ACROSS_HEADS ? (int64_t)Hq * D : D;
    const int64_t wk_len = norm_mode == QKROPE_NORM_ACROSS_HEADS ? (int64_t)Hk * D : D;
    Range rq = span_of(q, T, q_token_stride, (int64_t)Hq * D, 2);
    Range rk = span_of(k, T, k_token_stride, (int64_t)Hk * D, 2);
    Range rqo = span_of(q_out, T, q_out_token_stride, (int64_t)Hq * D, 2);
    Range rko = span_of(k_out, T, k_out_token_stride, (int64_t)Hk * D, 2);
    Range rt = span_of(rope_table, R > 0 ? T : 0, table_token_stride, R, tsize);
    Range rwq = norm_mode != QKROPE_NORM_NONE ? span_of(q_weight, 1, 0, wq_len, 2) : Range{0, 0, 0, 0};
    Range rwk = norm_mode != QKROPE_NORM_NONE ? span_of(k_weight, 1, 0, wk_len, 2) : Range{0, 0, 0, 0};
    const bool q_inplace = q_out == q && q_out_token_stride == q_token_stride;
    const bool k_inplace = k_out == k && k_out_token_stride == k_token_stride;
    if ((!q_inplace && overlap(rqo, rq)) || overlap(rqo, rk) || overlap(rqo, rt) ||
        overlap(rqo, rwq) || overlap(rqo, rwk) || overlap(rqo, rko))
        return fail(QKROPE_ERR_INVALID, "q_out overlaps another argument");
    if ((!k_inplace && overlap(rko, rk)) || overlap(rko, rq) || overlap(rko, rt) ||
        overlap(rko, rwq) || overlap(rko, rwk))
        return fail(QKROPE_ERR_INVALID, "k_out overlaps another argument");

    const int L = next_pow2(D / 8);           // lanes per head: one 16-byte chunk each
    const int64_t n_units[2] = {(int64_t)Hq * L, (int64_t)Hk * L};
    LaunchShape shape;
    if (!choose_shape(n_units, 2, &shape))
        return fail(QKROPE_ERR_UNSUPPORTED, "too many heads for one workgroup per token");

    KernelArgs a;
    std::memset(&a, 0, sizeof a);
    a.in[kQ] = static_cast<const uint16_t *>(q);
    a.in[kK] = static_cast<const uint16_t *>(k);
    a.out[kQ] = q_out;
    a.out[kK] = k_out;
    a.in_stride[kQ] = q_token_stride;
    a.in_stride[kK] = k_token_stride;
    a.out_stride[kQ] = q_out_token_stride;
    a.out_stride[kK] = k_out_token_stride;
    a.heads[kQ] = Hq;
    a.heads[kK] = Hk;
    a.heads[kV] = 0;
    a.weight[0] = static_cast<const uint16_t *>(q_weight);
    a.weight[1] = static_cast<const uint16_t *>(k_weight);
    a.table = rope_table;
    a.table_stride = table_token_stride;
    a.num_tokens = T;
    a.head_dim = D;
    a.rotary_dim = R;
    a.lanes_per_head = L;
    a.eps = (float)eps;
    const bool across = norm_mode == QKROPE_NORM_ACROSS_HEADS;
    a.inv_count[0] = (float)(1.0 / (double)(across ? (int64_t)Hq * D : D));
    a.inv_count[1] = (float)(1.0 / (double)(across ? (int64_t)Hk * D : D));
    a.qk_scale = 1.0f;
    a.v_scale = 1.0f;
    shape.blocks = T;

    KernelKey key;
    key.head_dim_tpl = 0;
    key.half_split = half;
    key.norm = norm_mode == QKROPE_NORM_NONE ? kNormNone
             : norm_mode == QKROPE_NORM_PER_HEAD ? kNormPerHead : kNormAcross;
    key.src = table_dtype == QKROPE_TABLE_F32 ? kSrcTableF32 : kSrcTableBF16;
    key.fp8 = false;
    key.slots = shape.slots;
    key.slot_uniform = shape.slot_uniform;
    return do_launch(h, key, shape, a, stream);
}

int qkrope_run_3d(qkrope_handle h, const void *qkv, const void *q_weight, const void *k_weight,
                  int64_t num_tokens, int ppf, int pph, int ppw, int num_frame_channels,
                  int num_height_channels, int num_width_channels, int num_heads_q,
                  int num_heads_k, int num_heads_v, int head_dim, double eps, double base,
                  int interleave, double factor, double low, double high, double attention_factor,
                  int is_qk_norm, int output_fp8, double output_quant_scale, double v_quant_scale,
                  void *q_out, void *k_out, void *v_out, void *stream)
{
    if (!h) return fail(QKROPE_ERR_INVALID, "handle is NULL");
    const int D = head_dim, Hq = num_heads_q, Hk = num_heads_k, Hv = num_heads_v;
    const int C[3] = {num_frame_channels, num_height_channels, num_width_channels};
    const int64_t T = num_tokens;
    if (T < 0 || Hq < 0 || Hk < 0 || Hv < 0) return fail(QKROPE_ERR_INVALID, "negative size");
    if (D != 64 && D != 128 && D != 256) return fail(QKROPE_ERR_INVALID, "head_dim must be 64, 128 or 256");
    for (int i = 0; i < 3; ++i)
        if (C[i] < 0 || C[i] % 2) return fail(QKROPE_ERR_INVALID, "channel counts must be even and >= 0");
    if (C[0] + C[1] + C[2] != D) return fail(QKROPE_ERR_INVALID, "channel counts must sum to head_dim");
    if (ppf <= 0 || pph <= 0 || ppw <= 0) return fail(QKROPE_ERR_INVALID, "ppf, pph, ppw must be positive");
    const int64_t S = (int64_t)ppf * pph * ppw;
    if (T % S) return fail(QKROPE_ERR_INVALID, "num_tokens must be a multiple of ppf*pph*ppw");
    if (!(base > 0.0) || !std::isfinite(base)) return fail(QKROPE_ERR_INVALID, "base must be finite and > 0");
    if (!(eps >= 0.0) || !std::isfinite(eps)) return fail(QKROPE_ERR_INVALID, "eps must be finite and >= 0");
    if (!(factor > 0.0) || !std::isfinite(factor)) return fail(QKROPE_ERR_INVALID, "factor must be finite and > 0");
    if (!std::isfinite(attention_factor)) return fail(QKROPE_ERR_INVALID, "attention_factor must be finite");
    if (factor == 1.0 && attention_factor != 1.0)
        return fail(QKROPE_ERR_INVALID, "attention_factor must be 1.0 when factor is 1.0");
    if (factor != 1.0 && !(high > low) )
        return fail(QKROPE_ERR_INVALID, "YaRN needs high > low");
    if (factor != 1.0 && (!std::isfinite(low) || !std::isfinite(high)))
        return fail(QKROPE_ERR_INVALID, "YaRN low/high must be finite");
    if (output_fp8 && (!(output_quant_scale > 0.0) || !std::isfinite(output_quant_scale) ||
                       !(v_quant_scale > 0.0) || !std::isfinite(v_quant_scale)))
        return fail(QKROPE_ERR_INVALID, "FP8 scales must be finite and > 0");
    if (T >= (int64_t(1) << 31)) return fail(QKROPE_ERR_UNSUPPORTED, "num_tokens must be < 2^31");
    if (T == 0 || Hq + Hk + Hv == 0) return ok();

    if (!qkv) return fail(QKROPE_ERR_INVALID, "qkv is NULL");
    if ((Hq && !q_out) || (Hk && !k_out) || (Hv && !v_out)) return fail(QKROPE_ERR_INVALID, "output is NULL");
    if (is_qk_norm && ((Hq && !q_weight) || (Hk && !k_weight)))
        return fail(QKROPE_ERR_INVALID, "norm weights are NULL while is_qk_norm is set");
    const int osize = output_fp8 ? 1 : 2;
    const uintptr_t oalign = output_fp8 ? 8 : 16;
    if (!aligned(qkv, 16) || !aligned(q_out, oalign) || !aligned(k_out, oalign) || !aligned(v_out, oalign))
        return fail(QKROPE_ERR_UNSUPPORTED, "qkv must be 16-byte aligned, outputs %d-byte aligned", (int)oalign);
    if (is_qk_norm && (!aligned(q_weight, 16) || !aligned(k_weight, 16)))
        return fail(QKROPE_ERR_UNSUPPORTED, "norm weights must be 16-byte aligned");

    const int64_t row = (int64_t)(Hq + Hk + Hv) * D;
    Range rin = span_of(qkv, T, row, row, 2);
    Range rq = span_of(q_out, T, (int64_t)Hq * D, (int64_t)Hq * D, osize);
    Range rk = span_of(k_out, T, (int64_t)Hk * D, (int64_t)Hk * D, osize);
    Range rv = span_of(v_out, T, (int64_t)Hv * D, (int64_t)Hv * D, osize);
    Range rwq = is_qk_norm ? span_of(q_weight, 1, 0, (int64_t)Hq * D, 2) : Range{0, 0, 0, 0};
    Range rwk = is_qk_norm ? span_of(k_weight, 1, 0, (int64_t)Hk * D, 2) : Range{0, 0, 0, 0};
    const Range outs[3] = {rq, rk, rv};
    for (int i = 0; i < 3; ++i) {
        if (overlap(outs[i], rin) || overlap(outs[i], rwq) || overlap(outs[i], rwk))
            return fail(QKROPE_ERR_INVALID, "an output overlaps qkv or a weight");
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outs[j])) return fail(QKROPE_ERR_INVALID, "outputs overlap each other");
    }

    const bool half = !interleave;
    const int units = D / 8;                   // 16-byte chunks per head: 8, 16 or 32
    const int64_t n_units[3] = {(int64_t)Hq * units, (int64_t)Hk * units, (int64_t)Hv * units};
    LaunchShape shape;
    if (!choose_shape(n_units, 3, &shape))
        return fail(QKROPE_ERR_UNSUPPORTED, "too many heads for one workgroup per token");

    KernelArgs a;
    std::memset(&a, 0, sizeof a);
    const uint16_t *base_in = static_cast<const uint16_t *>(qkv);
    a.in[kQ] = base_in;
    a.in[kK] = base_in + (int64_t)Hq * D;
    a.in[kV] = base_in + (int64_t)(Hq + Hk) * D;
    a.out[kQ] = q_out;
    a.out[kK] = k_out;
    a.out[kV] = v_out;
    for (int r = 0; r < 3; ++r) a.in_stride[r] = row;
    a.out_stride[kQ] = (int64_t)Hq * D;
    a.out_stride[kK] = (int64_t)Hk * D;
    a.out_stride[kV] = (int64_t)Hv * D;
    a.heads[kQ] = Hq;
    a.heads[kK] = Hk;
    a.heads[kV] = Hv;
    a.weight[0] = static_cast<const uint16_t *>(q_weight);
    a.weight[1] = static_cast<const uint16_t *>(k_weight);
    a.num_tokens = T;
    a.head_dim = D;
    a.rotary_dim = D;
    a.lanes_per_head = units;
    a.eps = (float)eps;
    a.inv_count[0] = Hq ? (float)(1.0 / ((double)Hq * D)) : 0.0f;
    a.inv_count[1] = Hk ? (float)(1.0 / ((double)Hk * D)) : 0.0f;
    a.qk_scale = output_fp8 ? (float)output_quant_scale : 1.0f;
    a.v_scale = output_fp8 ? (float)v_quant_scale : 1.0f;
    a.seq_len = (uint32_t)S;
    a.hw = (uint32_t)((int64_t)pph * ppw);
    a.ppw = (uint32_t)ppw;
    a.pph = (uint32_t)pph;
    a.div_seq = make_fast_div(a.seq_len);
    a.div_hw = make_fast_div(a.hw);
    a.div_w = make_fast_div(a.ppw);
    a.attention_factor = (float)attention_factor;
    // Per pair k of the concatenated [frame | height | width] frequency vector: its axis and the
    // YaRN-blended angular frequency, in fp64, handed to the kernel as revolutions per position.
    const double two_pi = 2.0 * 3.14159265358979323846;
    for (int k = 0, axis = 0, j = 0; k < D / 2; ++k, ++j) {
        while (j >= C[axis] / 2) {
            j -= C[axis] / 2;
            ++axis;
        }
        double omega = std::pow(base, -2.0 * j / (double)C[axis]);
        if (factor != 1.0) {
            double rho = (j - low) / (high - low);
            rho = rho < 0.0 ? 0.0 : (rho > 1.0 ? 1.0 : rho);
            omega = (omega / factor) * rho + omega * (1.0 - rho);
        }
        a.omega_rev[k] = (float)(omega / two_pi);
        a.axis[k] = (uint8_t)axis;
    }
    shape.blocks = T;

    KernelKey key;
    key.head_dim_tpl = D;
    key.half_split = half;
    key.norm = is_qk_norm ? kNormAcross : kNormNone;
    key.src = kSrc3D;
    key.fp8 = output_fp8 != 0;
    key.slots = shape.slots;
    key.slot_uniform = shape.slot_uniform;
    return do_launch(h, key, shape, a, stream);
}

}  // extern "C"
