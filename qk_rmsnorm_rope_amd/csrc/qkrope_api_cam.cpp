// qkrope_api_cam.cpp -- qkrope_cam_prep (include/qkrope.h): the camera prologue of the
// SANA-WM UCPE branch. Argument validation, launch shape and block order; the kernel is in
// qkrope_kernels_cam.hip.
#include "qkrope.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdint>

#include "qkrope_cam.h"
#include "qkrope_host.h"

using namespace qkrope;
using namespace qkrope::host;

extern "C" {

int qkrope_cam_prep(qkrope_handle h, const void *q, const void *k, const void *v, int act_dtype,
                    const float *proj_q, const float *proj_kv, const float *rope_cos,
                    const float *rope_sin, float k_scale, int64_t batch, int64_t num_tokens,
                    int num_heads, int head_dim, int64_t q_stride, int64_t k_stride,
                    int64_t v_stride, void *q_out, void *k_out, void *v_out,
                    int64_t out_row_stride, float *inflation_sq, void *stream)
{
    if (!h) return fail(QKROPE_ERR_INVALID, "handle is NULL");
    const int64_t B = batch, N = num_tokens;
    const int H = num_heads, D = head_dim;
    if (B < 0 || N < 0 || H < 0 || D <= 0)
        return fail(QKROPE_ERR_INVALID, "negative size or non-positive head_dim");
    if (D % 4) return fail(QKROPE_ERR_INVALID, "head_dim must be a multiple of 4 (4x4 projection groups)");
    if (act_dtype != QKROPE_DTYPE_BF16 && act_dtype != QKROPE_DTYPE_F16)
        return fail(QKROPE_ERR_INVALID, "act_dtype must be QKROPE_DTYPE_BF16 or QKROPE_DTYPE_F16");
    if (D % 8 || D > 256) return fail(QKROPE_ERR_UNSUPPORTED, "head_dim must be a multiple of 8 and <= 256");
    if (N >= (int64_t(1) << 31) || B >= (int64_t(1) << 31) || B * N >= (int64_t(1) << 31))
        return fail(QKROPE_ERR_UNSUPPORTED, "batch * num_tokens must be < 2^31");
    const int64_t strides[3] = {q_stride, k_stride, v_stride};
    for (int r = 0; r < 3; ++r) {
        if (strides[r] < (int64_t)H * D) return fail(QKROPE_ERR_INVALID, "token stride smaller than num_heads * head_dim");
        if (strides[r] % 8 || strides[r] >= (int64_t(1) << 24))
            return fail(QKROPE_ERR_UNSUPPORTED, "token strides must be multiples of 8 elements and < 2^24");
    }
    if (out_row_stride < N) return fail(QKROPE_ERR_INVALID, "out_row_stride smaller than num_tokens");
    if (out_row_stride >= (int64_t(1) << 31)) return fail(QKROPE_ERR_UNSUPPORTED, "out_row_stride must be < 2^31");
    if (B * N == 0 || H == 0) return ok();
    const void *ins[3] = {q, k, v};
    void *outs[3] = {q_out, k_out, v_out};
    if (!q || !k || !v || !proj_q || !proj_kv || !rope_cos || !rope_sin || !q_out || !k_out || !v_out)
        return fail(QKROPE_ERR_INVALID, "a required pointer is NULL");
    for (int r = 0; r < 3; ++r) {
        if (!aligned(ins[r], 16)) return fail(QKROPE_ERR_UNSUPPORTED, "q, k, v must be 16-byte aligned");
        if (!aligned(outs[r], 2)) return fail(QKROPE_ERR_INVALID, "outputs must be 2-byte aligned");
    }
    if (!aligned(proj_q, 16) || !aligned(proj_kv, 16) || !aligned(rope_cos, 16) || !aligned(rope_sin, 16))
        return fail(QKROPE_ERR_UNSUPPORTED, "projections and tables must be 16-byte aligned");
    if (inflation_sq && !aligned(inflation_sq, 4)) return fail(QKROPE_ERR_INVALID, "inflation_sq must be 4-byte aligned");
    // outputs must not overlap an input or one another (row spans of B*H*D rows)
    const int64_t out_rows = B * H * (int64_t)D;
    Range ro[4] = {span_of(q_out, out_rows, out_row_stride, N, 2), span_of(k_out, out_rows, out_row_stride, N, 2),
                   span_of(v_out, out_rows, out_row_stride, N, 2),
                   span_of(inflation_sq, inflation_sq ? 1 : 0, B * H * N, B * H * N, 4)};
    Range ri[7] = {span_of(q, B * N, q_stride, (int64_t)H * D, 2), span_of(k, B * N, k_stride, (int64_t)H * D, 2),
                   span_of(v, B * N, v_stride, (int64_t)H * D, 2), span_of(proj_q, 1, B * N * 16, B * N * 16, 4),
                   span_of(proj_kv, 1, B * N * 16, B * N * 16, 4), span_of(rope_cos, 1, N * D / 2, N * D / 2, 4),
                   span_of(rope_sin, 1, N * D / 2, N * D / 2, 4)};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 7; ++j)
            if (overlap(ro[i], ri[j])) return fail(QKROPE_ERR_INVALID, "an output overlaps an input");
        for (int j = i + 1; j < 4; ++j)
            if (overlap(ro[i], ro[j])) return fail(QKROPE_ERR_INVALID, "outputs overlap");
    }

    CamArgs a;
    for (int r = 0; r < 3; ++r) {
        a.in[r] = static_cast<const uint16_t *>(ins[r]);
        a.in_stride[r] = strides[r];
        a.out[r] = static_cast<uint16_t *>(outs[r]);
    }
    a.proj[0] = proj_q;
    a.proj[1] = proj_kv;
    a.cos_table = rope_cos;
    a.sin_table = rope_sin;
    a.inflation = inflation_sq;
    a.num_tokens = N;
    a.batch = (int)B;
    a.heads = H;
    a.head_dim = D;
    // Workgroups of at most 512 lanes (8 per token): with ~100 VGPRs a 1024-lane workgroup is
    // alone on its CU and nothing overlaps its load, barrier and store phases (measured on
    // MI355X at 2 x 18480 tokens: head_dim 128 in 1024-lane workgroups 176 us, 41% of 8 TB/s).
    // Wider heads give each lane more 16-byte chunks instead.
    const int C = D / 8;
    const int cpl = C <= 8 ? 1 : (C + 7) / 8;
    const int lanes = C <= 8 ? next_pow2(C) : 8;
    a.lanes_per_token = lanes;
    // Heads per workgroup: groups of at most kCamMaxHeads / cpl, as even as possible. A group
    // shares its tokens' matrices and table values over 3 tensors x its heads; measured on
    // MI355X (2 x 18480 tokens x 20 heads x 64), 2 heads per group beat 1, 3 and 4.
    const int max_heads = std::max(1, kCamMaxHeads / cpl);
    const int ngroups = (H + max_heads - 1) / max_heads;
    a.heads_per_group = (H + ngroups - 1) / ngroups;
    a.groups = (H + a.heads_per_group - 1) / a.heads_per_group;
    a.tiles = (int)((N + kCamTile - 1) / kCamTile);
    // Block order: tiles fastest within each (batch, head group), whose tiles are padded to a
    // multiple of 8 (padding blocks exit at once) so that XCD x takes the x-th contiguous eighth
    // of every group's tiles. Each XCD then sees one eighth of the tokens, and every head group
    // re-reads those tokens' matrices and table rows from its own L2: measured on MI355X
    // (2 x 18480 x 20 x 64), 426 -> 302 MB read per launch for 293 MB algorithmic, 2% faster
    // than plain runs of 16 tiles.
    a.tiles_padded = a.tiles >= 8 ? (a.tiles + 7) / 8 * 8 : a.tiles;
    const int64_t blocks = B * a.tiles_padded * (int64_t)a.groups;
    // a dispatch holds at most 2^32 - 1 work-items per dimension (first reached with one head:
    // 2^29 (b, n) tokens at head_dim 64, 206 GB of inputs and outputs)
    if (blocks >= (int64_t(1) << 31) || blocks * 64 * lanes >= (int64_t(1) << 32))
        return fail(QKROPE_ERR_UNSUPPORTED, "grid too large");
    a.xcd_group = a.tiles >= 8 ? (uint32_t)(a.tiles_padded / 8) : 0u;
    a.div_tiles = make_fast_div((uint32_t)a.tiles_padded);
    a.div_groups = make_fast_div((uint32_t)a.groups);
    a.div_xcd = make_fast_div(a.xcd_group ? a.xcd_group : 1u);
    // LDS rows of a power-of-two chunk count, so the per-token chunk rotation is a mask
    a.row_chunks = next_pow2(C);
    a.out_row_stride = out_row_stride;
    a.vec_store = (out_row_stride % 8 == 0) && aligned(q_out, 16) && aligned(k_out, 16) && aligned(v_out, 16);
    // Rows that all start on a 128-byte line (a pitch that is a multiple of 64 elements, bases on
    // lines): each tile's run of a row is one whole line, written by one store instruction, and
    // non-temporal stores are faster (measured on MI355X, 2 x 18480 x 20 x 64 into rows of 18496:
    // 119.8 -> 113.8 us; 2 x 18432 contiguous: 116.4 -> 111.8 us). Rows at other phases keep
    // normal stores: the L2 completes the lines that their runs split between neighbouring tiles,
    // and non-temporal stores there ran 39% slower.
    a.nt_store = a.vec_store && out_row_stride % 64 == 0 && aligned(q_out, 128) && aligned(k_out, 128) &&
                 aligned(v_out, 128);
    a.k_scale = k_scale;
    const int lds_bytes = 2 * kCamTile * a.row_chunks * 16;
    DeviceGuard g(h->device);
    if (g.err != hipSuccess) return fail(QKROPE_ERR_DEVICE, "hipSetDevice: %s", hipGetErrorString(g.err));
    const hipError_t e = launch_cam(a, act_dtype == QKROPE_DTYPE_F16 ? kActF16 : kActBF16, cpl,
                                    blocks, lds_bytes, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(QKROPE_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
