// Camera prologue of the SANA-WM UCPE branch (vLLM-Omni "vllm_omni.diffusion.models.sana_wm.ucpe",
// cam_prep_func) for gfx950.
//
// The page gives the steps (ReLU, the K scale, the 4x4 ray projection, RoPE from separate
// (N, D/2) cos/sin tables) and the shapes ((B, N, H, D) in, (B, H, D, N) out, inflation_sq
// (B, H, N)); how they compose is the reading also stated in the library header:
//   Q' = RoPE(P_q . ReLU(q)),  K' = RoPE(P_kv . (k_scale * ReLU(k))),  V' = RoPE(P_kv . v),
// where P . x applies the token's 4x4 matrix to each group of four consecutive channels
// (y[4g+i] = sum_j P[i][j] x[4g+j]) and RoPE rotates the adjacent pairs (2i, 2i+1) by +theta;
// inflation_sq = |P_kv . k'|^2 / |k'|^2 for k' = k_scale * ReLU(k), 1 where k' = 0. ReLU keeps
// x when it is positive or a NaN (of either sign, as PyTorch's ReLU does: the page presents the
// op as a PyTorch module's native equivalent) and gives +0 otherwise.
//
// Work decomposition. The op streams 4 bytes per element (16-bit in, 16-bit out) for ~12 flops,
// and turns a token-major layout into a dim-major one: a token's heads arrive as contiguous
// 16-byte chunks, but each output row (b, h, d) runs along the tokens. A workgroup owns one
// batch, one tile of 64 consecutive tokens and a group of at most kCamMaxHeads heads, with Q,
// K and V of each:
//   * lane (token nl, chunk dl) loads its token's two 4x4 matrices and four (cos, sin) pairs
//     per chunk once (the fp32 tables are twice the size of a bf16 head, so sharing them over
//     the group's heads and tensors matters), then issues the 16-byte loads of all its chunks;
//   * per head and tensor: ReLU (Q, K) on the packed 16-bit pairs (three packed integer
//     operations per two values), the K scale, the projection and the rotation in fp32, rounding to 16 bits, one
//     16-byte LDS write of the chunk into the token's row of a [64 tokens][row_chunks] tile
//     (D/8 chunks rounded up to a power of two) whose chunks are rotated by token/8 modulo
//     row_chunks (so the column reads below hit distinct banks);
//   * after a barrier, lane (row d, token segment s) gathers 8 consecutive tokens of dim d for
//     one 16-byte store (issued after the last tensor): 8 lanes cover a row's 64-token run. The
//     tile is double-buffered, one barrier per tensor;
//   * K also sums the key's squared norms before and after the projection over the token's
//     lanes with DPP, for inflation_sq.
// Output rows are out_row_stride elements apart (>= N): with a pitch that is a multiple of 64
// elements every row starts on a 128-byte line, a tile's 128-byte run of a row fills one line,
// and the whole tiles store non-temporally; otherwise the runs straddle two lines, which the L2
// completes from the neighbouring tiles, so the stores stay normal (measured on MI355X: 2 x
// 18432 tokens, rows on lines, 64.7% of 8 TB/s; 2 x 18480 into rows padded to 18496, 63.7%;
// 2 x 18480 contiguous, rows at four phases, 57.3%).
// Block order: token tiles fastest, so the workgroups that run together on one XCD write
// adjacent runs of the same output rows (measured on MI355X: 20% faster than head groups
// fastest); each (batch, head group) has its tiles padded to a multiple of 8 and XCD x takes
// the x-th contiguous eighth of them, so the tokens' matrices and table rows, re-read by every
// head group, come from that XCD's L2.
#include "qkrope_kernel_impl.h"
#include "qkrope_cam.h"

namespace qkrope {
namespace dev {

typedef short s16x2 __attribute__((ext_vector_type(2)));

// ReLU of two packed 16-bit floats (bf16 or binary16), NaNs kept. Read as int16, a negative
// number (-0 to -inf) is at most -C, C = 0x80 (bf16: -inf is 0xFF80) or 0x400 (binary16: 0xFC00),
// and the negative NaNs lie between -C and 0. Adding C - 1 with saturation leaves exactly the
// negative numbers below zero (positive patterns saturate at 0x7FFF instead of wrapping); the
// arithmetic shift turns that sign into a mask of the halves to clear. Three packed operations.
template <int ACT>
__device__ __forceinline__ uint32_t relu2(uint32_t u)
{
    constexpr short C1 = ACT == kActBF16 ? 0x7F : 0x3FF;
    const s16x2 t = __builtin_elementwise_add_sat(__builtin_bit_cast(s16x2, u), s16x2{C1, C1});
    const uint32_t clear = __builtin_bit_cast(uint32_t, t >> 15);
    return u & ~clear;
}

// y = P . x on each group of four channels of an 8-element chunk.
__device__ __forceinline__ void project8(const float P[16], const float x[8], float p[8])
{
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float acc = P[4 * i] * x[4 * g];
            acc = __builtin_fmaf(P[4 * i + 1], x[4 * g + 1], acc);
            acc = __builtin_fmaf(P[4 * i + 2], x[4 * g + 2], acc);
            p[4 * g + i] = __builtin_fmaf(P[4 * i + 3], x[4 * g + 3], acc);
        }
}

// ACT: activation format. CPL: 16-byte chunks per lane per head (1 for head_dim <= 64, else
// ceil(head_dim / 64)). LT: lanes per token (power of two >= head_dim / 8 / CPL, at most 8);
// workgroups are 64 * LT <= 512 lanes.
template <int ACT, int CPL, int LT>
__global__ void __launch_bounds__(64 * LT) qkrope_cam_kernel(const CamArgs a)
{
    extern __shared__ __align__(16) uint8_t s_tile[];   // 2 x [64 tokens][row_chunks x 8] 16-bit
    const int tid = threadIdx.x;
    constexpr int NTH = 64 * LT;

    // Every argument the first data loads depend on, taken by an empty asm statement at the
    // start: the compiler then fetches them in one batch of scalar loads, where it otherwise
    // spread them over five dependent round trips between the block decomposition's steps.
    asm volatile("" ::"s"(a.xcd_group), "s"(a.div_xcd.m), "s"(a.div_xcd.l), "s"(a.div_tiles.m),
                 "s"(a.div_tiles.l), "s"(a.tiles_padded), "s"(a.tiles), "s"(a.div_groups.m),
                 "s"(a.div_groups.l), "s"(a.groups), "s"(a.heads_per_group), "s"(a.heads),
                 "s"(a.head_dim), "s"(a.num_tokens), "s"(a.in[0]), "s"(a.in[1]), "s"(a.in[2]),
                 "s"(a.in_stride[0]), "s"(a.in_stride[1]), "s"(a.in_stride[2]), "s"(a.proj[0]),
                 "s"(a.proj[1]), "s"(a.cos_table), "s"(a.sin_table));
    // block -> (batch, head group, tile); uniform, with host-computed magic divisors; with
    // xcd_group G the grid is a whole number of 8*G runs and every block is renumbered
    // (branch-free: a select)
    uint32_t blk = blockIdx.x;
    {
        const uint32_t G = a.xcd_group, j = blk >> 3, x = blk & 7u;
        const uint32_t q = fast_div(j, a.div_xcd.m, a.div_xcd.l);
        const uint32_t r = q * (8u * G) + x * G + (j - q * G);
        blk = G ? r : blk;
    }
    const uint32_t bg = fast_div(blk, a.div_tiles.m, a.div_tiles.l);
    const uint32_t tile = blk - bg * (uint32_t)a.tiles_padded;
    if (tile >= (uint32_t)a.tiles) return;           // padding: no work (uniform)
    const uint32_t b = fast_div(bg, a.div_groups.m, a.div_groups.l);
    const uint32_t grp = bg - b * (uint32_t)a.groups;

    const int D = a.head_dim, C = D >> 3, H = a.heads;
    const int CP = a.row_chunks, RS = CP * 8;    // LDS row: CP chunks, RS 16-bit elements
    const int64_t N = a.num_tokens, RP = a.out_row_stride;   // RP: output row pitch, elements
    const int64_t n0 = (int64_t)tile * kCamTile;
    const int nvalid = (int)(N - n0 < kCamTile ? N - n0 : kCamTile);
    const int nl = tid / LT, dl = tid % LT;
    const int nlc = nl < nvalid ? nl : nvalid - 1;          // loads stay inside the tile's tokens
    const int64_t bn = (int64_t)b * N + n0 + nlc;
    const int h0 = (int)grp * a.heads_per_group;
    const int nh = a.heads_per_group < H - h0 ? a.heads_per_group : H - h0;
    const int iters = 3 * nh;

    // data loads first (every address valid: iterations past the group's heads reload its last
    // head, so the loads are unconditional and the compiler can wait for each one exactly)
    constexpr int MH = kCamMaxHeads / CPL > 0 ? kCamMaxHeads / CPL : 1;
    constexpr int MI = 3 * MH;
    const uint8_t *wg_in[3];
    uint32_t row_off[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        wg_in[r] = reinterpret_cast<const uint8_t *>(a.in[r] + ((int64_t)b * N + n0) * a.in_stride[r]);
        row_off[r] = (uint32_t)(nlc * a.in_stride[r] * 2) + (uint32_t)(h0 * D * 2);
    }
    bool chv[CPL];
    int chi[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int ch = dl + c * LT;
        chv[c] = ch < C;
        chi[c] = chv[c] ? ch : 0;
    }
    uint4 v[MI][CPL];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const int r = i % 3, hi = i / 3 < nh ? i / 3 : nh - 1;
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            v[i][c] = ld16_stream<true>(wg_in[r], row_off[r] + (uint32_t)(hi * D * 2) + 16u * (uint32_t)chi[c]);
    }
    // the token's matrices and the chunk's table values (normal loads: re-read by other groups)
    float pq[16], pk[16];
    {
        const f32x4 *P = reinterpret_cast<const f32x4 *>(a.proj[0] + bn * 16);
        const f32x4 *Q = reinterpret_cast<const f32x4 *>(a.proj[1] + bn * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 u = P[i], w = Q[i];
            pq[4 * i] = u.x; pq[4 * i + 1] = u.y; pq[4 * i + 2] = u.z; pq[4 * i + 3] = u.w;
            pk[4 * i] = w.x; pk[4 * i + 1] = w.y; pk[4 * i + 2] = w.z; pk[4 * i + 3] = w.w;
        }
    }
    float tc[CPL][4], ts[CPL][4];
    uint32_t ldsw[CPL];      // LDS byte offset of the chunk in the token's row (rotated)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const f32x4 cv = *reinterpret_cast<const f32x4 *>(a.cos_table + (n0 + nlc) * (D / 2) + 4 * chi[c]);
        const f32x4 sv = *reinterpret_cast<const f32x4 *>(a.sin_table + (n0 + nlc) * (D / 2) + 4 * chi[c]);
        tc[c][0] = cv.x; tc[c][1] = cv.y; tc[c][2] = cv.z; tc[c][3] = cv.w;
        ts[c][0] = sv.x; ts[c][1] = sv.y; ts[c][2] = sv.z; ts[c][3] = sv.w;
        ldsw[c] = (uint32_t)(nl * RS * 2 + ((chi[c] + (nl >> 3)) & (CP - 1)) * 16);
    }
    // the lane's output units (row d, 8-token segment s), 8 * D of them, and their LDS reads
    int ud[CPL], us[CPL];
    uint32_t ldsr[CPL];
    int64_t st_off[CPL];     // byte offset inside an output plane (b, h)
    bool uv[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int u = tid + j * NTH;
        uv[j] = u < 8 * D;
        const int uu = uv[j] ? u : 0;
        us[j] = uu & 7;
        ud[j] = uu >> 3;
        ldsr[j] = (uint32_t)((us[j] * 8 * RS + (((ud[j] >> 3) + us[j]) & (CP - 1)) * 8 + (ud[j] & 7)) * 2);
        st_off[j] = (ud[j] * RP + n0 + us[j] * 8) * 2;
    }
    // whole tiles of outputs with 16-byte aligned rows: 16-byte stores, issued after the loop
    // (measured slightly faster than storing each tensor as it is gathered); the last, partial
    // tile stores as it goes, 16 bytes per whole segment, and unaligned rows store elements
    const bool fast = a.vec_store && nvalid == kCamTile;
    // buffered outputs cost 4 * MI * CPL registers; past two chunks per lane they would cut the
    // occupancy below two workgroups per CU, so those variants store as they go
    constexpr bool kEndStores = CPL <= 2;
    uint4 o[kEndStores ? MI : 1][CPL];

#pragma unroll
    for (int i = 0; i < MI; ++i) {
        if (i >= iters) continue;          // uniform
        const int r = i % 3, h = h0 + i / 3;
        uint8_t *buf = s_tile + (i & 1) * (kCamTile * RS * 2);

        float na = 0.0f, np = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            uint4 raw = v[i][c];
            if (r < 2)
                raw = make_uint4(relu2<ACT>(raw.x), relu2<ACT>(raw.y), relu2<ACT>(raw.z), relu2<ACT>(raw.w));
            float x[8], p[8], y[8];
            unpack8<ACT>(raw, x);
            if (r == 0) {
                project8(pq, x, p);
            } else if (r == 1) {
                // |ReLU(k)|^2 from the packed pairs (products of 16-bit values are exact in
                // fp32); k_scale^2 is applied to the sum below
                if (chv[c]) na = sumsq_packed<ACT>(raw, na);
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] *= a.k_scale;
                project8(pk, x, p);
                if (chv[c]) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) np = __builtin_fmaf(p[e], p[e], np);
                }
            } else {
                project8(pk, x, p);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                y[2 * e] = __builtin_fmaf(p[2 * e], tc[c][e], -p[2 * e + 1] * ts[c][e]);
                y[2 * e + 1] = __builtin_fmaf(p[2 * e + 1], tc[c][e], p[2 * e] * ts[c][e]);
            }
            if (chv[c]) *reinterpret_cast<uint4 *>(buf + ldsw[c]) = pack8<ACT>(y);
        }
        if (r == 1 && a.inflation) {       // uniform
            na = group_sum(na, LT) * (a.k_scale * a.k_scale);
            np = group_sum(np, LT);
            if (dl == 0 && nl < nvalid)
                // 1 for a zero key; a NaN key keeps the quotient's NaN
                a.inflation[((int64_t)b * H + h) * N + n0 + nl] = na != 0.0f ? np * __builtin_amdgcn_rcpf(na) : 1.0f;
        }
        __syncthreads();

        uint16_t *out = a.out[r];
        uint8_t *plane = reinterpret_cast<uint8_t *>(out + ((int64_t)b * H + h) * D * RP);
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            if (!uv[j]) continue;
            const uint16_t *src = reinterpret_cast<const uint16_t *>(buf + ldsr[j]);
            uint16_t e8[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) e8[k] = src[k * RS];
            const uint4 w = make_uint4(e8[0] | (uint32_t)e8[1] << 16, e8[2] | (uint32_t)e8[3] << 16,
                                       e8[4] | (uint32_t)e8[5] << 16, e8[6] | (uint32_t)e8[7] << 16);
            if (fast) {
                if (kEndStores) o[i][j] = w;
                else *reinterpret_cast<uint4 *>(plane + st_off[j]) = w;
            } else if (a.vec_store && us[j] * 8 + 8 <= nvalid) {
                // the last, partial tile: its whole 8-token segments still take 16-byte stores
                *reinterpret_cast<uint4 *>(plane + st_off[j]) = w;
            } else {
                uint16_t *dst = reinterpret_cast<uint16_t *>(plane) + ud[j] * RP + n0 + us[j] * 8;
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if (us[j] * 8 + k < nvalid) dst[k] = e8[k];
            }
        }
    }
    if (kEndStores && fast) {
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            if (i >= iters) continue;
            const int r = i % 3, h = h0 + i / 3;
            uint8_t *plane = reinterpret_cast<uint8_t *>(a.out[r] + ((int64_t)b * H + h) * D * RP);
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                if (!uv[j]) continue;
                if (a.nt_store) {           // uniform: every row starts on a line
                    const uint4 ov = o[i][j];
                    const u32x4 w4 = {ov.x, ov.y, ov.z, ov.w};
                    __builtin_nontemporal_store(w4, reinterpret_cast<u32x4 *>(plane + st_off[j]));
                } else {
                    *reinterpret_cast<uint4 *>(plane + st_off[j]) = o[i][j];
                }
            }
        }
    }
}

template <int ACT, int CPL, int LT>
hipError_t go_cam(const CamArgs &a, int64_t blocks, int lds_bytes, hipStream_t st)
{
    hipLaunchKernelGGL((qkrope_cam_kernel<ACT, CPL, LT>), dim3((unsigned)blocks), dim3(64 * LT),
                       lds_bytes, st, a);
    return hipGetLastError();
}

template <int ACT>
hipError_t launch_cam_act(const CamArgs &a, int cpl, int64_t blocks, int lds_bytes, hipStream_t st)
{
    const int lt = a.lanes_per_token;
    if (cpl > 1 && lt != 8) return hipErrorInvalidValue;
    switch (cpl) {
    case 1: break;
    case 2: return go_cam<ACT, 2, 8>(a, blocks, lds_bytes, st);
    case 3: return go_cam<ACT, 3, 8>(a, blocks, lds_bytes, st);
    case 4: return go_cam<ACT, 4, 8>(a, blocks, lds_bytes, st);
    default: return hipErrorInvalidValue;
    }
    switch (lt) {
    case 1: return go_cam<ACT, 1, 1>(a, blocks, lds_bytes, st);
    case 2: return go_cam<ACT, 1, 2>(a, blocks, lds_bytes, st);
    case 4: return go_cam<ACT, 1, 4>(a, blocks, lds_bytes, st);
    case 8: return go_cam<ACT, 1, 8>(a, blocks, lds_bytes, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace dev

hipError_t launch_cam(const CamArgs &a, int act, int cpl, int64_t blocks, int lds_bytes,
                      hipStream_t st)
{
    if (act == kActBF16) return dev::launch_cam_act<kActBF16>(a, cpl, blocks, lds_bytes, st);
    if (act == kActF16) return dev::launch_cam_act<kActF16>(a, cpl, blocks, lds_bytes, st);
    return hipErrorInvalidValue;
}

}  // namespace qkrope
