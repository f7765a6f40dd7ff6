// Camera prologue of the SANA-WM UCPE branch (vLLM-Omni "vllm_omni.diffusion.models.sana_wm.ucpe",
// cam_prep_func) for gfx950.
//
// The page gives the steps (ReLU, the K scale, the 4x4 ray projection, RoPE from separate
// (N, D/2) cos/sin tables) and the shapes ((B, N, H, D) in, (B, H, D, N) out, inflation_sq
// (B, H, N)); how they compose is the reading also stated in the library header:
//   Q' = RoPE(P_q . ReLU(q)),  K' = RoPE(P_kv . (k_scale * ReLU(k))),  V' = RoPE(P_kv . v),
// where P . x applies the token's 4x4 matrix to each group of four consecutive channels
// (y[4g+i] = sum_j P[i][j] x[4g+j]) and RoPE rotates the adjacent pairs (2i, 2i+1) by +theta;
// inflation_sq = |P_kv . k'|^2 / |k'|^2 for k' = k_scale * ReLU(k), 1 where k' = 0.
//
// Work decomposition. The op streams 4 bytes per element (16-bit in, 16-bit out) for ~12 flops,
// so it is HBM-bound; what costs is the layout change: a token's heads arrive as contiguous
// 16-byte chunks, but each output row (b, h, d) runs along the tokens. A workgroup owns one
// batch, a tile of 64 consecutive tokens and a group of heads:
//   * lane (token nl, chunk dl) loads its token's two 4x4 matrices and its four (cos, sin)
//     pairs once, then for each head of the group and each of Q, K, V: one 16-byte load,
//     ReLU / scale / projection / rotation in fp32 registers, round to 16 bits, and one 16-byte
//     LDS write of the token's chunk (the next iteration's load is already in flight);
//   * after a barrier, lane (row d, token segment s) gathers 8 consecutive tokens of dim d
//     from LDS and writes them with one 16-byte non-temporal store: eight lanes cover a row's
//     64-token run, so every store instruction writes whole 128-byte lines;
//   * the LDS tile is double-buffered (one barrier per tensor) and its chunks are rotated by
//     token/8, which makes the column reads of the 8 segments of a wave fall in distinct banks;
//   * K's squared norms before and after the projection are summed over the token's lanes
//     with DPP, giving inflation_sq without another pass.
#include "qkrope_kernel_impl.h"

namespace qkrope {
namespace dev {

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

template <int ACT, int CPL>
__global__ void __launch_bounds__(1024) qkrope_cam_kernel(const CamArgs a)
{
    extern __shared__ __align__(16) uint8_t s_tile[];   // 2 x [64 tokens][D] 16-bit values
    const int tid = threadIdx.x, nth = blockDim.x;

    uint32_t blk = blockIdx.x;
    if (a.xcd_group) {
        const uint32_t G = a.xcd_group, S = 8u * G, full = gridDim.x / S * S;
        if (blk < full) {
            const uint32_t j = blk >> 3, x = blk & 7u;
            blk = (j / G) * S + x * G + j % G;
        }
    }
    const uint32_t grp = blk % (uint32_t)a.groups;
    const uint32_t bt = blk / (uint32_t)a.groups;
    const uint32_t tile = bt % (uint32_t)a.tiles;
    const uint32_t b = bt / (uint32_t)a.tiles;

    const int D = a.head_dim, C = D >> 3, H = a.heads;
    const int64_t N = a.num_tokens;
    const int64_t n0 = (int64_t)tile * kCamTile;
    const int nvalid = (int)(N - n0 < kCamTile ? N - n0 : kCamTile);
    const int LT = a.lanes_per_token;
    const int nl = tid >> a.lpt_shift, dl = tid & (LT - 1);
    const int nlc = nl < nvalid ? nl : nvalid - 1;          // loads stay inside the tile's tokens
    const int64_t bn = (int64_t)b * N + n0 + nlc;

    // the token's projections (normal loads: every head group of the tile re-reads them)
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
    // the lane's chunks: pairs 4*ch .. 4*ch+3 of the token's table row
    float tc[CPL][4], ts[CPL][4];
    bool chv[CPL];
    uint32_t choff[CPL];     // byte offset of the chunk inside a head
    uint32_t ldsw[CPL];      // LDS byte offset of the chunk in the token's row (rotated)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int ch = dl + c * LT;
        chv[c] = ch < C;
        const int chc = chv[c] ? ch : 0;
        choff[c] = 16u * (uint32_t)chc;
        ldsw[c] = (uint32_t)(nl * D * 2 + ((chc + (nl >> 3)) % C) * 16);
        const f32x4 cv = *reinterpret_cast<const f32x4 *>(a.cos_table + (n0 + nlc) * (D / 2) + 4 * chc);
        const f32x4 sv = *reinterpret_cast<const f32x4 *>(a.sin_table + (n0 + nlc) * (D / 2) + 4 * chc);
        tc[c][0] = cv.x; tc[c][1] = cv.y; tc[c][2] = cv.z; tc[c][3] = cv.w;
        ts[c][0] = sv.x; ts[c][1] = sv.y; ts[c][2] = sv.z; ts[c][3] = sv.w;
    }
    // the lane's output units (row d, 8-token segment s) and their rotated LDS reads
    int ud[CPL], us[CPL];
    uint32_t ldsr[CPL];
    bool uv[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int u = tid + j * nth;
        uv[j] = u < 8 * D;
        const int uu = uv[j] ? u : 0;
        us[j] = uu & 7;
        ud[j] = uu >> 3;
        const int ch = ud[j] >> 3, e = ud[j] & 7;
        ldsr[j] = (uint32_t)((us[j] * 8 * D + ((ch + us[j]) % C) * 8 + e) * 2);
    }

    const int h0 = (int)grp * a.heads_per_group;
    const int nh = a.heads_per_group < H - h0 ? a.heads_per_group : H - h0;
    const int iters = 3 * nh;
    const uint8_t *wg_in[3];
    uint32_t row_off[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        wg_in[r] = reinterpret_cast<const uint8_t *>(a.in[r] + ((int64_t)b * N + n0) * a.in_stride[r]);
        row_off[r] = (uint32_t)(nlc * a.in_stride[r] * 2);
    }

    auto load = [&](int it, uint4 v[CPL]) {
        const int hi = it / 3, r = it - 3 * hi;
        const uint8_t *base = sel3(r, wg_in[0], wg_in[1], wg_in[2]);
        const uint32_t off = sel3(r, row_off[0], row_off[1], row_off[2]) +
                             (uint32_t)((h0 + hi) * D * 2);
#pragma unroll
        for (int c = 0; c < CPL; ++c) v[c] = ld16_stream<true>(base, off + choff[c]);
    };

    uint4 cur[CPL];
    load(0, cur);
    for (int it = 0; it < iters; ++it) {
        const int hi = it / 3, r = it - 3 * hi, h = h0 + hi;
        uint4 nxt[CPL];
        if (it + 1 < iters) load(it + 1, nxt);
        uint8_t *buf = s_tile + (it & 1) * (kCamTile * D * 2);

        float na = 0.0f, np = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            float x[8], p[8], y[8];
            unpack8<ACT>(cur[c], x);
            if (r == 0) {
#pragma unroll
                for (int i = 0; i < 8; ++i) x[i] = x[i] > 0.0f ? x[i] : 0.0f;
                project8(pq, x, p);
            } else if (r == 1) {
#pragma unroll
                for (int i = 0; i < 8; ++i) x[i] = (x[i] > 0.0f ? x[i] : 0.0f) * a.k_scale;
                project8(pk, x, p);
                if (chv[c]) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        na = __builtin_fmaf(x[i], x[i], na);
                        np = __builtin_fmaf(p[i], p[i], np);
                    }
                }
            } else {
                project8(pk, x, p);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                y[2 * i] = __builtin_fmaf(p[2 * i], tc[c][i], -p[2 * i + 1] * ts[c][i]);
                y[2 * i + 1] = __builtin_fmaf(p[2 * i + 1], tc[c][i], p[2 * i] * ts[c][i]);
            }
            if (chv[c]) *reinterpret_cast<uint4 *>(buf + ldsw[c]) = pack8<ACT>(y);
        }
        if (r == 1 && a.inflation) {
            na = group_sum(na, LT);
            np = group_sum(np, LT);
            if (dl == 0 && nl < nvalid)
                a.inflation[((int64_t)b * H + h) * N + n0 + nl] = na > 0.0f ? np / na : 1.0f;
        }
        __syncthreads();

        uint16_t *out = sel3(r, a.out[0], a.out[1], a.out[2]);
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            if (!uv[j]) continue;
            const uint16_t *src = reinterpret_cast<const uint16_t *>(buf + ldsr[j]);
            uint16_t v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = src[k * D];
            uint16_t *dst = out + (((int64_t)b * H + h) * D + ud[j]) * N + n0 + us[j] * 8;
            if (a.vec_store && us[j] * 8 + 8 <= nvalid) {
                const uint4 w = make_uint4(v[0] | (uint32_t)v[1] << 16, v[2] | (uint32_t)v[3] << 16,
                                           v[4] | (uint32_t)v[5] << 16, v[6] | (uint32_t)v[7] << 16);
                st16_stream(reinterpret_cast<uint8_t *>(dst), w);
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if (us[j] * 8 + k < nvalid) dst[k] = v[k];
            }
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c) cur[c] = nxt[c];
    }
}

}  // namespace dev

hipError_t launch_cam(const CamArgs &a, int act, int cpl, int64_t blocks, int threads,
                      int lds_bytes, hipStream_t st)
{
    const dim3 grid((unsigned)blocks), block((unsigned)threads);
    if (act == kActBF16 && cpl == 1)
        hipLaunchKernelGGL((dev::qkrope_cam_kernel<kActBF16, 1>), grid, block, lds_bytes, st, a);
    else if (act == kActBF16 && cpl == 2)
        hipLaunchKernelGGL((dev::qkrope_cam_kernel<kActBF16, 2>), grid, block, lds_bytes, st, a);
    else if (act == kActF16 && cpl == 1)
        hipLaunchKernelGGL((dev::qkrope_cam_kernel<kActF16, 1>), grid, block, lds_bytes, st, a);
    else if (act == kActF16 && cpl == 2)
        hipLaunchKernelGGL((dev::qkrope_cam_kernel<kActF16, 2>), grid, block, lds_bytes, st, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace qkrope
