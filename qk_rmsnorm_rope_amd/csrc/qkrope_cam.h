// qkrope_cam.h -- internal interface between qkrope_api_cam.cpp and the camera prologue kernel
// (qkrope_kernels_cam.hip). Not installed.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "qkrope_internal.h"

namespace qkrope {

// Camera prologue (UCPE cam_prep_func): per token of [B, N, H, D] Q/K/V, ReLU (Q, K), K scale,
// a per-token 4x4 projection on groups of four channels (proj_q for Q, proj_kv for K and V),
// interleaved RoPE from split [N, D/2] fp32 tables; outputs [B, H, D, N] and the key's
// squared-norm growth under the projection, [B, H, N] fp32. One workgroup per (batch, tile of
// kCamTile tokens, group of heads); see qkrope_kernels_cam.hip.
constexpr int kCamTile = 64;        // tokens per tile: 128-byte runs of each output row
constexpr int kCamMaxHeads = 2;     // heads per workgroup at one 16-byte chunk per lane
struct CamArgs {
    const uint16_t *in[3];          // q, k, v: token (b, n) row at in[r] + (b*N + n)*in_stride[r]
    int64_t in_stride[3];           // elements; multiple of 8, >= H*D, < 2^24
    const float *proj[2];           // proj_q, proj_kv: [B, N, 4, 4] row-major per token
    const float *cos_table;         // [N, D/2]
    const float *sin_table;
    uint16_t *out[3];               // [B, H, D, N]: row (b, h, d) at ((b*H + h)*D + d)*out_row_stride
    int64_t out_row_stride;         // elements, >= N
    float *inflation;               // [B, H, N], or null
    int64_t num_tokens;             // N
    int batch, heads, head_dim;
    int lanes_per_token;            // power of two >= head_dim / 8 / chunks-per-lane
    int heads_per_group, groups;    // head groups of <= kCamMaxHeads / chunks-per-lane heads
    int tiles;                      // token tiles per batch
    int tiles_padded;               // block-index stride of a (batch, group): tiles rounded up
    uint32_t xcd_group;             // as KernelArgs::xcd_group, over tile-fastest blocks
    FastDiv div_tiles, div_groups, div_xcd;   // n / tiles_padded, n / groups, n / xcd_group
    int row_chunks;                 // LDS tile row: 16-byte chunks, next power of two >= D/8
    int vec_store;                  // outputs take 16-byte stores (row stride % 8 == 0, aligned bases)
    int nt_store;                   // every output row starts on a 128-byte line: whole tiles store non-temporally
    float k_scale;
};
// cpl: 16-byte chunks per lane (1 for head_dim <= 64, else ceil(head_dim / 64), with 8 lanes per
// token); threads = 64 * lanes_per_token;
// lds_bytes = 2 * kCamTile * row_chunks * 16.
hipError_t launch_cam(const CamArgs &args, int act, int cpl, int64_t blocks, int lds_bytes,
                      hipStream_t stream);

}  // namespace qkrope
