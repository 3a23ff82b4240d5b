// ssd_block_kernels.hpp -- the Mamba-2 block's prologue around the SSD for
// gfx950: causal depthwise conv1d + SiLU over the xBC channels, split into x, B
// and C.  ("SSM 家族全景图（下）：Mamba-2 与 Jamba", the block data flow of section
// five: the main path passes a one-dimensional causal convolution, then SiLU,
// before it is split into heads for the SSD.)  The gate epilogue, y * SiLU(z),
// is fused into chunk_scan (its GATE mode).
#pragma once

#include "ssd_kernels.hpp"

namespace ssd {

// A 16-byte vector of E as floats (8 for bf16, 4 for fp32), and back (bf16:
// round to nearest even).
__device__ __forceinline__ void unpack16_f32(uint4 r, float *v, const bf16 *)
{
    const floatx8 f = __builtin_convertvector(__builtin_bit_cast(bf16x8, r), floatx8);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = f[i];
}
__device__ __forceinline__ void unpack16_f32(uint4 r, float *v, const float *)
{
    v[0] = __uint_as_float(r.x); v[1] = __uint_as_float(r.y);
    v[2] = __uint_as_float(r.z); v[3] = __uint_as_float(r.w);
}
__device__ __forceinline__ uint4 pack16_f32(const float *v, const bf16 *)
{
    return uint4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
}
__device__ __forceinline__ uint4 pack16_f32(const float *v, const float *)
{
    return uint4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
}

// out[b,t,c] = SiLU(bias[c] + sum_{k<K} w[c][k] in[b, t-(K-1)+k, c]) with in = 0
// before the start of t's sequence (t' < 0, or with seq_idx a position of an
// earlier segment).  Channels c: [0, CX) -> x (row = H*P), [CX, CX+CG) -> B,
// [CX+CG, CX+2CG) -> C (rows = G*N).
//
// One thread per 16-byte channel vector (8 bf16 or 4 fp32 channels; CX and CG
// are multiples of 16, so a vector never straddles two outputs) and kConvTB
// tokens.  Consecutive threads take consecutive vectors of one token block, so
// every load and store of a wave is one contiguous run of 1 KiB.  All
// K-1+kConvTB input vectors of a thread are issued before any arithmetic (the
// token loop is unrolled at compile time); the K-1 rows before each block (the
// halo) are the only re-reads.
constexpr int kConvTB = 16;   // tokens per thread

template <typename E, int K, bool PACKED>
__global__ __launch_bounds__(kThreads) void k_conv1d_silu(
    const E *__restrict__ xbc, const float *__restrict__ w, const float *__restrict__ bias,
    const int32_t *__restrict__ seq_idx, E *__restrict__ xo, E *__restrict__ bo, E *__restrict__ co, int T, int CX,
    int CG, int64_t items)
{
    constexpr int V = 16 / (int)sizeof(E);   // channels per thread
    constexpr int R = K - 1 + kConvTB;      // input rows per thread
    // XCD-aware order: each XCD takes a contiguous range of workgroups, so the
    // halo rows of a token block were fetched into the same L2 by the workgroup
    // of the block before it
    const int64_t it = (int64_t)xcd_remap(blockIdx.x, gridDim.x) * kThreads + threadIdx.x;
    if (it >= items) return;
    const int CC = CX + 2 * CG, GV = CC / V;
    const int nb = (T + kConvTB - 1) / kConvTB;
    const int c = (int)(it % GV) * V;
    const int64_t r = it / GV;
    const int tb = (int)(r % nb), b = (int)(r / nb);
    const int t0 = tb * kConvTB;
    const E *src = xbc + (int64_t)b * T * CC + c;
    uint4 raw[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int tt = t0 - (K - 1) + i;
        raw[i] = tt >= 0 && tt < T ? *reinterpret_cast<const uint4 *>(src + (int64_t)tt * CC) : uint4{0, 0, 0, 0};
    }
    int sid[R];
    if constexpr (PACKED) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int tt = t0 - (K - 1) + i;
            sid[i] = tt >= 0 && tt < T ? seq_idx[tt] : -1;
        }
    }
    float wk[V][K], bv[V];
#pragma unroll
    for (int q = 0; q < V; ++q) {
        bv[q] = bias ? bias[c + q] : 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) wk[q][k] = w[(int64_t)(c + q) * K + k];
    }
    E *dst;
    int dc, ld;
    if (c < CX) { dst = xo; dc = c; ld = CX; }
    else if (c < CX + CG) { dst = bo; dc = c - CX; ld = CG; }
    else { dst = co; dc = c - CX - CG; ld = CG; }
    dst += ((int64_t)b * T + t0) * ld + dc;
#pragma unroll
    for (int j = 0; j < kConvTB; ++j) {
        float o[V];
#pragma unroll
        for (int q = 0; q < V; ++q) o[q] = bv[q];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int i = j + k;   // input row t-(K-1)+k of output row t = t0+j
            const bool in = !PACKED || sid[i] == sid[j + K - 1];
            float v[V];
            unpack16_f32(raw[i], v, (const E *)nullptr);
#pragma unroll
            for (int q = 0; q < V; ++q) o[q] += in ? wk[q][k] * v[q] : 0.f;
        }
#pragma unroll
        for (int q = 0; q < V; ++q) o[q] = silu(o[q]);
        if (t0 + j < T) *reinterpret_cast<uint4 *>(dst + (int64_t)j * ld) = pack16_f32(o, (const E *)nullptr);
    }
}

}  // namespace ssd
