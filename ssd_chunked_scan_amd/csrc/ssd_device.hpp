// ssd_device.hpp -- device-side building blocks shared by the SSD kernels (gfx950).
//
// Matrix-core convention used by every kernel.  One "fragment" is what a lane
// feeds one 16x16 output block per 32-wide K step:
//   lane l holds row (l % 16) of its operand and the 8 K-slots 8*(l/16) .. 8*(l/16)+7.
// For bf16 the fragment is 8 bf16 and one v_mfma_f32_16x16x32_bf16 consumes it.
// For fp32 it is 8 floats consumed by eight v_mfma_f32_16x16x4_f32, the j-th of
// which takes K-slot (l/16) <-> k = 8*(l/16) + j; A and B use the same map, so
// the sum over k is unchanged.  The 16x16 fp32 result sits in 4 registers per
// lane: acc[r] = D[row 4*(l/16) + r][col l % 16].
// Operands therefore need their K index contiguous per row; tiles whose K index
// is the slow axis in memory (time, for x and B in the state step) are
// transposed in registers on their way into LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef short shortx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;   // every kernel runs 4 waves of 64 lanes
constexpr int kMaxStateDim = 256;   // largest supported N (state size per head)
constexpr float kLog2e = 1.4426950408889634f;

// e^x through the hardware base-2 exponential (v_exp_f32).  Used only for
// arguments <= 0 (decays) where the result is in [0, 1].
__device__ __forceinline__ float exp_neg(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
// 2^x for arguments already scaled by log2(e) (v_exp_f32 alone).
__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }
// A float from another lane of the same 16-lane row (DPP move; every source
// lane is inside the row).  Controls: rotate the row by 8 (lane i <- i ^ 8),
// mirror each half row (i <- i ^ 7 within the half), and the quad permutes
// i <- i ^ 2 and i <- i ^ 1.
constexpr int kDppRowRor8 = 0x128, kDppRowHalfMirror = 0x141, kDppQuadXor2 = 0x4E, kDppQuadXor1 = 0xB1;
template <int CTRL> __device__ __forceinline__ float dpp_mov(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
// SiLU(v) = v / (1 + e^-v) with the hardware exponential and reciprocal
// (v_exp_f32, v_rcp_f32: about 1 ulp each) instead of a correctly rounded
// divide.  v -> -inf gives -0 (the reciprocal of inf is 0).
__device__ __forceinline__ float silu(float v) { return v * __builtin_amdgcn_rcpf(1.f + exp2_(-v * kLog2e)); }

template <typename E> struct Frag;
template <> struct Frag<bf16> { using type = bf16x8; };
template <> struct Frag<float> { using type = floatx8; };
template <typename E> using frag_t = typename Frag<E>::type;

// Elements per 16-byte vector.
template <typename E> constexpr int kVec16 = 16 / (int)sizeof(E);

__device__ __forceinline__ void mma(floatx4 &acc, const bf16x8 &a, const bf16x8 &b)
{
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ void mma(floatx4 &acc, const floatx8 &a, const floatx8 &b)
{
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], acc, 0, 0, 0);
}

// Fragment loads from a 16-byte aligned address (LDS or global).
__device__ __forceinline__ bf16x8 load_frag(const bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ floatx8 load_frag(const float *p)
{
    const floatx4 lo = *reinterpret_cast<const floatx4 *>(p);
    const floatx4 hi = *reinterpret_cast<const floatx4 *>(p + 4);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Fragment stores to a 16-byte aligned address.
__device__ __forceinline__ void store_frag(bf16 *p, const bf16x8 &v) { *reinterpret_cast<bf16x8 *>(p) = v; }
__device__ __forceinline__ void store_frag(float *p, const floatx8 &v)
{
    *reinterpret_cast<floatx4 *>(p) = __builtin_shufflevector(v, v, 0, 1, 2, 3);
    *reinterpret_cast<floatx4 *>(p + 4) = __builtin_shufflevector(v, v, 4, 5, 6, 7);
}

// A fragment with the K slots whose flag is off replaced by zero (a select, so
// a non-finite value in a dropped slot cannot reach the product).
__device__ __forceinline__ bf16x8 mask_frag(const bf16x8 &v, const bool (&keep)[8])
{
    const uint4 u = __builtin_bit_cast(uint4, v);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = w[i] & ((keep[2 * i] ? 0x0000ffffu : 0u) | (keep[2 * i + 1] ? 0xffff0000u : 0u));
    return __builtin_bit_cast(bf16x8, uint4{o[0], o[1], o[2], o[3]});
}
__device__ __forceinline__ floatx8 mask_frag(const floatx8 &v, const bool (&keep)[8])
{
    floatx8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = keep[e] ? v[e] : 0.f;
    return o;
}

__device__ __forceinline__ floatx8 to_f32(const bf16x8 &v) { return __builtin_convertvector(v, floatx8); }
__device__ __forceinline__ floatx8 to_f32(const floatx8 &v) { return v; }

template <typename F> __device__ __forceinline__ F from_f32(const floatx8 &v);
template <> __device__ __forceinline__ bf16x8 from_f32<bf16x8>(const floatx8 &v)
{
    return __builtin_convertvector(v, bf16x8);   // round to nearest even
}
template <> __device__ __forceinline__ floatx8 from_f32<floatx8>(const floatx8 &v) { return v; }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const bf16x2 v = __builtin_convertvector(floatx2{lo, hi}, bf16x2);   // round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float to_float(float v) { return v; }
__device__ __forceinline__ float to_float(bf16 v) { return (float)v; }
template <typename E> __device__ __forceinline__ E from_float(float v) { return (E)v; }

// Four floats to a 16-byte fp32 vector.
__device__ __forceinline__ void store16_f32(float *p, const float *in)
{
    *reinterpret_cast<floatx4 *>(p) = floatx4{in[0], in[1], in[2], in[3]};
}

// Four consecutive elements <-> floats (8-byte bf16 or 16-byte fp32 access).
__device__ __forceinline__ void load4_f32(const float *p, float *out)
{
    const floatx4 v = *reinterpret_cast<const floatx4 *>(p);
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
}
__device__ __forceinline__ void load4_f32(const bf16 *p, float *out)
{
    const floatx4 v = __builtin_convertvector(*reinterpret_cast<const bf16x4 *>(p), floatx4);
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
}
__device__ __forceinline__ void store4_f32(float *p, const float *in)
{
    *reinterpret_cast<floatx4 *>(p) = floatx4{in[0], in[1], in[2], in[3]};
}
__device__ __forceinline__ void store4_f32(bf16 *p, const float *in)
{
    *reinterpret_cast<bf16x4 *>(p) = __builtin_convertvector(floatx4{in[0], in[1], in[2], in[3]}, bf16x4);
}

// Raw buffer resource over [base, base + bytes) (base must be wave-uniform).
// A load whose offset falls outside the range returns zero, so masked or
// out-of-range lanes need no branch: they use kOffNone.
constexpr uint32_t kOffNone = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes)
{
    const int n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}
// The same with the range already clamped to [0, 2^31) by the caller (formed
// once outside a loop, so the loop only swaps the base address).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_n(const void *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ int rsrc_bytes(int64_t bytes)
{
    return bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : (int)bytes);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// A load of data read for the last time (the non-temporal cache policy), so it
// does not displace data that later loads will hit in L2 or the MALL.
constexpr int kCpolNonTemporal = 2;
__device__ __forceinline__ uint4 bload16_last(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolNonTemporal));
}
// 16-byte stores of results nothing in this pass reads again (non-temporal).
__device__ __forceinline__ void store16_stream(void *p, uint4 v)
{
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4 *>(p));
}
// The same with a wave-uniform extra offset in the scalar offset field (only for
// accesses known to be in range: the scalar part is not range-checked).
__device__ __forceinline__ uint4 bload16s(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
}
__device__ __forceinline__ uint2 bload8s(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff)
{
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0));
}
__device__ __forceinline__ void bstore8s(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff, uint2 v)
{
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((__vector_size__(8))) unsigned int, v),
                                          r, off, soff, 0);
}
__device__ __forceinline__ void bstore16s(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff, uint4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(
        __builtin_bit_cast(__attribute__((__vector_size__(16))) unsigned int, v), r, off, soff, 0);
}
// Fragment (16 or 32 bytes) from a buffer at a byte offset.
__device__ __forceinline__ void bload_frag(__amdgpu_buffer_rsrc_t r, uint32_t off, bf16x8 &f)
{
    f = __builtin_bit_cast(bf16x8, bload16(r, off));
}
__device__ __forceinline__ void bload_frag(__amdgpu_buffer_rsrc_t r, uint32_t off, floatx8 &f)
{
    const floatx4 lo = __builtin_bit_cast(floatx4, bload16(r, off));
    const floatx4 hi = __builtin_bit_cast(floatx4, bload16(r, off == kOffNone ? kOffNone : off + 16));
    f = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Workgroups are dispatched round-robin over the 8 XCDs (XCD = id % 8), each with
// its own L2.  Map the hardware id to a logical id so that every XCD works on one
// contiguous range of logical ids: neighbouring tiles (same chunk, same B/C
// group) then share an L2.
// floor(n / d) for wave-uniform 0 <= n < 2^23 and d >= 1, from the hardware
// reciprocal (1 ulp): n is exact in fp32, the reciprocal and the product add a
// relative error of at most 1.5 * 2^-23, so for d >= 3 (quotient below 2^23 / 3)
// the float quotient is within 0.5 of n / d, its truncation within one of the
// true quotient, and one integer step corrects it; for d = 1 or 2 the
// reciprocal and the product are exact.  A scalar 32-bit integer division costs
// about twenty scalar instructions per wave, and the scalar unit is shared by
// all the waves of a SIMD; this is a handful of vector ones.
__device__ __forceinline__ int udiv23(int n, int d)
{
    int q = (int)((float)n * __builtin_amdgcn_rcpf((float)d));
    const int r = n - q * d;
    q += (r >= d ? 1 : 0) - (r < 0 ? 1 : 0);
    return __builtin_amdgcn_readfirstlane(q);
}

// q = n / d and r = n % d for wave-uniform n >= 0 and d >= 1; `small` (uniform)
// promises n < 2^23 and takes the reciprocal division.
__device__ __forceinline__ void udivmod(int n, int d, bool small, int &q, int &r)
{
    if (small) q = udiv23(n, d);
    else q = n / d;
    r = n - q * d;
}

// The coordinates of workgroup unit u of a per-(chunk or segment, head, 64-p
// tile) grid: u = (k * H + h) * ntp + tp, and the group g = floor(h G / H) of
// head h.  Wave-uniform; the reciprocal division when every numerator stays
// below 2^23 (units = K H ntp and H G), else the integer one.
__device__ __forceinline__ void unit_coords(int u, int units, int ntp, int H, int G, int &tp, int &h, int &k, int &g)
{
    if (units < (1 << 23) && (int64_t)H * G < (1 << 23)) {
        const int q = udiv23(u, ntp);
        tp = u - q * ntp;
        k = udiv23(q, H);
        h = q - k * H;
        g = udiv23(h * G, H);
    } else {
        tp = u % ntp;
        const int q = u / ntp;
        h = q % H;
        k = q / H;
        g = h / (H / G);
    }
}

__device__ __forceinline__ int xcd_remap(int bid, int nblocks)
{
    const int x = bid & 7, k = bid >> 3;
    const int q = nblocks >> 3, r = nblocks & 7;
    return x * q + (x < r ? x : r) + k;
}

}  // namespace ssd
