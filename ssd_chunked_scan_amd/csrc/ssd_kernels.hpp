// ssd_kernels.hpp -- HIP kernels of the chunked SSD forward pass for gfx950.
//
// The pass follows the four-step block decomposition described in section 3.4 of
// "SSM 家族全景图（下）：Mamba-2 与 Jamba" (scwacadex) and section 4.1 of the
// "Mamba 2 -- Transformers are SSMs" paper story (ai.tomabc.com):
//   chunk_cumsum   Delta = softplus(dt) and the within-chunk log-decay prefix cs
//   chunk_cb       C B^T per chunk and B/C group (shared by the group's heads)
//   chunk_state    each chunk's end state from its own inputs (step 2)
//   state_passing  the short scan over chunk states (step 3)
//   chunk_scan     intra-chunk quadratic form (step 1) plus the decayed entering
//                  state (step 4) plus the D skip term
//   seq_final      per-sequence final states of a packed stream
//
// Layouts (row-major): x, y [b,T,H,P]; dt [b,T,H]; B, C [b,T,G,N];
// delta, cs [b,H,nc,Q] fp32; cb [b,nc,G,Q,Q]; states [b,nc,H,P,N].
#pragma once

#include <type_traits>

#include "ssd_device.hpp"

namespace ssd {

// The tokens of chunk c: t0 = its first one, len = how many.  Without a chunk
// map the chunks tile the sequence (t0 = c Q, the last one ragged).  With one
// (the packed backward's layout, in which every segment starts a chunk)
// cmap[c] = (first token, count) in the caller's own stream, count 0 for a
// chunk of padding only; the positions of a chunk past its count read as zero,
// which is what padding tokens are, so the padded stream is never copied.
__device__ __forceinline__ void chunk_rows(int c, int Q, int T, const int2 *cmap, int &t0, int &len)
{
    if (cmap) {
        const int2 m = cmap[c];
        t0 = m.x;
        len = m.y;
    } else {
        t0 = c * Q;
        len = min(Q, T - t0);
    }
}

// ---------------------------------------------------------------------------
// chunk_cumsum
// ---------------------------------------------------------------------------
constexpr int kCumsumHeads = 4;   // one wave per head

// softplus(z) = log(1 + e^z) = max(z, 0) + log1p(u) with u = e^-|z| in (0, 1],
// from the hardware base-2 exponential and logarithm.  log1p(u) is taken as
// log(w) u / (w - 1) with w = fl(1 + u): w - 1 is exact, and the quotient
// cancels the rounding of 1 + u, so the result keeps a few-ulp relative error
// however small u is (w == 1 means u is below half an ulp of 1: log1p(u) = u).
__device__ __forceinline__ float softplus_f(float z)
{
    const float u = __builtin_amdgcn_exp2f(-fabsf(z) * kLog2e);
    const float w = 1.f + u;
    const float l1p = w == 1.f ? u : __builtin_amdgcn_logf(w) * 0.6931471805599453f * (u / (w - 1.f));
    return fmaxf(z, 0.f) + l1p;
}

// Inclusive segmented scan over the 64 lanes of a wave: lane i ends with the
// sum of v over lanes j <= i back to (and including) the nearest lane whose
// flag is set, and f = whether any lane in 0..i has it.  Hillis-Steele steps
// with DPP moves: shifts by 1, 2, 4, 8 inside each 16-lane row (a lane with no
// source reads the identity (0, 0)), then row 15's last lane into row 1 and 3,
// and lane 31 into rows 2 and 3.  A double moves as two 32-bit halves.
template <int CTRL, int ROWS>
__device__ __forceinline__ void dpp_seg_step(double &v, int &f)
{
    const int64_t bits = __builtin_bit_cast(int64_t, v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)bits, CTRL, ROWS, 0xf, true);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(bits >> 32), CTRL, ROWS, 0xf, true);
    const int fo = __builtin_amdgcn_update_dpp(0, f, CTRL, ROWS, 0xf, true);
    const double vo = __builtin_bit_cast(double, ((int64_t)hi << 32) | (uint32_t)lo);
    v = f ? v : v + vo;
    f |= fo;
}
__device__ __forceinline__ void wave_segmented_scan(double &v, int &f)
{
    dpp_seg_step<0x111, 0xf>(v, f);   // row_shr:1
    dpp_seg_step<0x112, 0xf>(v, f);   // row_shr:2
    dpp_seg_step<0x114, 0xf>(v, f);   // row_shr:4
    dpp_seg_step<0x118, 0xf>(v, f);   // row_shr:8
    dpp_seg_step<0x142, 0xa>(v, f);   // row_bcast:15 into rows 1 and 3
    dpp_seg_step<0x143, 0xc>(v, f);   // row_bcast:31 into rows 2 and 3
}

// The loads of chunk_cumsum_wave (issued early by callers that have other
// loads to overlap): raw dt (softplus not yet applied) and sequence ids of the
// chunk's len tokens from t0 (T is the stream length, for addressing).
template <typename E>
__device__ __forceinline__ void chunk_cumsum_load(const E *__restrict__ dt, const int32_t *__restrict__ seq_idx,
                                                  int b, int t0, int len, int h, int T, int H, int Q,
                                                  float (&zv)[4], int (&sv)[4])
{
    const int lane = threadIdx.x & 63;
    const int per = Q >> 6;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        zv[j] = 0.f;
        sv[j] = 0;
        const int i = lane * per + j, t = t0 + i;
        if (j < per && i < len) {
            zv[j] = to_float(dt[((int64_t)b * T + t) * H + h]);
            if (seq_idx) sv[j] = seq_idx[t];
        }
    }
}

// The arithmetic of chunk_cumsum_wave on loaded values (the chunk's len
// tokens); zv becomes Delta.
__device__ __forceinline__ void chunk_cumsum_compute(const float *__restrict__ A, bool packed, int len, int h,
                                                     int Q, int softplus, float (&zv)[4], float (&cv)[4],
                                                     const int (&sv)[4])
{
    const int lane = threadIdx.x & 63;
    const int per = Q >> 6;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (j < per && lane * per + j < len && softplus) zv[j] = softplus_f(zv[j]);
    const int last_sv = per == 4 ? sv[3] : (per == 2 ? sv[1] : sv[0]);
    const int before = __shfl_up(last_sv, 1);   // id of the token just before this lane's first
    const double a = (double)A[h];
    double loc[4];
    int flg[4];
    double run = 0.0;
    int restarted = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        loc[j] = 0.0;
        flg[j] = 0;
        if (j < per) {
            const int i = lane * per + j;
            const int prev = j == 0 ? before : sv[j - 1];
            if (packed && i > 0 && i < len && sv[j] != prev) {
                run = 0.0;
                restarted = 1;
            }
            run += (double)zv[j] * a;
            loc[j] = run;
            flg[j] = restarted;
        }
    }
    // segmented inclusive scan of (restarted, run) over the 64 lanes
    double v = run;
    int f = restarted;
    wave_segmented_scan(v, f);
    double carry = __shfl_up(v, 1);
    if (lane == 0) carry = 0.0;
#pragma unroll
    for (int j = 0; j < 4; ++j) cv[j] = (float)(flg[j] ? loc[j] : carry + loc[j]);
}

// One wave computes Delta and cs of one (b, chunk, head): every lane owns Q/64
// consecutive tokens (per = 1, 2 or 4), sums them sequentially, and a segmented
// wave scan (a segment restarts at a packed-sequence boundary) combines the
// lanes.  Sums run in fp64 and are rounded once, so a stored cs carries a single
// rounding.  On return lane l holds, for token l*per + j (j < per), dv[j] = Delta
// (0 past the sequence end), cv[j] = cs and sv[j] = its sequence id (0 without
// seq_idx).  Used by the cumsum kernel and by chunk_state, which must agree bit
// for bit.
template <typename E>
__device__ __forceinline__ void chunk_cumsum_wave(const E *__restrict__ dt, const float *__restrict__ A,
                                                  const int32_t *__restrict__ seq_idx, int b, int c, int h,
                                                  int T, int H, int Q, int softplus, float (&dv)[4],
                                                  float (&cv)[4], int (&sv)[4])
{
    const int t0 = c * Q, len = min(Q, T - t0);
    chunk_cumsum_load<E>(dt, seq_idx, b, t0, len, h, T, H, Q, dv, sv);
    chunk_cumsum_compute(A, seq_idx != nullptr, len, h, Q, softplus, dv, cv, sv);
}

// Delta and cs rows of one (b, chunk, head) as left by chunk_cumsum_wave.
__device__ __forceinline__ void store_cumsum_wave(float *__restrict__ delta, float *__restrict__ cs, int64_t row,
                                                  int Q, const float (&dv)[4], const float (&cv)[4])
{
    const int per = Q >> 6;
    const int64_t o = row * Q + (threadIdx.x & 63) * per;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (j < per) {
            delta[o + j] = dv[j];
            cs[o + j] = cv[j];
        }
    }
}

// Grid (nc, ceil(H/4), b): one wave per (chunk, head).
template <typename E>
__global__ __launch_bounds__(kThreads) void k_chunk_cumsum(
    const E *__restrict__ dt, const float *__restrict__ A, const int32_t *__restrict__ seq_idx,
    float *__restrict__ delta, float *__restrict__ cs, int T, int H, int Q, int nc, int softplus)
{
    const int c = blockIdx.x, b = blockIdx.z;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = blockIdx.y * kCumsumHeads + wave;
    if (h >= H) return;   // whole wave; no barriers below
    float dv[4], cv[4];
    int sv[4];
    chunk_cumsum_wave<E>(dt, A, seq_idx, b, c, h, T, H, Q, softplus, dv, cv, sv);
    store_cumsum_wave(delta, cs, ((int64_t)b * H + h) * nc + c, Q, dv, cv);
}


// ---------------------------------------------------------------------------
// chunk_cb: C B^T and a copy of C per (b, c, g), in fragment-major order
// ---------------------------------------------------------------------------
// Fragment-major order stores a row-major matrix as 16-row x 32-column blocks
// (one MFMA K step), block (rb, kb) at (rb * NCOL/32 + kb) * 512 elements, each
// block as the 64 lanes' fragments: lane l = r % 16 + 16 ((col % 32) / 8) holds
// the 8 consecutive columns 8 ((col % 32) / 8) .. +7 of row r.  chunk_scan then
// fetches a fragment as one contiguous 1 KB (bf16) per wave instead of 16 rows x
// 64 bytes.  Per (b, c, g) the chunk_cb buffer holds the Q x Q matrix CB[t][s] =
// sum_n C[t][n] B[s][n] (only the 64 x 64 tiles with s-tile <= t-tile are
// written), then the chunk's C rows as a Q x NT matrix, then B^T as an NT x Q
// matrix (rows n, columns s) for chunk_state; rows past the sequence end and
// columns past N are zero.
template <int Q, int NT> constexpr int64_t cb_group_elems() { return (int64_t)Q * Q + 2 * (int64_t)Q * NT; }

// One workgroup per 64x64 (t, s) tile with s-tile <= t-tile.  The B rows of the
// s-tile and the C rows of the t-tile are loaded with row-contiguous 16-byte
// loads into LDS (row pitch 32 bytes past a multiple of 256, which keeps the
// 16-byte fragment reads conflict-free); each wave computes 32x32 as D[s][t]
// (A = B rows, B = C rows, K = n).  The result goes through LDS to leave in
// fragment-major order; the tiles of the first s-tile also copy their C rows,
// and the diagonal tiles write B^T of their s rows.
// REV reads every chunk's rows in reversed order (row i of a chunk of len rows
// is source row len - 1 - i), which is the backward pass's time-reversed
// problem, without a reversed copy of B and C.
template <typename E, int Q, int NT, bool REV = false>
__global__ __launch_bounds__(kThreads) void k_chunk_cb(const E *__restrict__ Bm, const E *__restrict__ Cm,
                                                       E *__restrict__ cbuf, int T, int G, int N, int nc,
                                                       const int32_t *__restrict__ cseg = nullptr,
                                                       const int2 *__restrict__ cmap = nullptr)
{
    using F = frag_t<E>;
    constexpr int V = kVec16<E>, ES = (int)sizeof(E);
    constexpr int QT = Q / 64, NTRI = QT * (QT + 1) / 2;
    constexpr int PITCH = NT + 2 * V;
    constexpr int NKS = NT / 32;
    __shared__ __align__(16) E bs[64 * PITCH];
    __shared__ __align__(16) E csm[64 * PITCH];
    const int units = NTRI * nc * G;
    const int u = xcd_remap(blockIdx.x, units);
    const int b = blockIdx.y;
    int tile = u % NTRI;
    int c, g;
    udivmod(u / NTRI, G, units < (1 << 23), c, g);
    if (cseg && cseg[c] < 0) return;   // a chunk of padding only (cseg: see k_state_passing)
    int ti = 0;
    while (tile > ti) {
        tile -= ti + 1;
        ++ti;
    }
    const int si = tile;
    int t0, len;
    chunk_rows(c, Q, T, cmap, t0, len);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;

    // ---- B rows si*64.. and C rows ti*64.. into LDS (zero past len and past N) ----
    constexpr int VL = NT / V, RPP = kThreads / VL, NPASS = 64 / RPP, PG = NPASS < 8 ? NPASS : 8;
    const int hv = threadIdx.x % VL, hr = threadIdx.x / VL;
    const uint32_t voff = hv * V < N ? (uint32_t)(hr * G * N * ES + hv * 16) : kOffNone;
    auto rows_rsrc = [&](const E *m, int r0) {
        const int rows = min(64, len - r0);
        return make_rsrc(m + (((int64_t)b * T + t0 + r0) * G + g) * N,
                         rows > 0 ? ((int64_t)(rows - 1) * G * N + N) * ES : 0);
    };
    // REV: the whole chunk's rows, tile row i of tile r0 at source row len - 1 - (r0 + i)
    const auto chunk_rsrc = [&](const E *m) {
        return make_rsrc(m + (((int64_t)b * T + t0) * G + g) * N, ((int64_t)(len - 1) * G * N + N) * ES);
    };
    auto rev_off = [&](int r0, int i) {
        const int q = r0 + hr + i * RPP;
        return (voff == kOffNone || q >= len) ? kOffNone
                                              : (uint32_t)((int64_t)(len - 1 - q) * G * N * ES + hv * 16);
    };
    const auto brs = REV ? chunk_rsrc(Bm) : rows_rsrc(Bm, si * 64), crs = REV ? chunk_rsrc(Cm) : rows_rsrc(Cm, ti * 64);
#pragma unroll
    for (int i0 = 0; i0 < NPASS; i0 += PG) {
        uint4 rb[PG], rc[PG];
#pragma unroll
        for (int i = 0; i < PG; ++i) {
            if constexpr (REV) {
                rb[i] = bload16(brs, rev_off(si * 64, i0 + i));
                rc[i] = bload16(crs, rev_off(ti * 64, i0 + i));
            } else {
                const uint32_t o = voff == kOffNone ? kOffNone : voff + (uint32_t)((i0 + i) * RPP * G * N * ES);
                rb[i] = bload16(brs, o);
                rc[i] = bload16(crs, o);
            }
        }
#pragma unroll
        for (int i = 0; i < PG; ++i) {
            *reinterpret_cast<uint4 *>(bs + (hr + (i0 + i) * RPP) * PITCH + hv * V) = rb[i];
            *reinterpret_cast<uint4 *>(csm + (hr + (i0 + i) * RPP) * PITCH + hv * V) = rc[i];
        }
    }
    __syncthreads();

    E *group = cbuf + (((int64_t)b * nc + c) * G + g) * cb_group_elems<Q, NT>();
    if (si == 0) {
        // the C rows of this t-tile, fragment-major: 4 row blocks x NKS K steps
        E *cf = group + (int64_t)Q * Q;
#pragma unroll
        for (int blk = wave; blk < 4 * NKS; blk += 4) {
            const int rb = blk / NKS, kb = blk % NKS;
            const F v = load_frag(csm + (16 * rb + li) * PITCH + kb * 32 + 8 * lg);
            store_frag(cf + ((int64_t)((4 * ti + rb) * NKS + kb) * 64 + lane) * 8, v);
        }
    }
    if (si == ti) {
        // B^T of this s-tile, fragment-major: NT/16 row blocks (n) x 2 K steps (s);
        // lane (li, lg) needs column n = 16 nb + li over rows s = 32 kb + 8 lg ..
        // +7: in bf16 two transposing reads (rows +0..3, +4..7; lane j of each
        // 16-lane group points at row j/4, columns 4 (j%4) ..), in fp32 8 reads
        E *bt = group + (int64_t)Q * Q + (int64_t)Q * NT;
#pragma unroll
        for (int blk = wave; blk < (NT / 16) * 2; blk += 4) {
            const int nb = blk >> 1, kb = blk & 1;
            F v;
            if constexpr (sizeof(E) == 2) {
                typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
                E *q = bs + (32 * kb + 8 * lg + (li >> 2)) * PITCH + 16 * nb + 4 * (li & 3);
                const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)q);
                const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(q + 4 * PITCH));
                v = __builtin_bit_cast(F, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = bs[(32 * kb + 8 * lg + e) * PITCH + 16 * nb + li];
            }
            store_frag(bt + ((int64_t)(nb * (Q / 32) + 2 * si + kb) * 64 + lane) * 8, v);
        }
    }

    // ---- D[s][t] over K = n ----
    const int s_w = (wave & 1) * 32, t_w = (wave >> 1) * 32;
    floatx4 acc[2][2] = {};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        F fa[2], fb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            fa[i] = load_frag(bs + (s_w + 16 * i + li) * PITCH + ks * 32 + 8 * lg);
            fb[i] = load_frag(csm + (t_w + 16 * i + li) * PITCH + ks * 32 + 8 * lg);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) mma(acc[i][j], fa[i], fb[j]);
    }

    // ---- through LDS (bs reused as st[t][s]) to fragment-major CB ----
    constexpr int SP = 64 + 2 * V;
    __syncthreads();   // every wave is done reading bs
    E *st = bs;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float o[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
            store4_f32(st + (t_w + 16 * j + li) * SP + s_w + 16 * i + 4 * lg, o);
        }
    __syncthreads();
#pragma unroll
    for (int blk = wave; blk < 8; blk += 4) {
        const int rb = blk >> 1, kb = blk & 1;
        const F v = load_frag(st + (16 * rb + li) * SP + 32 * kb + 8 * lg);
        store_frag(group + ((int64_t)((4 * ti + rb) * (Q / 32) + 2 * si + kb) * 64 + lane) * 8, v);
    }
}


// ---------------------------------------------------------------------------
// K tiles: LDS tiles whose MFMA K index (time) is the slow axis in memory
// ---------------------------------------------------------------------------
// KTile<E, KR, COLS> holds rows 0..KR-1 (time) and columns 0..COLS-1 of a
// row-major global array.  init() fixes each thread's byte offsets (row r,
// 16-byte column vector c) once; load(rsrc) issues the buffer loads into
// registers, where rsrc (see rsrc()) starts at the tile's first element and ends
// after its last valid row, so rows past it read as zero with no per-load
// arithmetic; columns >= ncols are masked in init().  store() writes LDS
// (optionally scaling row r by w[r], and with SEL zeroing rows whose m[r] == 0
// by a select, so a masked non-finite input cannot leak), and
// frag(tile, k0, col0) returns the MFMA fragment for K rows k0..k0+31 and
// columns col0..col0+15.
//
// bf16: the tile stays row-major in LDS (plain 16-byte copies) and fragments are
// read with ds_read_b64_tr_b16.  Within each 16-lane group, lane j points at
// row k0 + 8*(lane/16) + j/4, column col0 + 4*(j%4); the instruction hands lane
// j column col0 + j of those four rows, i.e. four consecutive K values of one
// column.  Two reads (rows +0..3 and +4..7) make the 8-wide fragment.  To keep
// both these reads (32 lanes x 8 bytes per LDS cycle) and the 16-byte row writes
// free of bank conflicts on 64 banks, the 8-byte column chunks of row r are
// stored XOR-swizzled by swz(r) (an even value, so a 16-byte vector stays
// contiguous): for 64-column tiles swz = 6*((r>>1)&7) mod 16 with no row padding,
// for wider tiles rows are padded by 32 bytes and swz = 16*((r>>3)&1).
// fp32: there is no 32-bit transpose read, so the tile is transposed in registers
// on its way into LDS ([col][row], rows padded by 16 bytes) and fragments are
// plain 32-byte reads.
template <typename E, int KR, int COLS, int TH = kThreads> struct KTile;

// The range ends with the last row's last valid column: the tile's own columns
// never exceed the row pitch, and with a pitch below COLS a longer range would
// let the rows past `rows` (which must read as zero) start inside it.
template <typename E, int COLS>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ktile_rsrc(const E *src, int64_t ld, int rows)
{
    return make_rsrc(src, rows > 0 ? ((int64_t)(rows - 1) * ld + (ld < COLS ? ld : COLS)) * (int64_t)sizeof(E) : 0);
}

template <int KR, int COLS, int TH>
struct KTile<bf16, KR, COLS, TH> {
    static constexpr int PITCH = COLS == 64 ? 64 : COLS + 16;
    static __device__ __forceinline__ int swz(int r)
    {
        return COLS == 64 ? ((6 * ((r >> 1) & 7)) & 14) : (((r >> 3) & 1) << 4);
    }
    static constexpr int SIZE = KR * PITCH;
    static constexpr int VPR = COLS / 8;   // 16-byte vectors per row
    static constexpr int NV = KR * VPR;
    static constexpr int PER = (NV + TH - 1) / TH;
    uint4 raw[PER];
    uint32_t voff[PER];

    static __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const bf16 *src, int64_t ld, int rows)
    {
        return ktile_rsrc<bf16, COLS>(src, ld, rows);
    }

    __device__ __forceinline__ void init(int64_t ld, int ncols)
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int v = threadIdx.x + i * TH;
            const int r = v / VPR, c = v % VPR;
            voff[i] = (v < NV && c * 8 < ncols) ? (uint32_t)(r * ld * 2 + c * 16) : kOffNone;
        }
    }
    // The first `len` rows in reversed order (tile row r = source row len - 1 - r),
    // rows from len on zero.
    __device__ __forceinline__ void init_rev(int64_t ld, int ncols, int len)
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int v = threadIdx.x + i * TH;
            const int r = v / VPR, c = v % VPR;
            voff[i] = (v < NV && c * 8 < ncols && r < len) ? (uint32_t)((len - 1 - r) * ld * 2 + c * 16) : kOffNone;
        }
    }

    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs)
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) raw[i] = bload16(rs, voff[i]);
    }

    template <bool SCALE, bool SEL>
    __device__ __forceinline__ void store(bf16 *dst, const float *w, const int *m) const
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int v = threadIdx.x + i * TH;
            if (NV % TH != 0 && v >= NV) continue;
            const int r = v / VPR, c = v % VPR;
            uint4 o = raw[i];
            if constexpr (SCALE) {
                const float ws = w[r];
                const bool keep = !SEL || m[r] != 0;
                uint32_t q[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lo = __uint_as_float(q[e] << 16) * ws;
                    const float hi = __uint_as_float(q[e] & 0xffff0000u) * ws;
                    q[e] = keep ? pack_bf16x2(lo, hi) : 0u;
                }
                o = uint4{q[0], q[1], q[2], q[3]};
            } else if constexpr (SEL) {
                if (m[r] == 0) o = uint4{0u, 0u, 0u, 0u};
            }
            *reinterpret_cast<uint4 *>(dst + r * PITCH + 4 * ((2 * c) ^ swz(r))) = o;
        }
    }

    // Per-lane element offsets of the fragment for columns col0..col0+15 at K row 0.
    // The swizzle has a period of 16 rows, so the fragment at K row k0 (a multiple
    // of 32) is at the same offsets plus k0 * PITCH: hoisting these out of the K
    // loops leaves one LDS immediate offset per read.
    struct Off {
        int lo, hi;
    };
    __device__ __forceinline__ static Off frag_off(int col0)
    {
        const int lane = threadIdx.x & 63, j = lane & 15, g = lane >> 4;
        const int r0 = 8 * g + (j >> 2), r1 = r0 + 4, c8 = (col0 >> 2) + (j & 3);
        return Off{r0 * PITCH + 4 * (c8 ^ swz(r0)), r1 * PITCH + 4 * (c8 ^ swz(r1))};
    }
    __device__ __forceinline__ static bf16x8 frag_at(const bf16 *tile, Off o, int k0)
    {
        typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
        bf16 *t = const_cast<bf16 *>(tile) + k0 * PITCH;
        const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(t + o.lo));
        const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(t + o.hi));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    __device__ __forceinline__ static bf16x8 frag(const bf16 *tile, int k0, int col0)
    {
        return frag_at(tile, frag_off(col0), k0);
    }
};

template <int KR, int COLS, int TH>
struct KTile<float, KR, COLS, TH> {
    static constexpr int PITCH = KR + 4;
    static constexpr int SIZE = COLS * PITCH;
    static constexpr int CBK = COLS / 4;
    static constexpr int NB = (KR / 4) * CBK;   // 4x4 blocks
    static constexpr int PER = (NB + TH - 1) / TH;
    uint4 raw[PER][4];
    uint32_t voff[PER];   // offset of the block's first row

    static __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const float *src, int64_t ld, int rows)
    {
        return ktile_rsrc<float, COLS>(src, ld, rows);
    }

    int64_t ldb;
    bool rev;
    int rtop[PER];   // reversed tiles: the source row of each block's first tile row
    __device__ __forceinline__ void init(int64_t ld, int ncols)
    {
        ldb = ld * 4;
        rev = false;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int blk = threadIdx.x + i * TH;
            const int cbk = blk % CBK, sb = blk / CBK;
            voff[i] = (blk < NB && cbk * 4 < ncols) ? (uint32_t)(sb * 4 * ldb + cbk * 16) : kOffNone;
        }
    }
    // The first `len` rows in reversed order (tile row r = source row len - 1 - r),
    // rows from len on zero.
    __device__ __forceinline__ void init_rev(int64_t ld, int ncols, int len)
    {
        ldb = ld * 4;
        rev = true;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int blk = threadIdx.x + i * TH;
            const int cbk = blk % CBK, sb = blk / CBK;
            rtop[i] = len - 1 - sb * 4;
            voff[i] = (blk < NB && cbk * 4 < ncols) ? (uint32_t)(cbk * 16) : kOffNone;
        }
    }

    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs)
    {
#pragma unroll
        for (int i = 0; i < PER; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (rev) {
                    const int gr = rtop[i] - r;
                    raw[i][r] = bload16(rs, voff[i] == kOffNone || gr < 0 ? kOffNone : voff[i] + (uint32_t)(gr * ldb));
                } else {
                    raw[i][r] = bload16(rs, voff[i] == kOffNone ? kOffNone : voff[i] + (uint32_t)(r * ldb));
                }
            }
    }

    template <bool SCALE, bool SEL>
    __device__ __forceinline__ void store(float *dst, const float *w, const int *m) const
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int blk = threadIdx.x + i * TH;
            if (NB % TH != 0 && blk >= NB) continue;
            const int cbk = blk % CBK, sb = blk / CBK;
            float f[4][4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t q[4] = {raw[i][r].x, raw[i][r].y, raw[i][r].z, raw[i][r].w};
                float ws = 1.f;
                bool keep = true;
                if constexpr (SCALE) ws = w[sb * 4 + r];
                if constexpr (SEL) keep = m[sb * 4 + r] != 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v = __uint_as_float(q[e]);
                    f[r][e] = keep ? (SCALE ? v * ws : v) : 0.f;
                }
            }
#pragma unroll
            for (int cc = 0; cc < 4; ++cc)
                *reinterpret_cast<floatx4 *>(dst + (cbk * 4 + cc) * PITCH + sb * 4) =
                    floatx4{f[0][cc], f[1][cc], f[2][cc], f[3][cc]};
        }
    }

    struct Off {
        int lo, hi;
    };
    __device__ __forceinline__ static Off frag_off(int col0)
    {
        const int lane = threadIdx.x & 63;
        return Off{(col0 + (lane & 15)) * PITCH + 8 * (lane >> 4), 0};
    }
    __device__ __forceinline__ static floatx8 frag_at(const float *tile, Off o, int k0)
    {
        return load_frag(tile + o.lo + k0);
    }
    __device__ __forceinline__ static floatx8 frag(const float *tile, int k0, int col0)
    {
        return frag_at(tile, frag_off(col0), k0);
    }
};

// ---------------------------------------------------------------------------
// chunk_state / seq_final: the staged state product
// ---------------------------------------------------------------------------
// One workgroup covers 64 p x NT n (NT = N rounded up to 64, so all of N) of one
// (chunk, head), streamed over time in 64-step K chunks; the next chunk's global
// loads are issued before the current chunk's MFMAs.  The product is
// D[n][p] = sum_s B^T[n][s] (w_s x_s)[p]; wave w owns n rows w*NT/4 .. +NT/4:
//   acc[i][j][r]  <->  n = w*NT/4 + i*16 + 4*(lane/16) + r,  p = j*16 + lane%16.
// w and m (per-token weights and keep flags, length Q) must be in LDS and
// visible before the call.
template <typename E, int NT>
struct StateSmem {
    using XT = KTile<E, 64, 64>;
    using BT = KTile<E, 64, NT>;
    E x[XT::SIZE];
    E b[BT::SIZE];
};

// The caller has run xs.init/bs.init and issued the loads of the first K chunk.
template <typename E, int NT, bool SEL>
__device__ __forceinline__ void state_product(StateSmem<E, NT> &sm, const E *xsrc, int64_t ldx, const E *bsrc,
                                              int64_t ldb, int slen, const float *w, const int *m,
                                              typename StateSmem<E, NT>::XT &xs,
                                              typename StateSmem<E, NT>::BT &bs, floatx4 (&acc)[NT / 64][4])
{
    using XT = typename StateSmem<E, NT>::XT;
    using BT = typename StateSmem<E, NT>::BT;
    constexpr int NI = NT / 64;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    typename BT::Off aoff[NI];
    typename XT::Off xoff[4];
#pragma unroll
    for (int i = 0; i < NI; ++i) aoff[i] = BT::frag_off(wave * (NT / 4) + i * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) xoff[j] = XT::frag_off(j * 16);
    for (int kb = 0; kb < slen; kb += 64) {
        xs.template store<true, SEL>(sm.x, w + kb, m + kb);
        bs.template store<false, SEL>(sm.b, nullptr, m + kb);
        __syncthreads();
        if (kb + 64 < slen) {
            xs.load(XT::rsrc(xsrc + (int64_t)(kb + 64) * ldx, ldx, slen - kb - 64));
            bs.load(BT::rsrc(bsrc + (int64_t)(kb + 64) * ldb, ldb, slen - kb - 64));
        }
        const int kend = min(64, ((slen - kb) + 31) & ~31);
#pragma unroll
        for (int ks = 0; ks < 64; ks += 32) {
            if (ks >= kend) break;
            frag_t<E> a[NI], bb[4];
#pragma unroll
            for (int i = 0; i < NI; ++i) a[i] = BT::frag_at(sm.b, aoff[i], ks);
#pragma unroll
            for (int j = 0; j < 4; ++j) bb[j] = XT::frag_at(sm.x, xoff[j], ks);
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) mma(acc[i][j], a[i], bb[j]);
        }
        __syncthreads();
    }
}

// Writes the 64 x NT state tile held in MFMA layout (acc[i][j][r] <-> n = w*NT/4 +
// i*16 + 4*(lane/16) + r, p = j*16 + lane%16) to out[p][n] (row pitch N), rows
// p < prows and columns n < N only.  bf16 goes through LDS (`stage`, at least
// 64 * NT elements, free on entry; the caller's last barrier covers earlier
// readers) so that whole rows leave as 16-byte vectors: the 8-byte writes put
// 16-byte chunk c of row p at c ^ (p mod min(NT/8, 16)), which spreads 16 rows
// over all banks, and each read instruction covers 64 consecutive chunks in a
// lane order (bits 3 and 4 of the lane swapped) that gives every LDS pass 256
// contiguous bytes.  fp32 lanes already hold 16 bytes and store directly.
template <typename E, int NT>
__device__ __forceinline__ void store_state_tile(E *stage, const floatx4 (&acc)[NT / 64][4], E *out, int prows,
                                                 int N)
{
    constexpr int NI = NT / 64;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
    if constexpr (sizeof(E) == 2) {
        constexpr int CPR = NT / 8;                       // 16-byte chunks per row
        constexpr int GM = (CPR < 16 ? CPR : 16) - 1;     // chunk swizzle mask
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = wave * (NT / 4) + i * 16 + 4 * lg, p = j * 16 + li;
                const uint2 v{pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3])};
                *reinterpret_cast<uint2 *>(stage + p * NT + 8 * ((n >> 3) ^ (p & GM)) + (n & 7)) = v;
            }
        __syncthreads();
        const int f = (lane & 7) | ((lane & 16) >> 1) | ((lane & 8) << 1) | (lane & 32);
#pragma unroll
        for (int m = 0; m < NT / 32; ++m) {
            const int F = (wave + 4 * m) * 64 + f;
            const int p = F / CPR, ch = F % CPR;
            const uint4 v = *reinterpret_cast<const uint4 *>(stage + p * NT + 8 * (ch ^ (p & GM)));
            if (p < prows && 8 * ch < N) *reinterpret_cast<uint4 *>(out + (int64_t)p * N + 8 * ch) = v;
        }
    } else {
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = wave * (NT / 4) + i * 16 + 4 * lg, p = j * 16 + li;
                if (p < prows && n < N) {
                    float o[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
                    store4_f32(out + (int64_t)p * N + n, o);
                }
            }
    }
}

// seg_end[s] = the last position of segment id s, or -1 for an id that never
// occurs, from non-decreasing ids in [0, nseq): position t writes the entry of
// its id if the id changes after t, and -1 for the ids it skips (those between
// its id and the next position's, those below the first id at t = 0, those past
// the last id at t = T-1).  Every id is written exactly once, so no pass has to
// clear the array first.  Ids are clamped to [0, nseq), so no write leaves the
// array whatever the ids hold.
__device__ __forceinline__ void seg_end_mark(const int32_t *__restrict__ seq_idx, int32_t *__restrict__ seg_end,
                                             int t, int T, int nseq)
{
    const int sid = seq_idx[t];
    if (t == 0)
        for (int id = 0; id < min(sid, nseq); ++id) seg_end[id] = -1;
    const int nxt = t == T - 1 ? nseq : seq_idx[t + 1];
    if (nxt != sid) {
        if (sid >= 0 && sid < nseq) seg_end[sid] = t;
        for (int id = max(sid + 1, 0); id < min(nxt, nseq); ++id) seg_end[id] = -1;
    }
}

// chunk_state: states[b,c,h,p,n] = sum_s w_s x_s[p] B_s[n], w_s = exp(cs_last -
// cs_s) delta_s for s in the segment of the chunk's last token (0 elsewhere).
// One workgroup per (b, c, h, 64-p tile).  Wave 0 first runs the cumsum step
// for (b, c, h) (Delta, cs and the weights); with packed streams and seg_end
// given, wave 1 of the (c, h = 0, first p-tile) workgroup marks the segment ends
// of the chunk (seg_end_mark).  The weighted x tile of all Q tokens
// is staged in LDS once (its K index, time, read back transposed); the B^T
// fragments (rows n, K = s) are streamed fragment-major from the chunk_cb
// buffer, RING K steps ahead, one contiguous block per wave and step.  Wave w
// owns n rows w*NT/4 .. +NT/4 of D[n][p] (A = B^T, B = (w x)^T):
//   acc[i][j][r]  <->  n = w*NT/4 + i*16 + 4*(lane/16) + r,  p = j*16 + lane%16.
// GRAD = true is the same product for the backward pass's per-chunk gradient
// states U_c = sum_t exp(cs_t) dy_t C_t^T, run on the chunk's tokens in reversed
// order: x = dy is passed in its own order and its rows are read reversed here,
// B^T = C^T comes reversed from the caller; the weight of reversed position s
// is exp(cs[len-1-s]) from the given cs, no cumsum step runs, and delta and cs
// are only read.
template <typename E, int Q, int NT, bool PACKED, bool GRAD = false>
__global__ __launch_bounds__(kThreads, 4) void k_chunk_state(
    const E *__restrict__ x, const E *__restrict__ cbuf, const E *__restrict__ dt, const float *__restrict__ A,
    const int32_t *__restrict__ seq_idx, float *__restrict__ delta, float *__restrict__ cs,
    E *__restrict__ states, int32_t *__restrict__ seg_end, int nseq, int T, int H, int G, int P, int N, int nc,
    int ntp, int softplus, const int32_t *__restrict__ cseg = nullptr, const int2 *__restrict__ cmap = nullptr)
{
    using F = frag_t<E>;
    using XT = KTile<E, Q, 64>;
    constexpr int NI = NT / 64;
    constexpr int NKS = Q / 32;
    constexpr int RING = 2;   // deep enough with four waves per SIMD, small enough to allow them
    constexpr int ES = (int)sizeof(E);
    constexpr int XSZ = XT::SIZE > 64 * NT ? XT::SIZE : 64 * NT;   // the x tile, then the result
    __shared__ __align__(16) E xt[XSZ];
    __shared__ float w[Q];
    __shared__ int m[Q];
    const int units = nc * H * ntp;
    const int u = xcd_remap(blockIdx.x, units);
    const int b = blockIdx.y;
    int tp, h, c, g;
    unit_coords(u, units, ntp, H, G, tp, h, c, g);
    if (cseg && cseg[c] < 0) return;   // a chunk of padding only (cseg: see k_state_passing)
    int t0, len;
    chunk_rows(c, Q, T, cmap, t0, len);
    const int p0 = tp * 64;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;

    // wave 0's dt loads go first: vector loads complete in issue order, and the
    // cumsum step below must not wait for the tiles
    float dv[4], cv[4];
    int sv[4];
    if (!GRAD && wave == 0) chunk_cumsum_load<E>(dt, seq_idx, b, t0, len, h, T, H, Q, dv, sv);
    const int64_t ldx = (int64_t)H * P;
    XT xs;
    if constexpr (GRAD) xs.init_rev(ldx, P - p0, len);   // the chunk's tokens in reversed order
    else xs.init(ldx, P - p0);
    xs.load(XT::rsrc(x + (((int64_t)b * T + t0) * H + h) * P + p0, ldx, len));

    // B^T fragments of this chunk and group; K steps past the sequence end are skipped
    const E *group = cbuf + (((int64_t)b * nc + c) * G + g) * cb_group_elems<Q, NT>();
    const auto brs = make_rsrc(group + (int64_t)Q * Q + (int64_t)Q * NT, (int64_t)NT * Q * ES);
    constexpr uint32_t BLK = 512 * ES;   // bytes per fragment block
    const int kend = (len + 31) / 32;
    uint32_t bbase[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) bbase[i] = (uint32_t)((wave * NI + i) * NKS) * BLK + lane * 8 * ES;
    auto b_off = [&](int i, int ks) -> uint32_t { return ks < kend ? bbase[i] + (uint32_t)ks * BLK : kOffNone; };
    F ra[RING][NI];
#pragma unroll
    for (int r = 0; r < RING; ++r)
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            if (r < NKS) bload_frag(brs, b_off(i, r), ra[r][i]);
            else ra[r][i] = F{};
        }

    // Packed streams: wave 1 of one workgroup per chunk records the segment ends
    // among the chunk's positions (for the per-segment final states), while wave
    // 0 runs the cumsum step.
    if (!GRAD && PACKED && seg_end && h == 0 && tp == 0 && wave == 1)
        for (int t = t0 + lane; t < t0 + len; t += 64) seg_end_mark(seq_idx, seg_end, t, T, nseq);

    // Delta and cs of this chunk and head (the cumsum step, bit-identical to
    // k_chunk_cumsum) by wave 0 while the loads above fly; the first p-tile's
    // workgroup also stores them for state_passing and chunk_scan
    if (GRAD && wave == 0) {
        const int64_t row = (((int64_t)b * H + h) * nc + c) * Q;
        for (int s = lane; s < Q; s += 64) {
            const bool keep = s < len;
            m[s] = keep;
            w[s] = keep ? __builtin_amdgcn_exp2f(cs[row + (len - 1 - s)] * kLog2e) : 0.f;
        }
    } else if (wave == 0) {
        chunk_cumsum_compute(A, PACKED, len, h, Q, softplus, dv, cv, sv);
        if (tp == 0) store_cumsum_wave(delta, cs, ((int64_t)b * H + h) * nc + c, Q, dv, cv);
        constexpr int per = Q / 64;
        const int il = len - 1, ll = il / per, jl = il % per;   // lane and slot of the last token
        float cl = cv[0];
        int sl = sv[0];
#pragma unroll
        for (int j = 1; j < per; ++j) {
            cl = jl == j ? cv[j] : cl;
            sl = jl == j ? sv[j] : sl;
        }
        const float lam = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cl), ll));
        const int seq_last = __builtin_amdgcn_readlane(sl, ll);
#pragma unroll
        for (int j = 0; j < per; ++j) {
            const int s = lane * per + j;
            const bool keep = s < len && (!PACKED || sv[j] == seq_last);
            m[s] = keep;
            w[s] = keep ? exp_neg(lam - cv[j]) * dv[j] : 0.f;
        }
    }
    __syncthreads();
    xs.template store<true, PACKED>(xt, w, m);
    // A chunk that holds a segment boundary keeps only its tokens a .. len-1 (ids
    // never decrease, so the kept tokens are one run ending at the chunk's last
    // token): the x rows before a are already zero (a select); the K steps wholly
    // before a are skipped and the one that straddles a drops its B^T columns
    // before a by a select, so a non-finite B of another sequence cannot reach
    // this state.
    int first_kept = 0;
    if (PACKED && !GRAD) {
        for (int s = lane; s < Q; s += 64) {   // every wave finds it on its own
            const uint64_t kept = __ballot(m[s] != 0);
            if (kept) {
                first_kept = s - lane + __builtin_ctzll(kept);
                break;
            }
        }
        first_kept = __builtin_amdgcn_readfirstlane(first_kept);
    }
    __syncthreads();

    floatx4 acc[NI][4];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    typename XT::Off xoff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) xoff[j] = XT::frag_off(j * 16);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        if (ks < kend) {   // wave-uniform
            if (PACKED && ks * 32 < first_kept) {   // wave-uniform; only in a chunk with a boundary
                const int sb = ks * 32 + 8 * (lane >> 4);
                bool kp[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) kp[e] = sb + e >= first_kept;
#pragma unroll
                for (int i = 0; i < NI; ++i) ra[ks % RING][i] = mask_frag(ra[ks % RING][i], kp);
            }
            if (!PACKED || ks * 32 + 32 > first_kept) {
                F bx[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) bx[j] = XT::frag_at(xt, xoff[j], ks * 32);
#pragma unroll
                for (int i = 0; i < NI; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) mma(acc[i][j], ra[ks % RING][i], bx[j]);
            }
        }
        if (ks + RING < NKS) {
#pragma unroll
            for (int i = 0; i < NI; ++i) bload_frag(brs, b_off(i, ks + RING), ra[ks % RING][i]);
        }
    }

    __syncthreads();   // the x tile is no longer read: its memory stages the result
    E *out = states + (((int64_t)b * nc + c) * H + h) * (int64_t)P * N;
    store_state_tile<E, NT>(xt, acc, out + (int64_t)p0 * N, P - p0, N);
}

// ---------------------------------------------------------------------------
// state_passing: in place S_c -> h_{c-1}; h_c = exp(cs_last(c)) h_{c-1} + S_c
// ---------------------------------------------------------------------------
// Every (b, h, p, n) element is an independent length-nc scan.  Each thread owns
// VE = 4 consecutive elements (8 bytes of bf16, 16 of fp32) and walks the chunks
// with a ring of D loads in flight: the slot a chunk's state is read from is
// refilled with the state D chunks ahead before the arithmetic.  The carry is
// replaced by zero (a select) when the chunk holds a segment boundary.
// (Four bf16 per thread measured best: eight leave the latency-bound small
// shapes with too few waves, two waste bandwidth on 4-byte accesses.)  D is
// kPrefetch, or kPrefetchLong for chains longer than kPrefetch chunks: such
// shapes have few threads per chunk (batch 1 at 16K tokens: two waves per
// SIMD), and twice the loads in flight took state_passing from 27.2 to 25.2 us
// at 16384 tokens, 32 heads, N = 256, and from 73.0 to 66.6 us at 15872 tokens,
// 64 heads, N = 128; on the 16-chunk chains of 8 x 2048 tokens, 80 heads, the
// larger ring's registers cost occupancy (62.0 -> 65.9 us), so it is not used
// there.
constexpr int kPrefetch = 32;
constexpr int kPrefetchLong = 64;

template <typename E, int VE> struct RawVec;
template <> struct RawVec<bf16, 4> { using type = uint2; };
template <> struct RawVec<float, 4> { using type = uint4; };

__device__ __forceinline__ void unpack_raw(const uint2 &v, float *o)
{
    o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
}
__device__ __forceinline__ void unpack_raw(const uint4 &v, float *o)
{
    o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
}
template <typename E, int VE> __device__ __forceinline__ void unpack_vec(const typename RawVec<E, VE>::type &v, float *o)
{
    unpack_raw(v, o);
}
template <int VE> __device__ __forceinline__ void store_vec(float *p, const float *v) { store16_f32(p, v); }
template <int VE> __device__ __forceinline__ void store_vec(bf16 *p, const float *v) { store4_f32(p, v); }
template <int VE> __device__ __forceinline__ void load_init(const float *p, float *v)
{
#pragma unroll
    for (int i = 0; i < VE; i += 4) load4_f32(p + i, v + i);
}
template <int VE> __device__ __forceinline__ void store_final(float *p, const float *v)
{
#pragma unroll
    for (int i = 0; i < VE; i += 4) store4_f32(p + i, v + i);
}

// REV = true runs the same scan over the chunks in reverse order, which is the
// backward pass's gradient-state scan: with U_c in `states` and dL/d(final
// state) in `init`, slot c receives G_c = dL/d(state after chunk c) and
// `final_states` receives dL/d(initial state); G_{c-1} = exp(cs_last(c)) G_c +
// U_c has the same form as the forward step.  (REV takes no seq_idx.)  With
// `hin` (the states entering each chunk, laid out like `states`) it also forms
// the boundary term exp(cs_last(c)) <G_c, Hin_c> of the log-decay gradient:
// each wave's share of the dot product goes to bnd_part[(b, h, c), wave of the
// (b, h)], PN / (64 VE) partials per (b, h, c), in a fixed order.
//
// cseg (instead of seq_idx; batch 1): the segment id of every chunk, for a
// stream laid out so that every segment starts at a chunk start (-1 for chunks
// past the last segment).  Forward: the carry is cut where the id changes, and
// the state stored as entering such a chunk is zero.  REV: where the id changes
// between chunk c-1 and c, G_{c-1} restarts from slot c alone, where the caller
// has put segment cseg[c-1]'s own final-state gradient in place of U_c (which
// nothing reads there; k_bwd_inject_dfinal); the scan starts from segment
// cseg[nc-1]'s, `init` + cseg[nc-1] * H * PN (init is then [nseq, H, PN], and an
// id of -1 or a NULL init means zero).  The cut is a select on the same update
// as the forward's, so the loop holds no extra loads.
template <typename E, int VE, bool REV = false, int D = kPrefetch>
__global__ __launch_bounds__(kThreads) void k_state_passing(
    E *__restrict__ states, const float *__restrict__ cs, const float *__restrict__ init,
    float *__restrict__ final_states, const int32_t *__restrict__ seq_idx,
    int T, int H, int64_t PN, int nc, int Q, int64_t total_vecs,
    const E *__restrict__ hin = nullptr, float *__restrict__ bnd_part = nullptr,
    const int32_t *__restrict__ cseg = nullptr)
{
    using R = typename RawVec<E, VE>::type;
    static_assert(64 % D == 0, "the ring depth divides 64");
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (gid >= total_vecs) return;
    const int lane = threadIdx.x & 63;
    const int64_t vph = PN / VE;   // a multiple of 64: every wave lies inside one (b, h)
    // the wave's (b, h): waves are numbered across the grid, vph / 64 of them per (b, h)
    const int wgid = blockIdx.x * (kThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool small = gridDim.x * (kThreads / 64) < (1u << 23);
    int bh, wr, b, h;
    udivmod(wgid, (int)(vph / 64), small, bh, wr);
    udivmod(bh, H, small, b, h);
    const int64_t e0 = (gid - (int64_t)bh * vph) * VE;
    auto chunk = [&](int k) { return REV ? nc - 1 - k : k; };   // the k-th chunk visited
    float hs[VE];
#pragma unroll
    for (int v = 0; v < VE; ++v) hs[v] = 0.f;
    // the gradient of segment sg (REV with cseg), or zero
    auto seg_init = [&](int sg) {
#pragma unroll
        for (int v = 0; v < VE; ++v) hs[v] = 0.f;
        if (init && sg >= 0) load_init<VE>(init + ((int64_t)sg * H + h) * PN + e0, hs);
    };
    if (REV && cseg) seg_init(cseg[nc - 1]);
    else if (init) load_init<VE>(init + (int64_t)bh * PN + e0, hs);
    const float *lamp = cs + (int64_t)bh * nc * Q + (Q - 1);   // cs at each chunk's last position
    const int64_t cstride = (int64_t)H * PN;
    E *lane_base = states + ((int64_t)b * nc * H + h) * PN + e0;
    R buf[D];
#pragma unroll
    for (int k = 0; k < D; ++k)
        if (k < nc) buf[k] = *reinterpret_cast<const R *>(lane_base + (int64_t)chunk(k) * cstride);
    // the boundary term (REV with hin): Hin of the visited chunks, in a ring of
    // DH loads in flight (shallower than the states' ring, to keep registers)
    constexpr bool BND = REV;
    constexpr int DH = BND ? (sizeof(E) == 2 ? D / 2 : D / 4) : 1;   // divides D
    const bool bnd_on = BND && hin != nullptr;   // uniform
    const E *hin_base = BND && hin ? hin + ((int64_t)b * nc * H + h) * PN + e0 : nullptr;
    const int64_t nwv = PN / (64 * VE), wv = e0 / (64 * VE);
    R hbuf[DH];
    if constexpr (BND) {
        if (bnd_on) {
#pragma unroll
            for (int k = 0; k < DH; ++k)
                if (k < nc) hbuf[k] = *reinterpret_cast<const R *>(hin_base + (int64_t)chunk(k) * cstride);
        }
    }
    int sprev = seq_idx ? seq_idx[0] : 0;
    for (int cb = 0; cb < nc; cb += 64) {
        // the per-chunk scalars of 64 visited chunks: lane i holds visit cb + i
        const int cl = cb + lane;
        const float lamv = cl < nc ? lamp[(int64_t)chunk(cl) * Q] : 0.f;
        const int slv = (!REV && seq_idx && cl < nc) ? seq_idx[min(cl * Q + Q, T) - 1] : 0;
        // with cseg: whether chunk c-1 of the visited chunk c is in another segment
        int cut = 0;
        if (cseg && cl < nc) {
            const int c = chunk(cl);
            if (c > 0) cut = cseg[c] != cseg[c - 1];
        }
        for (int k0 = 0; k0 < 64 && cb + k0 < nc; k0 += D) {
#pragma unroll
            for (int j = 0; j < D; ++j) {
                const int k = cb + k0 + j;
                if (k < nc) {
                    float sv[VE];
                    unpack_vec<E, VE>(buf[j], sv);
                    if (k + D < nc) buf[j] = *reinterpret_cast<const R *>(lane_base + (int64_t)chunk(k + D) * cstride);
                    const bool kcut = __builtin_amdgcn_readlane(cut, k0 + j) != 0;   // uniform
                    {
                        // a chunk that starts a segment: nothing enters it (forward)
                        float hv[VE];
#pragma unroll
                        for (int v = 0; v < VE; ++v) hv[v] = (!REV && kcut) ? 0.f : hs[v];
                        store_vec<VE>(lane_base + (int64_t)chunk(k) * cstride, hv);
                    }
                    const float lm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lamv), k0 + j));
                    const int sc = __builtin_amdgcn_readlane(slv, k0 + j);
                    const bool keep = (REV || !seq_idx || sc == sprev) && !kcut;
                    sprev = sc;
                    const float d = exp_neg(lm);
                    if constexpr (BND) {
                        if (bnd_on) {
                            // hs is G_c here: its dot with Hin_c over this wave's elements
                            float hv[VE];
                            unpack_vec<E, VE>(hbuf[j % DH], hv);
                            if (k + DH < nc)
                                hbuf[j % DH] = *reinterpret_cast<const R *>(hin_base + (int64_t)chunk(k + DH) * cstride);
                            float dot = 0.f;
#pragma unroll
                            for (int v = 0; v < VE; ++v) dot += hs[v] * hv[v];
                            dot += dpp_mov<kDppQuadXor1>(dot);
                            dot += dpp_mov<kDppQuadXor2>(dot);
                            dot += dpp_mov<kDppRowHalfMirror>(dot);   // the other quad of the half row
                            dot += dpp_mov<kDppRowRor8>(dot);         // the other half row
                            const float tot = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dot), 0)) +
                                              __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dot), 16)) +
                                              __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dot), 32)) +
                                              __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dot), 48));
                            if (lane == 0) bnd_part[((int64_t)bh * nc + chunk(k)) * nwv + wv] = d * tot;
                        }
                    }
#pragma unroll
                    for (int v = 0; v < VE; ++v) hs[v] = (keep ? d * hs[v] : 0.f) + sv[v];
                }
            }
        }
    }
    if (final_states) store_final<VE>(final_states + (int64_t)bh * PN + e0, hs);
}

// ---------------------------------------------------------------------------
// Packed streams: segment ends and per-segment final states
// ---------------------------------------------------------------------------
// The packed-stream precondition, checked on the device (ssd_check_seq_idx):
// one workgroup scans the ids; *first_bad receives the first position t whose
// id is outside [0, nseq) or smaller than the id at t-1, or -1 when there is
// none.  Each thread keeps the smallest bad position it saw, and the workgroup
// takes the minimum, so the result does not depend on thread timing.
__global__ __launch_bounds__(1024) void k_check_seq_idx(const int32_t *__restrict__ seq_idx, int64_t T, int64_t nseq,
                                                        int32_t *__restrict__ first_bad)
{
    __shared__ int64_t wmin[16];
    int64_t bad = T;
    for (int64_t t = threadIdx.x; t < T; t += blockDim.x) {
        const int32_t id = seq_idx[t];
        if (id < 0 || id >= nseq || (t > 0 && id < seq_idx[t - 1])) {
            bad = t;   // t only grows, so the first hit is this thread's smallest
            break;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const int64_t v = __shfl_xor(bad, o);
        bad = v < bad ? v : bad;
    }
    if ((threadIdx.x & 63) == 0) wmin[threadIdx.x >> 6] = bad;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < (int)(blockDim.x >> 6); ++w) bad = wmin[w] < bad ? wmin[w] : bad;
        *first_bad = bad < T ? (int32_t)bad : -1;
    }
}

// seg_end for every segment, one thread per position (seg_end_mark).
__global__ void k_seg_end(const int32_t *__restrict__ seq_idx, int32_t *__restrict__ seg_end, int T, int nseq)
{
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t < T) seg_end_mark(seq_idx, seg_end, t, T, nseq);
}

// final_states[sg,h,p,n] = state right after segment sg's last token t_e:
//   sum_{s in t_e's chunk, s <= t_e, seq_s = sg} exp(cs_te - cs_s) delta_s x_s[p] B_s[n]
//   + [the segment was already open when the chunk started] exp(cs_te) Hin_c[p][n].
// An id that never occurs gets zeros.  Batch is 1 with packed streams.
template <typename E, int Q, int NT>
__global__ __launch_bounds__(kThreads, 2) void k_seq_final(
    const E *__restrict__ x, const E *__restrict__ Bm, const float *__restrict__ delta,
    const float *__restrict__ cs, const int32_t *__restrict__ seq_idx, const E *__restrict__ hin,
    const int32_t *__restrict__ seg_end, float *__restrict__ final_states,
    int T, int H, int G, int P, int N, int nc, int nseq, int ntp)
{
    constexpr int NI = NT / 64;
    __shared__ __align__(16) StateSmem<E, NT> sm;
    __shared__ float w[Q];
    __shared__ int m[Q];
    const int units = nseq * H * ntp;
    const int u = xcd_remap(blockIdx.x, units);
    int tp, h, sg, g;
    unit_coords(u, units, ntp, H, G, tp, h, sg, g);
    const int p0 = tp * 64;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
    float *out = final_states + ((int64_t)sg * H + h) * (int64_t)P * N;
    const int te = seg_end[sg];
    if (te < 0) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = wave * (NT / 4) + i * 16 + 4 * lg, p = p0 + j * 16 + li;
                float z[4] = {0.f, 0.f, 0.f, 0.f};
                if (p < P && n < N) store4_f32(out + (int64_t)p * N + n, z);
            }
        return;
    }
    const int c = te / Q, t0 = c * Q, ie = te - t0;
    // The entering-state tile is requested first, with the chunk's x and B rows
    // (one round trip less than after the product), and used only when the
    // segment was already open at the chunk start.
    using RV = typename RawVec<E, 4>::type;
    RV hraw[NI][4];
    const E *hc = hin + ((int64_t)c * H + h) * (int64_t)P * N;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = wave * (NT / 4) + i * 16 + 4 * lg, p = p0 + j * 16 + li;
            hraw[i][j] = (p < P && n < N) ? *reinterpret_cast<const RV *>(hc + (int64_t)p * N + n) : RV{};
        }
    const bool carry = seq_idx[c > 0 ? t0 - 1 : 0] == sg;
    const E *xsrc = x + ((int64_t)t0 * H + h) * P + p0;
    const E *bsrc = Bm + ((int64_t)t0 * G + g) * N;
    const int64_t ldx = (int64_t)H * P, ldb = (int64_t)G * N;
    using XT = typename StateSmem<E, NT>::XT;
    using BT = typename StateSmem<E, NT>::BT;
    XT xs;
    BT bs;
    xs.init(ldx, P - p0);
    bs.init(ldb, N);
    xs.load(XT::rsrc(xsrc, ldx, ie + 1));
    bs.load(BT::rsrc(bsrc, ldb, ie + 1));
    const int64_t cso = ((int64_t)h * nc + c) * Q;
    const float cse = cs[cso + ie];
    for (int s = threadIdx.x; s < Q; s += kThreads) {
        const bool keep = s <= ie && seq_idx[t0 + s] == sg;
        m[s] = keep;
        w[s] = keep ? exp_neg(cse - cs[cso + s]) * delta[cso + s] : 0.f;
    }
    __syncthreads();
    floatx4 acc[NI][4];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    state_product<E, NT, true>(sm, xsrc, ldx, bsrc, ldb, ie + 1, w, m, xs, bs, acc);

    const float dcar = exp_neg(cse);
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = wave * (NT / 4) + i * 16 + 4 * lg, p = p0 + j * 16 + li;
            if (p < P && n < N) {
                float hv[4];
                unpack_vec<E, 4>(hraw[i][j], hv);
                float o[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] = acc[i][j][q] + (carry ? dcar * hv[q] : 0.f);
                store4_f32(out + (int64_t)p * N + n, o);
            }
        }
}

// ---------------------------------------------------------------------------
// chunk_scan: y = intra-chunk quadratic form + decayed entering state + D x
// ---------------------------------------------------------------------------
// One workgroup of Q/32 waves per (b, c, h, 64-p tile).  The chunk's Q output
// rows are split into NJ = Q/16 sub-blocks j of 16 rows (t0 = 16 j); wave w owns
// j = w and j = NJ-1-w, which balances the causal triangle exactly (every wave
// has NJ/2 - 1 K steps strictly below its two diagonal steps).  Everything is
// computed transposed, D[p][t], so a per-token decay is a per-lane scale:
//   y_t = u_t [ e_{t0} (C_t . Hin) + sum_{s < S_j} CB[t][s] V_j[s] x_s ]
//         + sum_{S_j <= s <= t} (CB[t][s] exp(cs_t - cs_s) delta_s + [s = t] D) x_s
// with e_{t0} = exp(cs_{t0}), u_t = exp(cs_t - cs_{t0}), V_j[s] = exp(cs_{t0} -
// cs_s) delta_s, and S_j = 32 floor(j/2) the start of the 32-wide K step that
// holds t0.  Every factor is a decay <= 1, so nothing overflows, and
// per-element exponentials are needed only on the diagonal step, where the D
// skip term rides on the diagonal.  Segment masks (packed streams) are selects
// on the same factors.
// Memory: the entering-state tile and the x tile have LDS regions of their own
// and are stored as soon as their loads land, so one barrier publishes both.
// The entering-state tile is read for the last time here and y is not read
// again in the pass: both use the non-temporal cache policy, which keeps them
// from displacing the C and CB fragments that the chunk's other heads re-read
// from L2 (measured: chunk_scan 59 -> 54 us at 16384 tokens, 32 heads, N = 256).
// The C and CB fragments come from the chunk_cb buffer, fragment-major (one
// contiguous block per wave and K step), fetched RING K steps ahead.

// V_j rows are stored packed: row j holds 32 * floor(j/2) entries.
__host__ __device__ constexpr int vt_offset(int j)
{
    return 32 * ((j & 1) ? (j >> 1) * (j >> 1) : (j >> 1) * ((j >> 1) - 1));
}

template <int Q> constexpr int scan_threads() { return Q * 2; }

// NT = N rounded up to 64 (compile time, so every K loop unrolls and every LDS
// fragment offset is an immediate); columns N..NT-1 are masked.
// Dot modes (used by the backward pass; DOT = 0 is the forward): with v = `vec`
// at each token's position (DOT = 1) or at the mirrored position len-1-t of a
// chunk whose tokens were reversed (DOT = 2: x is passed in its own order and its
// rows are read reversed here; `cs` is the forward's, from which the reversed
// chunk's cs_rev[i] = cs[len-1] - cs[len-1-i] is formed here, with unit step
// sizes and `delta` unused; the chunk_cb buffer and the states come reversed
// from the caller), the kernel also writes, per token,
// fp32 dot products over this workgroup's 64 p (one [b,H,nc,Q] slice per p tile,
// indexed by the token's original position):
//   dot1 = v . (the entering-state term alone),  dot2 (DOT = 2) = v . (the whole
//   output before the D skip term).
// P1ONLY computes dot1 only: no x tile, no intra-chunk terms, no y.
// DOT = 2 writes, instead of the reversed problem's output y'_t, the gradient
// dx = dx_delta[t'] y'_t + dx_D[h] x_t at the token's original position t' =
// len-1-t (x = the reversed problem's input, here dy; dx_delta = the forward's
// step sizes in their own order; dx_D may be null), and x . v per token over
// this workgroup's 64 p to dxv (laid out like dot1).
// GATE multiplies every output by SiLU(z) (z = `gate`, laid out like y) before
// its one rounding to E: the gate of the Mamba-2 block ("SSM 家族全景图（下）",
// the block data flow of section five: the gated path passes a SiLU and the two
// paths are multiplied elementwise).
template <typename E, int Q, int NT, bool PACKED, int DOT = 0, bool P1ONLY = false, bool GATE = false>
__global__ __launch_bounds__(scan_threads<Q>(), 4) void k_chunk_scan(
    const E *__restrict__ x, const float *__restrict__ delta, const float *__restrict__ cs,
    const E *__restrict__ cbuf, const E *__restrict__ hin,
    const float *__restrict__ D, const int32_t *__restrict__ seq_idx, E *__restrict__ y,
    int T, int H, int G, int P, int N, int nc, int ntp, const E *__restrict__ vec = nullptr,
    float *__restrict__ dot1 = nullptr, float *__restrict__ dot2 = nullptr, const E *__restrict__ gate = nullptr,
    const float *__restrict__ dx_delta = nullptr, const float *__restrict__ dx_D = nullptr,
    float *__restrict__ dxv = nullptr, const int32_t *__restrict__ cseg = nullptr,
    const int2 *__restrict__ cmap = nullptr)
{
    using F = frag_t<E>;
    constexpr int TH = scan_threads<Q>();
    using XT = KTile<E, Q, 64, TH>;
    constexpr int V = kVec16<E>;
    constexpr int ES = (int)sizeof(E);
    constexpr int NJ = Q / 16;          // 16-row sub-blocks per chunk
    constexpr int NSB = 2;              // sub-blocks per wave
    constexpr int KSB = (NJ - 1) / 2;   // K steps strictly below some sub-block's diagonal step
    constexpr int NKS = NT / 32;        // K steps of the entering-state product
    // Pitch of the entering-state tile: rows 32 bytes apart modulo 256 keep its
    // 16-byte fragment reads free of bank conflicts (a 128-bit LDS read serves
    // lanes 0-7 with 16-23, 8-15 with 24-31, and so on, in one pass).
    constexpr int HP = NT + 2 * V;
    constexpr int RING = 3;             // C / CB fragments fetched RING K steps ahead
    // the entering-state tile; after step 4 the same memory stages y (bf16)
    constexpr int HSZ = 64 * HP > Q * 64 ? 64 * HP : Q * 64;
    __shared__ __align__(16) E hs[HSZ];
    __shared__ __align__(16) E xt[XT::SIZE];
    __shared__ __align__(16) float vt[vt_offset(NJ)];
    __shared__ __align__(16) float csb[Q];   // cs * log2(e)
    __shared__ __align__(16) float db[Q];
    __shared__ __align__(16) int sq[PACKED ? Q : 4];

    const int units = nc * H * ntp;
    const int u = xcd_remap(blockIdx.x, units);
    const int b = blockIdx.y;
    int tp, h, c, g;
    unit_coords(u, units, ntp, H, G, tp, h, c, g);
    if (cseg && cseg[c] < 0) return;   // a chunk of padding only (cseg: see k_state_passing)
    int t0, len;
    chunk_rows(c, Q, T, cmap, t0, len);
    const int p0 = tp * 64;
    const int64_t cso = (((int64_t)b * H + h) * nc + c) * Q;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform, in an SGPR
    const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
    int jb[NSB];
    jb[0] = wave;
    jb[1] = NJ - 1 - wave;

    // ---- issue the global loads ----
    // entering-state tile: VL lanes per row (one 16-byte vector each), RPP rows
    // per pass; at most HG passes are held in registers at once
    constexpr int VL = NT / V, RPP = TH / VL, HPASS = 64 / RPP, HG = HPASS < 8 ? HPASS : 8;
    const int vpr = N / V;
    const int hv = threadIdx.x % VL, hr = threadIdx.x / VL;
    const auto hrs = make_rsrc(hin + ((((int64_t)b * nc + c) * H + h) * P + p0) * (int64_t)N,
                               (int64_t)min(64, P - p0) * N * ES);
    const uint32_t hvoff = hv < vpr ? (uint32_t)(hr * N * ES + hv * 16) : kOffNone;
    auto hoff = [&](int i) -> uint32_t {
        return hvoff == kOffNone ? kOffNone : hvoff + (uint32_t)(i * RPP * N * ES);
    };
    uint4 hraw[HG];
#pragma unroll
    for (int i = 0; i < HG; ++i) hraw[i] = bload16_last(hrs, hoff(i));
    XT xs;
    if constexpr (DOT == 2) xs.init_rev((int64_t)H * P, P - p0, len);   // the chunk's tokens in reversed order
    else xs.init((int64_t)H * P, P - p0);
    if constexpr (!P1ONLY) xs.load(XT::rsrc(x + (((int64_t)b * T + t0) * H + h) * P + p0, (int64_t)H * P, len));
    float c_i = 0.f, d_i = 0.f;
    int s_i = 0;
    if (threadIdx.x < Q) {
        if constexpr (DOT == 2) {
            // the reversed chunk; past len cs_rev keeps its last value, with step size 0
            const int kk = (int)threadIdx.x < len ? (int)threadIdx.x : len - 1;
            c_i = (cs[cso + len - 1] - cs[cso + len - 1 - kk]) * kLog2e;
            d_i = (int)threadIdx.x < len ? 1.f : 0.f;
        } else {
            c_i = cs[cso + threadIdx.x] * kLog2e;   // decays below are exp2 of differences
            d_i = delta[cso + threadIdx.x];
        }
        if (PACKED) s_i = seq_idx[t0 + min((int)threadIdx.x, len - 1)];
    }
    const int seq_prev = PACKED ? seq_idx[c > 0 ? t0 - 1 : 0] : 0;

    // The chunk_cb buffer of this (b, c, g): CB then C, both fragment-major, so
    // the fragment of row block j and K step ks is the contiguous 64 x 8 block
    // (j * steps-per-row + ks); lane l takes elements 8 l .. 8 l + 7 of it.  A
    // dead sub-block (rows past the sequence end) reads nothing: its offset is
    // kOffNone, which stays outside the buffer after adding a block offset.
    const E *group = cbuf + (((int64_t)b * nc + c) * G + g) * cb_group_elems<Q, NT>();
    const auto cbrs = make_rsrc(group, (int64_t)Q * Q * ES);
    const auto crs = make_rsrc(group + (int64_t)Q * Q, (int64_t)Q * NT * ES);
    constexpr uint32_t BLK = 512 * ES;   // bytes per fragment block
    bool live[NSB];
    uint32_t cbase[NSB], cbbase[NSB];
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
        live[k] = 16 * jb[k] < len;   // wave-uniform
        cbase[k] = live[k] ? (uint32_t)(jb[k] * NKS) * BLK + lane * 8 * ES : kOffNone;
        cbbase[k] = (uint32_t)(jb[k] * (Q / 32)) * BLK + lane * 8 * ES;
    }
    auto c_off = [&](int k, int ks) -> uint32_t { return cbase[k] + (uint32_t)ks * BLK; };
    auto cb_off = [&](int k, int ks) -> uint32_t {
        return (live[k] && ks < (jb[k] >> 1)) ? cbbase[k] + (uint32_t)ks * BLK : kOffNone;
    };

    F cr[RING][NSB];
#pragma unroll
    for (int r = 0; r < RING; ++r)
#pragma unroll
        for (int k = 0; k < NSB; ++k) {
            if (r < NKS) bload_frag(crs, c_off(k, r), cr[r][k]);
            else cr[r][k] = F{};
        }

    // ---- entering-state tile, x tile and per-token values into LDS ----
#pragma unroll
    for (int i0 = 0; i0 < HPASS; i0 += HG) {
        if (i0 > 0) {
#pragma unroll
            for (int i = 0; i < HG; ++i) hraw[i] = bload16_last(hrs, hoff(i0 + i));
        }
        // lanes past column N loaded zeros: storing them zero-fills columns N..NT-1
#pragma unroll
        for (int i = 0; i < HG; ++i)
            *reinterpret_cast<uint4 *>(hs + (hr + (i0 + i) * RPP) * HP + hv * V) = hraw[i];
    }
    if constexpr (!P1ONLY) xs.template store<false, false>(xt, nullptr, nullptr);
    if (threadIdx.x < Q) {
        csb[threadIdx.x] = c_i;
        db[threadIdx.x] = d_i;
        if (PACKED) sq[threadIdx.x] = s_i;
    }
    __syncthreads();
    // V_j[s] for s < 32 floor(j/2): thread s fills its column for every row j that has it
    if (!P1ONLY && threadIdx.x < 32 * KSB) {
        const int s = threadIdx.x;
        const float css = csb[s], dss = db[s];
        const int sqs = PACKED ? sq[s] : 0;
        for (int j = 2 * (s / 32 + 1); j < NJ; ++j) {
            const int tj = 16 * j;
            vt[vt_offset(j) + s] = (!PACKED || sqs == sq[tj]) ? exp2_(csb[tj] - css) * dss : 0.f;
        }
    }

    floatx4 acc[NSB][4];
#pragma unroll
    for (int k = 0; k < NSB; ++k)
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) acc[k][pb] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Row-wise view of this wave's tile, used to turn y, the gate's z and the dot
    // modes' v around in LDS (bf16): lane (oct, chunk) takes 16 bytes, p0 +
    // 8 chunk .. + 7, of row 16 j + 8 half + rsel.  Rows sit in LDS with their 8
    // chunks of 16 bytes at chunk ^ ((t >> 1) & 7), so the 8-byte accesses of 16
    // rows in the accumulator layout spread over all banks; the 16-byte row
    // accesses take 8 rows per instruction, ordered so that the two lane octets
    // sharing an LDS pass (0-7 with 16-23, ...) touch rows of opposite parity,
    // i.e. opposite bank halves.
    auto yoff = [](int t, int ch) { return t * 64 + 8 * (ch ^ ((t >> 1) & 7)); };
    const int oct = lane >> 3, chunk = lane & 7;
    const int rsel = (oct & 4) + ((oct & 1) << 1) + ((oct >> 1) & 1);   // 0,2,1,3,4,6,5,7
    const bool pin = p0 + 8 * chunk < P;

    // Turn this wave's rows (row-wise view, rows[k][half]) around in the LDS
    // region buf (the wave's own rows t of it) into the accumulator layout.
    auto turn = [&](E *buf, const uint4 (&rows)[NSB][2], floatx4 (&out)[NSB][4]) {
#pragma unroll
        for (int k = 0; k < NSB; ++k)
#pragma unroll
            for (int half = 0; half < 2; ++half)
                *reinterpret_cast<uint4 *>(buf + yoff(16 * jb[k] + 8 * half + rsel, chunk)) = rows[k][half];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int k = 0; k < NSB; ++k) {
            const int t = 16 * jb[k] + li;
#pragma unroll
            for (int pb = 0; pb < 4; ++pb)
                out[k][pb] = __builtin_convertvector(
                    *reinterpret_cast<const bf16x4 *>(buf + yoff(t, 2 * pb + (lg >> 1)) + 4 * (lg & 1)), floatx4);
        }
        // every lane has read its values before the rows are written again
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    // The dot modes' v in the row-wise view (bf16): token t's vec row, at the
    // mirrored position for DOT = 2
    uint4 vrow[NSB][2];
    auto load_vrows = [&]() {
#pragma unroll
        for (int k = 0; k < NSB; ++k)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int t = 16 * jb[k] + 8 * half + rsel, tv = DOT == 2 ? len - 1 - t : t;
                vrow[k][half] = live[k] && t < len && pin
                                    ? *reinterpret_cast<const uint4 *>(
                                          vec + (((int64_t)b * T + t0 + tv) * H + h) * P + p0 + 8 * chunk)
                                    : uint4{0, 0, 0, 0};
            }
    };

    if constexpr (P1ONLY && sizeof(E) == 2) load_vrows();

    // ---- step 4 part: Hin C^T over n (columns N..NT-1 are zero in both) ----
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        F a[4];
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) a[pb] = load_frag(hs + (pb * 16 + li) * HP + ks * 32 + 8 * lg);
#pragma unroll
        for (int k = 0; k < NSB; ++k) {
            if (!live[k]) continue;
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) mma(acc[k][pb], a[pb], cr[ks % RING][k]);
        }
        if (ks + RING < NKS) {
#pragma unroll
            for (int k = 0; k < NSB; ++k) bload_frag(crs, c_off(k, ks + RING), cr[ks % RING][k]);
        }
    }

    // v . acc over this tile's 64 p for each token of the wave's live sub-blocks,
    // each acc scaled by a per-token factor; lane (li, lg) holds p = 16 pb + 4 lg + q
    // v either loaded here (vv = nullptr: four p of token t per lane) or given
    // in the accumulator layout (vv)
    auto dot_out = [&](float *dst, auto scale, const floatx4 (*vv)[4] = nullptr) {
        const int64_t rowb = ((((int64_t)tp * gridDim.y + b) * H + h) * nc + c) * Q;
#pragma unroll
        for (int k = 0; k < NSB; ++k) {
            if (!live[k]) continue;
            const int t = 16 * jb[k] + li;
            const int tv = DOT == 2 ? len - 1 - t : t;   // the token's original position
            const float f = scale(k, t);
            float sum = 0.f;
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) {
                const int p = p0 + 16 * pb + 4 * lg;
                float v[4] = {0.f, 0.f, 0.f, 0.f};
                if (vv) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[q] = vv[k][pb][q];
                } else if (t < len && p < P) {
                    load4_f32(vec + (((int64_t)b * T + t0 + tv) * H + h) * P + p, v);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) sum += v[q] * acc[k][pb][q];
            }
            sum += __shfl_xor(sum, 16);
            sum += __shfl_xor(sum, 32);
            if (lg == 0 && t < len) dst[rowb + tv] = sum * f;
        }
    };
    if constexpr (DOT != 0) {
        // after the e^{cs_t0} scale below, the entering-state term of token t is
        // acc * exp(cs_t - cs_t0): take its dot product now
        auto sc1 = [&](int k, int t) {
            const int tj = 16 * jb[k];
            const bool mo = !PACKED || sq[tj] == seq_prev;
            return mo ? exp2_(csb[tj]) * exp2_(csb[min(t, Q - 1)] - csb[tj]) : 0.f;
        };
        if constexpr (P1ONLY && sizeof(E) == 2) {
            // v (loaded before step 4) turns around in the entering-state region
            // once every wave is done with it
            floatx4 vv[NSB][4];
            __syncthreads();
            turn(hs, vrow, vv);
            dot_out(dot1, sc1, vv);
        } else {
            dot_out(dot1, sc1);
        }
        if constexpr (P1ONLY) return;
    }

    // CB fragments: the diagonal step of both sub-blocks, and the first RING
    // strictly-below steps (every row of cb is in bounds)
    F dcb[NSB];
#pragma unroll
    for (int k = 0; k < NSB; ++k)
        bload_frag(cbrs, live[k] ? cbbase[k] + (uint32_t)(jb[k] >> 1) * BLK : kOffNone, dcb[k]);
#pragma unroll
    for (int r = 0; r < RING; ++r)
#pragma unroll
        for (int k = 0; k < NSB; ++k) {
            if (r < KSB) bload_frag(cbrs, cb_off(k, r), cr[r][k]);
            else cr[r][k] = F{};
        }
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
        const int tj = 16 * jb[k];
        const bool mo = !PACKED || sq[tj] == seq_prev;
        const float e0 = exp2_(csb[tj]);
#pragma unroll
        for (int pb = 0; pb < 4; ++pb)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[k][pb][q] = mo ? acc[k][pb][q] * e0 : 0.f;
    }

    // The gate's z (GATE), loaded before the diagonal step so that the loads
    // overlap its MFMA work.  bf16: in the row-wise view above (whole 128-byte
    // rows, 8 per instruction), turned around in LDS before use; fp32: four
    // consecutive p of token t per (sub-block, p block), straight into the
    // accumulator layout.
    using E4 = E __attribute__((ext_vector_type(4)));
    constexpr bool ZROW = sizeof(E) == 2;
    E4 zr[NSB][4];
    uint4 zrow[NSB][2];
    auto load_z = [&](int k) {
        if constexpr (ZROW) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int t = 16 * jb[k] + 8 * half + rsel;
                zrow[k][half] = live[k] && t < len && pin
                                    ? *reinterpret_cast<const uint4 *>(
                                          gate + (((int64_t)b * T + t0 + t) * H + h) * P + p0 + 8 * chunk)
                                    : uint4{0, 0, 0, 0};
            }
        } else {
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) {
                const int t = 16 * jb[k] + li, p = p0 + 16 * pb + 4 * lg;
                zr[k][pb] = live[k] && t < len && p < P
                                ? *reinterpret_cast<const E4 *>(gate + (((int64_t)b * T + t0 + t) * H + h) * P + p)
                                : E4{};
            }
        }
    };

    __syncthreads();   // the V table is complete
    typename XT::Off xoff[4];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) xoff[pb] = XT::frag_off(pb * 16);

    // Packed streams: a chunk that holds a segment boundary (block-uniform) takes
    // selects wherever the common path relies on a zero weight, so that a
    // non-finite x or B of one sequence cannot reach another's outputs: in step 1
    // the x rows and CB columns of tokens outside the sub-block's segment are
    // dropped, and the diagonal step runs once per segment among the sub-block's
    // rows, each pass kept only for that segment's rows.
    const bool bnd = PACKED && sq[0] != sq[max(len, 1) - 1];
    // first_row[k]: the first row of the chunk in the segment of sub-block k's
    // first row (boundary chunks only; 0 otherwise)
    int first_row[NSB];
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
        first_row[k] = 0;
        if (PACKED && bnd) {   // binary search: ids never decrease along the chunk
            const int tj = 16 * jb[k], sj = sq[tj];
            int lo = 0, hi = tj;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (__builtin_amdgcn_readfirstlane(sq[mid]) < sj) lo = mid + 1;
                else hi = mid;
            }
            first_row[k] = lo;
        }
    }

    // ---- step 1, the K steps strictly below each sub-block's diagonal step ----
    // In a chunk with a segment boundary, the K steps before the start of the
    // segment of the sub-block's first row (first_row) contribute nothing: the
    // ones wholly before it are skipped, and the one that straddles it is done
    // after the loop with selects.
#pragma unroll
    for (int ks = 0; ks < KSB; ++ks) {
        F a[4];
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) a[pb] = XT::frag_at(xt, xoff[pb], ks * 32);
#pragma unroll
        for (int k = 0; k < NSB; ++k) {
            const int j = jb[k];
            if (ks >= (j >> 1) || !live[k]) continue;
            if (PACKED && ks * 32 < first_row[k]) continue;   // wave-uniform; 0 without a boundary
            const float *vrow = vt + vt_offset(j) + ks * 32 + 8 * lg;
            const floatx4 v0 = *reinterpret_cast<const floatx4 *>(vrow);
            const floatx4 v1 = *reinterpret_cast<const floatx4 *>(vrow + 4);
            const floatx8 vv = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
            const F wfr = from_f32<F>(to_f32(cr[ks % RING][k]) * vv);
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) mma(acc[k][pb], a[pb], wfr);
        }
        if (ks + RING < KSB) {
#pragma unroll
            for (int k = 0; k < NSB; ++k) bload_frag(cbrs, cb_off(k, ks + RING), cr[ks % RING][k]);
        }
    }
    if (PACKED && bnd) {
        // The straddling K step: the x rows and CB columns before first_row are
        // dropped by selects (its CB fragment is fetched again here).
#pragma unroll
        for (int k = 0; k < NSB; ++k) {
            const int j = jb[k], ks = first_row[k] >> 5;
            if (!live[k] || ks * 32 == first_row[k] || ks >= (j >> 1)) continue;   // wave-uniform
            F cbf;
            bload_frag(cbrs, cb_off(k, ks), cbf);
            const float *vrow = vt + vt_offset(j) + ks * 32 + 8 * lg;
            const floatx4 v0 = *reinterpret_cast<const floatx4 *>(vrow);
            const floatx4 v1 = *reinterpret_cast<const floatx4 *>(vrow + 4);
            const int sb = ks * 32 + 8 * lg;
            bool kp[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) kp[e] = sb + e >= first_row[k];
            const floatx8 cf = to_f32(cbf);
            floatx8 wf;
#pragma unroll
            for (int e = 0; e < 8; ++e) wf[e] = kp[e] ? cf[e] * (e < 4 ? v0[e] : v1[e - 4]) : 0.f;
            const F wfr = from_f32<F>(wf);
#pragma unroll
            for (int pb = 0; pb < 4; ++pb)
                mma(acc[k][pb], mask_frag(XT::frag_at(xt, xoff[pb], ks * 32), kp), wfr);
        }
    }

    if constexpr (GATE) {
#pragma unroll
        for (int k = 0; k < NSB; ++k) load_z(k);
    }
    if constexpr (DOT == 2 && sizeof(E) == 2) load_vrows();

    // ---- u_t scale, then the diagonal K step with per-element decays and D ----
    const float Dh = D ? D[h] : 0.f;
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
        const int j = jb[k];
        if (!live[k]) continue;
        const int tj = 16 * j, t = tj + li;
        const bool keep = !PACKED || sq[t] == sq[tj];
        const float ut = exp2_(csb[t] - csb[tj]);
#pragma unroll
        for (int pb = 0; pb < 4; ++pb)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[k][pb][q] = keep ? acc[k][pb][q] * ut : 0.f;

        const int ks = j >> 1;
        const int sb = ks * 32 + 8 * lg;
        const floatx8 cf = to_f32(dcb[k]);
        const floatx4 cs0 = *reinterpret_cast<const floatx4 *>(csb + sb);
        const floatx4 cs1 = *reinterpret_cast<const floatx4 *>(csb + sb + 4);
        const floatx4 d0 = *reinterpret_cast<const floatx4 *>(db + sb);
        const floatx4 d1 = *reinterpret_cast<const floatx4 *>(db + sb + 4);
        const floatx8 csv = __builtin_shufflevector(cs0, cs1, 0, 1, 2, 3, 4, 5, 6, 7);
        const floatx8 dv = __builtin_shufflevector(d0, d1, 0, 1, 2, 3, 4, 5, 6, 7);
        const float cst = csb[t];
        const int rel = t - sb;   // position of t in this lane's 8 K slots (valid if 0..7)
        floatx8 wf;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bool ok = e <= rel;
            if (PACKED) ok = ok && sq[sb + e] == sq[t];
            wf[e] = (ok ? cf[e] * exp2_(cst - csv[e]) * dv[e] : 0.f) + (e == rel ? Dh : 0.f);
        }
        const F wfr = from_f32<F>(wf);
        if (PACKED && bnd && sq[ks * 32] != sq[ks * 32 + 31]) {   // wave-uniform
            // The K step holds a segment boundary: one pass per segment id sig among
            // rows tj .. tj+15 (ids never decrease along the chunk; rows past the end
            // repeat the last id), with the x slots of other segments dropped, each
            // pass kept for the rows of sig only (one p block at a time)
            // Each pass covers the rows lo .. hi of one id (a contiguous run, found
            // from the per-lane ids by ballots; everything here is wave-uniform).
            const int sid = sq[t];
            int lo = tj;
            while (lo < tj + 16) {
                const int sig = __builtin_amdgcn_readfirstlane(sq[lo]);
                const uint64_t later = __ballot(sid > sig) & 0xffffull;
                const int hi = later ? tj + __builtin_ctzll(later) - 1 : tj + 15;
                // the K slots of this id: rows of sig before tj lie in the same K
                // step only when tj is its second half, and the id may run on past
                // hi into the K step's second half
                const uint64_t ks_in = __ballot(lane < 32 && sq[ks * 32 + (lane & 31)] == sig);
                const int slo = ks * 32 + __builtin_ctzll(ks_in), shi = ks * 32 + 63 - __builtin_clzll(ks_in);
                bool kp[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) kp[e] = sb + e >= slo && sb + e <= shi;
                const bool mine = t >= lo && t <= hi;
#pragma unroll
                for (int pb = 0; pb < 4; ++pb) {
                    floatx4 tmp = floatx4{0.f, 0.f, 0.f, 0.f};
                    mma(tmp, mask_frag(XT::frag_at(xt, xoff[pb], ks * 32), kp), wfr);
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[k][pb][q] += mine ? tmp[q] : 0.f;
                }
                lo = hi + 1;
            }
            continue;
        }
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) mma(acc[k][pb], XT::frag_at(xt, xoff[pb], ks * 32), wfr);
    }

    if constexpr (DOT == 2) {
        if constexpr (sizeof(E) == 2) {
            // the entering-state region is free since the barrier after step 4
            floatx4 vv[NSB][4];
            turn(hs, vrow, vv);
            dot_out(dot2, [](int, int) { return 1.f; }, vv);
        } else {
            dot_out(dot2, [](int, int) { return 1.f; });
        }
    }

    if constexpr (GATE) {
        // y *= SiLU(z) in fp32, before the one rounding of y
        if constexpr (ZROW) {
            floatx4 zf[NSB][4];
            turn(hs, zrow, zf);
#pragma unroll
            for (int k = 0; k < NSB; ++k)
#pragma unroll
                for (int pb = 0; pb < 4; ++pb)
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[k][pb][q] *= silu(zf[k][pb][q]);
        } else {
#pragma unroll
            for (int k = 0; k < NSB; ++k) {
                if (!live[k]) continue;
#pragma unroll
                for (int pb = 0; pb < 4; ++pb) {
                    const floatx4 zf = __builtin_convertvector(zr[k][pb], floatx4);
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[k][pb][q] *= silu(zf[q]);
                }
            }
        }
    }

    // ---- epilogue: store y (DOT = 2: dx at the mirrored rows) ----
    const float dxD = DOT == 2 && dx_D ? dx_D[h] : 0.f;
    if constexpr (DOT == 2) {
        // Delta y' in fp32 here; the D dy term joins in the row phase below
#pragma unroll
        for (int k = 0; k < NSB; ++k) {
            const int t = 16 * jb[k] + li;
            const float dl = t < len ? dx_delta[cso + len - 1 - t] : 0.f;
#pragma unroll
            for (int pb = 0; pb < 4; ++pb)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[k][pb][q] *= dl;
        }
    }
    if constexpr (sizeof(E) == 2) {
        // Each wave turns its own 32 rows around in the entering-state region (free
        // since the barrier after step 4) so that y leaves as whole 128-byte rows
        // (the row-wise view above).
#pragma unroll
        for (int k = 0; k < NSB; ++k) {
            const int t = 16 * jb[k] + li;
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) {
                const uint2 v{pack_bf16x2(acc[k][pb][0], acc[k][pb][1]), pack_bf16x2(acc[k][pb][2], acc[k][pb][3])};
                *reinterpret_cast<uint2 *>(hs + yoff(t, 2 * pb + (lg >> 1)) + 4 * (lg & 1)) = v;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int k = 0; k < NSB; ++k) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int t = 16 * jb[k] + 8 * half + rsel;
                uint4 v = *reinterpret_cast<const uint4 *>(hs + yoff(t, chunk));
                if constexpr (DOT == 2) {
                    // dy's row t (p0 + 8 chunk ..) from the x tile: + D dy, and dy . v
                    // with v's same row and columns (still in registers), summed
                    // over the octet of lanes that holds the row
                    const floatx8 xv = __builtin_convertvector(
                        *reinterpret_cast<const bf16x8 *>(xt + t * 64 + 4 * ((2 * chunk) ^ XT::swz(t))), floatx8);
                    const floatx8 vr = __builtin_convertvector(__builtin_bit_cast(bf16x8, vrow[k][half]), floatx8);
                    float dv = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) dv += xv[e] * vr[e];
                    dv += dpp_mov<kDppQuadXor1>(dv);
                    dv += dpp_mov<kDppQuadXor2>(dv);
                    dv += dpp_mov<kDppRowHalfMirror>(dv);   // the octet's other quad
                    if (chunk == 0 && t < len)
                        dxv[((((int64_t)tp * gridDim.y + b) * H + h) * nc + c) * Q + len - 1 - t] = dv;
                    if (dx_D) {
                        const floatx8 d = __builtin_convertvector(__builtin_bit_cast(bf16x8, v), floatx8);
                        float o[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) o[e] = d[e] + dxD * xv[e];
                        v = uint4{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                                  pack_bf16x2(o[6], o[7])};
                    }
                }
                const int tw = DOT == 2 ? len - 1 - t : t;   // the row written
                if (t < len && pin)
                    store16_stream(y + (((int64_t)b * T + t0 + tw) * H + h) * P + p0 + 8 * chunk, v);
            }
        }
    } else {
        // fp32: each lane writes 16 bytes (4 consecutive p of one t) directly
#pragma unroll
        for (int k = 0; k < NSB; ++k) {
            const int t = 16 * jb[k] + li;
            const int tw = DOT == 2 ? len - 1 - t : t;   // the row written
            float dpart = 0.f;
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) {
                const int p = p0 + pb * 16 + 4 * lg;
                if (t >= len || p >= P) continue;
                float o[4] = {acc[k][pb][0], acc[k][pb][1], acc[k][pb][2], acc[k][pb][3]};
                if constexpr (DOT == 2) {
                    float xv[4], vv[4];
                    load4_f32(x + (((int64_t)b * T + t0 + tw) * H + h) * P + p, xv);
                    load4_f32(vec + (((int64_t)b * T + t0 + tw) * H + h) * P + p, vv);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        dpart += xv[q] * vv[q];
                        o[q] += dxD * xv[q];
                    }
                }
                store16_stream(y + (((int64_t)b * T + t0 + tw) * H + h) * P + p,
                               uint4{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                                     __float_as_uint(o[3])});
            }
            if constexpr (DOT == 2) {
                // dy . v of token t over the four lane groups (all lanes take part)
                dpart += __shfl_xor(dpart, 16);
                dpart += __shfl_xor(dpart, 32);
                if (lg == 0 && t < len) dxv[((((int64_t)tp * gridDim.y + b) * H + h) * nc + c) * Q + tw] = dpart;
            }
        }
    }
}

// final_states for an empty sequence: a copy of the initial state (or zeros).
__global__ void k_fill_final(float *__restrict__ out, const float *__restrict__ init, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = init ? init[i] : 0.f;
}

// ---------------------------------------------------------------------------
// Decode step: one new token per batch row, the state updated in place
// ---------------------------------------------------------------------------
// The recurrence itself, one step of it (section 3.1 of "Mamba 2 --
// Transformers are SSMs"): with a = exp(Delta A_h),
//   state[p][n] <- a state[p][n] + Delta x_p B_n,   y_p = sum_n C_n state[p][n] + D_h x_p.
// One workgroup per (b, h, block of RP*PASSES rows p).  A state row of N fp32 is
// covered by NL lanes (the power of two >= N/4), four consecutive n per lane, so
// every state access is 16 bytes; RP = 256/NL rows per pass.  Every state load of
// the workgroup is issued before any arithmetic; y_p is the sum of the row's
// lanes, combined with xor shuffles inside each NL-lane group.
template <int NL> constexpr int step_passes() { return NL / 4 < 8 ? NL / 4 : 8; }
template <int NL> constexpr int step_rows() { return (kThreads / NL) * step_passes<NL>(); }

template <typename E, int NL>
__global__ __launch_bounds__(kThreads) void k_ssd_step(
    const E *__restrict__ x, const E *__restrict__ dt, const float *__restrict__ A, const E *__restrict__ Bm,
    const E *__restrict__ Cm, const float *__restrict__ D, float *__restrict__ state, E *__restrict__ y, int H,
    int G, int P, int N, int softplus)
{
    constexpr int RP = kThreads / NL, PASSES = step_passes<NL>();
    const int bh = blockIdx.x;   // b * H + h
    const bool small = gridDim.x < (1u << 23);
    int b, h, g, gr;
    udivmod(bh, H, small, b, h);
    udivmod(h * G, H, small && (int64_t)H * G < (1 << 23), g, gr);
    const int p0 = blockIdx.y * RP * PASSES;
    const int li = threadIdx.x % NL, r = threadIdx.x / NL;
    const int n = 4 * li;
    const bool nin = n < N;   // N is a multiple of 16, so n + 3 < N too
    float *srow = state + (int64_t)bh * P * N;

    floatx4 hv[PASSES];
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
        const int p = p0 + r + i * RP;
        hv[i] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (p < P && nin) hv[i] = *reinterpret_cast<const floatx4 *>(srow + (int64_t)p * N + n);
    }
    float bv[4] = {0.f, 0.f, 0.f, 0.f}, cv[4] = {0.f, 0.f, 0.f, 0.f};
    if (nin) {
        load4_f32(Bm + ((int64_t)b * G + g) * N + n, bv);
        load4_f32(Cm + ((int64_t)b * G + g) * N + n, cv);
    }
    float xv[PASSES];
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
        const int p = p0 + r + i * RP;
        xv[i] = p < P ? to_float(x[(int64_t)bh * P + p]) : 0.f;
    }
    const float z = to_float(dt[bh]);
    const float delta = softplus ? softplus_f(z) : z;
    const float a = exp2_(delta * A[h] * kLog2e);
    const float Dh = D ? D[h] : 0.f;

#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
        const int p = p0 + r + i * RP;
        const float dx = delta * xv[i];
        floatx4 hn;
#pragma unroll
        for (int q = 0; q < 4; ++q) hn[q] = fmaf(a, hv[i][q], dx * bv[q]);
        if (p < P && nin) *reinterpret_cast<floatx4 *>(srow + (int64_t)p * N + n) = hn;
        float part = cv[0] * hn[0] + cv[1] * hn[1] + cv[2] * hn[2] + cv[3] * hn[3];
#pragma unroll
        for (int m = NL / 2; m > 0; m >>= 1) part += __shfl_xor(part, m, NL);
        if (li == 0 && p < P) y[(int64_t)bh * P + p] = from_float<E>(part + Dh * xv[i]);
    }
}

}  // namespace ssd
