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

#include "ssd_device.hpp"

namespace ssd {

// ---------------------------------------------------------------------------
// chunk_cumsum
// ---------------------------------------------------------------------------
constexpr int kCumsumHeads = 16;   // heads per workgroup

__device__ __forceinline__ float softplus_f(float z)
{
    // log(1 + e^z); above 20 the correction e^-z is below 2e-9 relative.
    return z > 20.f ? z : log1pf(expf(z));
}

// Grid (nc, ceil(H/16), b).  The workgroup reads the chunk's dt rows for 16
// heads (coalesced along heads), applies softplus, and each wave then runs one
// head at a time: every lane owns Q/64 consecutive tokens, sums them
// sequentially, and a segmented wave scan (a segment restarts at a packed
// sequence boundary) combines the lanes.  Sums run in fp64 and are rounded
// once, so a stored cs carries a single rounding.
template <typename E>
__global__ __launch_bounds__(kThreads) void k_chunk_cumsum(
    const E *__restrict__ dt, const float *__restrict__ A, const int32_t *__restrict__ seq_idx,
    float *__restrict__ delta, float *__restrict__ cs, int T, int H, int Q, int nc, int softplus)
{
    __shared__ float tile[256][kCumsumHeads + 1];
    __shared__ int sq[256];
    const int c = blockIdx.x, h0 = blockIdx.y * kCumsumHeads, b = blockIdx.z;
    const int t0 = c * Q;
    const int nh = min(kCumsumHeads, H - h0);
    for (int idx = threadIdx.x; idx < Q * kCumsumHeads; idx += kThreads) {
        const int i = idx / kCumsumHeads, hh = idx % kCumsumHeads;
        const int t = t0 + i;
        float v = 0.f;
        if (t < T && hh < nh) {
            const float z = to_float(dt[((int64_t)b * T + t) * H + h0 + hh]);
            v = softplus ? softplus_f(z) : z;
        }
        tile[i][hh] = v;
    }
    if (seq_idx)
        for (int i = threadIdx.x; i < Q; i += kThreads) sq[i] = (t0 + i < T) ? seq_idx[t0 + i] : 0;
    __syncthreads();

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int per = Q >> 6;   // 1, 2 or 4 tokens per lane
    for (int hh = wave; hh < nh; hh += 4) {
        const int h = h0 + hh;
        const double a = (double)A[h];
        double loc[4];
        int flg[4];
        double run = 0.0;
        int restarted = 0;
        for (int j = 0; j < per; ++j) {
            const int i = lane * per + j;
            if (seq_idx && i > 0 && t0 + i < T && sq[i] != sq[i - 1]) {
                run = 0.0;
                restarted = 1;
            }
            run += (double)tile[i][hh] * a;
            loc[j] = run;
            flg[j] = restarted;
        }
        // segmented inclusive scan of (restarted, run) over the 64 lanes
        double v = run;
        int f = restarted;
        for (int off = 1; off < 64; off <<= 1) {
            const double vo = __shfl_up(v, off);
            const int fo = __shfl_up(f, off);
            if (lane >= off) {
                if (!f) v += vo;
                f |= fo;
            }
        }
        double carry = __shfl_up(v, 1);
        if (lane == 0) carry = 0.0;
        const int64_t o = (((int64_t)b * H + h) * nc + c) * Q + lane * per;
        for (int j = 0; j < per; ++j) {
            delta[o + j] = tile[lane * per + j][hh];
            cs[o + j] = (float)(flg[j] ? loc[j] : carry + loc[j]);
        }
    }
}

// ---------------------------------------------------------------------------
// chunk_cb: cb[b,c,g,t,s] = sum_n C[t,n] B[s,n] for the lower block triangle
// ---------------------------------------------------------------------------
// One workgroup per 64x64 (t, s) tile with s-tile <= t-tile; four waves of 32x32.
// The MFMA computes D[s][t] (A = B rows, B = C rows, K = n, both K-contiguous in
// memory), so each lane ends with 4 consecutive s of one t: a vector store.
template <typename E>
__global__ __launch_bounds__(kThreads) void k_chunk_cb(
    const E *__restrict__ Bm, const E *__restrict__ Cm, E *__restrict__ cb,
    int T, int G, int N, int Q, int nc, int ntri)
{
    using F = frag_t<E>;
    const int units = ntri * nc * G;
    const int u = xcd_remap(blockIdx.x, units);
    const int b = blockIdx.y;
    int tile = u % ntri;
    const int cg = u / ntri, g = cg % G, c = cg / G;
    int ti = 0;
    while (tile > ti) { tile -= ti + 1; ++ti; }
    const int si = tile;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
    const int s_base = si * 64 + (wave & 1) * 32;
    const int t_base = ti * 64 + (wave >> 1) * 32;
    const int t0 = c * Q, len = min(Q, T - t0);

    const E *brow[2], *crow[2];
    bool bv[2], cv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int s = s_base + i * 16 + li, t = t_base + i * 16 + li;
        bv[i] = s < len;
        cv[i] = t < len;
        brow[i] = Bm + (((int64_t)b * T + t0 + (bv[i] ? s : 0)) * G + g) * N;
        crow[i] = Cm + (((int64_t)b * T + t0 + (cv[i] ? t : 0)) * G + g) * N;
    }
    floatx4 acc[2][2] = {};
    for (int k0 = 0; k0 < N; k0 += 32) {
        const int k = k0 + 8 * lg;
        const bool kin = k < N;
        F a[2], bb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            a[i] = (bv[i] && kin) ? load_frag(brow[i] + k) : F{};
            bb[i] = (cv[i] && kin) ? load_frag(crow[i] + k) : F{};
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) mma(acc[i][j], a[i], bb[j]);
    }
    E *out = cb + (((int64_t)b * nc + c) * G + g) * (int64_t)Q * Q;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int s = s_base + i * 16 + 4 * lg, t = t_base + j * 16 + li;
            float o[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
            store4_f32(out + (int64_t)t * Q + s, o);
        }
}

// ---------------------------------------------------------------------------
// Shared pieces of the state kernels
// ---------------------------------------------------------------------------

// Copy a [Q rows (time) x 64 cols] tile from global memory (row stride `ld`
// elements; rows >= slen and cols >= ncols read as zero) into LDS transposed,
// dst[col][row] with a pitch of Q + 16 bytes, optionally scaling row s by w[s]
// where m[s] != 0 and zeroing it where m[s] == 0 (a select, so a non-finite input
// in a masked row cannot leak).  Each thread moves V x V blocks (V = 16 B / elem).
template <typename E, int Q, bool SCALE>
__device__ __forceinline__ void stage_transposed(E *__restrict__ dst, const E *__restrict__ src, int64_t ld,
                                                 int slen, int ncols, const float *w, const int *m)
{
    constexpr int V = kVec16<E>;
    constexpr int PITCH = Q + V;
    constexpr int CB = 64 / V;
    constexpr int NB = (Q / V) * CB;
    for (int blk = threadIdx.x; blk < NB; blk += kThreads) {
        const int cbk = blk % CB, sb = blk / CB;
        const int col0 = cbk * V;
        float v[V][V];
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const int s = sb * V + i;
            if (s < slen && col0 < ncols) {
                load16_f32(src + (int64_t)s * ld + col0, v[i]);
            } else {
#pragma unroll
                for (int j = 0; j < V; ++j) v[i][j] = 0.f;
            }
            if (SCALE) {
                const float ws = w[s];
                const bool keep = m[s] != 0;
#pragma unroll
                for (int j = 0; j < V; ++j) v[i][j] = keep ? v[i][j] * ws : 0.f;
            }
        }
#pragma unroll
        for (int j = 0; j < V; ++j) {
            float col[V];
#pragma unroll
            for (int i = 0; i < V; ++i) col[i] = v[i][j];
            store16_f32(dst + (col0 + j) * PITCH + sb * V, col);
        }
    }
}

// acc[i][j][r] += sum_s bt[n][s] * xt[p][s] for the wave's 32x32 (n, p) quadrant,
// n = wn*32 + i*16 + 4*(lane/16) + r, p = wp*32 + j*16 + lane%16.
template <typename E, int Q>
__device__ __forceinline__ void state_mma(const E *bt, const E *xt, floatx4 (&acc)[2][2], int kend)
{
    constexpr int PITCH = Q + kVec16<E>;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
    const int wn = wave >> 1, wp = wave & 1;
    const E *a0p = bt + (wn * 32 + li) * PITCH + 8 * lg;
    const E *a1p = a0p + 16 * PITCH;
    const E *b0p = xt + (wp * 32 + li) * PITCH + 8 * lg;
    const E *b1p = b0p + 16 * PITCH;
    for (int ks = 0; ks < kend; ks += 32) {
        const auto a0 = load_frag(a0p + ks), a1 = load_frag(a1p + ks);
        const auto b0 = load_frag(b0p + ks), b1 = load_frag(b1p + ks);
        mma(acc[0][0], a0, b0);
        mma(acc[0][1], a0, b1);
        mma(acc[1][0], a1, b0);
        mma(acc[1][1], a1, b1);
    }
}

// ---------------------------------------------------------------------------
// chunk_state: states[b,c,h,p,n] = sum_s w_s x_s[p] B_s[n]
// ---------------------------------------------------------------------------
// w_s = exp(cs_last - cs_s) * delta_s for s in the segment of the chunk's last
// token (0 elsewhere).  One workgroup per (c, h, 64-p tile, 64-n tile); the
// product runs as D[n][p] = sum_s B^T[n][s] X'^T[p][s] so each lane stores 4
// consecutive n of one p.
template <typename E, int Q>
__global__ __launch_bounds__(kThreads) void k_chunk_state(
    const E *__restrict__ x, const E *__restrict__ Bm, const float *__restrict__ delta,
    const float *__restrict__ cs, const int32_t *__restrict__ seq_idx, E *__restrict__ states,
    int T, int H, int G, int P, int N, int nc, int ntp, int ntn)
{
    constexpr int PITCH = Q + kVec16<E>;
    __shared__ __align__(16) E xt[64 * PITCH];
    __shared__ __align__(16) E bt[64 * PITCH];
    __shared__ float w[Q];
    __shared__ int m[Q];
    const int units = nc * H * ntp * ntn;
    const int u = xcd_remap(blockIdx.x, units);
    const int b = blockIdx.y;
    int r = u;
    const int tn = r % ntn; r /= ntn;
    const int tp = r % ntp; r /= ntp;
    const int h = r % H;
    const int c = r / H;
    const int g = h / (H / G);
    const int t0 = c * Q, len = min(Q, T - t0);
    const int64_t cso = (((int64_t)b * H + h) * nc + c) * Q;
    const float lam = cs[cso + len - 1];
    const int seq_last = seq_idx ? seq_idx[t0 + len - 1] : 0;
    for (int s = threadIdx.x; s < Q; s += kThreads) {
        const bool keep = s < len && (!seq_idx || seq_idx[t0 + s] == seq_last);
        m[s] = keep;
        w[s] = keep ? exp_neg(lam - cs[cso + s]) * delta[cso + s] : 0.f;
    }
    __syncthreads();
    const int p0 = tp * 64, n0 = tn * 64;
    stage_transposed<E, Q, true>(xt, x + (((int64_t)b * T + t0) * H + h) * P + p0, (int64_t)H * P, len,
                                 P - p0, w, m);
    stage_transposed<E, Q, false>(bt, Bm + (((int64_t)b * T + t0) * G + g) * N + n0, (int64_t)G * N, len,
                                  N - n0, nullptr, nullptr);
    __syncthreads();
    floatx4 acc[2][2] = {};
    state_mma<E, Q>(bt, xt, acc, (len + 31) & ~31);

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
    const int wn = wave >> 1, wp = wave & 1;
    E *out = states + (((int64_t)b * nc + c) * H + h) * (int64_t)P * N;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + wn * 32 + i * 16 + 4 * lg, p = p0 + wp * 32 + j * 16 + li;
            if (p < P && n < N) {
                float o[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
                store4_f32(out + (int64_t)p * N + n, o);
            }
        }
}

// ---------------------------------------------------------------------------
// state_passing: in place S_c -> h_{c-1}; h_c = exp(cs_last(c)) h_{c-1} + S_c
// ---------------------------------------------------------------------------
// Every (b, h, p, n) element is an independent length-nc scan, so each thread
// owns one 16-byte vector of elements and walks the chunks, loading kPrefetch
// chunk states ahead of the arithmetic to keep many loads in flight.  The
// carry is replaced by zero (a select) when the chunk holds a segment boundary.
constexpr int kPrefetch = 8;

template <typename E>
__global__ __launch_bounds__(kThreads) void k_state_passing(
    E *__restrict__ states, const float *__restrict__ cs, const float *__restrict__ init,
    float *__restrict__ final_states, const int32_t *__restrict__ seq_idx,
    int T, int H, int64_t PN, int nc, int Q, int64_t total_vecs)
{
    constexpr int V = kVec16<E>;
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (gid >= total_vecs) return;
    const int64_t vecs_per_head = PN / V;
    const int64_t e0 = (gid % vecs_per_head) * V;
    const int64_t bh = gid / vecs_per_head;
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    float hs[V];
    if (init) {
#pragma unroll
        for (int v = 0; v < V; v += 4) load16_f32(init + bh * PN + e0 + v, hs + v);
    } else {
#pragma unroll
        for (int v = 0; v < V; ++v) hs[v] = 0.f;
    }
    const float *lam_ptr = cs + bh * (int64_t)nc * Q + (Q - 1);
    const int64_t cstride = (int64_t)H * PN;
    E *base = states + (b * nc * H + h) * PN + e0;
    for (int c0 = 0; c0 < nc; c0 += kPrefetch) {
        float sv[kPrefetch][V];
#pragma unroll
        for (int k = 0; k < kPrefetch; ++k)
            if (c0 + k < nc) load16_f32(base + (int64_t)(c0 + k) * cstride, sv[k]);
#pragma unroll
        for (int k = 0; k < kPrefetch; ++k) {
            const int c = c0 + k;
            if (c < nc) {
                store16_f32(base + (int64_t)c * cstride, hs);
                const float d = exp_neg(lam_ptr[(int64_t)c * Q]);
                bool keep = true;
                if (seq_idx) {
                    const int last = min(c * Q + Q, T) - 1;
                    keep = seq_idx[last] == seq_idx[c > 0 ? c * Q - 1 : 0];
                }
#pragma unroll
                for (int v = 0; v < V; ++v) hs[v] = (keep ? d * hs[v] : 0.f) + sv[k][v];
            }
        }
    }
    if (final_states) {
#pragma unroll
        for (int v = 0; v < V; v += 4) store16_f32(final_states + bh * PN + e0 + v, hs + v);
    }
}

// ---------------------------------------------------------------------------
// Packed streams: segment ends and per-segment final states
// ---------------------------------------------------------------------------
__global__ void k_seg_end_init(int32_t *seg_end, int nseq)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < nseq) seg_end[i] = -1;
}

// seg_end[s] = last position of segment id s (ids outside [0, nseq) are ignored).
__global__ void k_seg_end(const int32_t *__restrict__ seq_idx, int32_t *__restrict__ seg_end, int T, int nseq)
{
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T) return;
    const int s = seq_idx[t];
    if ((t == T - 1 || seq_idx[t + 1] != s) && s >= 0 && s < nseq) seg_end[s] = t;
}

// final_states[sg,h,p,n] = state right after segment sg's last token t_e:
//   sum_{s in t_e's chunk, s <= t_e, seq_s = sg} exp(cs_te - cs_s) delta_s x_s[p] B_s[n]
//   + [the segment was already open when the chunk started] exp(cs_te) Hin_c[p][n].
// An id that never occurs gets zeros.
template <typename E, int Q>
__global__ __launch_bounds__(kThreads) void k_seq_final(
    const E *__restrict__ x, const E *__restrict__ Bm, const float *__restrict__ delta,
    const float *__restrict__ cs, const int32_t *__restrict__ seq_idx, const E *__restrict__ hin,
    const int32_t *__restrict__ seg_end, float *__restrict__ final_states,
    int T, int H, int G, int P, int N, int nc, int nseq, int ntp, int ntn)
{
    constexpr int PITCH = Q + kVec16<E>;
    __shared__ __align__(16) E xt[64 * PITCH];
    __shared__ __align__(16) E bt[64 * PITCH];
    __shared__ float w[Q];
    __shared__ int m[Q];
    const int units = nseq * H * ntp * ntn;
    const int u = xcd_remap(blockIdx.x, units);
    int r = u;
    const int tn = r % ntn; r /= ntn;
    const int tp = r % ntp; r /= ntp;
    const int h = r % H;
    const int sg = r / H;
    const int g = h / (H / G);
    const int p0 = tp * 64, n0 = tn * 64;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
    const int wn = wave >> 1, wp = wave & 1;
    float *out = final_states + ((int64_t)sg * H + h) * (int64_t)P * N;
    const int te = seg_end[sg];
    if (te < 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int n = n0 + wn * 32 + i * 16 + 4 * lg, p = p0 + wp * 32 + j * 16 + li;
                float z[4] = {0.f, 0.f, 0.f, 0.f};
                if (p < P && n < N) store4_f32(out + (int64_t)p * N + n, z);
            }
        return;
    }
    const int c = te / Q, t0 = c * Q, ie = te - t0;
    const int64_t cso = ((int64_t)h * nc + c) * Q;   // batch is 1 with seq_idx
    const float cse = cs[cso + ie];
    for (int s = threadIdx.x; s < Q; s += kThreads) {
        const bool keep = s <= ie && seq_idx[t0 + s] == sg;
        m[s] = keep;
        w[s] = keep ? exp_neg(cse - cs[cso + s]) * delta[cso + s] : 0.f;
    }
    __syncthreads();
    stage_transposed<E, Q, true>(xt, x + ((int64_t)t0 * H + h) * P + p0, (int64_t)H * P, ie + 1, P - p0, w, m);
    stage_transposed<E, Q, false>(bt, Bm + ((int64_t)t0 * G + g) * N + n0, (int64_t)G * N, ie + 1, N - n0,
                                  nullptr, nullptr);
    __syncthreads();
    floatx4 acc[2][2] = {};
    state_mma<E, Q>(bt, xt, acc, (ie + 1 + 31) & ~31);

    const bool carry = seq_idx[c > 0 ? t0 - 1 : 0] == sg;
    const float dcar = exp_neg(cse);
    const E *hc = hin + ((int64_t)c * H + h) * (int64_t)P * N;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + wn * 32 + i * 16 + 4 * lg, p = p0 + wp * 32 + j * 16 + li;
            if (p < P && n < N) {
                float hv[4] = {0.f, 0.f, 0.f, 0.f};
                if (carry) load4_f32(hc + (int64_t)p * N + n, hv);
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
// One workgroup per (b, c, h, 64-p tile).  The chunk's Q output rows are split
// into 16-row sub-blocks j (t0 = 16 j); wave w owns j = w, w+4, ... so the
// causal work is balanced.  Everything is computed transposed, D[p][t], so the
// per-head decay enters as a per-column (per-lane) scale:
//   y_t = u_t [ e_{t0} (C_t . Hin) + sum_{s < S_j} CB[t][s] V_j[s] x_s ]
//         + sum_{S_j <= s <= t} CB[t][s] exp(cs_t - cs_s) delta_s x_s  + D x_t
// with e_{t0} = exp(cs_{t0}), u_t = exp(cs_t - cs_{t0}), V_j[s] = exp(cs_{t0} -
// cs_s) delta_s, and S_j = 32 floor(j/2) the start of the 32-wide K step that
// holds t0.  Every factor is a decay <= 1, so nothing overflows, and the
// per-element exponentials are needed only on the diagonal step.  Segment
// masks (packed streams) are selects on the same factors.
template <typename E, int Q>
__global__ __launch_bounds__(kThreads) void k_chunk_scan(
    const E *__restrict__ x, const E *__restrict__ Cm, const float *__restrict__ delta,
    const float *__restrict__ cs, const E *__restrict__ cb, const E *__restrict__ hin,
    const float *__restrict__ D, const int32_t *__restrict__ seq_idx, E *__restrict__ y,
    int T, int H, int G, int P, int N, int nc, int ntp)
{
    using F = frag_t<E>;
    constexpr int V = kVec16<E>;
    constexpr int XP = Q + V;     // pitch of the x^T tile
    constexpr int NJ = Q / 16;    // 16-row sub-blocks per chunk
    constexpr int NSB = Q / 64;   // sub-blocks per wave
    __shared__ __align__(16) E xt[64 * XP];
    __shared__ __align__(16) float vt[NJ * Q];
    __shared__ float csb[Q], db[Q];
    __shared__ int sq[Q];
    extern __shared__ __align__(16) char dyn_smem[];
    E *hs = reinterpret_cast<E *>(dyn_smem);   // entering state tile [64 p][N], pitch N + V
    const int HP = N + V;

    const int units = nc * H * ntp;
    const int u = xcd_remap(blockIdx.x, units);
    const int b = blockIdx.y;
    const int tp = u % ntp;
    const int h = (u / ntp) % H;
    const int c = u / (ntp * H);
    const int g = h / (H / G);
    const int t0 = c * Q, len = min(Q, T - t0);
    const int p0 = tp * 64;
    const int64_t cso = (((int64_t)b * H + h) * nc + c) * Q;

    for (int i = threadIdx.x; i < Q; i += kThreads) {
        csb[i] = cs[cso + i];
        db[i] = delta[cso + i];
        sq[i] = seq_idx ? seq_idx[t0 + min(i, len - 1)] : 0;
    }
    const int seq_prev = seq_idx ? seq_idx[c > 0 ? t0 - 1 : 0] : 0;
    {
        const E *src = hin + ((((int64_t)b * nc + c) * H + h) * P + p0) * (int64_t)N;
        const int vpr = N / V;
        for (int idx = threadIdx.x; idx < 64 * vpr; idx += kThreads) {
            const int pr = idx / vpr, nv = idx % vpr;
            uint4 v = {0u, 0u, 0u, 0u};
            if (p0 + pr < P) v = *reinterpret_cast<const uint4 *>(src + (int64_t)pr * N + nv * V);
            *reinterpret_cast<uint4 *>(hs + pr * HP + nv * V) = v;
        }
    }
    stage_transposed<E, Q, false>(xt, x + (((int64_t)b * T + t0) * H + h) * P + p0, (int64_t)H * P, len,
                                  P - p0, nullptr, nullptr);
    __syncthreads();
    for (int idx = threadIdx.x; idx < NJ * Q; idx += kThreads) {
        const int j = idx / Q, s = idx % Q;
        if (s < 32 * (j >> 1)) {
            const int tj = 16 * j;
            const bool keep = sq[s] == sq[tj];
            vt[idx] = keep ? exp_neg(csb[tj] - csb[s]) * db[s] : 0.f;
        }
    }
    __syncthreads();

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
    floatx4 acc[NSB][4];
    const E *crow[NSB];
    const E *cbrow[NSB];
    bool tval[NSB];
    const E *cbase = cb + (((int64_t)b * nc + c) * G + g) * (int64_t)Q * Q;
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
        const int t = 16 * (wave + 4 * k) + li;
        tval[k] = t < len;
        crow[k] = Cm + (((int64_t)b * T + t0 + (tval[k] ? t : 0)) * G + g) * N;
        cbrow[k] = cbase + (int64_t)t * Q;
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) acc[k][pb] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    // step 4 part: Hin C^T over n
    for (int k0 = 0; k0 < N; k0 += 32) {
        const int kk = k0 + 8 * lg;
        const bool kin = kk < N;
        F a[4];
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) a[pb] = kin ? load_frag(hs + (pb * 16 + li) * HP + kk) : F{};
#pragma unroll
        for (int k = 0; k < NSB; ++k) {
            if (16 * (wave + 4 * k) >= len) continue;
            const F bf = (tval[k] && kin) ? load_frag(crow[k] + kk) : F{};
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) mma(acc[k][pb], a[pb], bf);
        }
    }
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
        const int tj = 16 * (wave + 4 * k);
        const bool mo = !seq_idx || sq[tj] == seq_prev;
        const float e0 = exp_neg(csb[tj]);
#pragma unroll
        for (int pb = 0; pb < 4; ++pb)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[k][pb][q] = mo ? acc[k][pb][q] * e0 : 0.f;
    }

    // step 1, K steps strictly below each sub-block's diagonal step
    for (int ks = 0; ks < (NJ - 1) / 2; ++ks) {
        F a[4];
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) a[pb] = load_frag(xt + (pb * 16 + li) * XP + ks * 32 + 8 * lg);
#pragma unroll
        for (int k = 0; k < NSB; ++k) {
            const int j = wave + 4 * k;
            if (ks >= (j >> 1) || 16 * j >= len) continue;
            const floatx8 cf = to_f32(load_frag(cbrow[k] + ks * 32 + 8 * lg));
            const float *vrow = vt + j * Q + ks * 32 + 8 * lg;
            const floatx4 v0 = *reinterpret_cast<const floatx4 *>(vrow);
            const floatx4 v1 = *reinterpret_cast<const floatx4 *>(vrow + 4);
            const floatx8 vv = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
            const F wfr = from_f32<F>(cf * vv);
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) mma(acc[k][pb], a[pb], wfr);
        }
    }
    // u_t scale, then the diagonal K step with per-element decays
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
        const int j = wave + 4 * k;
        if (16 * j >= len) continue;
        const int tj = 16 * j, t = tj + li;
        const bool keep = sq[t] == sq[tj];
        const float ut = exp_neg(csb[t] - csb[tj]);
#pragma unroll
        for (int pb = 0; pb < 4; ++pb)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[k][pb][q] = keep ? acc[k][pb][q] * ut : 0.f;

        const int ks = j >> 1;
        const floatx8 cf = to_f32(load_frag(cbrow[k] + ks * 32 + 8 * lg));
        floatx8 wf;
        const float cst = csb[t];
        const int sqt = sq[t];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int s = ks * 32 + 8 * lg + e;
            const bool ok = s <= t && sq[s] == sqt;
            wf[e] = ok ? cf[e] * exp_neg(cst - csb[s]) * db[s] : 0.f;
        }
        const F wfr = from_f32<F>(wf);
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) {
            const F a = load_frag(xt + (pb * 16 + li) * XP + ks * 32 + 8 * lg);
            mma(acc[k][pb], a, wfr);
        }
    }

    // epilogue: + D x, store y (4 consecutive p of one t per lane)
    const float Dh = D ? D[h] : 0.f;
#pragma unroll
    for (int k = 0; k < NSB; ++k) {
        const int t = 16 * (wave + 4 * k) + li;
        if (t >= len) continue;
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) {
            const int p = p0 + pb * 16 + 4 * lg;
            if (p >= P) continue;
            const int64_t off = (((int64_t)b * T + t0 + t) * H + h) * P + p;
            float xv[4], o[4];
            load4_f32(x + off, xv);
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = acc[k][pb][q] + Dh * xv[q];
            store4_f32(y + off, o);
        }
    }
}

// final_states for an empty sequence: a copy of the initial state (or zeros).
__global__ void k_fill_final(float *__restrict__ out, const float *__restrict__ init, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = init ? init[i] : 0.f;
}

}  // namespace ssd
