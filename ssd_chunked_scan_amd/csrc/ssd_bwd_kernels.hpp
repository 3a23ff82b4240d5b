// ssd_bwd_kernels.hpp -- device code of the backward pass (gradients of the chunked
// SSD forward) for gfx950.
//
// The backward is the chain rule applied to the recurrence h_t = a_t h_{t-1} +
// Delta_t x_t B_t^T, y_t = h_t C_t + D x_t (section 3.1 of "Mamba 2 --
// Transformers are SSMs"), organised by chunks like the forward (section 4.1 of
// that page; "SSM 家族全景图（下）" section 3.4).  With g_t = dL/dh_t and, per
// chunk c, G_c = dL/d(state after chunk c):
//
//   y'_s  = g_s B_s = sum_{t >= s in c} exp(cs_t - cs_s) (C_t . B_s) dy_t
//                     + exp(cs_last - cs_s) G_c B_s              (anti-causal scan)
//   dx_s  = Delta_s y'_s + D dy_s
//   U_c   = sum_{t in c} exp(cs_t) dy_t C_t^T,  G_{c-1} = exp(cs_last(c)) G_c + U_c,
//   dinit = exp(cs_last(0)) G_0 + U_0                            (reverse state scan)
//   M[t][s] = sum_{heads of the group} exp(cs_t - cs_s) Delta_s (dy_t . x_s), s <= t
//   dC_t  = sum_s M[t][s] B_s + sum_h exp(cs_t) Hin_c^T dy_t
//   dB_s  = sum_t M[t][s] C_t + sum_h Delta_s exp(cs_last - cs_s) G_c^T x_s
//   dl_k  = a_k <g_k, h_{k-1}>  (l_k = Delta_k A, the log-decay), for k in chunk c:
//         = sum_{t >= k > s in c} S[t][s] + sum_{t >= k} dy_t . yoff_t
//           + sum_{s < k} Delta_s x_s . y'off_s + e^{cs_last} <G_c, Hin_c>
//     where S[t][s] = e^{cs_t - cs_s} Delta_s (dy_t . x_s) (C_t . B_s) is the
//     contribution of source s to dy_t . y_t, yoff / y'off the entering-state
//     terms of y / y';
//   dDelta_t = A dl_t + x_t . y'_t,   ddt_t = dDelta_t * sigmoid(dt_t) (softplus)
//   dA = sum_t Delta_t dl_t,   dD = sum_t dy_t . x_t
//
// The first sum of dl is the suffix sum of (row sums - column sums) of S inside
// the chunk, every term in fp32 from the same S, so no per-token state is ever
// stored and no rounded output is differenced.  The anti-causal scan runs on the
// forward's chunk_scan kernel with every chunk's tokens in reversed order; the
// kernels read dy, B, C and cs in that order themselves, so nothing is copied
// reversed.
#pragma once

#include "ssd_kernels.hpp"

namespace ssd {

// ---------------------------------------------------------------------------
// packed streams: a layout in which every segment starts at a chunk start
// ---------------------------------------------------------------------------
// The backward of a packed stream runs on a layout in which every segment
// occupies whole chunks: segment s (in id order) starts at padded position
// pstart[s], a multiple of Q, and is followed by padding up to the next
// multiple of Q.  Padding tokens have x = B = C = dy = 0 and a step size of
// zero, so they leave the state unchanged and contribute nothing; the state
// carry is cut where a chunk starts a new segment.  Positions past the last
// segment form chunks of no segment (id -1).  The layout is never built: each
// chunk reads its tokens from the caller's stream through a chunk map (first
// token, count; see chunk_rows), its positions past the count read as zero,
// and its gradients are written straight to the tokens' own rows.

// From seg_end (the last position of every id, -1 for an id that never occurs;
// ids never decrease along the stream): ostart[s] = the first position of s,
// len[s] its token count, pstart[s] its start in the padded layout.  One wave,
// ids in blocks of 64 with running carries.
__global__ void k_bwd_seg_ranges(const int32_t *__restrict__ seg_end, int32_t *__restrict__ ostart,
                                 int32_t *__restrict__ len, int32_t *__restrict__ pstart, int nseq, int Q)
{
    const int lane = threadIdx.x;
    int end_before = -1;   // the largest last position of the ids below the block
    int64_t pad_before = 0;
    for (int base = 0; base < nseq; base += 64) {
        const int s = base + lane;
        const int e = s < nseq ? seg_end[s] : -1;
        // inclusive max-scan of e and sum-scan of the padded lengths over the block
        int mx = e;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int u = __shfl_up(mx, o);
            if (lane >= o) mx = max(mx, u);
        }
        const int up = __shfl_up(mx, 1);
        const int first = 1 + max(end_before, lane > 0 ? up : -1);   // one past every earlier id's end
        const int n = e >= 0 ? e - first + 1 : 0;
        int64_t pad = (int64_t)((n + Q - 1) / Q) * Q;
        int64_t ps = pad;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int64_t u = __shfl_up(ps, o);
            if (lane >= o) ps += u;
        }
        if (s < nseq) {
            ostart[s] = first;
            len[s] = n;
            pstart[s] = (int32_t)(pad_before + ps - pad);
        }
        end_before = max(end_before, __shfl(mx, 63));
        pad_before += __shfl(ps, 63);
    }
}

// For every chunk c of the padded stream: cseg[c] = its segment (-1 past the
// last segment) and cmap[c] = (its first token in the caller's stream, its
// token count), (0, 0) for a chunk of padding only.  The segment of chunk c is
// the last id whose padded start is <= c Q (a binary search; an id without
// tokens has the same start as the next one).
__global__ void k_bwd_chunk_map(const int32_t *__restrict__ ostart, const int32_t *__restrict__ len,
                                const int32_t *__restrict__ pstart, int32_t *__restrict__ cseg,
                                int2 *__restrict__ cmap, int nseq, int Q, int ncp)
{
    const int c = blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= ncp) return;
    const int pp = c * Q;
    int lo = 0, hi = nseq - 1;   // the last s with pstart[s] <= pp (pstart[0] = 0)
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pstart[mid] <= pp) lo = mid;
        else hi = mid - 1;
    }
    const int off = pp - pstart[lo], n = len[lo];
    const int padded = (n + Q - 1) / Q * Q;
    if (off < padded) {
        cseg[c] = lo;
        cmap[c] = make_int2(ostart[lo] + off, min(Q, n - off));
    } else {
        cseg[c] = -1;
        cmap[c] = make_int2(0, 0);
    }
}

// The gradient state slot of the chunk right after segment sg's chunks in the
// padded stream (U_c, c = (pstart[sg] + len[sg] rounded up to Q) / Q: the first
// chunk of the next segment or of the trailing padding, where the reverse scan
// does not read U_c) takes sg's final-state gradient, zero without dfinal: the
// reverse scan restarts from that slot.  Segments without tokens own no chunk,
// and the last one's gradient enters the scan as its start instead when no chunk
// follows it.  nb blocks of 256 threads per segment (ceil(H*PN/4/256)), four
// elements per thread.
template <typename E>
__global__ void k_bwd_inject_dfinal(E *__restrict__ gstates, const float *__restrict__ dfinal,
                                    const int32_t *__restrict__ pstart, const int32_t *__restrict__ len, int H,
                                    int64_t PN, int nc, int Q, int nb)
{
    const int sg = blockIdx.x / nb, blk = blockIdx.x % nb;
    const int n = len[sg];
    if (n <= 0) return;   // uniform
    const int c = (pstart[sg] + (n + Q - 1) / Q * Q) / Q;
    if (c >= nc) return;
    const int64_t i = ((int64_t)blk * blockDim.x + threadIdx.x) * 4;
    if (i >= (int64_t)H * PN) return;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (dfinal) load4_f32(dfinal + (int64_t)sg * H * PN + i, v);
    store4_f32(gstates + (int64_t)c * H * PN + i, v);
}

// ---------------------------------------------------------------------------
// per (b, h): dl, ddt, and the dA / dD partial sums
// ---------------------------------------------------------------------------
// Inside chunk c (l_k enters through cs_j for j >= k in the chunk, and through
// the chunk's total decay):
//   dl_k = sum_{j >= k} (r_j - c_j + yo_j) + sum_{s < k} Delta_s zo_s + bnd_c
// with r_j / c_j the row / column sums of S (k_bwd_m), yo_j = dy_j . (entering-
// state term of y_j), zo_s = x_s . (the G_c term of y'_s), bnd_c = e^{cs_last}
// <G_c, Hin_c> (summed here from the nbp partials the reverse state scan left in
// bnd_part).  Then dDelta = A dl + x . y' and ddt = dDelta * sigmoid(dt).
// One wave per (b, h, c); lane l holds the tokens l*per .. l*per + per - 1 (per =
// Q/64); the scans run in fp64; dA and dD partials go to [b,H,nc].
__device__ __forceinline__ double wave_incl_scan(double v)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double u = __shfl_up(v, o);
        if (lane >= o) v += u;
    }
    return v;
}

template <typename E, int Q>
__global__ __launch_bounds__(kThreads) void k_bwd_dl(
    const float *__restrict__ rpart, const float *__restrict__ cpart, const float *__restrict__ yo,
    const float *__restrict__ zo, const float *__restrict__ xyp, const float *__restrict__ bnd_part,
    const float *__restrict__ dyx, const float *__restrict__ delta, const E *__restrict__ dt,
    const float *__restrict__ A, E *__restrict__ ddt, float *__restrict__ dA_part, float *__restrict__ dD_part, int T,
    int H, int nc, int ntp, int64_t rows, int softplus, int64_t nbp, const int32_t *__restrict__ cseg = nullptr,
    const int2 *__restrict__ cmap = nullptr)
{
    constexpr int per = Q / 64, QT = Q / 64;
    const int64_t wid = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);   // (b * H + h) * nc + c
    if (wid >= rows) return;   // whole wave
    const int lane = threadIdx.x & 63;
    const bool small = rows < (1 << 23);
    int bh32, c, b, h;
    udivmod((int)wid, nc, small, bh32, c);
    if (cseg && cseg[c] < 0) {   // a chunk of padding only: nothing of it enters dA or dD
        if (lane == 0) {
            dA_part[wid] = 0.f;
            dD_part[wid] = 0.f;
        }
        return;
    }
    udivmod(bh32, H, small, b, h);
    const int64_t slice = rows * Q;   // one tile / p-tile slice: [b,H,nc,Q]
    const float Ah = A[h];
    int t0, len;
    chunk_rows(c, Q, T, cmap, t0, len);
    const int64_t row = wid * Q;
    // Every value this lane needs is requested before any arithmetic (the
    // token loops unroll at compile time), so the wave waits for memory once:
    // the tile row sums of S (tiles si <= the token's tile), the column sums
    // (tiles ti >= it), the p-tile partials of the dot products, the step
    // sizes, dt and the boundary-term partials.
    float rv[per][QT], cv[per][QT], dlt[per], dtv[per];
    double y1v[per], z1v[per], xyv[per], dyv[per];
#pragma unroll
    for (int e = 0; e < per; ++e) {
        const int j = lane * per + e;
        const bool in = j < len;
        const int64_t o = row + j;
#pragma unroll
        for (int q = 0; q < QT; ++q) {
            rv[e][q] = in && q <= j / 64 ? rpart[q * slice + o] : 0.f;
            cv[e][q] = in && q >= j / 64 ? cpart[q * slice + o] : 0.f;
        }
        y1v[e] = in ? yo[o] : 0.f;
        z1v[e] = in ? zo[o] : 0.f;
        xyv[e] = in ? xyp[o] : 0.f;
        dyv[e] = in ? dyx[o] : 0.f;
        dlt[e] = in ? delta[o] : 0.f;
        dtv[e] = in && softplus ? to_float(dt[((int64_t)b * T + t0 + j) * H + h]) : 0.f;
    }
    float bv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) bv[i] = lane + 64 * i < nbp ? bnd_part[wid * nbp + lane + 64 * i] : 0.f;
    double bsum = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) bsum += bv[i];
    for (int64_t i = lane + 256; i < nbp; i += 64) bsum += bnd_part[wid * nbp + i];
    // further p tiles of the dot products (P > 64)
    for (int tp = 1; tp < ntp; ++tp)
#pragma unroll
        for (int e = 0; e < per; ++e) {
            const int j = lane * per + e;
            if (j >= len) continue;
            const int64_t o = tp * slice + row + j;
            y1v[e] += yo[o];
            z1v[e] += zo[o];
            xyv[e] += xyp[o];
            dyv[e] += dyx[o];
        }
    double av[per], zv[per];
    double asum = 0.0, zsum = 0.0;
#pragma unroll
    for (int e = 0; e < per; ++e) {
        double r = 0.0, cc = 0.0;
#pragma unroll
        for (int q = 0; q < QT; ++q) {
            r += rv[e][q];
            cc += cv[e][q];
        }
        av[e] = r - cc + y1v[e];
        zv[e] = dlt[e] * z1v[e];
        asum += av[e];
        zsum += zv[e];
    }
    // suffix sums of a (inclusive) and prefix sums of z (exclusive) over the chunk
    const double ain = wave_incl_scan(asum), zin = wave_incl_scan(zsum), bin = wave_incl_scan(bsum);
    const double atot = __shfl(ain, 63);
    double asuf = atot - ain + asum;   // sum of a over this lane's tokens and all later lanes
    double zpre = zin - zsum;          // sum of z over earlier lanes
    const double b0 = __shfl(bin, 63);
    double sa = 0.0, sd = 0.0;
#pragma unroll
    for (int e = 0; e < per; ++e) {
        const int j = lane * per + e;
        if (j < len) {
            const double dl = asuf + zpre + b0;
            const float dd = Ah * (float)dl + (float)xyv[e];
            float gr = dd;
            if (softplus) gr = dd / (1.f + __builtin_amdgcn_exp2f(-dtv[e] * kLog2e));   // dDelta * sigmoid(dt)
            ddt[((int64_t)b * T + t0 + j) * H + h] = from_float<E>(gr);
            sa += (double)dlt[e] * dl;
            sd += dyv[e];
        }
        asuf -= av[e];
        zpre += zv[e];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        sa += __shfl_xor(sa, o);
        sd += __shfl_xor(sd, o);
    }
    if (lane == 0) {
        dA_part[wid] = (float)sa;
        dD_part[wid] = (float)sd;
    }
}

// dA[h] = sum over (b, c) of dA_part[b, h, c], dD[h] likewise, one wave per head
// (a fixed order, so deterministic).
__global__ void k_bwd_sum_heads(const float *__restrict__ dA_part, const float *__restrict__ dD_part,
                                float *__restrict__ dA, float *__restrict__ dD, int batch, int H, int nc)
{
    const int h = blockIdx.x, lane = threadIdx.x;
    double a = 0.0, d = 0.0;
    for (int b = 0; b < batch; ++b)
        for (int c = lane; c < nc; c += 64) {
            const int64_t i = ((int64_t)b * H + h) * nc + c;
            a += dA_part[i];
            d += dD_part[i];
        }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        a += __shfl_xor(a, o);
        d += __shfl_xor(d, o);
    }
    if (lane == 0) {
        dA[h] = (float)a;
        if (dD) dD[h] = (float)d;
    }
}

// ---------------------------------------------------------------------------
// M[t][s] = sum over the group's heads of exp(cs_t - cs_s) Delta_s (dy_t . x_s)
// ---------------------------------------------------------------------------
// One workgroup per 64 x 64 (t, s) tile with s-tile <= t-tile of one (b, c, g).
// Each head's dy rows (t) and x rows (s) are staged in LDS 64 columns p at a
// time (the next step's rows are loaded into registers while the current step
// computes); each wave forms its 32 x 32 part of dy x^T with the matrix cores
// and adds it to the total with the exact per-element decay and step size, so
// no factor can overflow.  The tile is written twice, as M (rows t) and as M^T
// (rows s), each [b,nc,G,Q,Q] in E, so that both consumers read 16-byte
// fragments.  Entries with s > t, t >= len or s >= len are zero.
//
// The same per-head products give the intra-chunk part of the log-decay
// gradient: with S_h[t][s] = W_h[t][s] CB[t][s] (W_h the head's term of M, so S
// is exactly the contribution of source s to dy_t . y_t), each head's row sums
// rpart[si][t] = sum_{s in tile si} S[t][s] and column sums cpart[ti][s] = sum_{t
// in tile ti} S[t][s] are written per tile ([QT][b,H,nc,Q] fp32 each); rows and
// columns come from one S, so their difference cancels exactly where it should.
// Split over heads (hsplit > 1, grid x = ntiles * hsplit): workgroup (tile, k)
// takes the heads k*hpg/hsplit .. (k+1)*hpg/hsplit - 1 of the group and writes its
// partial sum of M as one fp32 64 x 64 tile (rows t) to mpart[k][tile unit]
// instead of mrow / mcol; k_bwd_m_reduce adds the parts in a fixed order.  The
// row and column sums are per head and go out as before.
template <typename E, int Q, int NT>
__global__ __launch_bounds__(kThreads) void k_bwd_m(
    const E *__restrict__ dy, const E *__restrict__ x, const float *__restrict__ delta, const float *__restrict__ cs,
    const E *__restrict__ cbuf, E *__restrict__ mrow, E *__restrict__ mcol, float *__restrict__ rpart,
    float *__restrict__ cpart, int T, int H, int G, int P, int nc, int hsplit, float *__restrict__ mpart,
    const int32_t *__restrict__ cseg = nullptr, const int2 *__restrict__ cmap = nullptr)
{
    using F = frag_t<E>;
    constexpr int V = kVec16<E>, ES = (int)sizeof(E);
    constexpr int QT = Q / 64, NTRI = QT * (QT + 1) / 2;
    constexpr int PITCH = 64 + 2 * V;   // rows 32 bytes past a multiple of 256 (bf16): conflict-free reads
    constexpr int VPR = 64 / V, RPP = kThreads / VPR, NPASS = 64 / RPP;
    __shared__ __align__(16) E ts[64 * PITCH];
    __shared__ __align__(16) E ss[64 * PITCH];
    __shared__ float stage[64 * 65];
    __shared__ float rsum[64], csum[64];
    __shared__ float hcs[2][64], hds[64];   // the head's cs at the t rows / s rows, delta at the s rows
    const int units = NTRI * nc * G;
    const int uu = xcd_remap(blockIdx.x, units * hsplit);
    const bool small = units * hsplit < (1 << 23);
    int u, sp;   // the split's workgroups sit next to each other
    udivmod(uu, hsplit, small, u, sp);
    const int b = blockIdx.y;
    int tile = u % NTRI;
    int c, g;
    udivmod(u / NTRI, G, small, c, g);
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
    const int hpg_all = H / G, PC = (P + 63) / 64;
    const int h_lo = sp * hpg_all / hsplit, hpg = (sp + 1) * hpg_all / hsplit - h_lo;   // this split's heads
    const int steps = hpg * PC;
    const int hv = threadIdx.x % VPR, hr = threadIdx.x / VPR;
    const int trows = min(64, len - ti * 64), srows = min(64, len - si * 64);

    uint4 rt[NPASS], rs[NPASS];
    float hval = 0.f;   // this thread's element of the next head's cs / delta rows (threads < 192)
    // Formed once (the loop only moves pointers by constant strides: all waves
    // of a CU share one scalar unit, and per-step 64-bit index products bound
    // this kernel): the first head's dy / x rows, buffer ranges, lane offsets.
    const int64_t ld = (int64_t)H * P;
    const int h0 = g * hpg_all + h_lo;
    const E *dy_ptr = dy + (((int64_t)b * T + t0 + ti * 64) * H + h0) * P;
    const E *x_ptr = x + (((int64_t)b * T + t0 + si * 64) * H + h0) * P;
    auto range = [&](int rows, int cols) { return rsrc_bytes(rows > 0 ? ((int64_t)(rows - 1) * ld + cols) * ES : 0); };
    const int ptail = P - (PC - 1) * 64;   // columns of the last p chunk
    const int tr_full = range(trows, 64), tr_tail = range(trows, ptail);
    const int sr_full = range(srows, 64), sr_tail = range(srows, ptail);
    uint32_t loff[NPASS];
#pragma unroll
    for (int i = 0; i < NPASS; ++i) loff[i] = (uint32_t)(((int64_t)(hr + i * RPP) * ld + hv * V) * ES);
    const int64_t hrow = (int64_t)nc * Q;
    // the cs / delta element this thread stages for each head (threads < 192)
    const float *hv_ptr = nullptr;
    if (threadIdx.x < 192) {
        const int part = threadIdx.x >> 6, e = threadIdx.x & 63;
        const int pos = (part == 0 ? ti : si) * 64 + e;
        hv_ptr = pos < len ? (part == 2 ? delta : cs) + (((int64_t)b * H + h0) * nc + c) * Q + pos : nullptr;
    }
    int ipc = 0;   // the p chunk of the next step issued
    auto issue = [&]() {
        if (ipc == 0 && threadIdx.x < 192) {
            hval = hv_ptr ? *hv_ptr : 0.f;
            if (hv_ptr) hv_ptr += hrow;
        }
        const bool last = ipc == PC - 1;
        const auto trs = make_rsrc_n(dy_ptr, last ? tr_tail : tr_full);
        const auto srs = make_rsrc_n(x_ptr, last ? sr_tail : sr_full);
        const bool cin = hv * V < P - ipc * 64;
#pragma unroll
        for (int i = 0; i < NPASS; ++i) {
            const uint32_t o = cin ? loff[i] : kOffNone;
            rt[i] = bload16(trs, o);
            rs[i] = bload16(srs, o);
        }
        if (last) {
            ipc = 0;
            dy_ptr += P - (PC - 1) * 64;
            x_ptr += P - (PC - 1) * 64;
        } else {
            ++ipc;
            dy_ptr += 64;
            x_ptr += 64;
        }
    };

    const int t_w = (wave >> 1) * 32, s_w = (wave & 1) * 32;
    floatx4 tot[2][2] = {}, acc[2][2] = {};
    // CB[t][s] of this lane's 16 elements, from the fragment-major CB of the chunk
    const E *cbg = cbuf + (((int64_t)b * nc + c) * G + g) * cb_group_elems<Q, NT>();
    float cbv[2][2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = ti * 64 + t_w + 16 * i + 4 * lg + r, s = si * 64 + s_w + 16 * j + li;
                const int64_t idx = ((int64_t)((t >> 4) * (Q / 32) + (s >> 5)) * 64 + (t & 15) + 16 * ((s & 31) >> 3)) * 8 + (s & 7);
                cbv[i][j][r] = to_float(cbg[idx]);
            }
    const int64_t bhnc = (int64_t)gridDim.y * H * nc * Q;   // one tile slice of rpart / cpart
    // this thread's row (threads < 64) or column (64..127) sum slot of the first
    // head; one head further is hrow further
    float *sum_ptr = nullptr;
    if (threadIdx.x < 128) {
        const int64_t row = (((int64_t)b * H + h0) * nc + c) * Q;
        sum_ptr = threadIdx.x < 64 ? rpart + si * bhnc + row + ti * 64 + threadIdx.x
                                   : cpart + ti * bhnc + row + si * 64 + (threadIdx.x - 64);
    }
    auto flush = [&]() {   // the finished head's row / column sums to memory, then cleared
        if (threadIdx.x < 64) {
            *sum_ptr = rsum[threadIdx.x];
            rsum[threadIdx.x] = 0.f;
        } else if (threadIdx.x < 128) {
            *sum_ptr = csum[threadIdx.x - 64];
            csum[threadIdx.x - 64] = 0.f;
        }
        if (threadIdx.x < 128) sum_ptr += hrow;
    };
    if (threadIdx.x < 64) rsum[threadIdx.x] = 0.f;
    else if (threadIdx.x < 128) csum[threadIdx.x - 64] = 0.f;
    issue();
    int kpc = 0;   // the p chunk of step k
    for (int k = 0; k < steps; ++k) {
        if (k > 0) __syncthreads();   // every wave is done reading the previous step's rows
        if (k > 0 && kpc == 0) flush();   // step k - 1 finished a head
#pragma unroll
        for (int i = 0; i < NPASS; ++i) {
            *reinterpret_cast<uint4 *>(ts + (hr + i * RPP) * PITCH + hv * V) = rt[i];
            *reinterpret_cast<uint4 *>(ss + (hr + i * RPP) * PITCH + hv * V) = rs[i];
        }
        if (kpc == 0 && threadIdx.x < 192) {
            const int part = threadIdx.x >> 6, e = threadIdx.x & 63;
            if (part == 2) hds[e] = hval;
            else hcs[part][e] = hval;
        }
        if (k + 1 < steps) issue();
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            F fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                fa[i] = load_frag(ts + (t_w + 16 * i + li) * PITCH + ks * 32 + 8 * lg);
                fb[i] = load_frag(ss + (s_w + 16 * i + li) * PITCH + ks * 32 + 8 * lg);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) mma(acc[i][j], fa[i], fb[j]);
        }
        const bool head_done = kpc == PC - 1;
        kpc = head_done ? 0 : kpc + 1;
        if (head_done) {
            // this head is complete: add it with its decays and step sizes, and
            // sum its S = W CB by rows and by columns
            float rs[2][4] = {}, cl[2] = {};
            if (si < ti && (ti + 1) * 64 <= len) {
                // a whole tile below the diagonal: W = e^{cs_t - ref} (Delta_s e^{ref - cs_s})
                // with ref = cs at the s tile's last row, so for A <= 0 (cs
                // non-increasing) both factors are at most 1 and none overflows
                const float ref = hcs[1][63];
                float at[2][4], bs[2];
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        at[i][r] = __builtin_amdgcn_exp2f((hcs[0][t_w + 16 * i + 4 * lg + r] - ref) * kLog2e);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    bs[j] = __builtin_amdgcn_exp2f((ref - hcs[1][s_w + 16 * j + li]) * kLog2e) * hds[s_w + 16 * j + li];
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float wv = acc[i][j][r] * at[i][r] * bs[j];
                            tot[i][j][r] += wv;
                            const float sv = wv * cbv[i][j][r];
                            rs[i][r] += sv;
                            cl[j] += sv;
                            acc[i][j][r] = 0.f;
                        }
            } else {
                // the diagonal tile or the ragged last one: the exact per-element
                // decay, and only s <= t < len.  Selects, not branches: an entry
                // outside takes a harmless exponent and contributes zero.
                float ht[2][4];
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) ht[i][r] = hcs[0][t_w + 16 * i + 4 * lg + r];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int s = si * 64 + s_w + 16 * j + li;
                    const float css = hcs[1][s_w + 16 * j + li], ds = hds[s_w + 16 * j + li];
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int t = ti * 64 + t_w + 16 * i + 4 * lg + r;
                            const bool in = s <= t && t < len;
                            float w = __builtin_amdgcn_exp2f((in ? ht[i][r] - css : -64.f) * kLog2e) * ds;
                            asm volatile("" : "+v"(w));   // keeps the compiler from branching around it
                            const float wv = in ? acc[i][j][r] * w : 0.f;
                            tot[i][j][r] += wv;
                            const float sv = wv * cbv[i][j][r];
                            rs[i][r] += sv;
                            cl[j] += sv;
                            acc[i][j][r] = 0.f;
                        }
                }
            }
            // Rows t (value m = 4 i + r) are summed over the 16 lanes li of a row
            // group, columns s (value j) over the 4 groups lg, each by halving
            // exchanges: at every step a lane keeps half of its values and adds
            // its partner's copy of that half.  The row partners are li ^ 8, li ^ 7,
            // li ^ 2 and li ^ 1 (DPP row rotate by 8, half-row mirror, and quad
            // permutes: register moves inside a 16-lane row, no LDS); each step's
            // partner differs in the bit that chose the kept half and agrees in the
            // bits chosen before, so the four steps cover all 16 lanes once.  In
            // the end lane li holds row value m = (li >> 1) & 7 and lane group lg
            // column value j = lg >> 1.
            float v8[8];
#pragma unroll
            for (int m = 0; m < 8; ++m) v8[m] = rs[m >> 2][m & 3];
            float v4[4], v2[2], v1, c1;
            {
                const bool up = li & 8;
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    v4[m] = (up ? v8[m + 4] : v8[m]) + dpp_mov<kDppRowRor8>(up ? v8[m] : v8[m + 4]);
            }
            {
                const bool up = li & 4;
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    v2[m] = (up ? v4[m + 2] : v4[m]) + dpp_mov<kDppRowHalfMirror>(up ? v4[m] : v4[m + 2]);
            }
            {
                const bool up = li & 2;
                v1 = (up ? v2[1] : v2[0]) + dpp_mov<kDppQuadXor2>(up ? v2[0] : v2[1]);
            }
            v1 += dpp_mov<kDppQuadXor1>(v1);
            {
                const bool up = lg & 2;
                c1 = (up ? cl[1] : cl[0]) + __shfl_xor(up ? cl[0] : cl[1], 32);
            }
            c1 += __shfl_xor(c1, 16);
            if ((li & 1) == 0) {
                const int m = (li >> 1) & 7;
                atomicAdd(&rsum[t_w + 16 * (m >> 2) + 4 * lg + (m & 3)], v1);
            }
            if ((lg & 1) == 0) atomicAdd(&csum[s_w + 16 * (lg >> 1) + li], c1);
        }
    }
    __syncthreads();
    flush();

    if (hsplit > 1) {
        // this split's part of the tile, fp32 rows t
        float *mp = mpart + ((int64_t)sp * gridDim.y * units + (int64_t)b * units + u) * 4096;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    mp[(t_w + 16 * i + 4 * lg + r) * 64 + s_w + 16 * j + li] = tot[i][j][r];
        return;
    }
    // M^T rows s: the four t of a lane are consecutive
    E *tcol = mcol + (((int64_t)b * nc + c) * G + g) * (int64_t)Q * Q;
    E *trow = mrow + (((int64_t)b * nc + c) * G + g) * (int64_t)Q * Q;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int s = si * 64 + s_w + 16 * j + li, t = ti * 64 + t_w + 16 * i + 4 * lg;
            const float o[4] = {tot[i][j][0], tot[i][j][1], tot[i][j][2], tot[i][j][3]};
            store4_f32(tcol + (int64_t)s * Q + t, o);
            // stage for the row-major copy
#pragma unroll
            for (int r = 0; r < 4; ++r) stage[(t_w + 16 * i + 4 * lg + r) * 65 + s_w + 16 * j + li] = tot[i][j][r];
        }
    __syncthreads();
    // M rows t: 64 rows x 64 columns, four consecutive s per thread and pass
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
        const int e = pass * kThreads + threadIdx.x;   // 0 .. 1023
        const int rr = e / 16, cc = (e % 16) * 4;
        const float o[4] = {stage[rr * 65 + cc], stage[rr * 65 + cc + 1], stage[rr * 65 + cc + 2], stage[rr * 65 + cc + 3]};
        store4_f32(trow + (int64_t)(ti * 64 + rr) * Q + si * 64 + cc, o);
    }
}

// M as the sum of k_bwd_m's hsplit parts (in split order, so the result does not
// depend on timing), written as M (rows t) and M^T (rows s) like the unsplit
// kernel.  One workgroup per tile unit of k_bwd_m.
template <typename E, int Q>
__global__ __launch_bounds__(kThreads) void k_bwd_m_reduce(const float *__restrict__ mpart, E *__restrict__ mrow,
                                                           E *__restrict__ mcol, int G, int nc, int hsplit,
                                                           const int32_t *__restrict__ cseg = nullptr)
{
    constexpr int QT = Q / 64, NTRI = QT * (QT + 1) / 2;
    __shared__ float stage[64 * 65];
    const int units = NTRI * nc * G;
    const int u = blockIdx.x, b = blockIdx.y;
    int tile = u % NTRI;
    const int cg = u / NTRI, g = cg % G, c = cg / G;
    if (cseg && cseg[c] < 0) return;   // a chunk of padding only (cseg: see k_state_passing)
    int ti = 0;
    while (tile > ti) {
        tile -= ti + 1;
        ++ti;
    }
    const int si = tile;
    const int64_t slice = (int64_t)gridDim.y * units * 4096;
    const float *src = mpart + ((int64_t)b * units + u) * 4096;
    E *trow = mrow + (((int64_t)b * nc + c) * G + g) * (int64_t)Q * Q;
    E *tcol = mcol + (((int64_t)b * nc + c) * G + g) * (int64_t)Q * Q;
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
        const int e = (pass * kThreads + threadIdx.x) * 4;   // 4 consecutive s of row rr
        const int rr = e / 64, cc = e % 64;
        floatx4 v = *reinterpret_cast<const floatx4 *>(src + e);
        for (int k = 1; k < hsplit; ++k) {
            const floatx4 w = *reinterpret_cast<const floatx4 *>(src + k * slice + e);
            v[0] += w[0]; v[1] += w[1]; v[2] += w[2]; v[3] += w[3];
        }
        const float o[4] = {v[0], v[1], v[2], v[3]};
        store4_f32(trow + (int64_t)(ti * 64 + rr) * Q + si * 64 + cc, o);
#pragma unroll
        for (int q = 0; q < 4; ++q) stage[(cc + q) * 65 + rr] = o[q];
    }
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
        const int e = (pass * kThreads + threadIdx.x) * 4;   // 4 consecutive t of column s = rr
        const int rr = e / 64, cc = e % 64;
        const float o[4] = {stage[rr * 65 + cc], stage[rr * 65 + cc + 1], stage[rr * 65 + cc + 2],
                            stage[rr * 65 + cc + 3]};
        store4_f32(tcol + (int64_t)(si * 64 + rr) * Q + ti * 64 + cc, o);
    }
}

// ---------------------------------------------------------------------------
// dC (MODE 0) and dB (MODE 1) of one (b, c, g), 64 rows x 64 columns n
// ---------------------------------------------------------------------------
// The output tile is computed transposed, D[n][r] (r = the output token), as one
// long K loop of steps; each step stages a 64 (K) x 64 (n) operand tile (read
// transposed) and the matching 64 (r) x 64 (K) tile of the other operand in
// LDS, both loaded one step ahead into registers with row-contiguous 16-byte
// loads (whole 128-byte rows; loading the second operand as MFMA fragments,
// 16 rows x 64 bytes per instruction, made the kernel three times slower):
//   MODE 0, dC:  K = s over the s-tiles <= this tile:  B rows s   x  M[t][s]
//                K = p over the group's heads:         exp(cs_t) (Hin_h[p]  x  dy_h[t][p])
//   MODE 1, dB:  K = t over the t-tiles >= this tile:  C rows t   x  M^T[s][t]
//                K = p over the group's heads:         Delta_s exp(cs_last - cs_s) (G_h[p]  x  x_h[s][p])
// (the per-row factor of a head multiplies its finished product, in fp32).
// Hin / G are the states entering / leaving the chunk ([b,nc,H,P,N] in E).
template <typename E, int Q, int MODE>
__global__ __launch_bounds__(kThreads) void k_bwd_bc(
    const E *__restrict__ src_bc /* B (dC) or C (dB) */, const E *__restrict__ mm /* M (dC) or M^T (dB) */,
    const E *__restrict__ states /* Hin (dC) or G (dB) */, const E *__restrict__ vec /* dy (dC) or x (dB) */,
    const float *__restrict__ delta, const float *__restrict__ cs, E *__restrict__ out, int T, int H, int G, int P,
    int N, int nc, int nnt, const int32_t *__restrict__ cseg = nullptr, const int2 *__restrict__ cmap = nullptr)
{
    using F = frag_t<E>;
    using KT = KTile<E, 64, 64>;
    constexpr int ES = (int)sizeof(E);
    constexpr int QT = Q / 64;
    constexpr int V = kVec16<E>;
    constexpr int PITCH = 64 + 2 * V;   // rows 32 bytes past a multiple of 256 (bf16): conflict-free reads
    constexpr int VPR = 64 / V, RPP = kThreads / VPR, NPASS = 64 / RPP;
    __shared__ __align__(16) E kt[KT::SIZE];
    __shared__ __align__(16) E bt[64 * PITCH];   // the second operand, rows r
    const int units = nc * G * QT * nnt;
    const int u = xcd_remap(blockIdx.x, units);
    const int b = blockIdx.y;
    const bool small = units < (1 << 23);
    int q1, nt, c, g;
    udivmod(u, nnt, small, q1, nt);
    const int rt = q1 % QT;
    udivmod(q1 / QT, G, small, c, g);
    if (cseg && cseg[c] < 0) return;   // a chunk of padding only (cseg: see k_state_passing)
    int t0, len;
    chunk_rows(c, Q, T, cmap, t0, len);
    const int n0 = nt * 64, r0 = rt * 64;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
    const int n_w = (wave & 1) * 32, c_w = (wave >> 1) * 32;
    const int hpg = H / G, PC = (P + 63) / 64;
    const int ntile = (len + 63) / 64;
    // steps: the M part (tiles q), then (head, p chunk) pairs
    const int q_lo = MODE == 0 ? 0 : rt, q_hi = MODE == 0 ? min(rt, ntile - 1) : ntile - 1;
    const int nq = max(0, q_hi - q_lo + 1);
    const int steps = r0 < len ? nq + hpg * PC : 0;
    if (steps == 0) return;   // the whole tile lies past the sequence end: nothing to write

    KT ka, kb;   // the M-part and the state-part operand tiles (different row pitches)
    ka.init((int64_t)G * N, N - n0);
    kb.init(N, N - n0);
    // the second operand of the next step: rows r0 + hr + i RPP, 16 bytes at column hv V
    const int hv = threadIdx.x % VPR, hr = threadIdx.x / VPR;
    uint4 rb[NPASS];
    float sc[2];     // the per-row scales of this lane's fragment rows (state part)
    // What does not change from step to step is formed once: base pointers,
    // buffer ranges, per-lane offsets.  A step only moves pointers by constant
    // strides (64 columns p, or one head), which keeps the loop's scalar work
    // small: all waves of a CU share one scalar unit, and the 64-bit index
    // products of every step used to bound this kernel.
    const E *bc_base = src_bc + (((int64_t)b * T + t0) * G + g) * N + n0;
    const int64_t bc_q = (int64_t)64 * G * N;   // one 64-row M-part tile
    const auto mrs = make_rsrc(mm + (((int64_t)b * nc + c) * G + g) * (int64_t)Q * Q, (int64_t)Q * Q * ES);
    uint32_t moff[NPASS], voff[NPASS];
#pragma unroll
    for (int i = 0; i < NPASS; ++i) {
        const int r = r0 + hr + i * RPP;
        moff[i] = r < len ? (uint32_t)((r * Q + hv * V) * ES) : kOffNone;
        voff[i] = r < len ? (uint32_t)(((int64_t)r * H * P + hv * V) * ES) : kOffNone;
    }
    // state part: the (head, p chunk) of the next step
    const E *st_ptr = states + (((int64_t)b * nc + c) * H + g * hpg) * (int64_t)P * N + n0;
    const E *vec_ptr = vec + (((int64_t)b * T + t0) * H + g * hpg) * P;
    const float *cs_ptr = cs + (((int64_t)b * H + g * hpg) * nc + c) * Q;
    const float *dl_ptr = delta + (((int64_t)b * H + g * hpg) * nc + c) * Q;
    const int64_t hrow = (int64_t)nc * Q, st_pc = (int64_t)64 * N, st_head = (int64_t)P * N - (PC - 1) * st_pc;
    const int vbytes = rsrc_bytes(((int64_t)(len - 1) * H * P + P) * ES);
    const int kb_full = rsrc_bytes((63 * (int64_t)N + min(N, 64)) * ES);
    const int kb_tail = rsrc_bytes(((int64_t)(P - (PC - 1) * 64 - 1) * N + min(N, 64)) * ES);
    int rrj[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = r0 + c_w + 16 * j + li;
        rrj[j] = r < len ? r : 0;
    }
    int pc = 0;
    auto issue = [&](int k) {
        if (k < nq) {
            const int q = q_lo + k, rows = min(64, len - q * 64);
            ka.load(KT::rsrc(bc_base + q * bc_q, (int64_t)G * N, rows));
            const uint32_t qo = (uint32_t)(q * 64 * ES);
#pragma unroll
            for (int i = 0; i < NPASS; ++i) rb[i] = bload16(mrs, moff[i] == kOffNone ? kOffNone : moff[i] + qo);
#pragma unroll
            for (int j = 0; j < 2; ++j) sc[j] = 1.f;
        } else {
            const int p0 = pc * 64;
            kb.load(make_rsrc_n(st_ptr, pc == PC - 1 ? kb_tail : kb_full));
            const auto vrs = make_rsrc_n(vec_ptr, vbytes);
            const bool pin = hv * V < P - p0;
#pragma unroll
            for (int i = 0; i < NPASS; ++i)
                rb[i] = bload16(vrs, (voff[i] != kOffNone && pin) ? voff[i] + (uint32_t)(p0 * ES) : kOffNone);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                sc[j] = MODE == 0 ? __builtin_amdgcn_exp2f(cs_ptr[rrj[j]] * kLog2e)
                                  : dl_ptr[rrj[j]] * __builtin_amdgcn_exp2f((cs_ptr[Q - 1] - cs_ptr[rrj[j]]) * kLog2e);
            if (++pc == PC) {
                pc = 0;
                st_ptr += st_head;
                vec_ptr += P;
                cs_ptr += hrow;
                dl_ptr += hrow;
            } else {
                st_ptr += st_pc;
            }
        }
    };

    floatx4 acc[2][2] = {};
    typename KT::Off aoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) aoff[i] = KT::frag_off(n_w + 16 * i);
    // The state part's per-row scale is the same for every column of a row and
    // every p of a head, so each head's product is formed unscaled in `part`
    // and added to the total with the scale of its rows (column r = lane's
    // c_w + 16 j + li of D) once the head's last p chunk is in; M-part steps
    // are added unscaled.
    floatx4 part[2][2] = {};
    issue(0);
    int kpc = 0;   // the p chunk of a state-part step
    for (int k = 0; k < steps; ++k) {
        if (k > 0) __syncthreads();   // every wave is done reading the previous tile
        const bool mpart = k < nq;
        if (mpart) ka.template store<false, false>(kt, nullptr, nullptr);
        else kb.template store<false, false>(kt, nullptr, nullptr);
#pragma unroll
        for (int i = 0; i < NPASS; ++i) *reinterpret_cast<uint4 *>(bt + (hr + i * RPP) * PITCH + hv * V) = rb[i];
        float cs_[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) cs_[j] = sc[j];
        if (k + 1 < steps) issue(k + 1);
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            F fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) fa[i] = KT::frag_at(kt, aoff[i], ks * 32);
#pragma unroll
            for (int j = 0; j < 2; ++j) fb[j] = load_frag(bt + (c_w + 16 * j + li) * PITCH + ks * 32 + 8 * lg);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) mma(part[i][j], fa[i], fb[j]);
        }
        bool fold = mpart;
        if (!mpart) {
            fold = kpc == PC - 1;
            kpc = fold ? 0 : kpc + 1;
        }
        if (fold) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[i][j][e] += part[i][j][e] * cs_[j];
                        part[i][j][e] = 0.f;
                    }
        }
    }

    // D[n][r] -> out[b, t0 + r, g, n .. n+3]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = r0 + c_w + 16 * j + li, n = n0 + n_w + 16 * i + 4 * lg;
            if (r < len && n < N) {
                const float o[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
                store4_f32(out + (((int64_t)b * T + t0 + r) * G + g) * N + n, o);
            }
        }
}

}  // namespace ssd
