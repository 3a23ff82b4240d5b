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
// forward's chunk_scan kernel with every chunk's tokens in reversed order
// (kernels below build the reversed copies).
#pragma once

#include "ssd_kernels.hpp"

namespace ssd {

// ---------------------------------------------------------------------------
// token order reversed inside every chunk
// ---------------------------------------------------------------------------
// out[b, c*Q + (len_c - 1 - i), :] = in[b, c*Q + i, :] for the len_c tokens of
// chunk c; rows hold R elements (R * sizeof(E) a multiple of 16 bytes).
template <typename E>
__global__ void k_bwd_reverse_rows(const E *__restrict__ in, E *__restrict__ out, int T, int Q, int64_t R,
                                   int64_t total_vecs)
{
    constexpr int V = kVec16<E>;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total_vecs) return;
    const int64_t vpr = R / V;
    const int64_t row = i / vpr, v = i % vpr;   // row = b * T + t
    const int b = (int)(row / T), t = (int)(row % T);
    const int c = t / Q, k = t % Q, len = min(Q, T - c * Q);
    const int tr = c * Q + (len - 1 - k);
    *reinterpret_cast<uint4 *>(out + ((int64_t)b * T + tr) * R + v * V) =
        *reinterpret_cast<const uint4 *>(in + row * R + v * V);
}

// For the reversed chunk (rows [b,H,nc,Q]): cs_rev[i] = cs[len-1] - cs[len-1-i]
// and delta_rev[i] = 1 for i < len; past len cs_rev keeps its last value and
// delta_rev is 0 (as the forward leaves positions past the sequence end).
__global__ void k_bwd_reverse_cs(const float *__restrict__ cs, float *__restrict__ cs_rev,
                                 float *__restrict__ delta_rev, int T, int Q, int nc, int64_t total)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int64_t row = i / Q;   // (b * H + h) * nc + c
    const int k = (int)(i % Q), c = (int)(row % nc);
    const int len = min(Q, T - c * Q);
    const float *r = cs + row * Q;
    const int kk = k < len ? k : len - 1;
    cs_rev[i] = r[len - 1] - r[len - 1 - kk];
    delta_rev[i] = k < len ? 1.f : 0.f;
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

template <typename E>
__global__ __launch_bounds__(kThreads) void k_bwd_dl(
    const float *__restrict__ rpart, const float *__restrict__ cpart, const float *__restrict__ yo,
    const float *__restrict__ zo, const float *__restrict__ xyp, const float *__restrict__ bnd_part,
    const float *__restrict__ dyx, const float *__restrict__ delta, const E *__restrict__ dt,
    const float *__restrict__ A, E *__restrict__ ddt, float *__restrict__ dA_part, float *__restrict__ dD_part, int T,
    int H, int Q, int nc, int ntp, int64_t rows, int softplus, int64_t nbp)
{
    const int64_t wid = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);   // (b * H + h) * nc + c
    if (wid >= rows) return;   // whole wave
    const int lane = threadIdx.x & 63;
    const int c = (int)(wid % nc);
    const int64_t bh = wid / nc;
    const int h = (int)(bh % H), b = (int)(bh / H);
    const int per = Q / 64, QT = Q / 64;
    const int64_t slice = rows * Q;   // one tile / p-tile slice: [b,H,nc,Q]
    const float Ah = A[h];
    const int len = min(Q, T - c * Q);
    const int64_t row = wid * Q;
    double av[4] = {0, 0, 0, 0}, zv[4] = {0, 0, 0, 0};
    float xv[4] = {0, 0, 0, 0};
    double asum = 0.0, zsum = 0.0;
    for (int e = 0; e < per; ++e) {
        const int j = lane * per + e;
        if (j >= len) continue;
        double r = 0.0, cc = 0.0, y1 = 0.0, z1 = 0.0, xy = 0.0;
        for (int si = 0; si <= j / 64; ++si) r += rpart[si * slice + row + j];
        for (int ti = j / 64; ti < QT; ++ti) cc += cpart[ti * slice + row + j];
        for (int tp = 0; tp < ntp; ++tp) {
            y1 += yo[tp * slice + row + j];
            z1 += zo[tp * slice + row + j];
            xy += xyp[tp * slice + row + j];
        }
        av[e] = r - cc + y1;
        zv[e] = delta[row + j] * z1;
        xv[e] = (float)xy;
        asum += av[e];
        zsum += zv[e];
    }
    // suffix sums of a (inclusive) and prefix sums of z (exclusive) over the chunk
    double bsum = 0.0;
    for (int64_t i = lane; i < nbp; i += 64) bsum += bnd_part[wid * nbp + i];
    const double ain = wave_incl_scan(asum), zin = wave_incl_scan(zsum), bin = wave_incl_scan(bsum);
    const double atot = __shfl(ain, 63);
    double asuf = atot - ain + asum;   // sum of a over this lane's tokens and all later lanes
    double zpre = zin - zsum;          // sum of z over earlier lanes
    const double b0 = __shfl(bin, 63);
    double sa = 0.0, sd = 0.0;
    for (int e = 0; e < per; ++e) {
        const int j = lane * per + e;
        if (j < len) {
            const double dl = asuf + zpre + b0;
            const float dd = Ah * (float)dl + xv[e];
            const int t = c * Q + j;
            float gr = dd;
            if (softplus) {
                const float zt = to_float(dt[((int64_t)b * T + t) * H + h]);
                gr = dd / (1.f + __builtin_amdgcn_exp2f(-zt * kLog2e));   // dDelta * sigmoid(dt)
            }
            ddt[((int64_t)b * T + t) * H + h] = from_float<E>(gr);
            sa += (double)delta[row + j] * dl;
            for (int tp = 0; tp < ntp; ++tp) sd += dyx[tp * slice + row + j];
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
template <typename E, int Q, int NT>
__global__ __launch_bounds__(kThreads) void k_bwd_m(
    const E *__restrict__ dy, const E *__restrict__ x, const float *__restrict__ delta, const float *__restrict__ cs,
    const E *__restrict__ cbuf, E *__restrict__ mrow, E *__restrict__ mcol, float *__restrict__ rpart,
    float *__restrict__ cpart, int T, int H, int G, int P, int nc)
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
    const int u = xcd_remap(blockIdx.x, units);
    const int b = blockIdx.y;
    int tile = u % NTRI;
    const int cg = u / NTRI, g = cg % G, c = cg / G;
    int ti = 0;
    while (tile > ti) {
        tile -= ti + 1;
        ++ti;
    }
    const int si = tile;
    const int t0 = c * Q, len = min(Q, T - t0);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
    const int hpg = H / G, PC = (P + 63) / 64, steps = hpg * PC;
    const int hv = threadIdx.x % VPR, hr = threadIdx.x / VPR;
    const int trows = min(64, len - ti * 64), srows = min(64, len - si * 64);

    uint4 rt[NPASS], rs[NPASS];
    float hval = 0.f;   // this thread's element of the next head's cs / delta rows (threads < 192)
    auto issue = [&](int k) {
        if (k % PC == 0 && threadIdx.x < 192) {
            const int h = g * hpg + k / PC, part = threadIdx.x >> 6, e = threadIdx.x & 63;
            const int64_t row = (((int64_t)b * H + h) * nc + c) * Q;
            const int pos = (part == 0 ? ti : si) * 64 + e;
            hval = pos < len ? (part == 2 ? delta[row + pos] : cs[row + pos]) : 0.f;
        }
        const int h = g * hpg + k / PC, p0 = (k % PC) * 64;
        const int64_t ld = (int64_t)H * P;
        const auto trs = make_rsrc(dy + (((int64_t)b * T + t0 + ti * 64) * H + h) * P + p0,
                                   trows > 0 ? ((int64_t)(trows - 1) * ld + min(64, P - p0)) * ES : 0);
        const auto srs = make_rsrc(x + (((int64_t)b * T + t0 + si * 64) * H + h) * P + p0,
                                   srows > 0 ? ((int64_t)(srows - 1) * ld + min(64, P - p0)) * ES : 0);
        const bool cin = p0 + hv * V < P;
#pragma unroll
        for (int i = 0; i < NPASS; ++i) {
            const uint32_t o = cin ? (uint32_t)(((int64_t)(hr + i * RPP) * ld + hv * V) * ES) : kOffNone;
            rt[i] = bload16(trs, o);
            rs[i] = bload16(srs, o);
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
    auto flush = [&](int h) {   // this head's row / column sums to memory, then cleared
        const int64_t row = (((int64_t)b * H + h) * nc + c) * Q;
        if (threadIdx.x < 64) {
            rpart[si * bhnc + row + ti * 64 + threadIdx.x] = rsum[threadIdx.x];
            rsum[threadIdx.x] = 0.f;
        } else if (threadIdx.x < 128) {
            const int e = threadIdx.x - 64;
            cpart[ti * bhnc + row + si * 64 + e] = csum[e];
            csum[e] = 0.f;
        }
    };
    if (threadIdx.x < 64) rsum[threadIdx.x] = 0.f;
    else if (threadIdx.x < 128) csum[threadIdx.x - 64] = 0.f;
    issue(0);
    for (int k = 0; k < steps; ++k) {
        if (k > 0) __syncthreads();   // every wave is done reading the previous step's rows
        if (k > 0 && (k - 1) % PC == PC - 1) flush(g * hpg + (k - 1) / PC);
#pragma unroll
        for (int i = 0; i < NPASS; ++i) {
            *reinterpret_cast<uint4 *>(ts + (hr + i * RPP) * PITCH + hv * V) = rt[i];
            *reinterpret_cast<uint4 *>(ss + (hr + i * RPP) * PITCH + hv * V) = rs[i];
        }
        if (k % PC == 0 && threadIdx.x < 192) {
            const int part = threadIdx.x >> 6, e = threadIdx.x & 63;
            if (part == 2) hds[e] = hval;
            else hcs[part][e] = hval;
        }
        if (k + 1 < steps) issue(k + 1);
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
        if (k % PC == PC - 1) {
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
                // decay, and only s <= t < len
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int s = si * 64 + s_w + 16 * j + li;
                    const float css = hcs[1][s_w + 16 * j + li], ds = hds[s_w + 16 * j + li];
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int t = ti * 64 + t_w + 16 * i + 4 * lg + r;
                            if (s <= t && t < len) {
                                const float w =
                                    __builtin_amdgcn_exp2f((hcs[0][t_w + 16 * i + 4 * lg + r] - css) * kLog2e) * ds;
                                const float wv = acc[i][j][r] * w;
                                tot[i][j][r] += wv;
                                const float sv = wv * cbv[i][j][r];
                                rs[i][r] += sv;
                                cl[j] += sv;
                            }
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
    flush(g * hpg + (steps - 1) / PC);

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
//                K = p over the group's heads:         Hin_h[p]   x  exp(cs_t) dy_h[t][p]
//   MODE 1, dB:  K = t over the t-tiles >= this tile:  C rows t   x  M^T[s][t]
//                K = p over the group's heads:         G_h[p]     x  Delta_s exp(cs_last - cs_s) x_h[s][p]
// Hin / G are the states entering / leaving the chunk ([b,nc,H,P,N] in E).
template <typename E, int Q, int MODE>
__global__ __launch_bounds__(kThreads) void k_bwd_bc(
    const E *__restrict__ src_bc /* B (dC) or C (dB) */, const E *__restrict__ mm /* M (dC) or M^T (dB) */,
    const E *__restrict__ states /* Hin (dC) or G (dB) */, const E *__restrict__ vec /* dy (dC) or x (dB) */,
    const float *__restrict__ delta, const float *__restrict__ cs, E *__restrict__ out, int T, int H, int G, int P,
    int N, int nc, int nnt)
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
    const int nt = u % nnt, rt = (u / nnt) % QT, cg = u / (nnt * QT), g = cg % G, c = cg / G;
    const int t0 = c * Q, len = min(Q, T - t0);
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
    auto issue = [&](int k) {
        if (k < nq) {
            const int q = q_lo + k, rows = min(64, len - q * 64);
            ka.load(KT::rsrc(src_bc + (((int64_t)b * T + t0 + q * 64) * G + g) * N + n0, (int64_t)G * N, rows));
            const E *mb = mm + (((int64_t)b * nc + c) * G + g) * (int64_t)Q * Q;
            const auto mrs = make_rsrc(mb, (int64_t)Q * Q * ES);
#pragma unroll
            for (int i = 0; i < NPASS; ++i) {
                const int r = r0 + hr + i * RPP;
                rb[i] = bload16(mrs, r < len ? (uint32_t)(((int64_t)r * Q + q * 64 + hv * V) * ES) : kOffNone);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) sc[j] = 1.f;
        } else {
            const int hk = k - nq, h = g * hpg + hk / PC, p0 = (hk % PC) * 64;
            kb.load(KT::rsrc(states + ((((int64_t)b * nc + c) * H + h) * P + p0) * N + n0, N, min(64, P - p0)));
            const auto vrs = make_rsrc(vec + (((int64_t)b * T + t0) * H + h) * P,
                                       ((int64_t)(len - 1) * H * P + P) * ES);
            const bool pin = p0 + hv * V < P;
#pragma unroll
            for (int i = 0; i < NPASS; ++i) {
                const int r = r0 + hr + i * RPP;
                rb[i] = bload16(vrs, (r < len && pin) ? (uint32_t)(((int64_t)r * H * P + p0 + hv * V) * ES) : kOffNone);
            }
            const int64_t row = (((int64_t)b * H + h) * nc + c) * Q;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int r = r0 + c_w + 16 * j + li;
                const int rr = r < len ? r : 0;
                sc[j] = MODE == 0 ? __builtin_amdgcn_exp2f(cs[row + rr] * kLog2e)
                                  : delta[row + rr] * __builtin_amdgcn_exp2f((cs[row + Q - 1] - cs[row + rr]) * kLog2e);
            }
        }
    };

    floatx4 acc[2][2] = {};
    typename KT::Off aoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) aoff[i] = KT::frag_off(n_w + 16 * i);
    issue(0);
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
            F fa[2], fbv[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) fa[i] = KT::frag_at(kt, aoff[i], ks * 32);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const F f = load_frag(bt + (c_w + 16 * j + li) * PITCH + ks * 32 + 8 * lg);
                fbv[j] = mpart ? f : from_f32<F>(to_f32(f) * cs_[j]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) mma(acc[i][j], fa[i], fbv[j]);
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
