// ssd_api.hip -- host side of libssd.so: argument validation, workspace layout
// and kernel launches behind the C ABI declared in include/ssd.h.
//
// Validation is pure host code and runs before any HIP call.  Nothing here
// allocates, frees or synchronises; every launch goes to the caller's stream.
#include "ssd.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "ssd_kernels.hpp"
#include "ssd_bwd_kernels.hpp"
#include "ssd_block_kernels.hpp"

using namespace ssd;

namespace {

struct Shape {
    int64_t b, T, H, P, N, G, Q, nc;
    int dtype;
    size_t esz;   // bytes per element of x, dt, B, C, y and the chunk intermediates
    bool packed;
    int64_t nseq;
};

constexpr int64_t kMaxDim = (int64_t)1 << 30;

ssd_status parse_shape(const ssd_fwd_args *a, Shape *s)
{
    if (!a) return SSD_ERR_NULL_POINTER;
    if (a->dtype != SSD_DTYPE_F32 && a->dtype != SSD_DTYPE_BF16) return SSD_ERR_BAD_DTYPE;
    if (a->batch < 1 || a->seqlen < 0 || a->nheads < 1 || a->headdim < 16 || a->dstate < 16 ||
        a->ngroups < 1)
        return SSD_ERR_BAD_SHAPE;
    if (a->headdim % 16 != 0 || a->dstate % 16 != 0 || a->dstate > kMaxStateDim) return SSD_ERR_BAD_SHAPE;
    if (a->batch > kMaxDim || a->seqlen > kMaxDim || a->nheads > kMaxDim || a->headdim > 4096)
        return SSD_ERR_BAD_SHAPE;
    if (a->nheads % a->ngroups != 0) return SSD_ERR_GROUPS;
    if (a->chunk != 64 && a->chunk != 128 && a->chunk != 256) return SSD_ERR_BAD_CHUNK;
    if (a->seq_idx && (a->batch != 1 || a->nseq < 1 || a->nseq > kMaxDim)) return SSD_ERR_SEQ_IDX;
    s->b = a->batch;
    s->T = a->seqlen;
    s->H = a->nheads;
    s->P = a->headdim;
    s->N = a->dstate;
    s->G = a->ngroups;
    s->Q = a->chunk;
    s->nc = (a->seqlen + a->chunk - 1) / a->chunk;
    s->dtype = a->dtype;
    s->esz = a->dtype == SSD_DTYPE_BF16 ? 2 : 4;
    s->packed = a->seq_idx != nullptr;
    s->nseq = a->seq_idx ? a->nseq : 0;
    // every grid dimension and every int32 index used inside the kernels must fit
    const int64_t units = s->nc * s->H * ((s->P + 63) / 64) * ((s->N + 63) / 64);
    if (units > INT32_MAX || s->nc * s->Q > INT32_MAX) return SSD_ERR_BAD_SHAPE;
    return SSD_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

struct Range {
    const void *p;
    size_t n;
};

bool overlaps(Range a, Range b)
{
    if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

// Sizes in bytes of the tensors in the args struct.
struct Sizes {
    size_t x, dt, A, bc, D, init, seq, y, fin;
};

Sizes tensor_sizes(const Shape &s)
{
    Sizes z;
    z.x = (size_t)(s.b * s.T * s.H * s.P) * s.esz;
    z.dt = (size_t)(s.b * s.T * s.H) * s.esz;
    z.A = (size_t)s.H * 4;
    z.bc = (size_t)(s.b * s.T * s.G * s.N) * s.esz;
    z.D = (size_t)s.H * 4;
    z.init = (size_t)(s.b * s.H * s.P * s.N) * 4;
    z.seq = (size_t)s.T * 4;
    z.y = z.x;
    z.fin = (size_t)((s.packed ? s.nseq : s.b) * s.H * s.P * s.N) * 4;
    return z;
}

// Which pointers an entry point reads or writes.
enum : unsigned {
    kNeedX = 1u << 0,
    kNeedDt = 1u << 1,
    kNeedB = 1u << 2,
    kNeedC = 1u << 3,
    kNeedY = 1u << 4,
    kCheckFinal = 1u << 5,   // final_states written if non-NULL
};

ssd_status check_pointers(const ssd_fwd_args *a, const Shape &s, unsigned need)
{
    const bool empty = s.T == 0;
    if (!a->A) return SSD_ERR_NULL_POINTER;
    if (!empty) {
        if ((need & kNeedX) && !a->x) return SSD_ERR_NULL_POINTER;
        if ((need & kNeedDt) && !a->dt) return SSD_ERR_NULL_POINTER;
        if ((need & kNeedB) && !a->B) return SSD_ERR_NULL_POINTER;
        if ((need & kNeedC) && !a->C) return SSD_ERR_NULL_POINTER;
        if ((need & kNeedY) && !a->y) return SSD_ERR_NULL_POINTER;
    }
    const void *ptrs[] = {a->x, a->dt, a->A, a->B, a->C, a->D, a->initial_states, a->seq_idx, a->y,
                          a->final_states, a->workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return SSD_ERR_MISALIGNED;
    const Sizes z = tensor_sizes(s);
    const Range ins[] = {{a->x, z.x}, {a->dt, z.dt}, {a->A, z.A}, {a->B, z.bc}, {a->C, z.bc},
                         {a->D, z.D}, {a->initial_states, z.init}, {a->seq_idx, z.seq}};
    const Range outs[] = {{(need & kNeedY) ? a->y : nullptr, z.y},
                          {(need & kCheckFinal) ? a->final_states : nullptr, z.fin}};
    for (const Range &o : outs)
        for (const Range &i : ins)
            if (overlaps(o, i)) return SSD_ERR_ALIASING;
    if (overlaps(outs[0], outs[1])) return SSD_ERR_ALIASING;
    return SSD_OK;
}

// Workspace carve-up for ssd_fwd (256-byte aligned pieces).
struct Workspace {
    size_t delta, cs, cb, states, seg_end, total;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// N rounded up to 64: the state width the kernels are compiled for.
int64_t nt_of(int64_t N) { return N <= 64 ? 64 : N <= 128 ? 128 : 256; }

Workspace workspace_layout(const Shape &s)
{
    Workspace w;
    const size_t dcs = (size_t)(s.b * s.H * s.nc * s.Q) * 4;
    const size_t cbs = (size_t)(s.b * s.nc * s.G * s.Q * (s.Q + 2 * nt_of(s.N))) * s.esz;
    const size_t sts = (size_t)(s.b * s.nc * s.H * s.P * s.N) * s.esz;
    w.delta = 0;
    w.cs = align256(w.delta + dcs);
    w.cb = align256(w.cs + dcs);
    w.states = align256(w.cb + cbs);
    w.seg_end = align256(w.states + sts);
    w.total = align256(w.seg_end + (s.packed ? (size_t)s.nseq * 4 : 0));
    return w;
}

ssd_status launched() { return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP; }

unsigned grid1(int64_t n, int threads) { return (unsigned)((n + threads - 1) / threads); }

// ---- per-step launches (typed) ----


// The state kernels cover all of N in one workgroup: NT = N rounded up to 64.
template <typename F>
ssd_status with_nt(int64_t N, F &&f)
{
    if (N <= 64) return f(std::integral_constant<int, 64>{});
    if (N <= 128) return f(std::integral_constant<int, 128>{});
    return f(std::integral_constant<int, 256>{});
}

template <typename F>
ssd_status with_q(int64_t Q, F &&f)
{
    if (Q == 64) return f(std::integral_constant<int, 64>{});
    if (Q == 128) return f(std::integral_constant<int, 128>{});
    return f(std::integral_constant<int, 256>{});
}

template <typename E>
ssd_status run_cumsum(const Shape &s, const ssd_fwd_args *a, float *delta, float *cs, hipStream_t st)
{
    dim3 grid((unsigned)s.nc, (unsigned)((s.H + kCumsumHeads - 1) / kCumsumHeads), (unsigned)s.b);
    hipLaunchKernelGGL(k_chunk_cumsum<E>, grid, dim3(kThreads), 0, st, (const E *)a->dt, a->A, a->seq_idx,
                       delta, cs, (int)s.T, (int)s.H, (int)s.Q, (int)s.nc, (int)a->dt_softplus);
    return launched();
}

// rev: every chunk's rows of a->B and a->C taken in reversed order.  cseg (the
// packed backward's layout, see run_passing): chunks of padding only are
// skipped, here and in the other per-chunk launches that take it.
template <typename E>
ssd_status run_cb(const Shape &s, const ssd_fwd_args *a, E *cb, hipStream_t st, bool rev = false,
                  const int32_t *cseg = nullptr, const int2 *cmap = nullptr)
{
    const int qt = (int)(s.Q / 64), ntri = qt * (qt + 1) / 2;
    dim3 grid((unsigned)(ntri * s.nc * s.G), (unsigned)s.b);
    return with_q(s.Q, [&](auto q) {
        return with_nt(s.N, [&](auto nt) {
            constexpr int Q = decltype(q)::value, NT = decltype(nt)::value;
            if (rev)
                hipLaunchKernelGGL((k_chunk_cb<E, Q, NT, true>), grid, dim3(kThreads), 0, st, (const E *)a->B,
                                   (const E *)a->C, cb, (int)s.T, (int)s.G, (int)s.N, (int)s.nc, cseg, cmap);
            else
                hipLaunchKernelGGL((k_chunk_cb<E, Q, NT>), grid, dim3(kThreads), 0, st, (const E *)a->B,
                                   (const E *)a->C, cb, (int)s.T, (int)s.G, (int)s.N, (int)s.nc, cseg, cmap);
            return launched();
        });
    });
}


template <typename E>
ssd_status run_state(const Shape &s, const ssd_fwd_args *a, float *delta, float *cs, const E *cb, E *states,
                     int32_t *seg_end, hipStream_t st, const int32_t *cseg = nullptr, const int2 *cmap = nullptr)
{
    const int ntp = (int)((s.P + 63) / 64);
    dim3 grid((unsigned)(s.nc * s.H * ntp), (unsigned)s.b);
    return with_q(s.Q, [&](auto q) {
        return with_nt(s.N, [&](auto nt) {
            constexpr int Q = decltype(q)::value, NT = decltype(nt)::value;
            auto launch = [&](auto kern) {
                hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, st, (const E *)a->x, cb, (const E *)a->dt, a->A,
                                   a->seq_idx, delta, cs, states, seg_end, (int)s.nseq, (int)s.T, (int)s.H,
                                   (int)s.G, (int)s.P, (int)s.N, (int)s.nc, ntp, (int)a->dt_softplus, cseg, cmap);
            };
            if (s.packed) launch(k_chunk_state<E, Q, NT, true>);
            else launch(k_chunk_state<E, Q, NT, false>);
            return launched();
        });
    });
}

// cseg: the per-chunk segment ids of a stream whose segments start at chunk
// starts (the packed backward's layout; seq_idx is then not read), or NULL.
template <typename E>
ssd_status run_passing(const Shape &s, const ssd_fwd_args *a, const float *cs, E *states, float *final_states,
                       hipStream_t st, const int32_t *cseg = nullptr)
{
    const int64_t PN = s.P * s.N;   // a multiple of 256
    constexpr int VE = 4;            // elements per thread
    const int64_t vecs = s.b * s.H * PN / VE;
    auto launch = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(grid1(vecs, kThreads)), dim3(kThreads), 0, st, states, cs, a->initial_states,
                           final_states, cseg ? nullptr : a->seq_idx, (int)s.T, (int)s.H, PN, (int)s.nc, (int)s.Q,
                           vecs, (const E *)nullptr, (float *)nullptr, cseg);
    };
    // a deeper ring of loads for bf16 chains longer than the default one (fp32
    // states would need twice its registers)
    if (sizeof(E) == 2 && s.nc > kPrefetch) launch(k_state_passing<E, VE, false, kPrefetchLong>);
    else launch(k_state_passing<E, VE>);
    return launched();
}

// `marked`: seg_end already holds the segment ends (chunk_state marks them in the
// forward); otherwise they are marked here first.
template <typename E>
ssd_status run_seq_final(const Shape &s, const ssd_fwd_args *a, const float *delta, const float *cs,
                         const E *hin, int32_t *seg_end, bool marked, hipStream_t st)
{
    if (!marked) {
        hipLaunchKernelGGL(k_seg_end, dim3(grid1(s.T, 256)), dim3(256), 0, st, a->seq_idx, seg_end, (int)s.T,
                           (int)s.nseq);
        if (launched() != SSD_OK) return SSD_ERR_HIP;
    }
    const int ntp = (int)((s.P + 63) / 64);
    dim3 grid((unsigned)(s.nseq * s.H * ntp));
    return with_q(s.Q, [&](auto q) {
        return with_nt(s.N, [&](auto nt) {
            constexpr int Q = decltype(q)::value, NT = decltype(nt)::value;
            hipLaunchKernelGGL((k_seq_final<E, Q, NT>), grid, dim3(kThreads), 0, st, (const E *)a->x,
                               (const E *)a->B, delta, cs, a->seq_idx, hin, seg_end, a->final_states, (int)s.T,
                               (int)s.H, (int)s.G, (int)s.P, (int)s.N, (int)s.nc, (int)s.nseq, ntp);
            return launched();
        });
    });
}

template <typename E>
ssd_status run_scan(const Shape &s, const ssd_fwd_args *a, const float *delta, const float *cs, const E *cb,
                    const E *hin, hipStream_t st)
{
    const int ntp = (int)((s.P + 63) / 64);
    dim3 grid((unsigned)(s.nc * s.H * ntp), (unsigned)s.b);
    return with_q(s.Q, [&](auto q) {
        return with_nt(s.N, [&](auto nt) {
            constexpr int Q = decltype(q)::value, NT = decltype(nt)::value;
            if (s.packed)
                hipLaunchKernelGGL((k_chunk_scan<E, Q, NT, true>), grid, dim3(scan_threads<Q>()), 0, st, (const E *)a->x,
                                   delta, cs, cb, hin, a->D, a->seq_idx, (E *)a->y, (int)s.T,
                                   (int)s.H, (int)s.G, (int)s.P, (int)s.N, (int)s.nc, ntp, (const E *)nullptr,
                                   (float *)nullptr, (float *)nullptr, (const E *)nullptr, (const float *)nullptr,
                                   (const float *)nullptr, (float *)nullptr);
            else
                hipLaunchKernelGGL((k_chunk_scan<E, Q, NT, false>), grid, dim3(scan_threads<Q>()), 0, st, (const E *)a->x,
                                   delta, cs, cb, hin, a->D, a->seq_idx, (E *)a->y, (int)s.T,
                                   (int)s.H, (int)s.G, (int)s.P, (int)s.N, (int)s.nc, ntp, (const E *)nullptr,
                                   (float *)nullptr, (float *)nullptr, (const E *)nullptr, (const float *)nullptr,
                                   (const float *)nullptr, (float *)nullptr);
            return launched();
        });
    });
}

// chunk_scan in a dot mode (non-packed): DOT = 1 with P1ONLY (entering-state dot
// only, no y), or DOT = 2 (both dots) on a chunk-reversed problem, writing
// dx = dx_delta y' + dx_D x to a->y at the original token order.
template <typename E, int DOT, bool P1ONLY>
ssd_status run_scan_dot(const Shape &s, const ssd_fwd_args *a, const float *delta, const float *cs, const E *cb,
                        const E *hin, const E *vec, float *dot1, float *dot2, hipStream_t st,
                        const float *dx_delta = nullptr, const float *dx_D = nullptr, float *dxv = nullptr,
                        const int32_t *cseg = nullptr, const int2 *cmap = nullptr)
{
    const int ntp = (int)((s.P + 63) / 64);
    dim3 grid((unsigned)(s.nc * s.H * ntp), (unsigned)s.b);
    return with_q(s.Q, [&](auto q) {
        return with_nt(s.N, [&](auto nt) {
            constexpr int Q = decltype(q)::value, NT = decltype(nt)::value;
            hipLaunchKernelGGL((k_chunk_scan<E, Q, NT, false, DOT, P1ONLY>), grid, dim3(scan_threads<Q>()), 0, st,
                               (const E *)a->x, delta, cs, cb, hin, a->D, (const int32_t *)nullptr, (E *)a->y,
                               (int)s.T, (int)s.H, (int)s.G, (int)s.P, (int)s.N, (int)s.nc, ntp, vec, dot1, dot2,
                               (const E *)nullptr, dx_delta, dx_D, dxv, cseg, cmap);
            return launched();
        });
    });
}

// chunk_scan with the SiLU(z) gate fused into its epilogue.
template <typename E>
ssd_status run_scan_gated(const Shape &s, const ssd_fwd_args *a, const float *delta, const float *cs, const E *cb,
                          const E *hin, const E *z, hipStream_t st)
{
    const int ntp = (int)((s.P + 63) / 64);
    dim3 grid((unsigned)(s.nc * s.H * ntp), (unsigned)s.b);
    return with_q(s.Q, [&](auto q) {
        return with_nt(s.N, [&](auto nt) {
            constexpr int Q = decltype(q)::value, NT = decltype(nt)::value;
            auto launch = [&](auto kern) {
                hipLaunchKernelGGL(kern, grid, dim3(scan_threads<Q>()), 0, st, (const E *)a->x, delta, cs, cb, hin,
                                   a->D, a->seq_idx, (E *)a->y, (int)s.T, (int)s.H, (int)s.G, (int)s.P, (int)s.N,
                                   (int)s.nc, ntp, (const E *)nullptr, (float *)nullptr, (float *)nullptr, z,
                                   (const float *)nullptr, (const float *)nullptr, (float *)nullptr,
                                   (const int32_t *)nullptr, (const int2 *)nullptr);
            };
            if (s.packed) launch(k_chunk_scan<E, Q, NT, true, 0, false, true>);
            else launch(k_chunk_scan<E, Q, NT, false, 0, false, true>);
            return launched();
        });
    });
}

ssd_status fill_final(const Shape &s, const ssd_fwd_args *a, hipStream_t st)
{
    if (!a->final_states) return SSD_OK;
    const int64_t n = (s.packed ? s.nseq : s.b) * s.H * s.P * s.N;
    // an empty packed stream has no segment that could receive the initial state
    const float *init = s.packed ? nullptr : a->initial_states;
    hipLaunchKernelGGL(k_fill_final, dim3(grid1(n, 256)), dim3(256), 0, st, a->final_states, init, n);
    return launched();
}

template <typename E>
ssd_status fwd_typed(const Shape &s, const ssd_fwd_args *a, const Workspace &w, hipStream_t st,
                     const E *gate = nullptr)
{
    char *ws = static_cast<char *>(a->workspace);
    float *delta = reinterpret_cast<float *>(ws + w.delta);
    float *cs = reinterpret_cast<float *>(ws + w.cs);
    E *cb = reinterpret_cast<E *>(ws + w.cb);
    E *states = reinterpret_cast<E *>(ws + w.states);
    int32_t *seg_end = reinterpret_cast<int32_t *>(ws + w.seg_end);
    ssd_status r;
    if ((r = run_cb<E>(s, a, cb, st)) != SSD_OK) return r;   // the cumsum step runs inside chunk_state
    const bool seq_final = s.packed && a->final_states;   // chunk_state then marks the segment ends
    if ((r = run_state<E>(s, a, delta, cs, cb, states, seq_final ? seg_end : nullptr, st)) != SSD_OK) return r;
    if ((r = run_passing<E>(s, a, cs, states, s.packed ? nullptr : a->final_states, st)) != SSD_OK) return r;
    if (seq_final)
        if ((r = run_seq_final<E>(s, a, delta, cs, states, seg_end, true, st)) != SSD_OK) return r;
    if (gate) return run_scan_gated<E>(s, a, delta, cs, cb, states, gate, st);
    return run_scan<E>(s, a, delta, cs, cb, states, st);
}

template <typename E>
ssd_status run_step(const ssd_step_args *a, hipStream_t st)
{
    const int N = (int)a->dstate, P = (int)a->headdim;
    const int need = N / 4;   // lanes per state row
    auto launch = [&](auto nl) {
        constexpr int NL = decltype(nl)::value;
        const dim3 grid((unsigned)(a->batch * a->nheads), (unsigned)((P + step_rows<NL>() - 1) / step_rows<NL>()));
        hipLaunchKernelGGL((k_ssd_step<E, NL>), grid, dim3(kThreads), 0, st, (const E *)a->x, (const E *)a->dt,
                           a->A, (const E *)a->B, (const E *)a->C, a->D, a->state, (E *)a->y, (int)a->nheads,
                           (int)a->ngroups, P, N, (int)a->dt_softplus);
        return launched();
    };
    if (need <= 4) return launch(std::integral_constant<int, 4>{});
    if (need <= 8) return launch(std::integral_constant<int, 8>{});
    if (need <= 16) return launch(std::integral_constant<int, 16>{});
    if (need <= 32) return launch(std::integral_constant<int, 32>{});
    return launch(std::integral_constant<int, 64>{});
}

template <typename E>
ssd_status run_conv(const ssd_conv_args *a, hipStream_t st)
{
    const int CX = (int)(a->nheads * a->headdim), CG = (int)(a->ngroups * a->dstate);
    const int64_t nb = (a->seqlen + kConvTB - 1) / kConvTB;
    const int64_t items = a->batch * nb * ((CX + 2 * CG) / (16 / (int)sizeof(E)));   // one 16-byte vector each
    auto launch = [&](auto kk) {
        constexpr int K = decltype(kk)::value;
        if (a->seq_idx)
            hipLaunchKernelGGL((k_conv1d_silu<E, K, true>), dim3(grid1(items, kThreads)), dim3(kThreads), 0, st,
                               (const E *)a->xbc, a->weight, a->bias, a->seq_idx, (E *)a->x, (E *)a->B,
                               (E *)a->C, (int)a->seqlen, CX, CG, items);
        else
            hipLaunchKernelGGL((k_conv1d_silu<E, K, false>), dim3(grid1(items, kThreads)), dim3(kThreads), 0, st,
                               (const E *)a->xbc, a->weight, a->bias, a->seq_idx, (E *)a->x, (E *)a->B,
                               (E *)a->C, (int)a->seqlen, CX, CG, items);
        return launched();
    };
    switch (a->width) {
    case 1: return launch(std::integral_constant<int, 1>{});
    case 2: return launch(std::integral_constant<int, 2>{});
    case 3: return launch(std::integral_constant<int, 3>{});
    default: return launch(std::integral_constant<int, 4>{});
    }
}

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------
struct BwdWorkspace {
    size_t delta, cs, cb, states, gstates, cbr, yo, zo, xyp, rpart, cpart, bnd, dyx,
        mrow, mcol, dA_part, dD_part, mpart, total;
};

// Workgroups of k_bwd_m split the group's heads hsplit ways when its tiles alone
// would leave the GPU short of workgroups (about 1024 wanted: 256 CUs, four
// each; every split adds an fp32 tile of partial sums to write and read back);
// every split keeps at least one head.
int64_t bwd_m_hsplit(const Shape &s)
{
    const int64_t qt = s.Q / 64, tiles = qt * (qt + 1) / 2 * s.nc * s.G * s.b;
    const int64_t hpg = s.H / s.G;
    int64_t k = (1024 + tiles - 1) / tiles;
    if (k > hpg) k = hpg;
    return k < 1 ? 1 : k;
}

BwdWorkspace bwd_workspace_layout(const Shape &s)
{
    BwdWorkspace w;
    const size_t dcs = (size_t)(s.b * s.H * s.nc * s.Q) * 4;
    const size_t cbs = (size_t)(s.b * s.nc * s.G * s.Q * (s.Q + 2 * nt_of(s.N))) * s.esz;
    const size_t sts = (size_t)(s.b * s.nc * s.H * s.P * s.N) * s.esz;
    const size_t ms = (size_t)(s.b * s.nc * s.G * s.Q * s.Q) * s.esz;
    const size_t bh = (size_t)(s.b * s.H) * 4;
    const size_t ntp = (size_t)((s.P + 63) / 64), qt = (size_t)(s.Q / 64);
    size_t o = 0;
    auto take = [&](size_t n) { const size_t at = o; o = align256(o + n); return at; };
    w.delta = take(dcs);
    w.cs = take(dcs);
    w.cb = take(cbs);
    w.states = take(sts);
    w.gstates = take(sts);
    w.cbr = take(cbs);
    w.yo = take(ntp * dcs);
    w.zo = take(ntp * dcs);
    w.xyp = take(ntp * dcs);
    w.rpart = take(qt * dcs);
    w.cpart = take(qt * dcs);
    w.bnd = take((size_t)(s.b * s.H * s.nc) * (size_t)(s.P * s.N / 256) * 4);   // per (b, h, c): PN / 256 partials
    w.dyx = take(dcs * ntp);   // one slice per 64-wide p tile
    w.mrow = take(ms);
    w.mcol = take(ms);
    w.dA_part = take(bh * (size_t)s.nc);
    w.dD_part = take(bh * (size_t)s.nc);
    const int64_t hs = bwd_m_hsplit(s);
    w.mpart = take(hs > 1 ? (size_t)hs * (size_t)(s.b * qt * (qt + 1) / 2 * s.nc * s.G) * 4096 * 4 : 0);
    w.total = o;
    return w;
}

template <typename E>
ssd_status run_state_grad(const Shape &s, const ssd_fwd_args *ar, const float *cs, const E *cbr, E *u,
                          hipStream_t st, const int32_t *cseg = nullptr, const int2 *cmap = nullptr)
{
    const int ntp = (int)((s.P + 63) / 64);
    dim3 grid((unsigned)(s.nc * s.H * ntp), (unsigned)s.b);
    return with_q(s.Q, [&](auto q) {
        return with_nt(s.N, [&](auto nt) {
            constexpr int Q = decltype(q)::value, NT = decltype(nt)::value;
            hipLaunchKernelGGL((k_chunk_state<E, Q, NT, false, true>), grid, dim3(kThreads), 0, st, (const E *)ar->x,
                               cbr, (const E *)nullptr, ar->A, (const int32_t *)nullptr, (float *)nullptr,
                               const_cast<float *>(cs), u, (int32_t *)nullptr, 0, (int)s.T, (int)s.H, (int)s.G,
                               (int)s.P, (int)s.N, (int)s.nc, ntp, 0, cseg, cmap);
            return launched();
        });
    });
}

template <typename E>
ssd_status run_passing_rev(const Shape &s, const float *cs, E *gstates, const float *dfinal, float *dinit,
                           const E *hin, float *bnd_part, hipStream_t st, const int32_t *cseg = nullptr)
{
    const int64_t PN = s.P * s.N;
    constexpr int VE = 4;   // so PN / (64 VE) = PN / 256 boundary partials per (b, h, c)
    const int64_t vecs = s.b * s.H * PN / VE;
    hipLaunchKernelGGL((k_state_passing<E, VE, true>), dim3(grid1(vecs, kThreads)), dim3(kThreads), 0, st, gstates,
                       cs, dfinal, dinit, (const int32_t *)nullptr, (int)s.T, (int)s.H, PN, (int)s.nc, (int)s.Q,
                       vecs, hin, bnd_part, cseg);
    return launched();
}

// The stage boundaries of one backward call, for ssd_bwd_stage_times: an event
// recorded on the stream before the first stage and after each named one.
// The events are made by start(), after every argument check has passed.
struct StageMarks {
    hipEvent_t ev[SSD_BWD_MAX_STAGES + 1];
    const char *name[SSD_BWD_MAX_STAGES];
    int made = 0, n = 0;
    bool ok = true;
    hipStream_t st = nullptr;
    ssd_status start(hipStream_t stream)
    {
        st = stream;
        for (; made <= SSD_BWD_MAX_STAGES; ++made)
            if (hipEventCreate(&ev[made]) != hipSuccess) return SSD_ERR_HIP;
        return hipEventRecord(ev[0], st) == hipSuccess ? SSD_OK : SSD_ERR_HIP;
    }
    ~StageMarks()
    {
        for (int i = 0; i < made; ++i) (void)hipEventDestroy(ev[i]);
    }
    void mark(const char *nm)
    {
        if (n >= SSD_BWD_MAX_STAGES || hipEventRecord(ev[n + 1], st) != hipSuccess) {
            ok = false;
            return;
        }
        name[n++] = nm;
    }
};

// Packed streams, on the layout in which every segment starts at a chunk start:
// cseg = the per-chunk segment ids, cmap = each chunk's first token and token
// count in the caller's stream (see chunk_rows), pstart / plen = each segment's
// padded start and token count (nseq of them); g->dfinal_states is then
// [nseq,H,P,N] and g->fwd_workspace is not used.
struct PackedSegs {
    const int32_t *cseg;
    const int2 *cmap;
    const int32_t *pstart, *plen;
    int nseq;
};

template <typename E>
ssd_status bwd_typed(const Shape &s, const ssd_fwd_args *a, const ssd_bwd_args *g, const BwdWorkspace &w,
                     hipStream_t st, const PackedSegs *pk = nullptr, StageMarks *sm = nullptr)
{
    const int32_t *cseg = pk ? pk->cseg : nullptr;
    const int2 *cmap = pk ? pk->cmap : nullptr;
    auto mark = [&](const char *nm) { if (sm) sm->mark(nm); };
    char *ws = static_cast<char *>(g->workspace);
    auto F32 = [&](size_t off) { return reinterpret_cast<float *>(ws + off); };
    auto EP = [&](size_t off) { return reinterpret_cast<E *>(ws + off); };
    float *delta = F32(w.delta), *cs = F32(w.cs);
    float *yo = F32(w.yo), *zo = F32(w.zo), *xyp = F32(w.xyp), *rpart = F32(w.rpart), *cpart = F32(w.cpart);
    float *bnd = F32(w.bnd), *dyx = F32(w.dyx), *dA_part = F32(w.dA_part), *dD_part = F32(w.dD_part);
    E *cb = EP(w.cb), *states = EP(w.states), *gstates = EP(w.gstates), *cbr = EP(w.cbr);
    E *mrow = EP(w.mrow), *mcol = EP(w.mcol);
    ssd_status r;
    ssd_fwd_args f = *a;
    f.final_states = nullptr;
    if (g->fwd_workspace && !cseg) {
        // 1. the forward's chunk intermediates, as its own call left them (read only)
        const Workspace fw = workspace_layout(s);
        char *fws = const_cast<char *>(static_cast<const char *>(g->fwd_workspace));
        delta = reinterpret_cast<float *>(fws + fw.delta);
        cs = reinterpret_cast<float *>(fws + fw.cs);
        cb = reinterpret_cast<E *>(fws + fw.cb);
        states = reinterpret_cast<E *>(fws + fw.states);
    } else {
        // 1. the forward's chunk intermediates again: delta, cs, CB, the entering states
        if ((r = run_cb<E>(s, &f, cb, st, false, cseg, cmap)) != SSD_OK) return r;
        mark("chunk_cb");
        if ((r = run_state<E>(s, &f, delta, cs, cb, states, nullptr, st, cseg, cmap)) != SSD_OK) return r;
        mark("chunk_state");
        if ((r = run_passing<E>(s, &f, cs, states, nullptr, st, cseg)) != SSD_OK) return r;
        mark("state_passing");
    }
    // 2-3. reversed-order problem: every chunk's tokens in reversed order, x <- dy,
    //    B <- C, C <- B, unit step size, no skip term; its output is turned into
    //    dx = Delta y' + D dy in original order.  No reversed copies: the kernels
    //    read dy, B, C and cs reversed themselves.
    ssd_fwd_args rv = *a;
    rv.x = g->dy;
    rv.B = a->C;
    rv.C = a->B;
    rv.D = nullptr;
    rv.y = g->dx;
    rv.initial_states = nullptr;
    rv.final_states = nullptr;
    if ((r = run_cb<E>(s, &rv, cbr, st, true, cseg, cmap)) != SSD_OK) return r;
    mark("chunk_cb_rev");
    // 4. per-chunk gradient states U_c, then the reverse scan to G_c and dinit
    if ((r = run_state_grad<E>(s, &rv, cs, cbr, gstates, st, cseg, cmap)) != SSD_OK) return r;
    mark("chunk_state_grad");
    if (cseg) {
        // packed layout: each segment's dfinal into the U slot of the chunk after its last
        const int64_t PN = s.P * s.N;
        const unsigned nb = grid1(s.H * PN / 4, 256);
        hipLaunchKernelGGL(k_bwd_inject_dfinal<E>, dim3(nb * (unsigned)pk->nseq), dim3(256), 0, st, gstates,
                           g->dfinal_states, pk->pstart, pk->plen, (int)s.H, PN, (int)s.nc, (int)s.Q, (int)nb);
        if ((r = launched()) != SSD_OK) return r;
        mark("inject_dfinal");
    }
    //    (with the boundary terms e^{cs_last} <G_c, Hin_c> of dl, as partial sums)
    if ((r = run_passing_rev<E>(s, cs, gstates, g->dfinal_states, g->dinitial_states, states, bnd, st, cseg)) !=
        SSD_OK)
        return r;
    mark("state_passing_rev");
    // 5. y' (reversed order) by the forward's chunk scan, with x . (G term) and x . y';
    //    it writes dx = Delta y' + D dy, and dy . x per (token, head)
    if ((r = run_scan_dot<E, 2, false>(s, &rv, nullptr, cs, cbr, gstates, (const E *)a->x, zo, xyp, st, delta,
                                       a->D, dyx, cseg, cmap)) != SSD_OK)
        return r;
    mark("chunk_scan_dx");
    // 6. dy . (entering-state term of y), from the forward's entering states
    if ((r = run_scan_dot<E, 1, true>(s, &f, delta, cs, cb, states, (const E *)g->dy, yo, nullptr, st, nullptr,
                                      nullptr, nullptr, cseg, cmap)) != SSD_OK)
        return r;
    mark("chunk_scan_dy_hin");
    // 7. M (summed over the group's heads) with the row / column sums of S; with
    //    the heads split over several workgroups, their parts are added after
    const int qt = (int)(s.Q / 64), ntri = qt * (qt + 1) / 2;
    const int nnt = (int)((s.N + 63) / 64);
    const int hsplit = (int)bwd_m_hsplit(s);
    float *mpart = F32(w.mpart);
    if ((r = with_q(s.Q, [&](auto q) {
             return with_nt(s.N, [&](auto nt) {
                 constexpr int Q = decltype(q)::value, NT = decltype(nt)::value;
                 hipLaunchKernelGGL((k_bwd_m<E, Q, NT>), dim3((unsigned)(ntri * s.nc * s.G * hsplit), (unsigned)s.b),
                                    dim3(kThreads), 0, st, (const E *)g->dy, (const E *)a->x, delta, cs, (const E *)cb,
                                    mrow, mcol, rpart, cpart, (int)s.T, (int)s.H, (int)s.G, (int)s.P, (int)s.nc,
                                    hsplit, mpart, cseg, cmap);
                 if (hsplit > 1)
                     hipLaunchKernelGGL((k_bwd_m_reduce<E, Q>), dim3((unsigned)(ntri * s.nc * s.G), (unsigned)s.b),
                                        dim3(kThreads), 0, st, (const float *)mpart, mrow, mcol, (int)s.G, (int)s.nc,
                                        hsplit, cseg);
                 return launched();
             });
         })) != SSD_OK)
        return r;
    mark("m_rows_cols");
    // 8. dl, ddt, dA, dD
    const int64_t dlrows = s.b * s.H * s.nc;
    with_q(s.Q, [&](auto q) {
        constexpr int Q = decltype(q)::value;
        hipLaunchKernelGGL((k_bwd_dl<E, Q>), dim3(grid1(dlrows, kThreads / 64)), dim3(kThreads), 0, st, rpart, cpart,
                           yo, zo, xyp, bnd, dyx, delta, (const E *)a->dt, a->A, (E *)g->ddt, dA_part, dD_part,
                           (int)s.T, (int)s.H, (int)s.nc, (int)((s.P + 63) / 64), dlrows, (int)a->dt_softplus,
                           s.P * s.N / 256, cseg, cmap);
        return SSD_OK;
    });
    hipLaunchKernelGGL(k_bwd_sum_heads, dim3((unsigned)s.H), dim3(64), 0, st, dA_part, dD_part, g->dA, g->dD,
                       (int)s.b, (int)s.H, (int)s.nc);
    if ((r = launched()) != SSD_OK) return r;
    mark("dl_ddt_dA_dD");
    // 9. dC and dB
    return with_q(s.Q, [&](auto q) {
        constexpr int Q = decltype(q)::value;
        const dim3 grid((unsigned)(s.nc * s.G * qt * nnt), (unsigned)s.b);
        hipLaunchKernelGGL((k_bwd_bc<E, Q, 0>), grid, dim3(kThreads), 0, st, (const E *)a->B, (const E *)mrow,
                           (const E *)states, (const E *)g->dy, delta, cs, (E *)g->dC, (int)s.T, (int)s.H, (int)s.G,
                           (int)s.P, (int)s.N, (int)s.nc, nnt, cseg, cmap);
        mark("dC");
        hipLaunchKernelGGL((k_bwd_bc<E, Q, 1>), grid, dim3(kThreads), 0, st, (const E *)a->C, (const E *)mcol,
                           (const E *)gstates, (const E *)a->x, delta, cs, (E *)g->dB, (int)s.T, (int)s.H,
                           (int)s.G, (int)s.P, (int)s.N, (int)s.nc, nnt, cseg, cmap);
        mark("dB");
        return launched();
    });
}

// ---------------------------------------------------------------------------
// backward of a packed stream
// ---------------------------------------------------------------------------
// The chunked backward runs on a layout in which every segment starts at a
// chunk start (k_bwd_seg_ranges, k_bwd_chunk_map), with the state carry cut
// between segments and each segment's final-state gradient entering after its
// last chunk.  The layout is never built: each chunk reads its tokens from the
// caller's stream through the chunk map and writes its gradients to the tokens'
// own rows.  Tp bounds the padded length from the host side: each of at most
// nseq segments adds fewer than Q tokens of padding.
struct PackedBwd {
    Shape sp;   // the padded problem (batch 1, no seq_idx)
    size_t seg_end, ostart, len, pstart, cseg, cmap, inner, total;
    BwdWorkspace w;
};

PackedBwd packed_bwd_layout(const Shape &s)
{
    PackedBwd k;
    k.sp = s;
    k.sp.packed = false;
    k.sp.nseq = 0;
    const int64_t tp = ((s.T + s.nseq * (s.Q - 1)) + s.Q - 1) / s.Q * s.Q;
    k.sp.T = tp;
    k.sp.nc = tp / s.Q;
    const size_t ids = (size_t)s.nseq * 4;
    size_t o = 0;
    auto take = [&](size_t n) { const size_t at = o; o = align256(o + n); return at; };
    k.seg_end = take(ids);
    k.ostart = take(ids);
    k.len = take(ids);
    k.pstart = take(ids);
    k.cseg = take((size_t)k.sp.nc * 4);
    k.cmap = take((size_t)k.sp.nc * 8);
    k.inner = o;
    k.w = bwd_workspace_layout(k.sp);
    k.total = align256(o + k.w.total);
    return k;
}

template <typename E>
ssd_status bwd_packed(const Shape &s, const ssd_fwd_args *a, const ssd_bwd_args *g, const PackedBwd &k,
                      hipStream_t st, StageMarks *sm = nullptr)
{
    char *ws = static_cast<char *>(g->workspace);
    auto I32 = [&](size_t off) { return reinterpret_cast<int32_t *>(ws + off); };
    const int T = (int)s.T, Q = (int)s.Q, nseq = (int)s.nseq, ncp = (int)k.sp.nc;
    int32_t *seg_end = I32(k.seg_end), *ostart = I32(k.ostart), *len = I32(k.len), *pstart = I32(k.pstart);
    int32_t *cseg = I32(k.cseg);
    int2 *cmap = reinterpret_cast<int2 *>(ws + k.cmap);
    // the padded layout, as a map from its chunks to the caller's tokens
    hipLaunchKernelGGL(k_seg_end, dim3(grid1(T, 256)), dim3(256), 0, st, a->seq_idx, seg_end, T, nseq);
    hipLaunchKernelGGL(k_bwd_seg_ranges, dim3(1), dim3(64), 0, st, seg_end, ostart, len, pstart, nseq, Q);
    hipLaunchKernelGGL(k_bwd_chunk_map, dim3(grid1(ncp, 256)), dim3(256), 0, st, ostart, len, pstart, cseg, cmap,
                       nseq, Q, ncp);
    if (launched() != SSD_OK) return SSD_ERR_HIP;
    if (sm) sm->mark("chunk_map");
    // the chunked backward on the padded stream: every chunk reads its tokens
    // from the caller's tensors and writes their gradients in place
    ssd_fwd_args fp = *a;
    fp.seq_idx = nullptr;
    fp.nseq = 0;
    fp.y = nullptr;
    ssd_bwd_args gp = *g;
    gp.workspace = ws + k.inner;
    gp.workspace_bytes = k.w.total;
    gp.fwd_workspace = nullptr;
    const PackedSegs pk{cseg, cmap, pstart, len, nseq};
    return bwd_typed<E>(k.sp, &fp, &gp, k.w, st, &pk, sm);
}

// ---------------------------------------------------------------------------
// static scratch for ssd_fwd_noalloc
// ---------------------------------------------------------------------------
// The forward's workspace for callers that cannot allocate.  Every GPU the
// library runs on holds its own copy of this array from module load until the
// process ends.  In host code `scratch` only names the symbol: its device
// address on the current device comes from hipGetSymbolAddress, taken once per
// device and cached, and only that address is ever handed to a kernel.
constexpr size_t kScratchBytes = SSD_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (nullptr on failure).
void *scratch_address()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

const char *const kStatusText[] = {
    "ok",
    "a required pointer is NULL",
    "a size is outside the supported range (P and N multiples of 16, N <= 256)",
    "dtype must be SSD_DTYPE_F32 or SSD_DTYPE_BF16",
    "chunk must be 64, 128 or 256",
    "nheads must be a multiple of ngroups",
    "seq_idx requires batch == 1 and nseq >= 1",
    "workspace is smaller than ssd_fwd_workspace_size",
    "a tensor pointer is not 16-byte aligned",
    "an output overlaps an input or another output",
    "a HIP kernel launch failed",
    "the problem needs more scratch than the library's static buffer holds (ssd_fwd_noalloc)",
};

ssd_status bwd_entry(const ssd_fwd_args *args, const ssd_bwd_args *g, void *stream, StageMarks *sm)
{
    Shape s;
    ssd_status r = parse_shape(args, &s);
    if (r != SSD_OK) return r;
    if (!g) return SSD_ERR_NULL_POINTER;
    if ((r = check_pointers(args, s, kNeedX | kNeedDt | kNeedB | kNeedC)) != SSD_OK) return r;
    const bool empty = s.T == 0;
    if (!g->dA) return SSD_ERR_NULL_POINTER;
    if (!empty && (!args->y || !g->dy || !g->dx || !g->ddt || !g->dB || !g->dC)) return SSD_ERR_NULL_POINTER;
    const void *ptrs[] = {args->y, g->dy, g->dfinal_states, g->dx, g->ddt, g->dA, g->dB, g->dC, g->dD,
                          g->dinitial_states, g->workspace, g->fwd_workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return SSD_ERR_MISALIGNED;
    const Sizes z = tensor_sizes(s);
    const size_t st = (size_t)(s.b * s.H * s.P * s.N) * 4;   // dinitial_states
    // packed streams: the backward always recomputes on its own layout, so a
    // forward workspace is not read
    const void *fwd_ws = s.packed ? nullptr : g->fwd_workspace;
    const size_t wtotal = s.packed ? packed_bwd_layout(s).total : bwd_workspace_layout(s).total;
    const size_t fws = workspace_layout(s).total;
    if (!empty) {
        if (!g->workspace) return SSD_ERR_NULL_POINTER;
        if (g->workspace_bytes < wtotal) return SSD_ERR_WORKSPACE_TOO_SMALL;
        if (fwd_ws && g->fwd_workspace_bytes < fws) return SSD_ERR_WORKSPACE_TOO_SMALL;
    }
    const Range ins[] = {{args->x, z.x}, {args->dt, z.dt}, {args->A, z.A}, {args->B, z.bc}, {args->C, z.bc},
                         {args->D, z.D}, {args->initial_states, z.init}, {args->seq_idx, z.seq}, {args->y, z.y},
                         {g->dy, z.x}, {g->dfinal_states, z.fin}, {fwd_ws, fws}};
    const Range outs[] = {{g->dx, z.x}, {g->ddt, z.dt}, {g->dA, z.A}, {g->dB, z.bc}, {g->dC, z.bc},
                          {g->dD, z.D}, {g->dinitial_states, st}, {empty ? nullptr : g->workspace, wtotal}};
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        for (const Range &in : ins)
            if (overlaps(outs[i], in)) return SSD_ERR_ALIASING;
        for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
            if (overlaps(outs[i], outs[j])) return SSD_ERR_ALIASING;
    }
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (empty) {
        // no tokens: the final state is the initial state, nothing else depends on the inputs
        hipLaunchKernelGGL(k_fill_final, dim3(grid1(s.H, 256)), dim3(256), 0, hs, g->dA, (const float *)nullptr, s.H);
        if (g->dD)
            hipLaunchKernelGGL(k_fill_final, dim3(grid1(s.H, 256)), dim3(256), 0, hs, g->dD, (const float *)nullptr, s.H);
        // (an empty packed stream has no segment that could receive the initial state)
        if (g->dinitial_states)
            hipLaunchKernelGGL(k_fill_final, dim3(grid1(s.b * s.H * s.P * s.N, 256)), dim3(256), 0, hs,
                               g->dinitial_states, s.packed ? nullptr : g->dfinal_states, s.b * s.H * s.P * s.N);
        return launched();
    }
    if (sm && (r = sm->start(hs)) != SSD_OK) return r;
    if (s.packed) {
        const PackedBwd k = packed_bwd_layout(s);
        return s.dtype == SSD_DTYPE_BF16 ? bwd_packed<bf16>(s, args, g, k, hs, sm)
                                         : bwd_packed<float>(s, args, g, k, hs, sm);
    }
    const BwdWorkspace w = bwd_workspace_layout(s);
    return s.dtype == SSD_DTYPE_BF16 ? bwd_typed<bf16>(s, args, g, w, hs, nullptr, sm)
                                     : bwd_typed<float>(s, args, g, w, hs, nullptr, sm);
}

}  // namespace

extern "C" {

int ssd_abi_version(void) { return SSD_ABI_VERSION; }

const char *ssd_status_string(int32_t status)
{
    if (status < 0 || status >= (int32_t)(sizeof(kStatusText) / sizeof(kStatusText[0]))) return "unknown status";
    return kStatusText[status];
}

ssd_status ssd_fwd_workspace_size(const ssd_fwd_args *args, size_t *bytes)
{
    Shape s;
    ssd_status r = parse_shape(args, &s);
    if (r != SSD_OK) return r;
    if (!bytes) return SSD_ERR_NULL_POINTER;
    *bytes = workspace_layout(s).total;
    return SSD_OK;
}

ssd_status ssd_fwd(const ssd_fwd_args *args, void *stream)
{
    Shape s;
    ssd_status r = parse_shape(args, &s);
    if (r != SSD_OK) return r;
    if ((r = check_pointers(args, s, kNeedX | kNeedDt | kNeedB | kNeedC | kNeedY | kCheckFinal)) != SSD_OK)
        return r;
    const Workspace w = workspace_layout(s);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (s.T == 0) return fill_final(s, args, st);
    if (!args->workspace) return SSD_ERR_NULL_POINTER;
    if (args->workspace_bytes < w.total) return SSD_ERR_WORKSPACE_TOO_SMALL;
    const Sizes z = tensor_sizes(s);
    const Range ws{args->workspace, w.total};
    const Range others[] = {{args->x, z.x}, {args->dt, z.dt}, {args->A, z.A}, {args->B, z.bc}, {args->C, z.bc},
                            {args->D, z.D}, {args->initial_states, z.init}, {args->seq_idx, z.seq},
                            {args->y, z.y}, {args->final_states, z.fin}};
    for (const Range &o : others)
        if (overlaps(ws, o)) return SSD_ERR_ALIASING;
    return s.dtype == SSD_DTYPE_BF16 ? fwd_typed<bf16>(s, args, w, st) : fwd_typed<float>(s, args, w, st);
}

ssd_status ssd_fwd_noalloc(const ssd_fwd_args *args, void *stream)
{
    Shape s;
    ssd_status r = parse_shape(args, &s);
    if (r != SSD_OK) return r;
    if ((r = check_pointers(args, s, kNeedX | kNeedDt | kNeedB | kNeedC | kNeedY | kCheckFinal)) != SSD_OK)
        return r;
    const Workspace w = workspace_layout(s);
    if (w.total > kScratchBytes) return SSD_ERR_SCRATCH_TOO_SMALL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (s.T == 0) return fill_final(s, args, st);
    void *ws = scratch_address();
    if (!ws) return SSD_ERR_HIP;
    // The forward writes every workspace byte it later reads (delta, cs, the
    // chunk_cb buffer's lower tiles, the states, the segment ends), so nothing in
    // the static buffer has to be cleared between calls.
    ssd_fwd_args a = *args;
    a.workspace = ws;
    a.workspace_bytes = kScratchBytes;
    return s.dtype == SSD_DTYPE_BF16 ? fwd_typed<bf16>(s, &a, w, st) : fwd_typed<float>(s, &a, w, st);
}

ssd_status ssd_chunk_cumsum(const ssd_fwd_args *args, float *delta, float *cs, void *stream)
{
    Shape s;
    ssd_status r = parse_shape(args, &s);
    if (r != SSD_OK) return r;
    if ((r = check_pointers(args, s, kNeedDt)) != SSD_OK) return r;
    if (s.T == 0) return SSD_OK;
    if (!delta || !cs) return SSD_ERR_NULL_POINTER;
    if (!aligned16(delta) || !aligned16(cs)) return SSD_ERR_MISALIGNED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    return s.dtype == SSD_DTYPE_BF16 ? run_cumsum<bf16>(s, args, delta, cs, st)
                                     : run_cumsum<float>(s, args, delta, cs, st);
}

ssd_status ssd_chunk_cb(const ssd_fwd_args *args, void *cb, void *stream)
{
    Shape s;
    ssd_status r = parse_shape(args, &s);
    if (r != SSD_OK) return r;
    if ((r = check_pointers(args, s, kNeedB | kNeedC)) != SSD_OK) return r;
    if (s.T == 0) return SSD_OK;
    if (!cb) return SSD_ERR_NULL_POINTER;
    if (!aligned16(cb)) return SSD_ERR_MISALIGNED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    return s.dtype == SSD_DTYPE_BF16 ? run_cb<bf16>(s, args, (bf16 *)cb, st)
                                     : run_cb<float>(s, args, (float *)cb, st);
}

ssd_status ssd_chunk_state(const ssd_fwd_args *args, float *delta, float *cs, const void *cb, void *states,
                           void *stream)
{
    Shape s;
    ssd_status r = parse_shape(args, &s);
    if (r != SSD_OK) return r;
    if ((r = check_pointers(args, s, kNeedX | kNeedDt | kNeedB)) != SSD_OK) return r;
    if (s.T == 0) return SSD_OK;
    if (!delta || !cs || !cb || !states) return SSD_ERR_NULL_POINTER;
    if (!aligned16(delta) || !aligned16(cs) || !aligned16(cb) || !aligned16(states)) return SSD_ERR_MISALIGNED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    return s.dtype == SSD_DTYPE_BF16
               ? run_state<bf16>(s, args, delta, cs, (const bf16 *)cb, (bf16 *)states, nullptr, st)
               : run_state<float>(s, args, delta, cs, (const float *)cb, (float *)states, nullptr, st);
}

ssd_status ssd_state_passing(const ssd_fwd_args *args, const float *cs, void *states, void *stream)
{
    Shape s;
    ssd_status r = parse_shape(args, &s);
    if (r != SSD_OK) return r;
    if ((r = check_pointers(args, s, kCheckFinal)) != SSD_OK) return r;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (s.T == 0) return s.packed ? SSD_OK : fill_final(s, args, st);
    if (!cs || !states) return SSD_ERR_NULL_POINTER;
    if (!aligned16(cs) || !aligned16(states)) return SSD_ERR_MISALIGNED;
    float *fin = s.packed ? nullptr : args->final_states;
    return s.dtype == SSD_DTYPE_BF16 ? run_passing<bf16>(s, args, cs, (bf16 *)states, fin, st)
                                     : run_passing<float>(s, args, cs, (float *)states, fin, st);
}

ssd_status ssd_check_seq_idx(const int32_t *seq_idx, int64_t seqlen, int64_t nseq, int32_t *first_bad, void *stream)
{
    if (!first_bad || (seqlen > 0 && !seq_idx)) return SSD_ERR_NULL_POINTER;
    if (seqlen < 0 || seqlen > INT32_MAX) return SSD_ERR_BAD_SHAPE;
    if (nseq < 1) return SSD_ERR_SEQ_IDX;
    if (!aligned4(seq_idx) || !aligned4(first_bad)) return SSD_ERR_MISALIGNED;
    hipLaunchKernelGGL(k_check_seq_idx, dim3(1), dim3(1024), 0, static_cast<hipStream_t>(stream), seq_idx, seqlen,
                       nseq, first_bad);
    return launched();
}

ssd_status ssd_seq_final_states(const ssd_fwd_args *args, const float *delta, const float *cs,
                                const void *states, int32_t *seg_end, void *stream)
{
    Shape s;
    ssd_status r = parse_shape(args, &s);
    if (r != SSD_OK) return r;
    if (!s.packed) return SSD_ERR_SEQ_IDX;
    if ((r = check_pointers(args, s, kNeedX | kNeedB | kCheckFinal)) != SSD_OK) return r;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!args->final_states) return SSD_ERR_NULL_POINTER;
    if (s.T == 0) return fill_final(s, args, st);
    if (!delta || !cs || !states || !seg_end) return SSD_ERR_NULL_POINTER;
    if (!aligned16(delta) || !aligned16(cs) || !aligned16(states) || !aligned16(seg_end))
        return SSD_ERR_MISALIGNED;
    return s.dtype == SSD_DTYPE_BF16
               ? run_seq_final<bf16>(s, args, delta, cs, (const bf16 *)states, seg_end, false, st)
               : run_seq_final<float>(s, args, delta, cs, (const float *)states, seg_end, false, st);
}

ssd_status ssd_chunk_scan(const ssd_fwd_args *args, const float *delta, const float *cs, const void *cb,
                          const void *states, void *stream)
{
    Shape s;
    ssd_status r = parse_shape(args, &s);
    if (r != SSD_OK) return r;
    if ((r = check_pointers(args, s, kNeedX | kNeedC | kNeedY)) != SSD_OK) return r;
    if (s.T == 0) return SSD_OK;
    if (!delta || !cs || !cb || !states) return SSD_ERR_NULL_POINTER;
    if (!aligned16(delta) || !aligned16(cs) || !aligned16(cb) || !aligned16(states)) return SSD_ERR_MISALIGNED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    return s.dtype == SSD_DTYPE_BF16
               ? run_scan<bf16>(s, args, delta, cs, (const bf16 *)cb, (const bf16 *)states, st)
               : run_scan<float>(s, args, delta, cs, (const float *)cb, (const float *)states, st);
}

ssd_status ssd_step(const ssd_step_args *a, void *stream)
{
    if (!a) return SSD_ERR_NULL_POINTER;
    if (a->dtype != SSD_DTYPE_F32 && a->dtype != SSD_DTYPE_BF16) return SSD_ERR_BAD_DTYPE;
    if (a->batch < 1 || a->nheads < 1 || a->headdim < 16 || a->dstate < 16 || a->ngroups < 1)
        return SSD_ERR_BAD_SHAPE;
    if (a->headdim % 16 != 0 || a->dstate % 16 != 0 || a->dstate > kMaxStateDim || a->headdim > 4096)
        return SSD_ERR_BAD_SHAPE;
    if (a->batch > kMaxDim || a->nheads > kMaxDim || a->batch * a->nheads > INT32_MAX) return SSD_ERR_BAD_SHAPE;
    if (a->nheads % a->ngroups != 0) return SSD_ERR_GROUPS;
    if (!a->x || !a->dt || !a->A || !a->B || !a->C || !a->state || !a->y) return SSD_ERR_NULL_POINTER;
    const void *ptrs[] = {a->x, a->dt, a->A, a->B, a->C, a->D, a->state, a->y};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return SSD_ERR_MISALIGNED;
    const size_t esz = a->dtype == SSD_DTYPE_BF16 ? 2 : 4;
    const int64_t bH = a->batch * a->nheads;
    const Range xr{a->x, (size_t)(bH * a->headdim) * esz}, dtr{a->dt, (size_t)bH * esz},
        Ar{a->A, (size_t)a->nheads * 4}, Br{a->B, (size_t)(a->batch * a->ngroups * a->dstate) * esz},
        Cr{a->C, (size_t)(a->batch * a->ngroups * a->dstate) * esz}, Dr{a->D, (size_t)a->nheads * 4},
        sr{a->state, (size_t)(bH * a->headdim * a->dstate) * 4}, yr{a->y, xr.n};
    const Range ins[] = {xr, dtr, Ar, Br, Cr, Dr};
    for (const Range &o : ins)
        if (overlaps(sr, o) || overlaps(yr, o)) return SSD_ERR_ALIASING;
    if (overlaps(sr, yr)) return SSD_ERR_ALIASING;
    hipStream_t st = static_cast<hipStream_t>(stream);
    return a->dtype == SSD_DTYPE_BF16 ? run_step<bf16>(a, st) : run_step<float>(a, st);
}

ssd_status ssd_bwd_workspace_size(const ssd_fwd_args *args, size_t *bytes)
{
    Shape s;
    ssd_status r = parse_shape(args, &s);
    if (r != SSD_OK) return r;
    if (!bytes) return SSD_ERR_NULL_POINTER;
    *bytes = s.packed ? packed_bwd_layout(s).total : bwd_workspace_layout(s).total;
    return SSD_OK;
}

ssd_status ssd_bwd(const ssd_fwd_args *args, const ssd_bwd_args *g, void *stream)
{
    return bwd_entry(args, g, stream, nullptr);
}

ssd_status ssd_bwd_stage_times(const ssd_fwd_args *args, const ssd_bwd_args *grads, void *stream, int max_stages,
                               float *ms, const char **names, int *nstages)
{
    if (!ms || !names || !nstages) return SSD_ERR_NULL_POINTER;
    if (max_stages < SSD_BWD_MAX_STAGES) return SSD_ERR_BAD_SHAPE;
    *nstages = 0;
    StageMarks sm;
    ssd_status r = bwd_entry(args, grads, stream, &sm);
    if (r == SSD_OK && !sm.ok) r = SSD_ERR_HIP;
    // an empty problem records no event: no stages
    if (r != SSD_OK || sm.n == 0) return r;
    if (hipEventSynchronize(sm.ev[sm.n]) != hipSuccess) return SSD_ERR_HIP;
    for (int i = 0; i < sm.n; ++i) {
        if (hipEventElapsedTime(&ms[i], sm.ev[i], sm.ev[i + 1]) != hipSuccess) return SSD_ERR_HIP;
        names[i] = sm.name[i];
    }
    *nstages = sm.n;
    return SSD_OK;
}

ssd_status ssd_fwd_gated(const ssd_fwd_args *args, const void *z, void *stream)
{
    Shape s;
    ssd_status r = parse_shape(args, &s);
    if (r != SSD_OK) return r;
    if ((r = check_pointers(args, s, kNeedX | kNeedDt | kNeedB | kNeedC | kNeedY | kCheckFinal)) != SSD_OK)
        return r;
    if (s.T > 0 && !z) return SSD_ERR_NULL_POINTER;
    if (z && !aligned16(z)) return SSD_ERR_MISALIGNED;
    const Sizes zs = tensor_sizes(s);
    const Range zr{z, zs.x};
    if (overlaps(zr, Range{args->y, zs.y}) || overlaps(zr, Range{args->final_states, zs.fin}))
        return SSD_ERR_ALIASING;
    const Workspace w = workspace_layout(s);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (s.T == 0) return fill_final(s, args, st);
    if (!args->workspace) return SSD_ERR_NULL_POINTER;
    if (args->workspace_bytes < w.total) return SSD_ERR_WORKSPACE_TOO_SMALL;
    const Range ws{args->workspace, w.total};
    const Range others[] = {{args->x, zs.x}, {args->dt, zs.dt}, {args->A, zs.A}, {args->B, zs.bc}, {args->C, zs.bc},
                            {args->D, zs.D}, {args->initial_states, zs.init}, {args->seq_idx, zs.seq},
                            {args->y, zs.y}, {args->final_states, zs.fin}, zr};
    for (const Range &o : others)
        if (overlaps(ws, o)) return SSD_ERR_ALIASING;
    return s.dtype == SSD_DTYPE_BF16 ? fwd_typed<bf16>(s, args, w, st, (const bf16 *)z)
                                     : fwd_typed<float>(s, args, w, st, (const float *)z);
}

ssd_status ssd_conv1d_silu(const ssd_conv_args *a, void *stream)
{
    if (!a) return SSD_ERR_NULL_POINTER;
    if (a->dtype != SSD_DTYPE_F32 && a->dtype != SSD_DTYPE_BF16) return SSD_ERR_BAD_DTYPE;
    if (a->batch < 1 || a->seqlen < 0 || a->nheads < 1 || a->headdim < 16 || a->ngroups < 1 || a->dstate < 16 ||
        a->width < 1 || a->width > 4)
        return SSD_ERR_BAD_SHAPE;
    if (a->headdim % 16 != 0 || a->dstate % 16 != 0 || a->batch > kMaxDim || a->seqlen > kMaxDim ||
        a->nheads > kMaxDim || a->headdim > kMaxDim || a->ngroups > kMaxDim || a->dstate > kMaxDim)
        return SSD_ERR_BAD_SHAPE;
    const int64_t CC = a->nheads * a->headdim + 2 * a->ngroups * a->dstate;
    if (CC > INT32_MAX / 4 || a->batch * a->seqlen > ((int64_t)1 << 40) / CC)
        return SSD_ERR_BAD_SHAPE;
    if (a->nheads % a->ngroups != 0) return SSD_ERR_GROUPS;
    if (a->seq_idx && a->batch != 1) return SSD_ERR_SEQ_IDX;
    if (a->seqlen == 0) return SSD_OK;
    if (!a->xbc || !a->weight || !a->x || !a->B || !a->C) return SSD_ERR_NULL_POINTER;
    const void *ptrs[] = {a->xbc, a->weight, a->bias, a->seq_idx, a->x, a->B, a->C};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return SSD_ERR_MISALIGNED;
    const size_t esz = a->dtype == SSD_DTYPE_BF16 ? 2 : 4;
    const int64_t bt = a->batch * a->seqlen;
    const Range in[] = {{a->xbc, (size_t)(bt * CC) * esz}, {a->weight, (size_t)(CC * a->width) * 4},
                        {a->bias, (size_t)CC * 4}, {a->seq_idx, (size_t)a->seqlen * 4}};
    const Range out[] = {{a->x, (size_t)(bt * a->nheads * a->headdim) * esz},
                         {a->B, (size_t)(bt * a->ngroups * a->dstate) * esz},
                         {a->C, (size_t)(bt * a->ngroups * a->dstate) * esz}};
    for (size_t i = 0; i < 3; ++i) {
        for (const Range &r : in)
            if (overlaps(out[i], r)) return SSD_ERR_ALIASING;
        for (size_t j = i + 1; j < 3; ++j)
            if (overlaps(out[i], out[j])) return SSD_ERR_ALIASING;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    return a->dtype == SSD_DTYPE_BF16 ? run_conv<bf16>(a, st) : run_conv<float>(a, st);
}

}  // extern "C"
