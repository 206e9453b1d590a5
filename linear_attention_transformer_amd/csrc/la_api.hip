// la_api.hip -- C ABI of the linear-attention library (declared in
// include/la.h): argument validation, segment planning, workspace layout and
// kernel dispatch.  See la_kernels.hpp for the method and its sources.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <type_traits>

#include "la.h"
#include "la_kernels.hpp"
#include "la_kernels_nc.hpp"
#include "la_kernels_causal.hpp"
#include "la_kernels_bf16.hpp"
#include "la_kernels_decode.hpp"

namespace {

using namespace la;

// Segments are multiples of 64 rows (every chunk size divides 64).  The
// plan aims at >= 512 workgroups per launch (two per CU on 256 CUs) by
// splitting each head's sequence into segments.
constexpr int64_t kSegAlign = 64;
constexpr int64_t kTargetWorkgroups = 512;

struct Plan {
    int64_t BH, N, D, PS, nseg, seg_len;
    int causal;
    float n0;  // tokens carried in from outside the call, added to every row's count
};

bool supported_d(int64_t D)
{
    return D == 16 || D == 32 || D == 64 || D == 128 || D == 256;
}

Plan make_plan(int64_t B, int64_t H, int64_t N, int64_t D, int causal)
{
    Plan p;
    p.BH = B * H;
    p.N = N;
    p.D = D;
    p.PS = D * D + 2 * D;
    p.causal = causal;
    p.n0 = 0.f;
    const int64_t nchunks = std::max<int64_t>((N + kSegAlign - 1) / kSegAlign, 1);
    const int64_t want =
        p.BH >= kTargetWorkgroups ? 1 : (kTargetWorkgroups + p.BH - 1) / std::max<int64_t>(p.BH, 1);
    const int64_t ns = std::min(want, nchunks);
    const int64_t per = (nchunks + ns - 1) / ns;
    p.seg_len = per * kSegAlign;
    p.nseg = std::max<int64_t>((N + p.seg_len - 1) / p.seg_len, 1);
    return p;
}

// Workgroups of `kern` (`threads` each) resident on the current device at
// once: compute units x workgroups per unit.  Both factors are cached (the
// compute-unit count per device, the occupancy per kernel); 0 if unknown.
template <class K>
int64_t resident_wgs(K kern, int threads)
{
    static int cus[64];
    static int per_cu = -1;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 0;
    if (cus[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cus[dev] = v;
    }
    if (per_cu < 0) {
        int v = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kern, threads, 0) != hipSuccess)
            return 0;
        per_cu = v;
    }
    return (int64_t)per_cu * cus[dev];
}

// The plan re-segmented so that one pass of the kernel is a single batch of
// resident workgroups (for a kernel whose workgroups hold one segment of one
// head), never with more segments than the plan's (its workspace holds that
// many records per head).
Plan one_batch(const Plan &p, int64_t resident)
{
    Plan q = p;
    const int64_t want = resident > 0 ? std::max<int64_t>(resident / std::max<int64_t>(p.BH, 1), 1)
                                      : p.nseg;
    if (want >= p.nseg)
        return q;
    const int64_t nchunks = std::max<int64_t>((p.N + kSegAlign - 1) / kSegAlign, 1);
    const int64_t per = (nchunks + want - 1) / want;
    q.seg_len = per * kSegAlign;
    q.nseg = std::max<int64_t>((p.N + q.seg_len - 1) / q.seg_len, 1);
    return q;
}

// workspace regions, in floats, each rounded up to 64 floats (256 bytes)
struct Layout {
    int64_t part, tot, gpart, gtot, cbuf, total;
};

int64_t up64(int64_t x) { return (x + 63) / 64 * 64; }

Layout make_layout(const Plan &p)
{
    Layout l;
    int64_t off = 0;
    l.part = off;
    off += up64(p.BH * p.nseg * p.PS);
    l.tot = off;
    off += up64(p.BH * p.PS);
    l.gpart = off;
    off += up64(p.BH * p.nseg * p.PS);
    l.gtot = off;
    off += up64(p.BH * p.PS);
    l.cbuf = off;
    off += up64(p.BH * p.N * 2);
    l.total = off;
    return l;
}

int64_t state_floats(const Plan &p) { return p.BH * (p.causal ? p.nseg : 1) * p.PS; }

int check_sizes(int64_t B, int64_t H, int64_t N, int64_t D, int causal)
{
    if (causal != 0 && causal != 1)
        return LA_ERR_UNSUPPORTED;
    if (B < 0 || H < 0 || N < 0)
        return LA_ERR_SHAPE;
    if (!supported_d(D))
        return LA_ERR_UNSUPPORTED;
    int64_t t;
    if (__builtin_mul_overflow(B, H, &t) || __builtin_mul_overflow(t, N, &t) ||
        __builtin_mul_overflow(t, D, &t) || __builtin_mul_overflow(t, (int64_t)16, &t))
        return LA_ERR_SHAPE;
    // keeps every grid below 2^31 workgroups and row counts exact in fp32
    if (B * H > (int64_t)1 << 22 || N > (int64_t)1 << 24)
        return LA_ERR_SHAPE;
    return LA_OK;
}

struct Range {
    const char *p;
    size_t n;
};

bool overlap(const Range &a, const Range &b)
{
    if (a.p == nullptr || b.p == nullptr || a.n == 0 || b.n == 0)
        return false;
    return a.p < b.p + b.n && b.p < a.p + a.n;
}

bool aliased(const Range *outs, int nout, const Range *ins, int nin)
{
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j)
            if (overlap(outs[i], ins[j]))
                return true;
        for (int j = i + 1; j < nout; ++j)
            if (overlap(outs[i], outs[j]))
                return true;
    }
    return false;
}

bool misaligned(const void *p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u); }

int launched()
{
    return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

// Optional per-launch timing: caller-owned hipEvents recorded around each
// kernel launch (events[2i] before, events[2i+1] after launch i).
struct Tracer {
    void *const *ev;
    int nev;
    int n;
    const char **names;
};

template <class F>
int traced(Tracer *t, hipStream_t s, const char *name, F &&launch)
{
    const bool rec = t != nullptr && t->ev != nullptr && 2 * t->n + 1 < t->nev;
    if (rec && hipEventRecord(static_cast<hipEvent_t>(t->ev[2 * t->n]), s) != hipSuccess)
        return LA_ERR_HIP;
    launch();
    const int rc = launched();
    if (rec && hipEventRecord(static_cast<hipEvent_t>(t->ev[2 * t->n + 1]), s) != hipSuccess)
        return LA_ERR_HIP;
    if (t != nullptr) {
        if (t->names != nullptr && 2 * t->n + 1 < t->nev)
            t->names[t->n] = name;
        ++t->n;
    }
    return rc;
}

// segment records -> head total (mode 0), exclusive prefixes (1) or
// exclusive suffixes (2), starting from `init` and writing the inclusive
// total to `total` when given
int scan(float *part, float *out, const Plan &p, int mode, hipStream_t s, Tracer *t,
         const float *init = nullptr, float *total = nullptr)
{
    const int64_t bph = (p.PS / 4 + 255) / 256;  // 4 floats per thread
    return traced(t, s, "state_scan", [&] {
        k_state_scan<<<dim3((unsigned)(p.BH * bph)), dim3(256), 0, s>>>(
            part, out, (int)p.nseg, p.PS, bph, mode, init, total);
    });
}

// the non-causal fast path (la_kernels_nc.hpp) covers 32 <= D <= 128
template <int D>
constexpr bool nc_path()
{
    return D >= 32 && D <= 128;
}

// fp32 storage at D = 256: the fast reduction (four 128 x 128 blocks per
// segment) for both masks, the fast non-causal apply kernels (eight waves)
// and a dQ pass without the dS role (the gradient record then comes from
// the reduction)
template <class ST, int D>
constexpr bool wide_path()
{
    return std::is_same<ST, StF32>::value && D == 256;
}

template <class ST, int D>
int state_of_kv(const void *K, const void *V, float *part, float *tot, const Plan &p,
                hipStream_t s, Tracer *t, const float *init = nullptr, float *total = nullptr)
{
    typedef Cfg<D, DefCS<D>::value> C;
    typedef typename ST::T T;
    int rc = LA_OK;
    bool done = false;
    if constexpr (nc_path<D>() || wide_path<ST, D>()) {
        rc = traced(t, s, "state_local", [&] {
            if constexpr (std::is_same<ST, StBF16>::value)
                bf::k_reduce_bf<D, false><<<dim3((unsigned)(p.nseg * p.BH)), dim3(256), 0, s>>>(
                    static_cast<const T *>(K), static_cast<const T *>(V), nullptr, part, p.N,
                    p.seg_len, (int)p.nseg);
            else
                nc::k_reduce_nc<ST, D, false>
                    <<<dim3((unsigned)(p.nseg * p.BH * nc::reduce_blocks<D>())),
                       dim3(nc::kReduceThreads), 0, s>>>(
                        static_cast<const T *>(K), static_cast<const T *>(V), nullptr, part, p.N,
                        p.seg_len, (int)p.nseg);
        });
        done = true;
    }
    if (!done) {
        const dim3 grid((unsigned)(p.nseg * p.BH * C::CS));
        rc = traced(t, s, "state_local", [&] {
            k_state_local<ST, D><<<grid, dim3(C::NT), 0, s>>>(
                static_cast<const T *>(K), static_cast<const T *>(V), part, p.N, p.seg_len,
                (int)p.nseg);
        });
    }
    if (rc != LA_OK)
        return rc;
    return p.causal ? scan(part, nullptr, p, 1, s, t, init, total)
                    : scan(part, tot, p, 0, s, t, init, total);
}

// Carry: `cin` (or null) is the record [S | z | u] of p.n0 tokens outside
// the call that every row attends to; `cout` (or null) receives cin plus the
// call's own record.  O == null computes the state only.
template <class ST, int D>
int run_forward(const void *Q, const void *K, const void *V, void *O, float *den_out,
                void *state_out, float *ws, const Plan &p, hipStream_t s, Tracer *t,
                const float *cin, float *cout)
{
    typedef Cfg<D, DefCS<D>::value> C;
    typedef typename ST::T T;
    const Layout l = make_layout(p);
    float *rec;
    int rc;
    if (p.causal) {
        rec = state_out ? static_cast<float *>(state_out) : ws + l.part;
        rc = state_of_kv<ST, D>(K, V, rec, nullptr, p, s, t, cin, cout);
    } else {
        rec = state_out ? static_cast<float *>(state_out) : ws + l.tot;
        rc = state_of_kv<ST, D>(K, V, ws + l.part, rec, p, s, t, cin, cout);
    }
    if (rc != LA_OK || O == nullptr)
        return rc;
    if constexpr (nc_path<D>()) {
        if (!p.causal)
            return traced(t, s, "forward", [&] {
                if constexpr (std::is_same<ST, StBF16>::value)
                    bf::k_apply_bf<D, 0><<<dim3((unsigned)(p.nseg * p.BH)),
                                           dim3(bf::kApplyThreads), 0, s>>>(
                        static_cast<const T *>(Q), nullptr, static_cast<T *>(O), nullptr,
                        den_out, nullptr, rec, p.N, p.seg_len, (int)p.nseg, p.n0);
                else
                    nc::k_apply_nc<ST, D, 0><<<dim3((unsigned)(p.nseg * p.BH)),
                                               dim3(nc::kApplyThreads), 0, s>>>(
                        static_cast<const T *>(Q), nullptr, static_cast<T *>(O), nullptr,
                        den_out, rec, p.N, p.seg_len, (int)p.nseg, p.n0);
            });
        return traced(t, s, "forward", [&] {
            if constexpr (std::is_same<ST, StBF16>::value)
                bf::k_fwd_causal_bf<D><<<dim3((unsigned)(p.nseg * p.BH)),
                                         dim3(cz::threads<D>()), 0, s>>>(
                    static_cast<const T *>(Q), static_cast<const T *>(K),
                    static_cast<const T *>(V), static_cast<T *>(O), den_out, rec, p.N, p.seg_len,
                    (int)p.nseg, p.n0);
            else
                cz::k_fwd_causal<ST, D><<<dim3((unsigned)(p.nseg * p.BH)),
                                          dim3(cz::threads<D>()), 0, s>>>(
                    static_cast<const T *>(Q), static_cast<const T *>(K),
                    static_cast<const T *>(V), static_cast<T *>(O), den_out, rec, p.N, p.seg_len,
                    (int)p.nseg, p.n0);
        });
    }
    if constexpr (wide_path<ST, D>()) {
        if (!p.causal)
            return traced(t, s, "forward", [&] {
                nc::k_apply_nc<ST, D, 0><<<dim3((unsigned)(p.nseg * p.BH)),
                                           dim3(nc::apply_threads<D>()), 0, s>>>(
                    static_cast<const T *>(Q), nullptr, static_cast<T *>(O), nullptr, den_out,
                    rec, p.N, p.seg_len, (int)p.nseg, p.n0);
            });
    }
    const dim3 grid((unsigned)(p.nseg * p.BH * C::CS));
    return traced(t, s, "forward", [&] {
        if (p.causal)
            k_forward<ST, D, true><<<grid, dim3(C::NT), 0, s>>>(
                static_cast<const T *>(Q), static_cast<const T *>(K),
                static_cast<const T *>(V), static_cast<T *>(O), den_out, rec, p.N,
                p.seg_len, (int)p.nseg, p.n0);
        else
            k_forward<ST, D, false><<<grid, dim3(C::NT), 0, s>>>(
                static_cast<const T *>(Q), static_cast<const T *>(K),
                static_cast<const T *>(V), static_cast<T *>(O), den_out, rec, p.N,
                p.seg_len, (int)p.nseg, p.n0);
    });
}

// Carry: `cin` is the forward's carried-in record (read only when state_in
// is null, to recompute the state); `gin` (or null) is the gradient record
// [dS | r | t] of the rows outside the call that attend to its keys, and
// `gout` (or null) receives gin plus the call's own gradient record.
// dK == null skips the dK | dV pass.
template <class ST, int D, bool CAUSAL>
int run_backward_t(const void *Q, const void *K, const void *V, const void *G, void *dQ,
                   void *dK, void *dV, const void *state_in, float *ws, const Plan &p,
                   hipStream_t s, Tracer *t, const float *cin, const float *gin, float *gout)
{
    typedef Cfg<D, DefCS<D>::value> C;
    typedef Cfg<D, 1> CQ;
    typedef typename ST::T T;
    constexpr bool FUSE = (D != 256);
    const Layout l = make_layout(p);
    const float *fstate;
    int rc;
    if (state_in) {
        fstate = static_cast<const float *>(state_in);
    } else {
        rc = state_of_kv<ST, D>(K, V, ws + l.part, ws + l.tot, p, s, t, cin);
        if (rc != LA_OK)
            return rc;
        fstate = CAUSAL ? ws + l.part : ws + l.tot;
    }
    float *gpart = ws + l.gpart, *cbuf = ws + l.cbuf;
    const T *q = static_cast<const T *>(Q), *k = static_cast<const T *>(K),
            *v = static_cast<const T *>(V), *g = static_cast<const T *>(G);
    if constexpr (CAUSAL && nc_path<D>()) {
        const dim3 g1((unsigned)(p.nseg * p.BH)), nt(cz::threads<D>());
        // dQ and (c_i, 1/den_i), chunk by chunk from the saved prefix records
        rc = traced(t, s, "bwd_q", [&] {
            if constexpr (std::is_same<ST, StBF16>::value)
                bf::k_bwd_q_causal_bf<D><<<g1, nt, 0, s>>>(q, k, v, g, static_cast<T *>(dQ),
                                                           cbuf, fstate, p.N, p.seg_len,
                                                           (int)p.nseg, p.n0);
            else
                cz::k_bwd_q_causal<ST, D><<<g1, nt, 0, s>>>(q, k, v, g, static_cast<T *>(dQ),
                                                            cbuf, fstate, p.N, p.seg_len,
                                                            (int)p.nseg, p.n0);
        });
        if (rc != LA_OK)
            return rc;
        rc = traced(t, s, "grad_state_local", [&] {
            if constexpr (std::is_same<ST, StBF16>::value)
                bf::k_reduce_bf<D, true><<<g1, dim3(256), 0, s>>>(q, g, cbuf, gpart, p.N,
                                                                p.seg_len, (int)p.nseg);
            else
                nc::k_reduce_nc<ST, D, true><<<g1, dim3(nc::kReduceThreads), 0, s>>>(
                    q, g, cbuf, gpart, p.N, p.seg_len, (int)p.nseg);
        });
        if (rc != LA_OK)
            return rc;
        if ((rc = scan(gpart, nullptr, p, 2, s, t, gin, gout)) != LA_OK)  // exclusive suffix
            return rc;
        if (dK == nullptr)
            return LA_OK;
        return traced(t, s, "bwd_kv", [&] {
            if constexpr (std::is_same<ST, StBF16>::value)
                bf::k_bwd_kv_causal_bf<D><<<dim3((unsigned)(2 * p.nseg * p.BH)), nt, 0, s>>>(
                    q, k, v, g, static_cast<T *>(dK), static_cast<T *>(dV), cbuf, gpart, p.N,
                    p.seg_len, (int)p.nseg);
            else
                cz::k_bwd_kv_causal<ST, D><<<dim3((unsigned)(2 * p.nseg * p.BH)), nt, 0, s>>>(
                    q, k, v, g, static_cast<T *>(dK), static_cast<T *>(dV), cbuf, gpart, p.N,
                    p.seg_len, (int)p.nseg);
        });
    }
    if constexpr (!CAUSAL && wide_path<ST, D>()) {
        // dQ and (c_i, 1/den_i); the gradient records by the fast reduction;
        // dK | dV by the eight-wave apply kernel
        const dim3 g1((unsigned)(p.nseg * p.BH));
        rc = traced(t, s, "bwd_q", [&] {
            nc::k_bwd_q_nc<ST, D, false><<<g1, dim3(512), 0, s>>>(
                g, q, static_cast<T *>(dQ), cbuf, fstate, p.N, p.seg_len, (int)p.nseg, p.n0);
        });
        if (rc != LA_OK)
            return rc;
        rc = traced(t, s, "grad_state_local", [&] {
            nc::k_reduce_nc<ST, D, true>
                <<<dim3((unsigned)(p.nseg * p.BH * nc::reduce_blocks<D>())),
                   dim3(nc::kReduceThreads), 0, s>>>(q, g, cbuf, gpart, p.N, p.seg_len,
                                                     (int)p.nseg);
        });
        if (rc != LA_OK)
            return rc;
        if ((rc = scan(gpart, ws + l.gtot, p, 0, s, t, gin, gout)) != LA_OK)
            return rc;
        if (dK == nullptr)
            return LA_OK;
        return traced(t, s, "bwd_kv", [&] {
            nc::k_apply_nc<ST, D, 2><<<dim3((unsigned)(2 * p.nseg * p.BH)),
                                       dim3(nc::apply_threads<D>()), 0, s>>>(
                v, k, static_cast<T *>(dK), static_cast<T *>(dV), nullptr, ws + l.gtot, p.N,
                p.seg_len, (int)p.nseg, p.n0);
        });
    }
    if constexpr (!CAUSAL && nc_path<D>()) {
        const dim3 g1((unsigned)(p.nseg * p.BH));
        if constexpr (std::is_same<ST, StBF16>::value) {
            // bf16 matrix cores: dQ with (c_i, 1/den_i), then the gradient
            // records from a second (bf16, half-size) read of Q and dO
            rc = traced(t, s, "bwd_q", [&] {
                bf::k_apply_bf<D, 1><<<g1, dim3(bf::kApplyThreads), 0, s>>>(
                    g, q, static_cast<T *>(dQ), nullptr, nullptr, cbuf, fstate, p.N, p.seg_len,
                    (int)p.nseg, p.n0);
            });
            if (rc != LA_OK)
                return rc;
            rc = traced(t, s, "grad_state_local", [&] {
                bf::k_reduce_bf<D, true><<<g1, dim3(256), 0, s>>>(q, g, cbuf, gpart, p.N,
                                                                p.seg_len, (int)p.nseg);
            });
        } else {
            // dQ and the segment's gradient record in one pass over Q and dO,
            // its segments sized for one batch of resident workgroups
            const Plan pq = one_batch(p, resident_wgs(nc::k_bwd_q_nc<ST, D>, 512));
            rc = traced(t, s, "bwd_q", [&] {
                nc::k_bwd_q_nc<ST, D><<<dim3((unsigned)(pq.nseg * pq.BH)), dim3(512), 0, s>>>(
                    g, q, static_cast<T *>(dQ), gpart, fstate, pq.N, pq.seg_len, (int)pq.nseg,
                    pq.n0);
            });
            if (rc != LA_OK)
                return rc;
            if ((rc = scan(gpart, ws + l.gtot, pq, 0, s, t, gin, gout)) != LA_OK)
                return rc;
        }
        if (rc != LA_OK)
            return rc;
        if constexpr (std::is_same<ST, StBF16>::value)
            if ((rc = scan(gpart, ws + l.gtot, p, 0, s, t, gin, gout)) != LA_OK)
                return rc;
        if (dK == nullptr)
            return LA_OK;
        return traced(t, s, "bwd_kv", [&] {
            if constexpr (std::is_same<ST, StBF16>::value)
                bf::k_apply_bf<D, 2><<<dim3((unsigned)(2 * p.nseg * p.BH)),
                                       dim3(bf::kApplyThreads), 0, s>>>(
                    v, k, static_cast<T *>(dK), static_cast<T *>(dV), nullptr, nullptr,
                    ws + l.gtot, p.N, p.seg_len, (int)p.nseg, p.n0);
            else
                nc::k_apply_nc<ST, D, 2><<<dim3((unsigned)(2 * p.nseg * p.BH)),
                                           dim3(nc::kApplyThreads), 0, s>>>(
                    v, k, static_cast<T *>(dK), static_cast<T *>(dV), nullptr, ws + l.gtot, p.N,
                    p.seg_len, (int)p.nseg, p.n0);
        });
    }
    rc = traced(t, s, "bwd_q", [&] {
        k_bwd_q<ST, D, CAUSAL, FUSE><<<dim3((unsigned)(p.nseg * p.BH)), dim3(CQ::NT), 0, s>>>(
            q, k, v, g, static_cast<T *>(dQ), fstate, gpart, cbuf, p.N, p.seg_len,
            (int)p.nseg, p.n0);
    });
    if (rc != LA_OK)
        return rc;
    const dim3 grid((unsigned)(p.nseg * p.BH * C::CS));
    if constexpr (!FUSE) {
        rc = traced(t, s, "grad_state_local", [&] {
            k_grad_state_local<ST, D><<<grid, dim3(C::NT), 0, s>>>(q, g, cbuf, gpart, p.N,
                                                                   p.seg_len, (int)p.nseg);
        });
        if (rc != LA_OK)
            return rc;
    }
    const float *gstate;
    if (CAUSAL) {
        rc = scan(gpart, nullptr, p, 2, s, t, gin, gout);
        gstate = gpart;
    } else {
        rc = scan(gpart, ws + l.gtot, p, 0, s, t, gin, gout);
        gstate = ws + l.gtot;
    }
    if (rc != LA_OK)
        return rc;
    if (dK == nullptr)
        return LA_OK;
    return traced(t, s, "bwd_kv", [&] {
        k_bwd_kv<ST, D, CAUSAL><<<grid, dim3(C::NT), 0, s>>>(
            q, k, v, g, static_cast<T *>(dK), static_cast<T *>(dV), gstate, cbuf, p.N,
            p.seg_len, (int)p.nseg);
    });
}

template <class ST, int D>
int run_backward(const void *Q, const void *K, const void *V, const void *G, void *dQ,
                 void *dK, void *dV, const void *state_in, float *ws, const Plan &p,
                 hipStream_t s, Tracer *t, const float *cin, const float *gin, float *gout)
{
    if (p.causal)
        return run_backward_t<ST, D, true>(Q, K, V, G, dQ, dK, dV, state_in, ws, p, s, t, cin,
                                           gin, gout);
    return run_backward_t<ST, D, false>(Q, K, V, G, dQ, dK, dV, state_in, ws, p, s, t, cin,
                                        gin, gout);
}

template <class ST>
int dispatch_forward(const void *Q, const void *K, const void *V, void *O, float *den,
                     void *st, float *ws, const Plan &p, hipStream_t s, Tracer *t,
                     const float *cin, float *cout)
{
    switch (p.D) {
    case 16: return run_forward<ST, 16>(Q, K, V, O, den, st, ws, p, s, t, cin, cout);
    case 32: return run_forward<ST, 32>(Q, K, V, O, den, st, ws, p, s, t, cin, cout);
    case 64: return run_forward<ST, 64>(Q, K, V, O, den, st, ws, p, s, t, cin, cout);
    case 128: return run_forward<ST, 128>(Q, K, V, O, den, st, ws, p, s, t, cin, cout);
    case 256: return run_forward<ST, 256>(Q, K, V, O, den, st, ws, p, s, t, cin, cout);
    default: return LA_ERR_UNSUPPORTED;
    }
}

template <class ST>
int dispatch_backward(const void *Q, const void *K, const void *V, const void *G, void *dQ,
                      void *dK, void *dV, const void *st, float *ws, const Plan &p,
                      hipStream_t s, Tracer *t, const float *cin, const float *gin,
                      float *gout)
{
#define LA_BWD(d)                                                                          \
    run_backward<ST, d>(Q, K, V, G, dQ, dK, dV, st, ws, p, s, t, cin, gin, gout)
    switch (p.D) {
    case 16: return LA_BWD(16);
    case 32: return LA_BWD(32);
    case 64: return LA_BWD(64);
    case 128: return LA_BWD(128);
    case 256: return LA_BWD(256);
    default: return LA_ERR_UNSUPPORTED;
    }
#undef LA_BWD
}

size_t elem_size(int dtype) { return dtype == LA_BF16 ? 2 : 4; }

// tokens a carried-in record may stand for (counts enter the kernels as fp32)
constexpr int64_t kMaxCarry = (int64_t)1 << 40;

// A call over zero tokens passes the carried record through: out = in, or
// zero without one (the scan kernel over zero segments; no memset or copy
// node, so the call stays capturable).
int pass_record(const float *in, float *out, int64_t BH, int64_t D, hipStream_t s)
{
    if (out == nullptr)
        return LA_OK;
    const size_t rb = (size_t)(BH * (D * D + 2 * D)) * sizeof(float);
    if (misaligned(out) || misaligned(in))
        return LA_ERR_ALIGN;
    if (overlap({(const char *)out, rb}, {(const char *)in, rb}))
        return LA_ERR_ALIAS;
    Plan p{};
    p.BH = BH;
    p.D = D;
    p.PS = D * D + 2 * D;
    p.nseg = 0;
    return scan(out, out, p, 0, s, nullptr, in, nullptr);
}

int forward_impl(bool require_o, const void *Q, const void *K, const void *V, void *O,
                 int64_t B, int64_t H, int64_t N, int64_t D, int causal, int dtype,
                 const float *cin, int64_t n_carry, float *cout, float *den_out,
                 void *state_out, void *ws, size_t ws_bytes, void *stream,
                 void *const *events, int n_events, int *n_launched, const char **names)
{
    if (n_launched)
        *n_launched = 0;
    if (dtype != LA_FP32 && dtype != LA_BF16)
        return LA_ERR_DTYPE;
    int rc = check_sizes(B, H, N, D, causal);
    if (rc != LA_OK)
        return rc;
    if (n_carry < 0 || n_carry > kMaxCarry)
        return LA_ERR_SHAPE;
    if (B * H == 0)
        return LA_OK;
    if (N == 0)
        return pass_record(cin, cout, B * H, D, static_cast<hipStream_t>(stream));
    // O == null asks for the state only: something must receive it
    if (!Q || !K || !V || !ws || (!O && (require_o || den_out || (!cout && !state_out))))
        return LA_ERR_NULL;
    const size_t rb = (size_t)(B * H * (D * D + 2 * D)) * sizeof(float);
    Plan p = make_plan(B, H, N, D, causal);
    p.n0 = (float)n_carry;
    const size_t need = (size_t)make_layout(p).total * sizeof(float);
    if (ws_bytes < need)
        return LA_ERR_WORKSPACE;
    if (misaligned(Q) || misaligned(K) || misaligned(V) || misaligned(O) ||
        misaligned(den_out) || misaligned(state_out) || misaligned(ws) || misaligned(cin) ||
        misaligned(cout))
        return LA_ERR_ALIGN;
    const size_t tb = (size_t)(B * H * N * D) * elem_size(dtype);
    const Range ins[4] = {{(const char *)Q, tb},
                          {(const char *)K, tb},
                          {(const char *)V, tb},
                          {(const char *)cin, rb}};
    const Range outs[5] = {
        {(const char *)O, tb},
        {(const char *)den_out, (size_t)(B * H * N) * sizeof(float)},
        {(const char *)state_out, (size_t)state_floats(p) * sizeof(float)},
        {(const char *)ws, need},
        {(const char *)cout, rb}};
    if (aliased(outs, 5, ins, 4))
        return LA_ERR_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    float *w = static_cast<float *>(ws);
    Tracer t{events, events ? n_events : 0, 0, names};
    rc = (dtype == LA_FP32)
             ? dispatch_forward<StF32>(Q, K, V, O, den_out, state_out, w, p, s, &t, cin, cout)
             : dispatch_forward<StBF16>(Q, K, V, O, den_out, state_out, w, p, s, &t, cin, cout);
    if (n_launched)
        *n_launched = t.n;
    return rc;
}

int backward_impl(bool require_kv, const void *Q, const void *K, const void *V,
                  const void *dO, void *dQ, void *dK, void *dV, int64_t B, int64_t H,
                  int64_t N, int64_t D, int causal, int dtype, const float *cin,
                  int64_t n_carry, const float *gin, float *gout, const void *state_in,
                  void *ws, size_t ws_bytes, void *stream, void *const *events, int n_events,
                  int *n_launched, const char **names)
{
    if (n_launched)
        *n_launched = 0;
    if (dtype != LA_FP32 && dtype != LA_BF16)
        return LA_ERR_DTYPE;
    int rc = check_sizes(B, H, N, D, causal);
    if (rc != LA_OK)
        return rc;
    if (n_carry < 0 || n_carry > kMaxCarry)
        return LA_ERR_SHAPE;
    if (B * H == 0)
        return LA_OK;
    if (N == 0)
        return pass_record(gin, gout, B * H, D, static_cast<hipStream_t>(stream));
    // dK and dV: both given, or (segment calls only) both null
    if (!Q || !K || !V || !dO || !dQ || !ws || (dK == nullptr) != (dV == nullptr) ||
        (require_kv && dK == nullptr))
        return LA_ERR_NULL;
    const size_t rb = (size_t)(B * H * (D * D + 2 * D)) * sizeof(float);
    Plan p = make_plan(B, H, N, D, causal);
    p.n0 = (float)n_carry;
    const size_t need = (size_t)make_layout(p).total * sizeof(float);
    if (ws_bytes < need)
        return LA_ERR_WORKSPACE;
    if (misaligned(Q) || misaligned(K) || misaligned(V) || misaligned(dO) ||
        misaligned(dQ) || misaligned(dK) || misaligned(dV) || misaligned(state_in) ||
        misaligned(ws) || misaligned(cin) || misaligned(gin) || misaligned(gout))
        return LA_ERR_ALIGN;
    const size_t tb = (size_t)(B * H * N * D) * elem_size(dtype);
    const Range ins[7] = {{(const char *)Q, tb},
                          {(const char *)K, tb},
                          {(const char *)V, tb},
                          {(const char *)dO, tb},
                          {(const char *)state_in, (size_t)state_floats(p) * sizeof(float)},
                          {(const char *)cin, rb},
                          {(const char *)gin, rb}};
    const Range outs[5] = {{(const char *)dQ, tb},
                           {(const char *)dK, tb},
                           {(const char *)dV, tb},
                           {(const char *)ws, need},
                           {(const char *)gout, rb}};
    if (aliased(outs, 5, ins, 7))
        return LA_ERR_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    float *w = static_cast<float *>(ws);
    Tracer t{events, events ? n_events : 0, 0, names};
    rc = (dtype == LA_FP32) ? dispatch_backward<StF32>(Q, K, V, dO, dQ, dK, dV, state_in, w, p,
                                                       s, &t, cin, gin, gout)
                            : dispatch_backward<StBF16>(Q, K, V, dO, dQ, dK, dV, state_in, w,
                                                        p, s, &t, cin, gin, gout);
    if (n_launched)
        *n_launched = t.n;
    return rc;
}

template <class ST>
int launch_decode(const void *q, const void *k, const void *v, void *o, int64_t BH, int64_t H,
                  int64_t D, const float *rin, float *rout, const int64_t *counts, float n_all,
                  float *den, hipStream_t s)
{
    typedef typename ST::T T;
#define LA_DEC(d)                                                                          \
    dec::k_decode<ST, d><<<dim3((unsigned)(BH * dec::blocks_per_head<d>())),              \
                           dim3(dec::kThreads), 0, s>>>(                                   \
        static_cast<const T *>(q), static_cast<const T *>(k), static_cast<const T *>(v),   \
        static_cast<T *>(o), den, rin, rout, counts, n_all, (int)H)
    switch (D) {
    case 16: LA_DEC(16); break;
    case 32: LA_DEC(32); break;
    case 64: LA_DEC(64); break;
    case 128: LA_DEC(128); break;
    case 256: LA_DEC(256); break;
    default: return LA_ERR_UNSUPPORTED;
    }
#undef LA_DEC
    return launched();
}

}  // namespace

extern "C" {

int la_decode_step(const void *q, const void *k, const void *v, void *o, int64_t B, int64_t H,
                   int64_t D, int dtype, const float *state_in, float *state_out,
                   const int64_t *counts, int64_t n_prev, float *den_out, void *stream)
{
    if (dtype != LA_FP32 && dtype != LA_BF16)
        return LA_ERR_DTYPE;
    int rc = check_sizes(B, H, 1, D, 1);
    if (rc != LA_OK)
        return rc;
    if (n_prev < 0 || n_prev > kMaxCarry)
        return LA_ERR_SHAPE;
    if (B * H == 0)
        return LA_OK;
    if (!q || !k || !v || !o || !state_out)
        return LA_ERR_NULL;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) ||
        misaligned(state_in) || misaligned(state_out) || misaligned(counts) ||
        misaligned(den_out))
        return LA_ERR_ALIGN;
    const size_t tb = (size_t)(B * H * D) * elem_size(dtype);
    const size_t rb = (size_t)(B * H * (D * D + 2 * D)) * sizeof(float);
    const Range ins[5] = {{(const char *)q, tb},
                          {(const char *)k, tb},
                          {(const char *)v, tb},
                          {(const char *)state_in, rb},
                          {(const char *)counts, (size_t)B * sizeof(int64_t)}};
    const Range outs[3] = {{(const char *)o, tb},
                           {(const char *)state_out, rb},
                           {(const char *)den_out, (size_t)(B * H) * sizeof(float)}};
    if (aliased(outs, 3, ins, 5))
        return LA_ERR_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return dtype == LA_FP32 ? launch_decode<StF32>(q, k, v, o, B * H, H, D, state_in,
                                                   state_out, counts, (float)n_prev, den_out, s)
                            : launch_decode<StBF16>(q, k, v, o, B * H, H, D, state_in,
                                                    state_out, counts, (float)n_prev, den_out,
                                                    s);
}


const char *la_status_string(int status)
{
    switch (status) {
    case LA_OK: return "LA_OK";
    case LA_ERR_NULL: return "LA_ERR_NULL: a required pointer is NULL";
    case LA_ERR_SHAPE: return "LA_ERR_SHAPE: negative or too large size";
    case LA_ERR_DTYPE: return "LA_ERR_DTYPE: dtype must be LA_FP32 or LA_BF16";
    case LA_ERR_UNSUPPORTED:
        return "LA_ERR_UNSUPPORTED: D must be 16, 32, 64, 128 or 256 and causal 0 or 1";
    case LA_ERR_WORKSPACE: return "LA_ERR_WORKSPACE: workspace too small";
    case LA_ERR_ALIAS: return "LA_ERR_ALIAS: an output overlaps an input or another output";
    case LA_ERR_ALIGN: return "LA_ERR_ALIGN: device pointers must be 16-byte aligned";
    case LA_ERR_HIP: return "LA_ERR_HIP: a HIP launch failed";
    default: return "unknown la_status";
    }
}

int64_t la_num_segments(int64_t B, int64_t H, int64_t N, int64_t D, int causal)
{
    if (check_sizes(B, H, N, D, causal) != LA_OK)
        return 0;
    return make_plan(B, H, N, D, causal).nseg;
}

size_t la_workspace_size(int64_t B, int64_t H, int64_t N, int64_t D, int causal)
{
    if (check_sizes(B, H, N, D, causal) != LA_OK || B * H * N == 0)
        return 0;
    return (size_t)make_layout(make_plan(B, H, N, D, causal)).total * sizeof(float);
}

size_t la_state_size(int64_t B, int64_t H, int64_t N, int64_t D, int causal)
{
    if (check_sizes(B, H, N, D, causal) != LA_OK || B * H * N == 0)
        return 0;
    return (size_t)state_floats(make_plan(B, H, N, D, causal)) * sizeof(float);
}

size_t la_record_size(int64_t B, int64_t H, int64_t D)
{
    if (B < 0 || H < 0 || !supported_d(D) || B * H > (int64_t)1 << 22)
        return 0;
    return (size_t)(B * H * (D * D + 2 * D)) * sizeof(float);
}

int la_forward_traced(const void *Q, const void *K, const void *V, void *O, int64_t B,
                      int64_t H, int64_t N, int64_t D, int causal, int dtype, float *den_out,
                      void *state_out, void *ws, size_t ws_bytes, void *stream,
                      void *const *events, int n_events, int *n_launched, const char **names)
{
    return forward_impl(true, Q, K, V, O, B, H, N, D, causal, dtype, nullptr, 0, nullptr,
                        den_out, state_out, ws, ws_bytes, stream, events, n_events, n_launched,
                        names);
}

int la_forward(const void *Q, const void *K, const void *V, void *O, int64_t B, int64_t H,
               int64_t N, int64_t D, int causal, int dtype, float *den_out, void *state_out,
               void *ws, size_t ws_bytes, void *stream)
{
    return la_forward_traced(Q, K, V, O, B, H, N, D, causal, dtype, den_out, state_out, ws,
                             ws_bytes, stream, nullptr, 0, nullptr, nullptr);
}

int la_forward_segment(const void *Q, const void *K, const void *V, void *O, int64_t B,
                       int64_t H, int64_t N, int64_t D, int causal, int dtype,
                       const float *carry_in, int64_t n_carry, float *carry_out,
                       float *den_out, void *state_out, void *ws, size_t ws_bytes,
                       void *stream)
{
    return forward_impl(false, Q, K, V, O, B, H, N, D, causal, dtype, carry_in, n_carry,
                        carry_out, den_out, state_out, ws, ws_bytes, stream, nullptr, 0, nullptr,
                        nullptr);
}

int la_backward_traced(const void *Q, const void *K, const void *V, const void *dO, void *dQ,
                       void *dK, void *dV, int64_t B, int64_t H, int64_t N, int64_t D,
                       int causal, int dtype, const void *state_in, void *ws, size_t ws_bytes,
                       void *stream, void *const *events, int n_events, int *n_launched,
                       const char **names)
{
    return backward_impl(true, Q, K, V, dO, dQ, dK, dV, B, H, N, D, causal, dtype, nullptr, 0,
                         nullptr, nullptr, state_in, ws, ws_bytes, stream, events, n_events,
                         n_launched, names);
}

int la_backward(const void *Q, const void *K, const void *V, const void *dO, void *dQ,
                void *dK, void *dV, int64_t B, int64_t H, int64_t N, int64_t D, int causal,
                int dtype, const void *state_in, void *ws, size_t ws_bytes, void *stream)
{
    return la_backward_traced(Q, K, V, dO, dQ, dK, dV, B, H, N, D, causal, dtype, state_in, ws,
                              ws_bytes, stream, nullptr, 0, nullptr, nullptr);
}

int la_backward_segment(const void *Q, const void *K, const void *V, const void *dO, void *dQ,
                        void *dK, void *dV, int64_t B, int64_t H, int64_t N, int64_t D,
                        int causal, int dtype, const float *carry_in, int64_t n_carry,
                        const float *gcarry_in, float *gcarry_out, const void *state_in,
                        void *ws, size_t ws_bytes, void *stream)
{
    return backward_impl(false, Q, K, V, dO, dQ, dK, dV, B, H, N, D, causal, dtype, carry_in,
                         n_carry, gcarry_in, gcarry_out, state_in, ws, ws_bytes, stream, nullptr,
                         0, nullptr, nullptr);
}

}  // extern "C"
