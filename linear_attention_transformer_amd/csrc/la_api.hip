// la_api.hip -- C ABI of the linear-attention library (declared in
// include/la.h): argument validation, segment planning, workspace layout and
// kernel dispatch.  See la_kernels.hpp for the method and its sources.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "la.h"
#include "la_internal.hpp"
#include "la_kernels.hpp"
#include "la_kernels_nc.hpp"
#include "la_kernels_causal.hpp"
#include "la_kernels_bf16.hpp"
#include "la_kernels_decode.hpp"
#include "la_kernels_stage.hpp"

namespace {

using namespace la;

// Segments are multiples of 64 rows (every chunk size divides 64).  The
// plan aims at >= 512 workgroups per launch (two per CU on 256 CUs) by
// splitting each head's sequence into segments.
constexpr int64_t kSegAlign = 64;
constexpr int64_t kTargetWorkgroups = 512;
constexpr int64_t kMinSegChunks = 4;

struct Plan {
    int64_t BH, N, D, PS, nseg, seg_len;
    int64_t dl;  // columns of the caller's rows (D unless a narrow head runs at width D)
    int causal;
    float n0;  // tokens carried in from outside the call, added to every row's count
    OutLay ol; // where the outputs go (default: [B, H, N, D] contiguous)
};

// the plain [B, H, N, D] layout
OutLay plain_layout(int64_t H, int64_t N, int64_t D)
{
    return OutLay{std::max<int64_t>(H, 1) * N * D, N * D, D, std::max<int64_t>(H, 1)};
}

// head sizes the kernels take as they are (others are padded to the next)
bool supported_d(int64_t D)
{
    return D == 32 || D == 64 || D == 128 || D == 256;
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
    p.ol = plain_layout(H, N, D);
    p.dl = D;
    const int64_t nchunks = std::max<int64_t>((N + kSegAlign - 1) / kSegAlign, 1);
    // width 16 runs one-wave workgroups: four times as many fill the chip
    const int64_t target = D <= 16 ? 8 * kTargetWorkgroups : kTargetWorkgroups;
    const int64_t want =
        p.BH >= target ? 1 : (target + p.BH - 1) / std::max<int64_t>(p.BH, 1);
    const int64_t ns = std::min(want, nchunks);
    // Segments of at least kMinSegChunks chunks when that still gives one
    // workgroup per CU: shorter segments cost more in their 4(D^2 + 2D)-byte
    // records (written, scanned, read by the walks) than they gain in
    // parallelism.  (B4 H16 N1024: 8 segments of 128 rows -> 4 of 256, bf16
    // causal step 0.127 -> 0.117 ms; with 4 heads the short segments stay.)
    const int64_t at_min = (nchunks + kMinSegChunks - 1) / kMinSegChunks;
    const int64_t pmin = (D > 16 && p.BH * at_min >= kTargetWorkgroups / 2) ? kMinSegChunks : 1;
    const int64_t per = std::max<int64_t>((nchunks + ns - 1) / ns, pmin);
    p.seg_len = per * kSegAlign;
    p.nseg = std::max<int64_t>((N + p.seg_len - 1) / p.seg_len, 1);
    return p;
}

// Workgroups of kernel KERN (`threads` each) resident on the current device
// at once: compute units x workgroups per unit.  Both factors are cached (the
// compute-unit count per device, the occupancy per kernel: one cache per
// instantiation, i.e. per kernel); 0 if unknown.  (Concurrent first calls
// may both query; they store the same values.)
template <auto KERN>
int64_t resident_wgs(int threads)
{
    static std::atomic<int> cus[64];
    static std::atomic<int> per_cu{-1};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 0;
    int c = cus[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cus[dev].store(c, std::memory_order_relaxed);
    }
    int o = per_cu.load(std::memory_order_relaxed);
    if (o < 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, KERN, threads, 0) != hipSuccess)
            return 0;
        per_cu.store(o, std::memory_order_relaxed);
    }
    return (int64_t)o * c;
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

// Segments per workgroup for a walk over the suffix (or prefix) records of
// the plan: the smallest count that fits the launch into one batch of
// `resident` workgroups (the plan's segments when even one per head does
// not fit; 1 if the residency is unknown).  Records stay the plan's: a
// merged walk starts from the record of its last segment.
int merge_factor(const Plan &p, int64_t resident)
{
    if (resident <= 0)
        return 1;
    for (int64_t m = 1; m < p.nseg; ++m)
        if ((p.nseg + m - 1) / m * p.BH <= resident)
            return (int)m;
    return (int)std::max<int64_t>(p.nseg, 1);
}

// The plan re-segmented so that a launch of `per` workgroups per segment and
// head fills `resident` slots in one batch, for a kernel whose workgroups
// read only the head's total state (no record per segment): more or fewer
// segments than the plan's are both fine.
Plan rows_plan(const Plan &p, int64_t resident, int64_t per)
{
    if (resident <= 0)
        return p;
    Plan q = p;
    const int64_t want = std::max<int64_t>(resident / (per * std::max<int64_t>(p.BH, 1)), 1);
    const int64_t nchunks = std::max<int64_t>((p.N + kSegAlign - 1) / kSegAlign, 1);
    const int64_t ns = std::min(want, nchunks);
    const int64_t each = (nchunks + ns - 1) / ns;
    q.seg_len = each * kSegAlign;
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

// the head size the kernels run: D itself, or the next native size above it
// (the extra columns zero)
int64_t padded_d(int64_t D)
{
    for (int64_t d : {16, 32, 64, 128, 256})
        if (D <= d)
            return d;
    return 0;
}

int check_sizes(int64_t B, int64_t H, int64_t N, int64_t D, int causal)
{
    if (causal != 0 && causal != 1)
        return LA_ERR_UNSUPPORTED;
    if (B < 0 || H < 0 || N < 0)
        return LA_ERR_SHAPE;
    if (D < 1 || D > 256)
        return LA_ERR_UNSUPPORTED;
    int64_t t;
    if (__builtin_mul_overflow(B, H, &t) || __builtin_mul_overflow(t, N, &t) ||
        __builtin_mul_overflow(t, padded_d(D), &t) ||
        __builtin_mul_overflow(t, (int64_t)16, &t))
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

// outputs against inputs, and against each other unless `outs_checked`
// (outputs of a row layout that interleave by design, e.g. dQ, dK and dV
// side by side in each row: their spans overlap, their elements do not)
bool aliased(const Range *outs, int nout, const Range *ins, int nin, bool outs_checked = false)
{
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j)
            if (overlap(outs[i], ins[j]))
                return true;
        if (!outs_checked)
            for (int j = i + 1; j < nout; ++j)
                if (overlap(outs[i], outs[j]))
                    return true;
    }
    return false;
}

bool misaligned(const void *p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u); }

// elements an output of layout ol spans, from its pointer to one past its
// last element
int64_t out_extent(const OutLay &ol, int64_t B, int64_t H, int64_t N, int64_t D)
{
    return (B - 1) * ol.sb + (H - 1) * ol.sh + (N - 1) * ol.sn + D;
}

// An output layout the kernels can write: positive strides, rows of D
// elements that do not overlap (sn >= D), and, where the kernels store
// 16-byte pieces (every native head size), strides in whole 16 bytes.
bool layout_ok(const OutLay &ol, int64_t D, size_t esz, bool native_d)
{
    if (ol.sb <= 0 || ol.sh <= 0 || ol.sn < D || ol.H <= 0)
        return false;
    const int64_t v = (int64_t)(16 / esz);
    return !native_d || (ol.sb % v == 0 && ol.sh % v == 0 && ol.sn % v == 0);
}

int launched()
{
    return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

// Checked once per call before its first launch: an error that earlier HIP
// calls on this thread left pending is not this call's to report or to
// clear.  The call then launches nothing, leaves that error pending and
// returns LA_ERR_HIP_PENDING; with none pending, every error launched()
// reads afterwards is this call's own.  hipErrorNotReady (the answer of an
// earlier query, not a failure) is cleared.
int no_pending_error()
{
    const hipError_t e = hipPeekAtLastError();
    if (e == hipSuccess)
        return LA_OK;
    if (e == hipErrorNotReady) {
        (void)hipGetLastError();
        return LA_OK;
    }
    return LA_ERR_HIP_PENDING;
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
    // the first launch of a call (a call without a tracer makes one launch)
    if (t == nullptr || t->n == 0) {
        const int pend = no_pending_error();
        if (pend != LA_OK)
            return pend;
    }
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

// D = 256, every storage type (2-byte rows widened exactly to fp32): the
// fast reduction (four 128 x 128 blocks per segment) for both masks, the
// fast non-causal apply kernels (eight waves) and a dQ pass without the dS
// role (the gradient record then comes from the reduction)
template <class ST, int D>
constexpr bool wide_path()
{
    return D == 256;
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
            if constexpr (std::is_same<ST, StBF16>::value && D <= 128)
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
    if constexpr (D <= 16) {
        // width 16: the first-version kernels
        const dim3 grid((unsigned)(p.nseg * p.BH * C::CS));
        rc = traced(t, s, "state_local", [&] {
            k_state_local<ST, D><<<grid, dim3(C::NT), 0, s>>>(
                static_cast<const T *>(K), static_cast<const T *>(V), part, p.N, p.seg_len,
                (int)p.nseg, (int)p.dl);
        });
        done = true;
    }
    if (!done)
        return LA_ERR_UNSUPPORTED;
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
                if constexpr (std::is_same<ST, StBF16>::value) {
                    const Plan pf = rows_plan(
                        p, resident_wgs<bf::k_apply_bf<D, 0>>(bf::kApplyThreads), 1);
                    bf::k_apply_bf<D, 0><<<dim3((unsigned)(pf.nseg * pf.BH)),
                                           dim3(bf::kApplyThreads), 0, s>>>(
                        static_cast<const T *>(Q), nullptr, static_cast<T *>(O), nullptr,
                        den_out, nullptr, rec, pf.N, pf.seg_len, (int)pf.nseg, pf.n0, pf.ol);
                } else {
                    const Plan pf = rows_plan(
                        p, resident_wgs<nc::k_apply_nc<ST, D, 0>>(nc::kApplyThreads), 1);
                    nc::k_apply_nc<ST, D, 0><<<dim3((unsigned)(pf.nseg * pf.BH)),
                                               dim3(nc::kApplyThreads), 0, s>>>(
                        static_cast<const T *>(Q), nullptr, static_cast<T *>(O), nullptr,
                        den_out, rec, pf.N, pf.seg_len, (int)pf.nseg, pf.n0, pf.ol);
                }
            });
        return traced(t, s, "forward", [&] {
            if constexpr (std::is_same<ST, StBF16>::value)
                bf::k_fwd_causal_bf<D><<<dim3((unsigned)(p.nseg * p.BH)),
                                         dim3(cz::threads<D>()), 0, s>>>(
                    static_cast<const T *>(Q), static_cast<const T *>(K),
                    static_cast<const T *>(V), static_cast<T *>(O), den_out, rec, p.N, p.seg_len,
                    (int)p.nseg, p.n0, p.ol);
            else
                cz::k_fwd_causal<ST, D><<<dim3((unsigned)(p.nseg * p.BH)),
                                          dim3(cz::threads<D>()), 0, s>>>(
                    static_cast<const T *>(Q), static_cast<const T *>(K),
                    static_cast<const T *>(V), static_cast<T *>(O), den_out, rec, p.N, p.seg_len,
                    (int)p.nseg, p.n0, p.ol);
        });
    }
    if constexpr (wide_path<ST, D>()) {
        if (!p.causal)
            return traced(t, s, "forward", [&] {
                nc::k_apply_nc<ST, D, 0><<<dim3((unsigned)(p.nseg * p.BH)),
                                           dim3(nc::apply_threads<D>()), 0, s>>>(
                    static_cast<const T *>(Q), nullptr, static_cast<T *>(O), nullptr, den_out,
                    rec, p.N, p.seg_len, (int)p.nseg, p.n0, p.ol);
            });
        // causal: the chunk walk of la_kernels_causal.hpp with eight waves,
        // each holding a 256 x 32 slab of the running state (rows widened to
        // fp32 for every storage type)
        return traced(t, s, "forward", [&] {
            cz::k_fwd_causal<ST, D><<<dim3((unsigned)(p.nseg * p.BH)), dim3(cz::threads<D>()),
                                      0, s>>>(
                static_cast<const T *>(Q), static_cast<const T *>(K), static_cast<const T *>(V),
                static_cast<T *>(O), den_out, rec, p.N, p.seg_len, (int)p.nseg, p.n0, p.ol);
        });
    }
    if constexpr (D > 16) {
        return LA_ERR_UNSUPPORTED;  // every D from 32 up returned above
    } else {
        // width 16: the first-version kernels
        const dim3 grid((unsigned)(p.nseg * p.BH * C::CS));
        return traced(t, s, "forward", [&] {
            if (p.causal)
                k_forward<ST, D, true><<<grid, dim3(C::NT), 0, s>>>(
                    static_cast<const T *>(Q), static_cast<const T *>(K),
                    static_cast<const T *>(V), static_cast<T *>(O), den_out, rec, p.N,
                    p.seg_len, (int)p.nseg, p.n0, p.ol, (int)p.dl);
            else
                k_forward<ST, D, false><<<grid, dim3(C::NT), 0, s>>>(
                    static_cast<const T *>(Q), static_cast<const T *>(K),
                    static_cast<const T *>(V), static_cast<T *>(O), den_out, rec, p.N,
                    p.seg_len, (int)p.nseg, p.n0, p.ol, (int)p.dl);
        });
    }
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
                                                           (int)p.nseg, p.n0, p.ol);
            else
                cz::k_bwd_q_causal<ST, D><<<g1, nt, 0, s>>>(q, k, v, g, static_cast<T *>(dQ),
                                                            cbuf, fstate, p.N, p.seg_len,
                                                            (int)p.nseg, p.n0, p.ol);
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
            // one workgroup per CU: segments are merged so that the walk is
            // one batch of resident workgroups
            if constexpr (std::is_same<ST, StBF16>::value && D >= 64) {
                const int m = merge_factor(
                    p, resident_wgs<bf::k_bwd_kv_causal_bf2<D>>(128 * (D / 32)));
                bf::k_bwd_kv_causal_bf2<D>
                    <<<dim3((unsigned)((p.nseg + m - 1) / m * p.BH)), dim3(128 * (D / 32)), 0,
                       s>>>(q, k, v, g, static_cast<T *>(dK), static_cast<T *>(dV), cbuf, gpart,
                            p.N, p.seg_len, (int)p.nseg, m, p.ol);
            } else if constexpr (std::is_same<ST, StBF16>::value)
                bf::k_bwd_kv_causal_bf<D><<<dim3((unsigned)(2 * p.nseg * p.BH)), nt, 0, s>>>(
                    q, k, v, g, static_cast<T *>(dK), static_cast<T *>(dV), cbuf, gpart, p.N,
                    p.seg_len, (int)p.nseg, p.ol);
            else if constexpr (D >= 64) {
                const int m = merge_factor(
                    p, resident_wgs<cz::k_bwd_kv_causal2<ST, D>>(128 * (D / 32)));
                cz::k_bwd_kv_causal2<ST, D>
                    <<<dim3((unsigned)((p.nseg + m - 1) / m * p.BH)), dim3(128 * (D / 32)), 0,
                       s>>>(q, k, v, g, static_cast<T *>(dK), static_cast<T *>(dV), cbuf, gpart,
                            p.N, p.seg_len, (int)p.nseg, m, p.ol);
            } else
                cz::k_bwd_kv_causal<ST, D><<<dim3((unsigned)(2 * p.nseg * p.BH)), nt, 0, s>>>(
                    q, k, v, g, static_cast<T *>(dK), static_cast<T *>(dV), cbuf, gpart, p.N,
                    p.seg_len, (int)p.nseg, p.ol);
        });
    }
    if constexpr (CAUSAL && wide_path<ST, D>()) {
        // the causal walks with eight waves (a 256 x 32 state slab each), the
        // gradient records by the fast reduction, dK | dV by the two-parity
        // walk (the one-workgroup form would need the whole fp32 suffix state,
        // 256 KB, in LDS)
        const dim3 g1((unsigned)(p.nseg * p.BH)), nt(cz::threads<D>());
        rc = traced(t, s, "bwd_q", [&] {
            cz::k_bwd_q_causal<ST, D><<<g1, nt, 0, s>>>(q, k, v, g, static_cast<T *>(dQ), cbuf,
                                                        fstate, p.N, p.seg_len, (int)p.nseg,
                                                        p.n0, p.ol);
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
        if ((rc = scan(gpart, nullptr, p, 2, s, t, gin, gout)) != LA_OK)  // exclusive suffix
            return rc;
        if (dK == nullptr)
            return LA_OK;
        return traced(t, s, "bwd_kv", [&] {
            cz::k_bwd_kv_causal<ST, D><<<dim3((unsigned)(2 * p.nseg * p.BH)), nt, 0, s>>>(
                q, k, v, g, static_cast<T *>(dK), static_cast<T *>(dV), cbuf, gpart, p.N,
                p.seg_len, (int)p.nseg, p.ol);
        });
    }
    if constexpr (!CAUSAL && wide_path<ST, D>()) {
        // dQ and (c_i, 1/den_i); the gradient records by the fast reduction;
        // dK | dV by the eight-wave apply kernel
        const dim3 g1((unsigned)(p.nseg * p.BH));
        rc = traced(t, s, "bwd_q", [&] {
            nc::k_bwd_q_nc<ST, D, false><<<g1, dim3(512), 0, s>>>(
                g, q, static_cast<T *>(dQ), cbuf, fstate, p.N, p.seg_len, (int)p.nseg, p.n0, p.ol);
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
                p.seg_len, (int)p.nseg, p.n0, p.ol);
        });
    }
    if constexpr (!CAUSAL && nc_path<D>()) {
        const dim3 g1((unsigned)(p.nseg * p.BH));
        if constexpr (std::is_same<ST, StBF16>::value && D >= 64) {
            // bf16 matrix cores: dQ and the segment's gradient record in one
            // pass over Q and dO, segments sized for one batch of resident
            // workgroups
            const Plan pq = one_batch(p, resident_wgs<bf::k_bwd_q_bf<D>>(512));
            rc = traced(t, s, "bwd_q", [&] {
                bf::k_bwd_q_bf<D><<<dim3((unsigned)(pq.nseg * pq.BH)), dim3(512), 0, s>>>(
                    g, q, static_cast<T *>(dQ), gpart, fstate, pq.N, pq.seg_len, (int)pq.nseg,
                    pq.n0, pq.ol);
            });
            if (rc != LA_OK)
                return rc;
            if ((rc = scan(gpart, ws + l.gtot, pq, 0, s, t, gin, gout)) != LA_OK)
                return rc;
        } else if constexpr (std::is_same<ST, StBF16>::value) {
            // bf16 matrix cores: dQ with (c_i, 1/den_i), then the gradient
            // records from a second (bf16, half-size) read of Q and dO
            rc = traced(t, s, "bwd_q", [&] {
                bf::k_apply_bf<D, 1><<<g1, dim3(bf::kApplyThreads), 0, s>>>(
                    g, q, static_cast<T *>(dQ), nullptr, nullptr, cbuf, fstate, p.N, p.seg_len,
                    (int)p.nseg, p.n0, p.ol);
            });
            if (rc != LA_OK)
                return rc;
            rc = traced(t, s, "grad_state_local", [&] {
                bf::k_reduce_bf<D, true><<<g1, dim3(256), 0, s>>>(q, g, cbuf, gpart, p.N,
                                                                p.seg_len, (int)p.nseg);
            });
            if (rc != LA_OK)
                return rc;
            if ((rc = scan(gpart, ws + l.gtot, p, 0, s, t, gin, gout)) != LA_OK)
                return rc;
        } else {
            // dQ and the segment's gradient record in one pass over Q and dO,
            // its segments sized for one batch of resident workgroups
            const Plan pq = one_batch(p, resident_wgs<nc::k_bwd_q_nc<ST, D>>(512));
            rc = traced(t, s, "bwd_q", [&] {
                nc::k_bwd_q_nc<ST, D><<<dim3((unsigned)(pq.nseg * pq.BH)), dim3(512), 0, s>>>(
                    g, q, static_cast<T *>(dQ), gpart, fstate, pq.N, pq.seg_len, (int)pq.nseg,
                    pq.n0, pq.ol);
            });
            if (rc != LA_OK)
                return rc;
            if ((rc = scan(gpart, ws + l.gtot, pq, 0, s, t, gin, gout)) != LA_OK)
                return rc;
        }
        if (rc != LA_OK)
            return rc;
        if (dK == nullptr)
            return LA_OK;
        return traced(t, s, "bwd_kv", [&] {
            if constexpr (std::is_same<ST, StBF16>::value) {
                const Plan pk =
                    rows_plan(p, resident_wgs<bf::k_apply_bf<D, 2>>(bf::kApplyThreads), 2);
                bf::k_apply_bf<D, 2><<<dim3((unsigned)(2 * pk.nseg * pk.BH)),
                                       dim3(bf::kApplyThreads), 0, s>>>(
                    v, k, static_cast<T *>(dK), static_cast<T *>(dV), nullptr, nullptr,
                    ws + l.gtot, pk.N, pk.seg_len, (int)pk.nseg, pk.n0, pk.ol);
            } else {
                const Plan pk =
                    rows_plan(p, resident_wgs<nc::k_apply_nc<ST, D, 2>>(nc::kApplyThreads), 2);
                nc::k_apply_nc<ST, D, 2><<<dim3((unsigned)(2 * pk.nseg * pk.BH)),
                                           dim3(nc::kApplyThreads), 0, s>>>(
                    v, k, static_cast<T *>(dK), static_cast<T *>(dV), nullptr, ws + l.gtot, pk.N,
                    pk.seg_len, (int)pk.nseg, pk.n0, pk.ol);
            }
        });
    }
    if constexpr (D > 16) {
        return LA_ERR_UNSUPPORTED;  // every D from 32 up returned above
    } else {
        // width 16: the first-version kernels (dQ fused with the gradient record)
        rc = traced(t, s, "bwd_q", [&] {
            k_bwd_q<ST, D, CAUSAL><<<dim3((unsigned)(p.nseg * p.BH)), dim3(CQ::NT), 0, s>>>(
                q, k, v, g, static_cast<T *>(dQ), fstate, gpart, cbuf, p.N, p.seg_len,
                (int)p.nseg, p.n0, p.ol, (int)p.dl);
        });
        if (rc != LA_OK)
            return rc;
        const dim3 grid((unsigned)(p.nseg * p.BH * C::CS));
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
                p.seg_len, (int)p.nseg, p.ol, (int)p.dl);
        });
    }
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

size_t elem_size(int dtype) { return dtype == LA_FP32 ? 4 : 2; }

bool valid_dtype(int dtype) { return dtype == LA_FP32 || dtype == LA_BF16 || dtype == LA_FP16; }

// calls the matrix-core kernels take as they are; the others are padded
bool native(int64_t D) { return supported_d(D); }

// tokens a carried-in record may stand for (counts enter the kernels as fp32)
constexpr int64_t kMaxCarry = (int64_t)1 << 40;

// A call over zero tokens passes the carried record through: out = in, or
// zero without one (the scan kernel over zero segments; no memset or copy
// node, so the call stays capturable).
int pass_record(const float *in, float *out, int64_t BH, int64_t D, hipStream_t s)
{
    if (out == nullptr)
        return LA_OK;
    Plan p{};
    p.BH = BH;
    p.D = D;
    p.PS = D * D + 2 * D;
    p.nseg = 0;
    return scan(out, out, p, 0, s, nullptr, in, nullptr);
}

size_t record_bytes(int64_t BH, int64_t D) { return (size_t)(BH * (D * D + 2 * D)) * sizeof(float); }

// Native forward (supported D, fp32 or bf16).  Arguments are validated here.
int forward_impl(bool require_o, const void *Q, const void *K, const void *V, void *O,
                 int64_t B, int64_t H, int64_t N, int64_t D, int causal, int dtype,
                 const float *cin, int64_t n_carry, float *cout, float *den_out,
                 void *state_out, void *ws, size_t ws_bytes, hipStream_t s, Tracer *t,
                 const OutLay *ol = nullptr, int64_t dl = 0)
{
    if (!valid_dtype(dtype))
        return LA_ERR_DTYPE;
    int rc = check_sizes(B, H, N, D, causal);
    if (rc != LA_OK)
        return rc;
    // dl > 0: heads of dl <= 16 columns run at width D = 16 on the caller's
    // rows (dl elements apart); the records stay at width D
    if (!(supported_d(D) || (D == 16 && dl > 0 && dl <= 16)))
        return LA_ERR_UNSUPPORTED;
    if (n_carry < 0 || n_carry > kMaxCarry)
        return LA_ERR_SHAPE;
    if (B * H == 0)
        return LA_OK;
    const size_t rb = record_bytes(B * H, D);
    if (N == 0) {
        if (misaligned(cout) || misaligned(cin))
            return LA_ERR_ALIGN;
        if (overlap({(const char *)cout, rb}, {(const char *)cin, rb}))
            return LA_ERR_ALIAS;
        return pass_record(cin, cout, B * H, D, s);
    }
    // O == null asks for the state only: something must receive it
    if (!Q || !K || !V || !ws || (!O && (require_o || den_out || (!cout && !state_out))))
        return LA_ERR_NULL;
    Plan p = make_plan(B, H, N, D, causal);
    p.n0 = (float)n_carry;
    if (dl > 0) {
        p.dl = dl;
        p.ol = plain_layout(H, N, dl);
    }
    if (ol != nullptr) {
        if (!layout_ok(*ol, p.dl, elem_size(dtype), p.dl == D))
            return LA_ERR_ALIGN;
        p.ol = *ol;
    }
    // the forward uses the first two workspace regions (records, totals)
    const size_t need = (size_t)make_layout(p).gpart * sizeof(float);
    if (ws_bytes < need)
        return LA_ERR_WORKSPACE;
    if (misaligned(Q) || misaligned(K) || misaligned(V) || misaligned(O) ||
        misaligned(den_out) || misaligned(state_out) || misaligned(ws) || misaligned(cin) ||
        misaligned(cout))
        return LA_ERR_ALIGN;
    const size_t tb = (size_t)(B * H * N * p.dl) * elem_size(dtype);
    const size_t ob = (size_t)out_extent(p.ol, B, H, N, p.dl) * elem_size(dtype);
    const Range ins[4] = {{(const char *)Q, tb},
                          {(const char *)K, tb},
                          {(const char *)V, tb},
                          {(const char *)cin, rb}};
    const Range outs[5] = {
        {(const char *)O, ob},
        {(const char *)den_out, (size_t)(B * H * N) * sizeof(float)},
        {(const char *)state_out, (size_t)state_floats(p) * sizeof(float)},
        {(const char *)ws, need},
        {(const char *)cout, rb}};
    if (aliased(outs, 5, ins, 4))
        return LA_ERR_ALIAS;
    float *w = static_cast<float *>(ws);
    switch (dtype) {
    case LA_FP32:
        return dispatch_forward<StF32>(Q, K, V, O, den_out, state_out, w, p, s, t, cin, cout);
    case LA_BF16:
        return dispatch_forward<StBF16>(Q, K, V, O, den_out, state_out, w, p, s, t, cin, cout);
    default:
        return dispatch_forward<StF16>(Q, K, V, O, den_out, state_out, w, p, s, t, cin, cout);
    }
}

// Native backward (supported D, fp32 or bf16).  Arguments are validated here.
int backward_impl(bool require_kv, const void *Q, const void *K, const void *V,
                  const void *dO, void *dQ, void *dK, void *dV, int64_t B, int64_t H,
                  int64_t N, int64_t D, int causal, int dtype, const float *cin,
                  int64_t n_carry, const float *gin, float *gout, const void *state_in,
                  void *ws, size_t ws_bytes, hipStream_t s, Tracer *t,
                  const OutLay *ol = nullptr, int64_t dl = 0)
{
    if (!valid_dtype(dtype))
        return LA_ERR_DTYPE;
    int rc = check_sizes(B, H, N, D, causal);
    if (rc != LA_OK)
        return rc;
    // dl > 0: heads of dl <= 16 columns run at width D = 16 on the caller's
    // rows (dl elements apart); the records stay at width D
    if (!(supported_d(D) || (D == 16 && dl > 0 && dl <= 16)))
        return LA_ERR_UNSUPPORTED;
    if (n_carry < 0 || n_carry > kMaxCarry)
        return LA_ERR_SHAPE;
    if (B * H == 0)
        return LA_OK;
    const size_t rb = record_bytes(B * H, D);
    if (N == 0) {
        if (misaligned(gout) || misaligned(gin))
            return LA_ERR_ALIGN;
        if (overlap({(const char *)gout, rb}, {(const char *)gin, rb}))
            return LA_ERR_ALIAS;
        return pass_record(gin, gout, B * H, D, s);
    }
    // dK and dV: both given, or (segment calls only) both null
    if (!Q || !K || !V || !dO || !dQ || !ws || (dK == nullptr) != (dV == nullptr) ||
        (require_kv && dK == nullptr))
        return LA_ERR_NULL;
    Plan p = make_plan(B, H, N, D, causal);
    p.n0 = (float)n_carry;
    if (dl > 0) {
        p.dl = dl;
        p.ol = plain_layout(H, N, dl);
    }
    if (ol != nullptr) {
        if (!layout_ok(*ol, p.dl, elem_size(dtype), p.dl == D))
            return LA_ERR_ALIGN;
        p.ol = *ol;
    }
    const size_t need = (size_t)make_layout(p).total * sizeof(float);
    if (ws_bytes < need)
        return LA_ERR_WORKSPACE;
    if (misaligned(Q) || misaligned(K) || misaligned(V) || misaligned(dO) ||
        misaligned(dQ) || misaligned(dK) || misaligned(dV) || misaligned(state_in) ||
        misaligned(ws) || misaligned(cin) || misaligned(gin) || misaligned(gout))
        return LA_ERR_ALIGN;
    const size_t tb = (size_t)(B * H * N * p.dl) * elem_size(dtype);
    const size_t ob = (size_t)out_extent(p.ol, B, H, N, p.dl) * elem_size(dtype);
    const Range ins[7] = {{(const char *)Q, tb},
                          {(const char *)K, tb},
                          {(const char *)V, tb},
                          {(const char *)dO, tb},
                          {(const char *)state_in, (size_t)state_floats(p) * sizeof(float)},
                          {(const char *)cin, rb},
                          {(const char *)gin, rb}};
    const Range outs[5] = {{(const char *)dQ, ob},
                           {(const char *)dK, ob},
                           {(const char *)dV, ob},
                           {(const char *)ws, need},
                           {(const char *)gout, rb}};
    if (aliased(outs, 5, ins, 7, ol != nullptr) ||
        (ol != nullptr && (aliased(outs + 3, 2, outs, 3) || overlap(outs[3], outs[4]))))
        return LA_ERR_ALIAS;
    float *w = static_cast<float *>(ws);
    switch (dtype) {
    case LA_FP32:
        return dispatch_backward<StF32>(Q, K, V, dO, dQ, dK, dV, state_in, w, p, s, t, cin, gin,
                                        gout);
    case LA_BF16:
        return dispatch_backward<StBF16>(Q, K, V, dO, dQ, dK, dV, state_in, w, p, s, t, cin,
                                         gin, gout);
    default:
        return dispatch_backward<StF16>(Q, K, V, dO, dQ, dK, dV, state_in, w, p, s, t, cin, gin,
                                        gout);
    }
}

// ------------------------------------------------------------ staging
// Workspace of a padded call, in bytes: the native call's workspace at Dp,
// then seven padded [B,H,N,Dp] tensors, then three padded records, each
// region 256-byte aligned.  Heads of D <= 16 run at width Dp = 16 on the
// caller's own rows: no padded tensors, only the records.
struct Staging {
    int64_t Dp;
    size_t inner, tensor, record;
    size_t off_inner, off_tensor[7], off_record[3], total;
};

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

Staging make_staging(int64_t B, int64_t H, int64_t N, int64_t D, int causal, int dtype)
{
    Staging g{};
    g.Dp = padded_d(D);
    g.inner = N > 0 ? (size_t)make_layout(make_plan(B, H, N, g.Dp, causal)).total * sizeof(float)
                    : 0;
    g.tensor = g.Dp == 16 ? 0 : up256((size_t)(B * H * N * g.Dp) * elem_size(dtype));
    g.record = up256(record_bytes(B * H, g.Dp));
    size_t off = 0;
    g.off_inner = off;
    off += up256(g.inner);
    for (int i = 0; i < 7; ++i) {
        g.off_tensor[i] = off;
        off += g.tensor;
    }
    for (int i = 0; i < 3; ++i) {
        g.off_record[i] = off;
        off += g.record;
    }
    g.total = off;
    return g;
}

int grid_for(int64_t n)
{
    return (int)std::max<int64_t>(1, std::min<int64_t>((n + stg::kThreads - 1) / stg::kThreads,
                                                       (int64_t)1 << 16));
}

// [rows, D] <-> [rows, Dp] in storage `dtype` (pad: to_padded, else unpad)
// (unpad: rows r = bh * N + n go to row n of head bh in the layout `ol`, or
// to row r of a plain [rows, D] tensor)
int stage_tensor(const char *name, bool to_padded, const void *src, void *dst, int dtype,
                 int64_t D, int64_t Dp, int64_t rows, hipStream_t s, Tracer *t, int64_t N = 1,
                 const OutLay *ol = nullptr)
{
    const int64_t chunks = rows * (Dp * (int64_t)elem_size(dtype) / 16);
    const dim3 grid(grid_for(chunks)), blk(stg::kThreads);
    const OutLay lay = ol ? *ol : OutLay{N * D, N * D, D, 1};
    return traced(t, s, name, [&] {
        if (dtype == LA_FP32) {
            if (to_padded)
                stg::k_pad<StF32><<<grid, blk, 0, s>>>(static_cast<const float *>(src),
                                                       static_cast<float *>(dst), rows, (int)D,
                                                       (int)Dp);
            else
                stg::k_unpad<StF32><<<grid, blk, 0, s>>>(static_cast<const float *>(src),
                                                         static_cast<float *>(dst), rows,
                                                         (int)D, (int)Dp, N, lay);
        } else {
            // bf16 and fp16 move as the same 16-bit words
            if (to_padded)
                stg::k_pad<StBF16><<<grid, blk, 0, s>>>(static_cast<const uint16_t *>(src),
                                                        static_cast<uint16_t *>(dst), rows,
                                                        (int)D, (int)Dp);
            else
                stg::k_unpad<StBF16><<<grid, blk, 0, s>>>(static_cast<const uint16_t *>(src),
                                                          static_cast<uint16_t *>(dst), rows,
                                                          (int)D, (int)Dp, N, lay);
        }
    });
}

// a record of width Ds as one of width Dd (zero where Dd > Ds); `to` names
// the direction for the tracer
int stage_record(bool to, const float *src, int64_t Ds, float *dst, int64_t Dd, int64_t BH,
                 hipStream_t s, Tracer *t)
{
    return traced(t, s, to ? "stage_record" : "unstage_record", [&] {
        stg::k_stage_record<<<dim3(grid_for(BH * (Dd * Dd + 2 * Dd))), dim3(stg::kThreads), 0,
                              s>>>(src, dst, BH, (int)Ds, (int)Dd);
    });
}

// Forward of any supported call: native, or padded through the workspace.
int forward_any(bool require_o, const void *Q, const void *K, const void *V, void *O,
                int64_t B, int64_t H, int64_t N, int64_t D, int causal, int dtype,
                const float *cin, int64_t n_carry, float *cout, float *den_out,
                void *state_out, void *ws, size_t ws_bytes, hipStream_t s, Tracer *t,
                const OutLay *ol = nullptr)
{
    if (!valid_dtype(dtype))
        return LA_ERR_DTYPE;
    int rc = check_sizes(B, H, N, D, causal);
    if (rc != LA_OK)
        return rc;
    if (native(D))
        return forward_impl(require_o, Q, K, V, O, B, H, N, D, causal, dtype, cin, n_carry,
                            cout, den_out, state_out, ws, ws_bytes, s, t, ol);
    if (n_carry < 0 || n_carry > kMaxCarry)
        return LA_ERR_SHAPE;
    if (B * H == 0)
        return LA_OK;
    const int64_t BH = B * H;
    const size_t rb = record_bytes(BH, D);
    if (misaligned(cin) || misaligned(cout))
        return LA_ERR_ALIGN;
    if (N == 0) {
        if (overlap({(const char *)cout, rb}, {(const char *)cin, rb}))
            return LA_ERR_ALIAS;
        return cout ? stage_record(true, cin, D, cout, D, BH, s, t) : LA_OK;
    }
    if (!Q || !K || !V || !ws || (!O && (require_o || den_out || (!cout && !state_out))))
        return LA_ERR_NULL;
    const Staging g = make_staging(B, H, N, D, causal, dtype);
    if (ws_bytes < g.total)
        return LA_ERR_WORKSPACE;
    if (misaligned(Q) || misaligned(K) || misaligned(V) || misaligned(O) ||
        misaligned(den_out) || misaligned(state_out) || misaligned(ws))
        return LA_ERR_ALIGN;
    Plan pp = make_plan(B, H, N, g.Dp, causal);
    if (ol != nullptr && !layout_ok(*ol, D, elem_size(dtype), false))
        return LA_ERR_ALIGN;
    const size_t tb = (size_t)(BH * N * D) * elem_size(dtype);
    const size_t ob =
        (size_t)out_extent(ol ? *ol : plain_layout(H, N, D), B, H, N, D) * elem_size(dtype);
    const Range ins[4] = {{(const char *)Q, tb},
                          {(const char *)K, tb},
                          {(const char *)V, tb},
                          {(const char *)cin, rb}};
    const Range outs[5] = {
        {(const char *)O, ob},
        {(const char *)den_out, (size_t)(BH * N) * sizeof(float)},
        {(const char *)state_out, (size_t)state_floats(pp) * sizeof(float)},
        {(const char *)ws, g.total},
        {(const char *)cout, rb}};
    if (aliased(outs, 5, ins, 4))
        return LA_ERR_ALIAS;
    char *w = static_cast<char *>(ws);
    void *tq = w + g.off_tensor[0], *tk = w + g.off_tensor[1], *tv = w + g.off_tensor[2],
         *to = w + g.off_tensor[3];
    float *r_in = reinterpret_cast<float *>(w + g.off_record[0]);
    float *r_out = reinterpret_cast<float *>(w + g.off_record[1]);
    if (g.Dp == 16) {
        // D <= 16: the kernels read and write the caller's rows directly;
        // only the carried records change width
        if (cin && (rc = stage_record(true, cin, D, r_in, g.Dp, BH, s, t)) != LA_OK)
            return rc;
        rc = forward_impl(require_o, Q, K, V, O, B, H, N, g.Dp, causal, dtype,
                          cin ? r_in : nullptr, n_carry, cout ? r_out : nullptr, den_out,
                          state_out, w + g.off_inner, g.inner, s, t, ol, D);
        if (rc != LA_OK)
            return rc;
        return cout ? stage_record(false, r_out, g.Dp, cout, D, BH, s, t) : LA_OK;
    }
    const int64_t rows = BH * N;
    if ((rc = stage_tensor("stage", true, Q, tq, dtype, D, g.Dp, rows, s, t)) != LA_OK ||
        (rc = stage_tensor("stage", true, K, tk, dtype, D, g.Dp, rows, s, t)) != LA_OK ||
        (rc = stage_tensor("stage", true, V, tv, dtype, D, g.Dp, rows, s, t)) != LA_OK)
        return rc;
    if (cin && (rc = stage_record(true, cin, D, r_in, g.Dp, BH, s, t)) != LA_OK)
        return rc;
    rc = forward_impl(require_o, tq, tk, tv, O ? to : nullptr, B, H, N, g.Dp, causal, dtype,
                      cin ? r_in : nullptr, n_carry, cout ? r_out : nullptr, den_out,
                      state_out, w + g.off_inner, g.inner, s, t);
    if (rc != LA_OK)
        return rc;
    if (O && (rc = stage_tensor("unstage", false, to, O, dtype, D, g.Dp, rows, s, t, N, ol)) !=
                 LA_OK)
        return rc;
    if (cout && (rc = stage_record(false, r_out, g.Dp, cout, D, BH, s, t)) != LA_OK)
        return rc;
    return LA_OK;
}

// Backward of any supported call: native, or padded through the workspace.
int backward_any(bool require_kv, const void *Q, const void *K, const void *V,
                 const void *dO, void *dQ, void *dK, void *dV, int64_t B, int64_t H,
                 int64_t N, int64_t D, int causal, int dtype, const float *cin,
                 int64_t n_carry, const float *gin, float *gout, const void *state_in,
                 void *ws, size_t ws_bytes, hipStream_t s, Tracer *t,
                 const OutLay *ol = nullptr)
{
    if (!valid_dtype(dtype))
        return LA_ERR_DTYPE;
    int rc = check_sizes(B, H, N, D, causal);
    if (rc != LA_OK)
        return rc;
    if (native(D))
        return backward_impl(require_kv, Q, K, V, dO, dQ, dK, dV, B, H, N, D, causal, dtype,
                             cin, n_carry, gin, gout, state_in, ws, ws_bytes, s, t, ol);
    if (n_carry < 0 || n_carry > kMaxCarry)
        return LA_ERR_SHAPE;
    if (B * H == 0)
        return LA_OK;
    const int64_t BH = B * H;
    const size_t rb = record_bytes(BH, D);
    if (misaligned(gin) || misaligned(gout) || misaligned(cin))
        return LA_ERR_ALIGN;
    if (N == 0) {
        if (overlap({(const char *)gout, rb}, {(const char *)gin, rb}))
            return LA_ERR_ALIAS;
        return gout ? stage_record(true, gin, D, gout, D, BH, s, t) : LA_OK;
    }
    if (!Q || !K || !V || !dO || !dQ || !ws || (dK == nullptr) != (dV == nullptr) ||
        (require_kv && dK == nullptr))
        return LA_ERR_NULL;
    const Staging g = make_staging(B, H, N, D, causal, dtype);
    if (ws_bytes < g.total)
        return LA_ERR_WORKSPACE;
    if (misaligned(Q) || misaligned(K) || misaligned(V) || misaligned(dO) ||
        misaligned(dQ) || misaligned(dK) || misaligned(dV) || misaligned(state_in) ||
        misaligned(ws))
        return LA_ERR_ALIGN;
    Plan pp = make_plan(B, H, N, g.Dp, causal);
    if (ol != nullptr && !layout_ok(*ol, D, elem_size(dtype), false))
        return LA_ERR_ALIGN;
    const size_t tb = (size_t)(BH * N * D) * elem_size(dtype);
    const size_t ob =
        (size_t)out_extent(ol ? *ol : plain_layout(H, N, D), B, H, N, D) * elem_size(dtype);
    const Range ins[7] = {{(const char *)Q, tb},
                          {(const char *)K, tb},
                          {(const char *)V, tb},
                          {(const char *)dO, tb},
                          {(const char *)state_in, (size_t)state_floats(pp) * sizeof(float)},
                          {(const char *)cin, rb},
                          {(const char *)gin, rb}};
    const Range outs[5] = {{(const char *)dQ, ob},
                           {(const char *)dK, ob},
                           {(const char *)dV, ob},
                           {(const char *)ws, g.total},
                           {(const char *)gout, rb}};
    if (aliased(outs, 5, ins, 7, ol != nullptr) ||
        (ol != nullptr && (aliased(outs + 3, 2, outs, 3) || overlap(outs[3], outs[4]))))
        return LA_ERR_ALIAS;
    char *w = static_cast<char *>(ws);
    void *T_[7];
    for (int i = 0; i < 7; ++i)
        T_[i] = w + g.off_tensor[i];
    float *r_cin = reinterpret_cast<float *>(w + g.off_record[0]);
    float *r_gin = reinterpret_cast<float *>(w + g.off_record[1]);
    float *r_gout = reinterpret_cast<float *>(w + g.off_record[2]);
    if (g.Dp == 16) {
        // D <= 16: the kernels read and write the caller's rows directly;
        // only the carried records change width
        if (cin && !state_in && (rc = stage_record(true, cin, D, r_cin, g.Dp, BH, s, t)) != LA_OK)
            return rc;
        if (gin && (rc = stage_record(true, gin, D, r_gin, g.Dp, BH, s, t)) != LA_OK)
            return rc;
        rc = backward_impl(require_kv, Q, K, V, dO, dQ, dK, dV, B, H, N, g.Dp, causal, dtype,
                           (cin && !state_in) ? r_cin : nullptr, n_carry, gin ? r_gin : nullptr,
                           gout ? r_gout : nullptr, state_in, w + g.off_inner, g.inner, s, t, ol,
                           D);
        if (rc != LA_OK)
            return rc;
        return gout ? stage_record(false, r_gout, g.Dp, gout, D, BH, s, t) : LA_OK;
    }
    const int64_t rows = BH * N;
    const void *src[4] = {Q, K, V, dO};
    for (int i = 0; i < 4; ++i)
        if ((rc = stage_tensor("stage", true, src[i], T_[i], dtype, D, g.Dp, rows, s, t)) !=
            LA_OK)
            return rc;
    if (cin && !state_in && (rc = stage_record(true, cin, D, r_cin, g.Dp, BH, s, t)) != LA_OK)
        return rc;
    if (gin && (rc = stage_record(true, gin, D, r_gin, g.Dp, BH, s, t)) != LA_OK)
        return rc;
    const bool kv = dK != nullptr;
    rc = backward_impl(require_kv, T_[0], T_[1], T_[2], T_[3], T_[4], kv ? T_[5] : nullptr,
                       kv ? T_[6] : nullptr, B, H, N, g.Dp, causal, dtype,
                       (cin && !state_in) ? r_cin : nullptr, n_carry, gin ? r_gin : nullptr,
                       gout ? r_gout : nullptr, state_in, w + g.off_inner, g.inner, s, t);
    if (rc != LA_OK)
        return rc;
    if ((rc = stage_tensor("unstage", false, T_[4], dQ, dtype, D, g.Dp, rows, s, t, N, ol)) !=
        LA_OK)
        return rc;
    if (kv &&
        ((rc = stage_tensor("unstage", false, T_[5], dK, dtype, D, g.Dp, rows, s, t, N, ol)) !=
             LA_OK ||
         (rc = stage_tensor("unstage", false, T_[6], dV, dtype, D, g.Dp, rows, s, t, N, ol)) !=
             LA_OK))
        return rc;
    if (gout && (rc = stage_record(false, r_gout, g.Dp, gout, D, BH, s, t)) != LA_OK)
        return rc;
    return LA_OK;
}

template <class ST>
int launch_decode(const void *q, const void *k, const void *v, void *o, int64_t BH, int64_t H,
                  int64_t D, const float *rin, float *rout, const int64_t *counts, float n_all,
                  float *den, hipStream_t s)
{
    typedef typename ST::T T;
    const T *qq = static_cast<const T *>(q), *kk = static_cast<const T *>(k),
            *vv = static_cast<const T *>(v);
    T *oo = static_cast<T *>(o);
    const int pend = no_pending_error();
    if (pend != LA_OK)
        return pend;
#define LA_DEC(d)                                                                          \
    dec::k_decode<ST, d><<<dim3((unsigned)(BH * dec::blocks_per_head<d>())),              \
                           dim3(dec::kThreads), 0, s>>>(qq, kk, vv, oo, den, rin, rout,    \
                                                        counts, n_all, (int)H)
    switch (D) {
    case 16: LA_DEC(16); return launched();
    case 32: LA_DEC(32); return launched();
    case 64: LA_DEC(64); return launched();
    case 128: LA_DEC(128); return launched();
    case 256: LA_DEC(256); return launched();
    default: break;
    }
#undef LA_DEC
    dec::k_decode_any<ST><<<dim3((unsigned)(BH * ((D + 31) / 32))), dim3(dec::kThreads), 0, s>>>(
        qq, kk, vv, oo, den, rin, rout, counts, n_all, (int)H, (int)D);
    return launched();
}

// Workspace bytes of a forward call: the records and totals at a native
// head size, the whole staging layout for a padded one; 0 when there is
// nothing to do.  Arguments already validated.
size_t forward_ws_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int causal, int dtype)
{
    if (B * H * N == 0)
        return 0;
    if (native(D))
        return (size_t)make_layout(make_plan(B, H, N, D, causal)).gpart * sizeof(float);
    return make_staging(B, H, N, D, causal, dtype).total;
}

}  // namespace

// ------------------------------------------------- outputs in a given layout
namespace la_internal {

int forward_to(const void *Q, const void *K, const void *V, void *O, int64_t B, int64_t H,
               int64_t N, int64_t D, int causal, int dtype, void *state_out, void *ws,
               size_t ws_bytes, void *stream, OutStrides o)
{
    const la::OutLay ol{o.sb, o.sh, o.sn, std::max<int64_t>(H, 1)};
    Tracer t{nullptr, 0, 0, nullptr};
    return forward_any(true, Q, K, V, O, B, H, N, D, causal, dtype, nullptr, 0, nullptr,
                       nullptr, state_out, ws, ws_bytes, static_cast<hipStream_t>(stream), &t,
                       &ol);
}

int backward_to(const void *Q, const void *K, const void *V, const void *dO, void *dQ,
                void *dK, void *dV, int64_t B, int64_t H, int64_t N, int64_t D, int causal,
                int dtype, const void *state_in, void *ws, size_t ws_bytes, void *stream,
                OutStrides o)
{
    const la::OutLay ol{o.sb, o.sh, o.sn, std::max<int64_t>(H, 1)};
    Tracer t{nullptr, 0, 0, nullptr};
    return backward_any(true, Q, K, V, dO, dQ, dK, dV, B, H, N, D, causal, dtype, nullptr, 0,
                        nullptr, nullptr, state_in, ws, ws_bytes,
                        static_cast<hipStream_t>(stream), &t, &ol);
}

}  // namespace la_internal

// ------------------------------------------------- forward without a workspace
// The workspace of la_forward_noalloc: a static array in device memory, one
// copy on every device the library runs on, held until the process ends.  Host
// code never passes this name to a kernel or a copy (on the host it is only a
// stand-in for the symbol): the device address of each device's copy comes
// from hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) unsigned char scratch[LA_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_lock;
void *g_scratch_addr[64];

int scratch_on_current_device(void **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return LA_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_scratch_lock);
    if (g_scratch_addr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return LA_ERR_HIP;
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return LA_OK;
}

}  // namespace

extern "C" {

int la_forward_noalloc(const void *Q, const void *K, const void *V, void *O, int64_t B,
                       int64_t H, int64_t N, int64_t D, int causal, int dtype, float *den_out,
                       void *state_out, void *stream)
{
    if (!valid_dtype(dtype))
        return LA_ERR_DTYPE;
    int rc = check_sizes(B, H, N, D, causal);
    if (rc != LA_OK)
        return rc;
    const size_t need = forward_ws_bytes(B, H, N, D, causal, dtype);
    if (need > (size_t)LA_SCRATCH_BYTES)
        return LA_ERR_WORKSPACE;
    void *ws = nullptr;
    if (need > 0) {
        if ((rc = no_pending_error()) != LA_OK)
            return rc;
        if ((rc = scratch_on_current_device(&ws)) != LA_OK)
            return rc;
    }
    Tracer t{nullptr, 0, 0, nullptr};
    return forward_any(true, Q, K, V, O, B, H, N, D, causal, dtype, nullptr, 0, nullptr,
                       den_out, state_out, ws, (size_t)LA_SCRATCH_BYTES,
                       static_cast<hipStream_t>(stream), &t);
}

int la_decode_step(const void *q, const void *k, const void *v, void *o, int64_t B, int64_t H,
                   int64_t D, int dtype, const float *state_in, float *state_out,
                   const int64_t *counts, int64_t n_prev, float *den_out, void *stream)
{
    if (!valid_dtype(dtype))
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
    const size_t rb = record_bytes(B * H, D);
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
    switch (dtype) {
    case LA_FP32:
        return launch_decode<StF32>(q, k, v, o, B * H, H, D, state_in, state_out, counts,
                                    (float)n_prev, den_out, s);
    case LA_BF16:
        return launch_decode<StBF16>(q, k, v, o, B * H, H, D, state_in, state_out, counts,
                                     (float)n_prev, den_out, s);
    default:
        return launch_decode<StF16>(q, k, v, o, B * H, H, D, state_in, state_out, counts,
                                    (float)n_prev, den_out, s);
    }
}

const char *la_status_string(int status)
{
    switch (status) {
    case LA_OK: return "LA_OK";
    case LA_ERR_NULL: return "LA_ERR_NULL: a required pointer is NULL";
    case LA_ERR_SHAPE: return "LA_ERR_SHAPE: negative or too large size";
    case LA_ERR_DTYPE: return "LA_ERR_DTYPE: dtype must be LA_FP32, LA_BF16 or LA_FP16";
    case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED: D must be 1..256 and causal 0 or 1";
    case LA_ERR_WORKSPACE: return "LA_ERR_WORKSPACE: workspace too small";
    case LA_ERR_ALIAS: return "LA_ERR_ALIAS: an output overlaps an input or another output";
    case LA_ERR_ALIGN: return "LA_ERR_ALIGN: device pointers must be 16-byte aligned";
    case LA_ERR_HIP: return "LA_ERR_HIP: a HIP launch failed";
    case LA_ERR_HIP_PENDING:
        return "LA_ERR_HIP_PENDING: a HIP error from earlier work was pending; nothing was "
               "launched and the error was left pending";
    default: return "unknown la_status";
    }
}

int64_t la_num_segments(int64_t B, int64_t H, int64_t N, int64_t D, int causal)
{
    if (check_sizes(B, H, N, D, causal) != LA_OK)
        return 0;
    return make_plan(B, H, N, padded_d(D), causal).nseg;
}

size_t la_workspace_size_for(int64_t B, int64_t H, int64_t N, int64_t D, int causal,
                             int dtype)
{
    if (!valid_dtype(dtype) || check_sizes(B, H, N, D, causal) != LA_OK || B * H * N == 0)
        return 0;
    if (native(D))
        return (size_t)make_layout(make_plan(B, H, N, D, causal)).total * sizeof(float);
    return make_staging(B, H, N, D, causal, dtype).total;
}

size_t la_workspace_size(int64_t B, int64_t H, int64_t N, int64_t D, int causal)
{
    // padded fp32 tensors are the largest; native D needs the same for every
    // storage type
    return la_workspace_size_for(B, H, N, D, causal, LA_FP32);
}

size_t la_state_size(int64_t B, int64_t H, int64_t N, int64_t D, int causal)
{
    if (check_sizes(B, H, N, D, causal) != LA_OK || B * H * N == 0)
        return 0;
    return (size_t)state_floats(make_plan(B, H, N, padded_d(D), causal)) * sizeof(float);
}

size_t la_record_size(int64_t B, int64_t H, int64_t D)
{
    if (B < 0 || H < 0 || D < 1 || D > 256 || B * H > (int64_t)1 << 22)
        return 0;
    return record_bytes(B * H, D);
}

int la_forward_traced(const void *Q, const void *K, const void *V, void *O, int64_t B,
                      int64_t H, int64_t N, int64_t D, int causal, int dtype, float *den_out,
                      void *state_out, void *ws, size_t ws_bytes, void *stream,
                      void *const *events, int n_events, int *n_launched, const char **names)
{
    Tracer t{events, events ? n_events : 0, 0, names};
    const int rc = forward_any(true, Q, K, V, O, B, H, N, D, causal, dtype, nullptr, 0, nullptr,
                               den_out, state_out, ws, ws_bytes,
                               static_cast<hipStream_t>(stream), &t);
    if (n_launched)
        *n_launched = t.n;
    return rc;
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
    Tracer t{nullptr, 0, 0, nullptr};
    return forward_any(false, Q, K, V, O, B, H, N, D, causal, dtype, carry_in, n_carry,
                       carry_out, den_out, state_out, ws, ws_bytes,
                       static_cast<hipStream_t>(stream), &t);
}

int la_backward_traced(const void *Q, const void *K, const void *V, const void *dO, void *dQ,
                       void *dK, void *dV, int64_t B, int64_t H, int64_t N, int64_t D,
                       int causal, int dtype, const void *state_in, void *ws, size_t ws_bytes,
                       void *stream, void *const *events, int n_events, int *n_launched,
                       const char **names)
{
    Tracer t{events, events ? n_events : 0, 0, names};
    const int rc = backward_any(true, Q, K, V, dO, dQ, dK, dV, B, H, N, D, causal, dtype,
                                nullptr, 0, nullptr, nullptr, state_in, ws, ws_bytes,
                                static_cast<hipStream_t>(stream), &t);
    if (n_launched)
        *n_launched = t.n;
    return rc;
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
    Tracer t{nullptr, 0, 0, nullptr};
    return backward_any(false, Q, K, V, dO, dQ, dK, dV, B, H, N, D, causal, dtype, carry_in,
                        n_carry, gcarry_in, gcarry_out, state_in, ws, ws_bytes,
                        static_cast<hipStream_t>(stream), &t);
}

}  // extern "C"
