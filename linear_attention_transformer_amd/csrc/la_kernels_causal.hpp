// la_kernels_causal.hpp -- causal linear attention for 32 <= D <= 128 on gfx950.
//
// Same method as la_kernels.hpp, causal mask j <= i (pages about
// "Transformer Based Linear Attention with Optimized GPU Kernel
// Implementation": sciencestack.ai TL;DR and Figure 1 caption; the
// token-by-token state growth of the cloud.baidu.com article, section 2).
// Each head's sequence is cut into segments (one workgroup each) and each
// segment into chunks of C = 32 rows, processed in order.  A segment starts
// from the record of everything before it (forward, dQ: the exclusive prefix
// of the per-segment state records) or after it (dK, dV: the exclusive
// suffix of the gradient records).  For every chunk:
//   - the running state is applied to the chunk's rows (an MFMA product
//     over D, as in the non-causal kernels);
//   - the masked in-chunk block is formed densely: the C x C product (Q K^T
//     or dO V^T) is split into 16 x 16 tiles over all of D, spread over the
//     waves, written once to LDS, and applied with one more MFMA over the
//     chunk's rows;
//   - the running state is updated by the chunk (an MFMA over its rows).
//
// Wave cb of a workgroup owns output columns 32 cb .. 32 cb + 31 and the
// matching D x 32 slice of the running state, held as four (D / 32) MFMA
// accumulators st[t][i] <-> state[32 t + 8 (i / 4) + 4 h + i % 4][32 cb + j]
// (or its transpose).  With v_mfma_f32_32x32x2_f32 (lane l = 32 h + j
// supplies A[m = j][k = h] and B[k = h][n = j]; accumulator element i sits
// at row 8 (i / 4) + 4 h + i % 4, column j) that is exactly the A operand
// of the apply at k-block kb, step r: st[kb / 4][4 (kb % 4) + r].  So the
// state is applied and updated in place without leaving the registers.
//
// Rows are staged in LDS as fp32 from a register prefetch of the next chunk.
// Three barriers per chunk: after the product tiles are written (B1), after the
// last read of the chunk's rows (B2) and after the next chunk is staged
// (B3).  Tensors read only before B1 are restaged right after it, so at most
// two tensors' prefetch registers are live at a time.
#pragma once

#include "la_kernels_nc.hpp"

namespace la {
namespace cz {

using nc::dot4;
using nc::drain_loads;
using nc::f16v;
using nc::IO;
using nc::mma32;
using nc::zero16;

constexpr int kC = 32;  // rows per chunk
// word 3 of a raw buffer resource descriptor on gfx9-family GPUs (gfx950
// included): 32-bit data format, no swizzle, zero returned out of range
constexpr int kBufferWord3 = 0x00020000;

template <int D>
constexpr int threads() { return 64 * (D / 32); }

// Rows r0 .. r0 + kC - 1 of one head's [N, D] tensor: fetched into registers
// by the NT threads of the workgroup with 16-byte buffer loads through a
// descriptor that covers only the chunk's valid rows (base = row r0, range
// = the rows before `end`), so loads past the end return zeros and every
// access stays inside the tensor; then written to LDS as fp32.
template <class ST, int D, int NT>
struct Rows {
    typedef typename ST::T T;
    static constexpr int VEC = 16 / sizeof(T);
    static constexpr int CPR = D / VEC;
    static constexpr int PER = kC * CPR / NT;
    static constexpr int LDX = D + 4;
    static_assert(PER >= 1 && kC * CPR % NT == 0, "staging split");
    uint4 r[PER];

    __device__ __forceinline__ void fetch(const T *src, int64_t r0, int64_t end, int tid)
    {
        const int rows = (int)(end - r0 < kC ? end - r0 : kC);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<T *>(src + r0 * D), (short)0, rows * (int)(D * sizeof(T)), kBufferWord3);
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int c = tid + p * NT;
            r[p] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(
                           rs, (c / CPR) * (int)(D * sizeof(T)) + 16 * (c % CPR), 0, 0));
        }
    }
    __device__ __forceinline__ void stage(float *lds, int tid) const
    {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int c = tid + p * NT;
            float v[VEC];
            ST::widen(r[p], v);
            float *dst = lds + (c / CPR) * LDX + VEC * (c % CPR);
#pragma unroll
            for (int x = 0; x < VEC; x += 4)
                *reinterpret_cast<f4 *>(dst + x) = f4{v[x], v[x + 1], v[x + 2], v[x + 3]};
        }
    }
};

// Q_c K_c^T into wx and G_c V_c^T into gx (sh[i * WP + jj]; i: row of the
// first factor, jj: row of the second), each whole over the D columns, as
// eight 16 x 16 tiles (v_mfma_f32_16x16x4_f32) spread over the NCB waves:
// one copy of each product in LDS.  Lane
// (g = lane / 16, r = lane % 16) reads columns 16 s + 4 g .. + 3 of row r of
// a tile as one vector and supplies component c at MFMA step 4 s + c; both
// factors use the same order of the columns, so their sum is unchanged.
// Output element v of the lane sits at tile row 4 g + v, tile column r.
template <int D>
__device__ __forceinline__ void tiles_xyT(const float *qs, const float *ks, const float *gs,
                                          const float *vs, float *wx, float *gx, int cb,
                                          int lane)
{
    constexpr int NCB = D / 32, LDX = D + 4, WP = kC + 1, PER = 8 / NCB;
    static_assert(PER % 2 == 0 || PER == 1, "tiles per wave");
    constexpr int GRP = PER >= 2 ? 2 : 1;  // tiles in flight together
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int k0 = 0; k0 < PER; k0 += GRP) {
        const float *xa[GRP], *ya[GRP];
        float *dst[GRP];
#pragma unroll
        for (int u = 0; u < GRP; ++u) {
            const int tt = cb * PER + k0 + u;  // 0..3: Q K^T tiles, 4..7: G V^T
            const int ti = (tt >> 1) & 1, tj = tt & 1;
            xa[u] = (tt < 4 ? qs : gs) + (16 * ti + r) * LDX + 4 * g;
            ya[u] = (tt < 4 ? ks : vs) + (16 * tj + r) * LDX + 4 * g;
            dst[u] = (tt < 4 ? wx : gx) + (16 * ti + 4 * g) * WP + 16 * tj + r;
        }
        f4 a[GRP];
#pragma unroll
        for (int u = 0; u < GRP; ++u)
            a[u] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            f4 x[GRP], y[GRP];
#pragma unroll
            for (int u = 0; u < GRP; ++u) {
                x[u] = *reinterpret_cast<const f4 *>(xa[u] + 16 * st);
                y[u] = *reinterpret_cast<const f4 *>(ya[u] + 16 * st);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int u = 0; u < GRP; ++u)
                    a[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(x[u][c], y[u][c], a[u], 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < GRP; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                dst[u][v * WP] = a[u][v];
    }
}

// X_c Y_c^T into sh (as above, one product): its four 16 x 16 tiles spread
// over the NCB waves (D = 256: waves 0..3, one each; the others have none);
// a wave with a single tile runs its k-steps as two independent chains (even
// and odd column groups) and adds them at the end.
template <int D>
__device__ __forceinline__ void tile_xyT(const float *xs, const float *ys, float *sh, int cb,
                                         int lane)
{
    constexpr int NCB = D / 32, LDX = D + 4, WP = kC + 1, PER = NCB >= 4 ? 1 : 4 / NCB,
                  NST = D / 16;
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int tt = cb * PER + k;
        if (tt >= 4)
            break;
        const int ti = tt >> 1, tj = tt & 1;
        const float *xa = xs + (16 * ti + r) * LDX + 4 * g;
        const float *ya = ys + (16 * tj + r) * LDX + 4 * g;
        f4 a[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int st = 0; st < NST; ++st) {
            const f4 x = *reinterpret_cast<const f4 *>(xa + 16 * st);
            const f4 y = *reinterpret_cast<const f4 *>(ya + 16 * st);
#pragma unroll
            for (int c = 0; c < 4; ++c)
                a[st & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(x[c], y[c], a[st & 1], 0, 0, 0);
        }
        float *dst = sh + (16 * ti + 4 * g) * WP + 16 * tj + r;
#pragma unroll
        for (int v = 0; v < 4; ++v)
            dst[v * WP] = a[0][v] + a[1][v];
    }
}

// ============================================================ forward
// o_i = (u + S^T q_i + sum_{j in c, j <= i} (1 + q_i.k_j) v_j) / den_i,
// den_i = t0 + q_i.z + sum_{j in c, j <= i} (1 + q_i.k_j), with (S, z, u)
// over the rows before the chunk (t0 = its first row); then
// (S, z, u) += (K_c^T V_c, sum k, sum v).  st[t] = S[32t.., 32cb..].
template <class ST, int D>
__global__ __launch_bounds__(threads<D>()) void k_fwd_causal(
    const typename ST::T *__restrict__ Q, const typename ST::T *__restrict__ K,
    const typename ST::T *__restrict__ V, typename ST::T *__restrict__ O,
    float *__restrict__ den_out, const float *__restrict__ rec, int64_t N, int64_t seg_len,
    int nseg, float n0, OutLay ol)
{
    typedef typename ST::T T;
    typedef IO<ST> io;
    static_assert(D >= 32 && D <= 256, "32-column blocks, state in registers");
    constexpr int NCB = D / 32, NT = threads<D>(), KB = D / 8, LDX = D + 4, WP = kC + 1;
    __shared__ __attribute__((aligned(16))) float qs[kC * LDX];
    __shared__ __attribute__((aligned(16))) float ks[kC * LDX];
    __shared__ __attribute__((aligned(16))) float vs[kC * LDX];
    __shared__ float wx[kC * WP];  // Q_c K_c^T
    __shared__ __attribute__((aligned(16))) float vz[D];
    __shared__ __attribute__((aligned(16))) float vu[D];

    const int64_t bh = blockIdx.x / nseg;
    const int seg = (int)(blockIdx.x % nseg);
    const int tid = threadIdx.x, cb = tid >> 6, lane = tid & 63, j = lane & 31, h = lane >> 5;
    const int64_t beg = (int64_t)seg * seg_len;
    const int64_t end = (beg + seg_len < N) ? beg + seg_len : N;
    const int64_t hoff = bh * N * D;
    const float *st = rec + (bh * nseg + seg) * (int64_t)(D * D + 2 * D);
    const T *qh = Q + hoff, *kh = K + hoff, *vh = V + hoff;
    T *oh = O + ol.head(bh);

    Rows<ST, D, NT> rq, rk, rv;
    const int64_t nrounds = (end - beg + kC - 1) / kC;
    rq.fetch(qh, beg, end, tid);
    rk.fetch(kh, beg, end, tid);
    rv.fetch(vh, beg, end, tid);
    f16v sacc[NCB];
#pragma unroll
    for (int t = 0; t < NCB; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            sacc[t][i] = st[(32 * t + 8 * (i / 4) + 4 * h + (i % 4)) * D + 32 * cb + j];
    for (int e = tid; e < D; e += NT) {
        vz[e] = st[D * D + e];
        vu[e] = st[D * D + D + e];
    }
    rq.stage(qs, tid);
    rk.stage(ks, tid);
    rv.stage(vs, tid);
    drain_loads();
    if (nrounds > 1)
        rq.fetch(qh, beg + kC, end, tid);
    __syncthreads();

    f4 pend[4];
    int64_t prow = 0;
    bool pok = false;
    auto store_pending = [&](int q) {
        if (pok)
            io::store4(oh + prow * ol.sn + 32 * cb + 8 * q + 4 * h, pend[q]);
    };

    for (int64_t round = 0; round < nrounds; ++round) {
        const int64_t t0 = beg + round * kC;
        const bool more = round + 1 < nrounds;
        // (1) the prefix state applied to the chunk's queries, and q.z
        f16v acc = zero16();
        float qz = 0.f;
        {
            const float *xt = &qs[j * LDX + 4 * h];
            int zo = 4 * h;
            asm volatile("" : "+v"(zo));  // z changes per chunk: keep its reads here
            f4 xn = *reinterpret_cast<const f4 *>(xt);
            f4 zn = *reinterpret_cast<const f4 *>(&vz[zo]);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const f4 x = xn, z = zn;
                if (kb + 1 < KB) {
                    xn = *reinterpret_cast<const f4 *>(xt + (kb + 1) * 8);
                    zn = *reinterpret_cast<const f4 *>(&vz[zo + (kb + 1) * 8]);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc = mma32(sacc[kb / 4][4 * (kb % 4) + r], x[r], acc);
                qz += dot4(x, z);
                asm volatile("" : "+v"(qz));  // accumulate here, not after the loop
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (kb == q * (KB / 4))
                        store_pending(q);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // (2) this wave's tiles of Q_c K_c^T
        tile_xyT<D>(qs, ks, wx, cb, lane);
        __syncthreads();  // B1
        if (more) {
            rq.stage(qs, tid);
            rk.fetch(kh, t0 + kC, end, tid);
            rv.fetch(vh, t0 + kC, end, tid);
        }
        // (3) in-chunk term (key rows jr = 2kk + h of the MFMA step) and the
        // state update
        float rs = 0.f, zc = 0.f, uc = 0.f;
#pragma unroll
        for (int kk = 0; kk < kC / 2; ++kk) {
            const int jr = 2 * kk + h;
            const float vb = vs[jr * LDX + 32 * cb + j];
            const float wsum = wx[j * WP + jr];
            const float wm = (jr <= j) ? 1.f + wsum : 0.f;
            rs += wm;
            acc = mma32(vb, wm, acc);
#pragma unroll
            for (int t = 0; t < NCB; ++t)
                sacc[t] = mma32(ks[jr * LDX + 32 * t + j], vb, sacc[t]);
            // (this wave's K column read again: selecting it among the
            // unrolled operands would cost a select per block)
            zc += ks[jr * LDX + 32 * cb + j];
            uc += vb;
            __builtin_amdgcn_sched_barrier(0);
        }
        rs = swap32_sum(rs);
        zc = swap32_sum(zc);
        uc = swap32_sum(uc);
        qz = swap32_sum(qz);
        // (4) normalised rows of the chunk, stored during the next product
        const float den = (n0 + (float)t0) + qz + rs;
        const float inv = 1.f / den;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f4 u = *reinterpret_cast<const f4 *>(&vu[32 * cb + 8 * q + 4 * h]);
            pend[q] = f4{(acc[4 * q] + u[0]) * inv, (acc[4 * q + 1] + u[1]) * inv,
                         (acc[4 * q + 2] + u[2]) * inv, (acc[4 * q + 3] + u[3]) * inv};
        }
        prow = t0 + j;
        pok = prow < end;
        if (den_out != nullptr && pok && h == 0 && cb == 0)
            den_out[bh * N + prow] = den;
        __syncthreads();  // B2
        if (h == 0) {
            vz[32 * cb + j] += zc;
            vu[32 * cb + j] += uc;
        }
        if (more) {
            rk.stage(ks, tid);
            rv.stage(vs, tid);
            if (round + 2 < nrounds)
                rq.fetch(qh, t0 + 2 * kC, end, tid);
        }
        __syncthreads();  // B3
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
        store_pending(q);
}

// ============================================================ dQ
// With (S, z, u) over the rows before the chunk and, for row i of it,
//   W_ij = 1 + q_i.k_j, GV_ij = g_i.v_j (j in the chunk, j <= i),
//   den_i = t0 + q_i.z + sum_j W_ij,  y_i = S g_i,
//   c_i = (g_i.u + q_i.y_i + sum_j W_ij GV_ij) / den_i^2   (= a_i.o_i),
//   dq_i = (y_i + sum_j (GV_ij - c_i den_i) k_j) / den_i - c_i z,
// (S a_i - c_i z plus the in-chunk sum of (a_i.v_j - c_i) k_j), and
// cbuf[i] = (c_i, 1 / den_i) for the gradient record and the dK | dV pass.
// The product runs over S's rows: st[t] = S^T[32t.., 32cb..].
template <class ST, int D>
__global__ __launch_bounds__(threads<D>()) __attribute__((amdgpu_waves_per_eu(2))) void k_bwd_q_causal(
    const typename ST::T *__restrict__ Q, const typename ST::T *__restrict__ K,
    const typename ST::T *__restrict__ V, const typename ST::T *__restrict__ G,
    typename ST::T *__restrict__ dQ, float *__restrict__ cbuf, const float *__restrict__ rec,
    int64_t N, int64_t seg_len, int nseg, float n0, OutLay ol)
{
    typedef typename ST::T T;
    typedef IO<ST> io;
    static_assert(D >= 32 && D <= 256, "32-column blocks, state in registers");
    constexpr int NCB = D / 32, NT = threads<D>(), KB = D / 8, LDX = D + 4, WP = kC + 1;
    __shared__ __attribute__((aligned(16))) float qs[kC * LDX];
    __shared__ __attribute__((aligned(16))) float ks[kC * LDX];
    __shared__ __attribute__((aligned(16))) float vs[kC * LDX];
    __shared__ __attribute__((aligned(16))) float gs[kC * LDX];
    __shared__ float wx[kC * WP];       // Q_c K_c^T
    __shared__ float gx[kC * WP];       // G_c V_c^T
    __shared__ float xq[NCB][kC];       // shares of q_i.y_i
    __shared__ __attribute__((aligned(16))) float vz[D];
    __shared__ __attribute__((aligned(16))) float vu[D];

    const int64_t bh = blockIdx.x / nseg;
    const int seg = (int)(blockIdx.x % nseg);
    const int tid = threadIdx.x, cb = tid >> 6, lane = tid & 63, j = lane & 31, h = lane >> 5;
    const int64_t beg = (int64_t)seg * seg_len;
    const int64_t end = (beg + seg_len < N) ? beg + seg_len : N;
    const int64_t hoff = bh * N * D;
    const float *st = rec + (bh * nseg + seg) * (int64_t)(D * D + 2 * D);
    const T *qh = Q + hoff, *kh = K + hoff, *vh = V + hoff, *gh = G + hoff;
    T *oh = dQ + ol.head(bh);

    Rows<ST, D, NT> rq, rk, rv, rg;
    const int64_t nrounds = (end - beg + kC - 1) / kC;
    rq.fetch(qh, beg, end, tid);
    rk.fetch(kh, beg, end, tid);
    rv.fetch(vh, beg, end, tid);
    rg.fetch(gh, beg, end, tid);
    // sacc[t][i] = S[32cb + j][32t + 8(i/4) + 4h + i%4]
    f16v sacc[NCB];
#pragma unroll
    for (int t = 0; t < NCB; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f4 v = *reinterpret_cast<const f4 *>(st + (32 * cb + j) * D + 32 * t + 8 * q +
                                                       4 * h);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sacc[t][4 * q + r] = v[r];
        }
    for (int e = tid; e < D; e += NT) {
        vz[e] = st[D * D + e];
        vu[e] = st[D * D + D + e];
    }
    rq.stage(qs, tid);
    rk.stage(ks, tid);
    rv.stage(vs, tid);
    rg.stage(gs, tid);
    drain_loads();
    if (nrounds > 1) {
        rq.fetch(qh, beg + kC, end, tid);
        rg.fetch(gh, beg + kC, end, tid);
    }
    __syncthreads();

    for (int64_t round = 0; round < nrounds; ++round) {
        const int64_t t0 = beg + round * kC;
        const bool more = round + 1 < nrounds;
        // (1) y = S g for the chunk's rows, with g.u and q.z
        f16v acc = zero16();
        float gu = 0.f, qz = 0.f;
        {
            const float *xt = &gs[j * LDX + 4 * h];
            const float *qt = &qs[j * LDX + 4 * h];
            int vo = 4 * h;
            asm volatile("" : "+v"(vo));  // z and u change per chunk
            f4 xn = *reinterpret_cast<const f4 *>(xt);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const f4 x = xn;
                if (kb + 1 < KB)
                    xn = *reinterpret_cast<const f4 *>(xt + (kb + 1) * 8);
                const f4 qv = *reinterpret_cast<const f4 *>(qt + kb * 8);
                const f4 z = *reinterpret_cast<const f4 *>(&vz[vo + kb * 8]);
                const f4 u = *reinterpret_cast<const f4 *>(&vu[vo + kb * 8]);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc = mma32(sacc[kb / 4][4 * (kb % 4) + r], x[r], acc);
                gu += dot4(x, u);
                qz += dot4(qv, z);
                asm volatile("" : "+v"(gu), "+v"(qz));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // (2) Q_c K_c^T and G_c V_c^T (whole tiles), q.y over this wave's
        // columns
        tiles_xyT<D>(qs, ks, gs, vs, wx, gx, cb, lane);
        {
            float p = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f4 qv = *reinterpret_cast<const f4 *>(&qs[j * LDX + 32 * cb + 8 * q + 4 * h]);
                p += qv[0] * acc[4 * q] + qv[1] * acc[4 * q + 1] + qv[2] * acc[4 * q + 2] +
                     qv[3] * acc[4 * q + 3];
            }
            p = swap32_sum(p);
            if (h == 0)
                xq[cb][j] = p;
        }
        __syncthreads();  // B1
        if (more) {
            rq.stage(qs, tid);
            rg.stage(gs, tid);
            rk.fetch(kh, t0 + kC, end, tid);
            rv.fetch(vh, t0 + kC, end, tid);
        }
        // (3) den, c, then the in-chunk term and the state update (key rows
        // jr = 2kk + h of the MFMA step)
        float gvk[kC / 2];
        float rs = 0.f, cw = 0.f;
#pragma unroll
        for (int kk = 0; kk < kC / 2; ++kk) {
            const int jr = 2 * kk + h;
            const float w = wx[j * WP + jr], gv = gx[j * WP + jr];
            const bool m = jr <= j;
            const float wm = m ? 1.f + w : 0.f;
            rs += wm;
            cw += wm * gv;
            gvk[kk] = m ? gv : 0.f;
        }
        rs = swap32_sum(rs);
        cw = swap32_sum(cw);
        gu = swap32_sum(gu);
        qz = swap32_sum(qz);
        float qy = 0.f;
#pragma unroll
        for (int p = 0; p < NCB; ++p)
            qy += xq[p][j];
        const float den = (n0 + (float)t0) + qz + rs;
        const float inv = 1.f / den;
        const float c = (gu + qy + cw) * inv * inv;
        const float cden = c * den;
        float zc = 0.f, uc = 0.f;
#pragma unroll
        for (int kk = 0; kk < kC / 2; ++kk) {
            const int jr = 2 * kk + h;
            const float kv = ks[jr * LDX + 32 * cb + j];
            const float pm = (jr <= j) ? gvk[kk] - cden : 0.f;
            acc = mma32(kv, pm, acc);
#pragma unroll
            for (int t = 0; t < NCB; ++t)
                sacc[t] = mma32(vs[jr * LDX + 32 * t + j], kv, sacc[t]);
            uc += vs[jr * LDX + 32 * cb + j];  // (as in the forward)
            zc += kv;
            __builtin_amdgcn_sched_barrier(0);
        }
        zc = swap32_sum(zc);
        uc = swap32_sum(uc);
        // (4) dq rows (z of the rows before the chunk), stored right away
        // (held to be stored during the next product, they cost registers
        // that the product's operands then spilled)
        const int64_t row = t0 + j;
        if (row < end) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f4 z = *reinterpret_cast<const f4 *>(&vz[32 * cb + 8 * q + 4 * h]);
                io::store4(oh + row * ol.sn + 32 * cb + 8 * q + 4 * h,
                           f4{acc[4 * q] * inv - c * z[0], acc[4 * q + 1] * inv - c * z[1],
                              acc[4 * q + 2] * inv - c * z[2], acc[4 * q + 3] * inv - c * z[3]});
            }
            if (h == 0 && cb == 0)
                reinterpret_cast<float2 *>(cbuf)[bh * N + row] = float2{c, inv};
        }
        __syncthreads();  // B2
        if (h == 0) {
            vz[32 * cb + j] += zc;
            vu[32 * cb + j] += uc;
        }
        if (more) {
            rk.stage(ks, tid);
            rv.stage(vs, tid);
            if (round + 2 < nrounds) {
                rq.fetch(qh, t0 + 2 * kC, end, tid);
                rg.fetch(gh, t0 + 2 * kC, end, tid);
            }
        }
        __syncthreads();  // B3
    }
}

// ============================================================ dK | dV
// Chunks in reverse order.  With (R, r, t) = (sum q a^T, sum c q, sum a) over
// the rows after the chunk and, for row j of it (i in the chunk, i >= j),
//   dk_j = R v_j - r + sum_i (a_i.v_j - c_i) q_i,
//   dv_j = t + R^T k_j + sum_i (1 + q_i.k_j) a_i,
// a_i = g_i / den_i and (c_i, 1 / den_i) from cbuf; then (R, r, t) += the
// chunk's rows.  Workgroup parity 0 computes dK (st[t] = R^T[32t.., 32cb..],
// G_c V_c^T), parity 1 computes dV (st[t] = R[32t.., 32cb..], Q_c K_c^T).
// LDS of the dK | dV pass
template <int D>
struct KvLds {
    static constexpr int LDX = D + 4, WP = kC + 1, NCB = D / 32;
    float xs[kC * LDX];    // V (dK) or K (dV)
    float qs[kC * LDX];
    float gs[kC * LDX];
    float sh[kC * WP];     // G_c V_c^T (dK) or Q_c K_c^T (dV)
    float cs[kC], is[kC];  // c_i, 1/den_i of the chunk's rows
    float vr[D];           // r (dK) or t (dV)
};

template <class ST, int D, int PAR>
__device__ __forceinline__ void kv_pass(
    const typename ST::T *__restrict__ Q, const typename ST::T *__restrict__ K,
    const typename ST::T *__restrict__ V, const typename ST::T *__restrict__ G,
    typename ST::T *__restrict__ dK, typename ST::T *__restrict__ dV,
    const float *__restrict__ cbuf, const float *__restrict__ rec, int64_t N, int64_t seg_len,
    int nseg, OutLay ol, KvLds<D> &L)
{
    typedef typename ST::T T;
    typedef IO<ST> io;
    static_assert(D >= 32 && D <= 256, "32-column blocks, state in registers");
    constexpr int NCB = D / 32, NT = threads<D>(), KB = D / 8, LDX = D + 4, WP = kC + 1;
    float *xs = L.xs, *qs = L.qs, *gs = L.gs, *cs = L.cs, *is = L.is, *vr = L.vr;
    auto &sh = L.sh;

    const int64_t b = blockIdx.x >> 1;
    const int64_t bh = b / nseg;
    const int seg = (int)(b % nseg);
    const int tid = threadIdx.x, cb = tid >> 6, lane = tid & 63, j = lane & 31, h = lane >> 5;
    const int64_t beg = (int64_t)seg * seg_len;
    const int64_t end = (beg + seg_len < N) ? beg + seg_len : N;
    const int64_t hoff = bh * N * D;
    const float *st = rec + (bh * nseg + seg) * (int64_t)(D * D + 2 * D);
    const T *xh = (PAR == 0 ? V : K) + hoff, *qh = Q + hoff, *gh = G + hoff;
    T *oh = (PAR == 0 ? dK : dV) + ol.head(bh);
    const float2 *ch = reinterpret_cast<const float2 *>(cbuf) + bh * N;

    Rows<ST, D, NT> rx, rq, rg;
    float2 rc = float2{0.f, 0.f};
    auto fetch_c = [&](int64_t r0) {
        if (tid < kC) {
            int64_t row = r0 + tid;
            row = row < end ? row : end - 1;
            rc = ch[row];
        }
    };
    auto stage_c = [&](int64_t r0) {
        if (tid < kC) {
            const bool ok = r0 + tid < end;
            cs[tid] = ok ? rc.x : 0.f;
            is[tid] = ok ? rc.y : 0.f;
        }
    };
    const int64_t nrounds = (end - beg + kC - 1) / kC;
    const int64_t last = beg + (nrounds - 1) * kC;  // first row of the last chunk
    rx.fetch(xh, last, end, tid);
    rq.fetch(qh, last, end, tid);
    rg.fetch(gh, last, end, tid);
    fetch_c(last);
    // parity 0: sacc[t][i] = R[32cb + j][32t + 8(i/4) + 4h + i%4]
    // parity 1: sacc[t][i] = R[32t + 8(i/4) + 4h + i%4][32cb + j]
    f16v sacc[NCB];
#pragma unroll
    for (int t = 0; t < NCB; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int a = 32 * t + 8 * (i / 4) + 4 * h + (i % 4), o = 32 * cb + j;
            sacc[t][i] = (PAR == 0) ? st[o * D + a] : st[a * D + o];
        }
    for (int e = tid; e < D; e += NT)
        vr[e] = st[D * D + (PAR == 0 ? 0 : D) + e];
    rx.stage(xs, tid);
    rq.stage(qs, tid);
    rg.stage(gs, tid);
    stage_c(last);
    drain_loads();
    if (nrounds > 1)
        rx.fetch(xh, last - kC, end, tid);
    __syncthreads();


    for (int64_t round = 0; round < nrounds; ++round) {
        const int64_t t0 = last - round * kC;
        const bool more = round + 1 < nrounds;
        // (1) the suffix state applied to the chunk's rows of V (dK) or K (dV)
        f16v acc = zero16();
        {
            const float *xt = &xs[j * LDX + 4 * h];
            f4 xn = *reinterpret_cast<const f4 *>(xt);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const f4 x = xn;
                if (kb + 1 < KB)
                    xn = *reinterpret_cast<const f4 *>(xt + (kb + 1) * 8);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc = mma32(sacc[kb / 4][4 * (kb % 4) + r], x[r], acc);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // (2) G_c V_c^T (dK; xs holds V) or Q_c K_c^T (dV; xs holds K)
        if constexpr (PAR == 0)
            tile_xyT<D>(gs, xs, sh, cb, lane);
        else
            tile_xyT<D>(qs, xs, sh, cb, lane);
        __syncthreads();  // B1
        if (more) {
            rx.stage(xs, tid);
            rq.fetch(qh, t0 - kC, end, tid);
            rg.fetch(gh, t0 - kC, end, tid);
            fetch_c(t0 - kC);
        }
        // (3) in-chunk term over query rows ir = 2kk + h >= j, and the state
        // update
        float vc = 0.f;
        if constexpr (PAR == 0) {
#pragma unroll
            for (int kk = 0; kk < kC / 2; ++kk) {
                const int ir = 2 * kk + h;
                const float s = sh[ir * WP + j];
                const float ci = cs[ir], ii = is[ir];
                const float pm = (ir >= j) ? s * ii - ci : 0.f;
                const float qb = qs[ir * LDX + 32 * cb + j];
                acc = mma32(qb, pm, acc);
#pragma unroll
                for (int t = 0; t < NCB; ++t)
                    sacc[t] = mma32(gs[ir * LDX + 32 * t + j] * ii, qb, sacc[t]);
                vc += ci * qb;
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < kC / 2; ++kk) {
                const int ir = 2 * kk + h;
                const float s = sh[ir * WP + j];
                const float wm = (ir >= j) ? 1.f + s : 0.f;
                const float ab = gs[ir * LDX + 32 * cb + j] * is[ir];
                acc = mma32(ab, wm, acc);
#pragma unroll
                for (int t = 0; t < NCB; ++t)
                    sacc[t] = mma32(qs[ir * LDX + 32 * t + j], ab, sacc[t]);
                vc += ab;
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        vc = swap32_sum(vc);
        // (4) rows of dK (- r) or dV (+ t) with the vector of the rows after
        // the chunk (stored here: the next chunk's product covers them)
        const float sg = (PAR == 0) ? -1.f : 1.f;
        if (t0 + j < end)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f4 v = *reinterpret_cast<const f4 *>(&vr[32 * cb + 8 * q + 4 * h]);
                io::store4(oh + (t0 + j) * ol.sn + 32 * cb + 8 * q + 4 * h,
                           f4{acc[4 * q] + sg * v[0], acc[4 * q + 1] + sg * v[1],
                              acc[4 * q + 2] + sg * v[2], acc[4 * q + 3] + sg * v[3]});
            }
        __syncthreads();  // B2
        if (h == 0)
            vr[32 * cb + j] += vc;
        if (more) {
            rq.stage(qs, tid);
            rg.stage(gs, tid);
            stage_c(t0 - kC);
            if (round + 2 < nrounds)
                rx.fetch(xh, t0 - 2 * kC, end, tid);
        }
        __syncthreads();  // B3
    }
}


template <class ST, int D>
__global__ __launch_bounds__(threads<D>()) __attribute__((amdgpu_waves_per_eu(2))) void k_bwd_kv_causal(
    const typename ST::T *__restrict__ Q, const typename ST::T *__restrict__ K,
    const typename ST::T *__restrict__ V, const typename ST::T *__restrict__ G,
    typename ST::T *__restrict__ dK, typename ST::T *__restrict__ dV,
    const float *__restrict__ cbuf, const float *__restrict__ rec, int64_t N, int64_t seg_len,
    int nseg, OutLay ol)
{
    __shared__ __attribute__((aligned(16))) KvLds<D> lds;
    if (blockIdx.x & 1)
        kv_pass<ST, D, 1>(Q, K, V, G, dK, dV, cbuf, rec, N, seg_len, nseg, ol, lds);
    else
        kv_pass<ST, D, 0>(Q, K, V, G, dK, dV, cbuf, rec, N, seg_len, nseg, ol, lds);
}

// ============================================================ dK | dV, one workgroup
// The recurrences of kv_pass, with dK and dV of a segment formed by one
// workgroup of 2 NCB waves that holds the suffix state R once, so that R is
// updated once per chunk instead of once per output:
//   - waves NCB .. 2 NCB - 1 form dV columns 32 (w - NCB) .. (dv_j = R^T k_j
//     + t + in-chunk terms); each keeps its D x 32 column slab of R as MFMA
//     accumulators (the A operand of R^T k), adds the chunk to it in place
//     (R += Q_c^T A_c) and, after the chunk's last read of R, publishes it in
//     LDS as R[a][b] (a: column of Q, b: column of a);
//   - waves 0 .. NCB - 1 form dK columns 32 w .. (dk_j = R v_j - r + in-chunk
//     terms), reading R by rows from LDS, and the products Q_c K_c^T and
//     G_c V_c^T as 16 x 16 tiles;
//   - one loop per role, behind a scalar branch on the wave index, so that
//     each role's registers are allocated apart.
// Three barriers per chunk, as in kv_pass: after the product tiles (B1),
// after the chunk's last reads (B2), after the next chunk is staged (B3).
// K and V are read only before B1 and are restaged right after it.  When the
// launch has more workgroups than one batch holds, a workgroup walks several
// consecutive segments, starting from the suffix record of the last of them.
template <int D>
struct Kv2Lds {
    static constexpr int LDX = D + 4, RP = D + 4, WP = kC + 1;
    float qs[kC * LDX], ks[kC * LDX], vs[kC * LDX], gs[kC * LDX];
    float rs[D * RP];                // R[a][b] at a * RP + b
    float wx[kC * WP], gx[kC * WP];  // Q_c K_c^T, G_c V_c^T ([i][j] at i * WP + j)
    float cs[kC], is[kC];            // c_i, 1 / den_i of the chunk's rows
    float vr[D], vt[D];              // r, t of the rows after the chunk
};

template <class ST, int D>
__global__ __launch_bounds__(128 * (D / 32)) void k_bwd_kv_causal2(
    const typename ST::T *__restrict__ Q, const typename ST::T *__restrict__ K,
    const typename ST::T *__restrict__ V, const typename ST::T *__restrict__ G,
    typename ST::T *__restrict__ dK, typename ST::T *__restrict__ dV,
    const float *__restrict__ cbuf, const float *__restrict__ rec, int64_t N, int64_t seg_len,
    int nseg, int merge, OutLay ol)
{
    typedef typename ST::T T;
    typedef IO<ST> io;
    static_assert(D == 64 || D == 128, "two or four 32-column blocks");
    constexpr int NCB = D / 32, NW = 2 * NCB, NT = 64 * NW, KB = D / 8;
    constexpr int LDX = Kv2Lds<D>::LDX, RP = Kv2Lds<D>::RP, WP = Kv2Lds<D>::WP;
    __shared__ __attribute__((aligned(16))) Kv2Lds<D> L;

    // a workgroup walks `merge` consecutive segments of the plan, starting
    // from the suffix record of the last of them
    const int nsm = (nseg + merge - 1) / merge;
    const int64_t bh = blockIdx.x / nsm;
    const int sm = (int)(blockIdx.x % nsm);
    const int seg = (sm + 1) * merge - 1 < nseg ? (sm + 1) * merge - 1 : nseg - 1;
    const int tid = threadIdx.x, lane = tid & 63, j = lane & 31, h = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool isk = w < NCB;
    const int cb = isk ? w : w - NCB;
    const int64_t beg = (int64_t)sm * merge * seg_len;
    const int64_t end = (beg + merge * seg_len < N) ? beg + merge * seg_len : N;
    const int64_t hoff = bh * N * D;
    const float *st = rec + (bh * nseg + seg) * (int64_t)(D * D + 2 * D);
    const T *qh = Q + hoff, *kh = K + hoff, *vh = V + hoff, *gh = G + hoff;
    T *oh = (isk ? dK : dV) + ol.head(bh);
    const float2 *ch = reinterpret_cast<const float2 *>(cbuf) + bh * N;

    // chunk rows from registers: a chunk outside [beg, end) reads nothing
    // (its rows are zero), so the fetches past the walk need no branch
    Rows<ST, D, NT> rq, rk, rv, rg;
    float2 pc = float2{0.f, 0.f};
    auto fetch_kv = [&](int64_t r0) {
        const int64_t rb = r0 < beg ? end : r0;
        rk.fetch(kh, rb, end, tid);
        rv.fetch(vh, rb, end, tid);
    };
    auto fetch_qg = [&](int64_t r0) {
        const int64_t rb = r0 < beg ? end : r0;
        rq.fetch(qh, rb, end, tid);
        rg.fetch(gh, rb, end, tid);
        const int rows = (int)(end - rb < kC ? end - rb : kC);
        const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float2 *>(ch + rb), (short)0, rows * 8, kBufferWord3);
        pc = __builtin_bit_cast(float2,
                                __builtin_amdgcn_raw_buffer_load_b64(rc, (tid & (kC - 1)) * 8, 0, 0));
    };
    auto stage_kv = [&]() {
        rk.stage(L.ks, tid);
        rv.stage(L.vs, tid);
    };
    auto stage_qg = [&]() {
        rq.stage(L.qs, tid);
        rg.stage(L.gs, tid);
        if (tid < kC) {
            L.cs[tid] = pc.x;
            L.is[tid] = pc.y;
        }
    };

    // dV waves: their D x 32 column slab of R as MFMA accumulators,
    // sacc[t][i] <-> R[32 t + 8 (i / 4) + 4 h + i % 4][32 cb + j], which is
    // also the A operand of R^T k at k-block kb, step r: sacc[kb / 4][4 (kb %
    // 4) + r].  They add each chunk to it and publish it in LDS for the dK
    // waves, which read R by rows.
    f16v sacc[NCB];
    auto write_r = [&]() {
#pragma unroll
        for (int t = 0; t < NCB; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                L.rs[(32 * t + 8 * (i / 4) + 4 * h + (i % 4)) * RP + 32 * cb + j] = sacc[t][i];
    };

    const int64_t nrounds = (end - beg + kC - 1) / kC;
    const int64_t last = beg + (nrounds - 1) * kC;  // first row of the last chunk
    fetch_kv(last);
    fetch_qg(last);
    if (!isk) {
#pragma unroll
        for (int t = 0; t < NCB; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                sacc[t][i] = st[(32 * t + 8 * (i / 4) + 4 * h + (i % 4)) * D + 32 * cb + j];
        write_r();
    }
    for (int e = tid; e < D; e += NT) {
        L.vr[e] = st[D * D + e];
        L.vt[e] = st[D * D + D + e];
    }
    stage_kv();
    stage_qg();
    drain_loads();
    fetch_kv(last - kC);
    fetch_qg(last - kC);
    __syncthreads();

    // one loop per role (a scalar branch: each role's registers are
    // allocated apart), both through the same three barriers per chunk
    auto walk = [&](auto role) {
        constexpr bool DK = decltype(role)::value;
        for (int64_t round = 0; round < nrounds; ++round) {
            const int64_t t0 = last - round * kC;
            // (1) the suffix state applied to the chunk's rows: dK^T block
            // C[a][t] = sum_b R[a][b] V[t][b] (R by rows, from LDS) or dV^T
            // block C[b][t] = sum_a R[a][b] K[t][a] (the wave's own slab);
            // k-slot of lane (j, h) at k-block kb, step r: column 8 kb + 4 h + r
            f16v acc = zero16();
            if constexpr (DK) {
                const float *xt = &L.vs[j * LDX + 4 * h];
                const float *rt = &L.rs[(32 * cb + j) * RP + 4 * h];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const f4 x = *reinterpret_cast<const f4 *>(xt + 8 * kb);
                    const f4 a = *reinterpret_cast<const f4 *>(rt + 8 * kb);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc = mma32(a[r], x[r], acc);
                }
                // (2) Q_c K_c^T and G_c V_c^T, tiles over the dK waves (the dV
                // waves update R after B1)
                tiles_xyT<D>(L.qs, L.ks, L.gs, L.vs, L.wx, L.gx, cb, lane);
            } else {
                const float *xt = &L.ks[j * LDX + 4 * h];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const f4 x = *reinterpret_cast<const f4 *>(xt + 8 * kb);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc = mma32(sacc[kb / 4][4 * (kb % 4) + r], x[r], acc);
                }
            }
            __syncthreads();  // B1
            stage_kv();  // K, V are read only before B1
            fetch_kv(t0 - 2 * kC);
            // (3) in-chunk terms over rows ir = 2 kk + h >= j: dK^T[a][j] +=
            // sum_i Q[i][a] (a_i.v_j - c_i), dV^T[b][j] += sum_i A[i][b] (1 + q_i.k_j)
            float vc = 0.f;
            if constexpr (DK) {
#pragma unroll
                for (int kk = 0; kk < kC / 2; ++kk) {
                    const int ir = 2 * kk + h;
                    const float ci = L.cs[ir];
                    const float pm = (ir >= j) ? L.gx[ir * WP + j] * L.is[ir] - ci : 0.f;
                    const float qb = L.qs[ir * LDX + 32 * cb + j];
                    acc = mma32(qb, pm, acc);
                    vc += ci * qb;
                }
            } else {
                // and the slab of R takes the chunk in: R[a][32 cb ..] += Q_c^T A_c
#pragma unroll
                for (int kk = 0; kk < kC / 2; ++kk) {
                    const int ir = 2 * kk + h;
                    const float wm = (ir >= j) ? 1.f + L.wx[ir * WP + j] : 0.f;
                    const float ab = L.gs[ir * LDX + 32 * cb + j] * L.is[ir];
                    acc = mma32(ab, wm, acc);
#pragma unroll
                    for (int t = 0; t < NCB; ++t)
                        sacc[t] = mma32(L.qs[ir * LDX + 32 * t + j], ab, sacc[t]);
                    vc += ab;
                }
            }
            vc = swap32_sum(vc);
            // (4) rows of dK (- r) or dV (+ t) with the vectors of the rows after the chunk
            {
                constexpr float sg = DK ? -1.f : 1.f;
                const float *vec = DK ? L.vr : L.vt;
                if (t0 + j < end)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f4 v = *reinterpret_cast<const f4 *>(&vec[32 * cb + 8 * q + 4 * h]);
                        io::store4(oh + (t0 + j) * ol.sn + 32 * cb + 8 * q + 4 * h,
                                   f4{acc[4 * q] + sg * v[0], acc[4 * q + 1] + sg * v[1],
                                      acc[4 * q + 2] + sg * v[2], acc[4 * q + 3] + sg * v[3]});
                    }
            }
            // (5) the dV waves publish the updated R (every read of R for this
            // chunk was before B1)
            if constexpr (!DK)
                write_r();
            __syncthreads();  // B2
            if (h == 0)
                (DK ? L.vr : L.vt)[32 * cb + j] += vc;
            stage_qg();
            fetch_qg(t0 - 2 * kC);
            __syncthreads();  // B3
        }
    };
    if (isk)
        walk(std::true_type{});
    else
        walk(std::false_type{});
}

}  // namespace cz
}  // namespace la
