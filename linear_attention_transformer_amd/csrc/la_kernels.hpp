// la_kernels.hpp -- gfx950 (CDNA4) kernels of Transformer-based linear
// attention: forward and backward of one head-batch.
//
// The method (pages about "Transformer Based Linear Attention with Optimized
// GPU Kernel Implementation"; sciencestack.ai TL;DR and Figure 1 caption;
// cloud.baidu.com article, section 2): per head, the similarity of query i
// and key j is 1 + q_i.k_j; outputs are normalised by den_i = sum_j w_ij; the
// O(N D^2) evaluation goes through the D x D state S = sum_j k_j v_j^T and the
// vectors z = sum k, u = sum v:
//     den_i = n_i + q_i.z,   o_i = (u + S^T q_i) / den_i      (n_i = #visible)
// Causally the state is a prefix over the sequence (the token recurrence of
// the article's pseudocode); here it is grown chunk by chunk, with the
// masked in-chunk block done densely.  The backward uses a_i = g_i/den_i,
// c_i = a_i.o_i and the gradient states dS = sum q a^T, r = sum c q,
// t = sum a:  dq_i = S a_i - c_i z,  dk_j = dS v_j - r,  dv_j = t + dS^T k_j
// (prefix states for dq, suffix states for dk/dv when causal).  c_i is
// formed without reading o_i: c_i den_i = a_i.u + q_i.(S a_i) (+ the in-chunk
// terms when causal).
//
// Hardware mapping.  Every contraction runs on v_mfma_f32_16x16x4_f32 with
// fp32 operands (bf16 storage is widened when tiles are staged in LDS).  A
// D x D state lives in registers, spread over the waves of a workgroup: wave
// w owns 16-column blocks of the state and keeps every 16x16 tile of them in
// the MFMA accumulator layout (lane l holds rows 4*(l/16)+r, r=0..3, column
// l%16).  That layout is used as is for the B operand of X . State, by
// letting the four accumulator registers stand for four successive k-steps
// and reading the matching four columns of X with one 16-byte LDS read; the
// k order inside a 16-block is permuted identically on both operands, which
// leaves the sum unchanged.
//
// Each workgroup owns one (head, segment, column-slice) triple.  Segments are
// processed sequentially in chunks of rows staged through LDS, with the next
// chunk's global loads in flight while the current one is computed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef float f4 __attribute__((ext_vector_type(4)));

// Where a kernel writes a [B, H, N, D] output: element d of row n of head
// bh = b * H + h at (b * sb + h * sh + n * sn + d) elements from the output
// pointer.  The plain layout is {H N D, N D, D, H}; a row layout puts the
// heads of one token side by side ([B, N, H, D]: {N H D, D, H D, H}).  Row
// strides and head offsets keep 16-byte alignment wherever the kernels store
// 16-byte pieces (checked on the host).
struct OutLay {
    int64_t sb, sh, sn;
    int64_t H;
    __device__ __forceinline__ int64_t head(int64_t bh) const
    {
        return (bh / H) * sb + (bh % H) * sh;
    }
};

__device__ __forceinline__ f4 mma(float a, float b, f4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Lane-group sums without the LDS crossbar: DPP moves within rows of 16
// lanes (quad_perm [1,0,3,2] and [2,3,0,1], then the half-row and row
// mirrors), v_permlane16_swap between rows 2r and 2r+1, v_permlane32_swap
// between the wave's halves.  group_sum<N> sums aligned groups of N lanes
// (N = 1..64, a power of two) and leaves the sum in every lane of the group.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// v + (the same register of lane l ^ 16), i.e. the sum of rows 2r, 2r+1
__device__ __forceinline__ float swap16_sum(float v)
{
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// v + (the same register of lane l ^ 32)
__device__ __forceinline__ float swap32_sum(float v)
{
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Two sums for one exchange: a + (a of lane l ^ 16) in rows 0 and 2 of
// the wave, b + (b of lane l ^ 16) in rows 1 and 3 (v_permlane16_swap moves
// the odd rows of its first register and the even rows of its second)
__device__ __forceinline__ float pair16_sum(float a, float b)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, a),
                                                    __builtin_bit_cast(unsigned, b), false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// a + (a of lane l ^ 32) in the lower half, b + (b of lane l ^ 32) in the
// upper half
__device__ __forceinline__ float pair32_sum(float a, float b)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a),
                                                    __builtin_bit_cast(unsigned, b), false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

template <int N>
__device__ __forceinline__ float group_sum(float v)
{
    static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "power-of-two group");
    if constexpr (N >= 2)
        v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
    if constexpr (N >= 4)
        v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
    if constexpr (N >= 8)
        v += dpp_mov<0x141>(v);  // row_half_mirror
    if constexpr (N >= 16)
        v += dpp_mov<0x140>(v);  // row_mirror
    if constexpr (N >= 32)
        v = swap16_sum(v);
    if constexpr (N >= 64)
        v = swap32_sum(v);
    return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

// Workgroup b of a launch of `units` workgroups per head: its head bh and
// its unit u (0 <= u < units).  The dispatcher deals workgroups to the eight
// XCDs in turn (b mod 8); when the number of heads is a multiple of 8, the
// units of one head are all given workgroups on one XCD, so that the head's
// state record, which each of them reads, is fetched into one L2 instead of
// eight.  Otherwise the plain order (bh = b / units).
__device__ __forceinline__ void xcd_unit(int64_t b, int units, int64_t &bh, int &u)
{
    const int64_t heads = gridDim.x / units;
    if ((heads & 7) == 0) {
        const int64_t l = b >> 3;
        bh = (l / units) * 8 + (b & 7);
        u = (int)(l % units);
    } else {
        bh = b / units;
        u = (int)(b % units);
    }
}

// sum over the 16 lanes that share l/16
__device__ __forceinline__ float group16_sum(float v) { return group_sum<16>(v); }

// ------------------------------------------------------------ storage types
struct StF32 {
    typedef float T;
    static constexpr int VEC = 4;  // elements per 16-byte vector
    __device__ static __forceinline__ void widen(const uint4 &r, float *o)
    {
        o[0] = __uint_as_float(r.x);
        o[1] = __uint_as_float(r.y);
        o[2] = __uint_as_float(r.z);
        o[3] = __uint_as_float(r.w);
    }
    __device__ static __forceinline__ T narrow(float x) { return x; }
    __device__ static __forceinline__ float widen1(T x) { return x; }
};

struct StBF16 {
    typedef uint16_t T;
    static constexpr int VEC = 8;
    __device__ static __forceinline__ void widen(const uint4 &r, float *o)
    {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    // round-to-nearest-even to bfloat16 (gfx950 converts in hardware:
    // v_cvt_pk_bf16_f32, two values per instruction; NaN stays NaN)
    __device__ static __forceinline__ T narrow(float x)
    {
        return __builtin_bit_cast(uint16_t, (__bf16)x);
    }
    // a in the low half, b in the high half
    __device__ static __forceinline__ uint32_t narrow2(float a, float b)
    {
        typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
        const bf2 v = {(__bf16)a, (__bf16)b};
        return __builtin_bit_cast(uint32_t, v);
    }
    __device__ static __forceinline__ float widen1(T x) { return __uint_as_float((uint32_t)x << 16); }
    // the two elements of a 32-bit word (low half first)
    __device__ static __forceinline__ void widen2(uint32_t x, float *o)
    {
        o[0] = __uint_as_float(x << 16);
        o[1] = __uint_as_float(x & 0xffff0000u);
    }
};

// IEEE half storage: widened exactly to fp32 (v_cvt_f32_f16), narrowed with
// round to nearest even (v_cvt_f16_f32 in the default rounding mode)
struct StF16 {
    typedef uint16_t T;
    static constexpr int VEC = 8;
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    typedef float fl2 __attribute__((ext_vector_type(2)));
    __device__ static __forceinline__ void widen2(uint32_t x, float *o)
    {
        const fl2 f = __builtin_convertvector(__builtin_bit_cast(h2, x), fl2);
        o[0] = f.x;
        o[1] = f.y;
    }
    __device__ static __forceinline__ void widen(const uint4 &r, float *o)
    {
        widen2(r.x, o);
        widen2(r.y, o + 2);
        widen2(r.z, o + 4);
        widen2(r.w, o + 6);
    }
    __device__ static __forceinline__ float widen1(T x)
    {
        return (float)__builtin_bit_cast(_Float16, x);
    }
    __device__ static __forceinline__ T narrow(float x)
    {
        return __builtin_bit_cast(uint16_t, (_Float16)x);
    }
    __device__ static __forceinline__ uint32_t narrow2(float a, float b)
    {
        const h2 v = {(_Float16)a, (_Float16)b};
        return __builtin_bit_cast(uint32_t, v);
    }
};

// ------------------------------------------------------------ configuration
// D: head dimension.  CS: column slices (workgroups that share one head and
// segment, each owning D/CS columns of the state).
template <int D_, int CS_>
struct Cfg {
    static constexpr int D = D_;
    static_assert(D == 16 || D == 32 || D == 64 || D == 128 || D == 256,
                  "unsupported head dimension");
    static constexpr int CS = CS_;
    static constexpr int NW = (D <= 64) ? D / 16 : (D == 128 ? 4 : 8);  // waves
    static constexpr int NT = NW * 64;                                    // threads
    static constexpr int KB = D / 16;               // 16-blocks of D
    static constexpr int NBW = KB / (CS * NW);      // state column blocks per wave
    static constexpr int KPW = KB / NW;             // contraction blocks per wave (16x16 products)
    static constexpr int LD = D + 4;                // LDS row stride (floats)
    static constexpr int RN = (D >= 256) ? 32 : 64; // rows per chunk, non-causal
    static constexpr int RC = 16;                   // rows per chunk, causal
    static constexpr int PS = D * D + 2 * D;        // floats per state record
    static_assert(NBW >= 1 && NBW * CS * NW == KB, "bad column split");
    static_assert(KPW >= 1 && KPW * NW == KB, "bad contraction split");
    static_assert(2 * D <= NT, "column-sum threads");
};

// default slicing: D = 256 holds its state in two workgroups
template <int D>
struct DefCS {
    static constexpr int value = (D == 256) ? 2 : 1;
};

// threads per workgroup (independent of the column slicing); a function so
// that it can appear inside __launch_bounds__
template <int D>
constexpr int threads_for()
{
    return Cfg<D, 1>::NT;
}

// global column of n-block nb of wave w in column slice cs
template <class C>
__device__ __forceinline__ int ncol(int cs, int w, int nb)
{
    return (cs * (C::KB / C::CS) + w * C::NBW + nb) * 16;
}

// ---------------------------------------------------------------- tile I/O
// ROWS x D tile of one head, fetched with 16-byte loads into registers and
// committed to LDS as fp32 (row stride D + 4).  Rows at or beyond `lim` read
// as zero.  A head of dl < D columns (rows dl elements apart in memory) is
// read element by element, its columns dl .. D - 1 as zero.
template <class ST, class C, int ROWS>
struct Tile {
    typedef typename ST::T T;
    static constexpr int D = C::D;
    static constexpr int VPR = D / ST::VEC;
    static constexpr int NV = ROWS * VPR;
    static constexpr int PER = (NV + C::NT - 1) / C::NT;
    uint4 r[PER];

    __device__ __forceinline__ void fetch(const T *__restrict__ head, int64_t row0,
                                          int64_t lim, int dl = D)
    {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int idx = (int)threadIdx.x + p * C::NT;
            r[p] = make_uint4(0u, 0u, 0u, 0u);
            if (NV % C::NT == 0 || idx < NV) {
                const int row = idx / VPR, cv = idx % VPR;
                if (row0 + row < lim) {
                    if (dl == D) {
                        r[p] = *reinterpret_cast<const uint4 *>(
                            head + (row0 + row) * (int64_t)D + cv * ST::VEC);
                    } else {
                        T v[ST::VEC];
#pragma unroll
                        for (int x = 0; x < ST::VEC; ++x) {
                            const int col = cv * ST::VEC + x;
                            v[x] = col < dl ? head[(row0 + row) * (int64_t)dl + col] : T(0);
                        }
                        r[p] = __builtin_bit_cast(uint4, v);
                    }
                }
            }
        }
    }

    __device__ __forceinline__ void commit(float *lds) const
    {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int idx = (int)threadIdx.x + p * C::NT;
            if (NV % C::NT == 0 || idx < NV) {
                const int row = idx / VPR, cv = idx % VPR;
                float v[ST::VEC];
                ST::widen(r[p], v);
                float *dst = lds + row * C::LD + cv * ST::VEC;
#pragma unroll
                for (int x = 0; x < ST::VEC; x += 4)
                    *reinterpret_cast<f4 *>(dst + x) = f4{v[x], v[x + 1], v[x + 2], v[x + 3]};
            }
        }
    }
};

// ------------------------------------------------------- wave-level products
template <class C>
struct Acc {
    f4 t[C::KB][C::NBW];
    __device__ __forceinline__ void zero()
    {
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int nb = 0; nb < C::NBW; ++nb)
                t[kb][nb] = f4{0.f, 0.f, 0.f, 0.f};
    }
    // Mat[k][n] = rec[k*D + n]; lane holds Mat[kb*16+4lg+r][ncol+lr]
    __device__ __forceinline__ void load(const float *rec, int cs, int w, int lr, int lg)
    {
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int nb = 0; nb < C::NBW; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    t[kb][nb][r] = rec[(kb * 16 + 4 * lg + r) * C::D + ncol<C>(cs, w, nb) + lr];
    }
    // Mat[k][n] = rec[n*D + k] (the transpose of a stored record)
    __device__ __forceinline__ void load_t(const float *rec, int cs, int w, int lr, int lg)
    {
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int nb = 0; nb < C::NBW; ++nb)
                t[kb][nb] = *reinterpret_cast<const f4 *>(
                    rec + (ncol<C>(cs, w, nb) + lr) * C::D + kb * 16 + 4 * lg);
    }
    __device__ __forceinline__ void store(float *rec, int cs, int w, int lr, int lg) const
    {
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int nb = 0; nb < C::NBW; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    rec[(kb * 16 + 4 * lg + r) * C::D + ncol<C>(cs, w, nb) + lr] = t[kb][nb][r];
    }
};

// acc += X^T Y over ROWS staged rows: Mat[k][n] += sum_t X[t][k] Y[t][n],
// k over all D, n over this wave's columns.
template <class C, int ROWS>
__device__ __forceinline__ void reduce_rows(Acc<C> &acc, const float *xs, const float *ys,
                                            int cs, int w, int lr, int lg)
{
#pragma unroll
    for (int ts = 0; ts < ROWS / 4; ++ts) {
        float a[C::KB], b[C::NBW];
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
            a[kb] = xs[(ts * 4 + lg) * C::LD + kb * 16 + lr];
#pragma unroll
        for (int nb = 0; nb < C::NBW; ++nb)
            b[nb] = ys[(ts * 4 + lg) * C::LD + ncol<C>(cs, w, nb) + lr];
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int nb = 0; nb < C::NBW; ++nb)
                acc.t[kb][nb] = mma(a[kb], b[nb], acc.t[kb][nb]);
    }
}

// out[tb][nb] += Z[tb*16 + ., :] . Mat[:, wave columns] for staged rows Z.
template <class C, int TB>
__device__ __forceinline__ void apply_rows(f4 (&out)[TB][C::NBW], const float *zs,
                                           const Acc<C> &acc, int lr, int lg)
{
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
            const f4 z = *reinterpret_cast<const f4 *>(zs + (tb * 16 + lr) * C::LD +
                                                       kb * 16 + 4 * lg);
#pragma unroll
            for (int nb = 0; nb < C::NBW; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    out[tb][nb] = mma(z[r], acc.t[kb][nb][r], out[tb][nb]);
        }
}

// Partial of X Y^T (16 x 16, first 16 staged rows of each) over this wave's
// share of the D columns; stored to part[w*256 + i*16 + j].
template <class C>
__device__ __forceinline__ void pair_partial(float *part, const float *xs, const float *ys,
                                             int w, int lr, int lg)
{
    f4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < C::KPW; ++kk) {
        const int kb = w * C::KPW + kk;
        const f4 xa = *reinterpret_cast<const f4 *>(xs + lr * C::LD + kb * 16 + 4 * lg);
        const f4 yb = *reinterpret_cast<const f4 *>(ys + lr * C::LD + kb * 16 + 4 * lg);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            p = mma(xa[r], yb[r], p);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
        part[w * 256 + (4 * lg + r) * 16 + lr] = p[r];
}

// out[nb] += A16 . Y: A16 is 16x16 in LDS (row stride 20; row = output row,
// column = contraction index), Y is staged rows.
template <class C>
__device__ __forceinline__ void small_apply(f4 (&out)[C::NBW], const float *a16,
                                            const float *ys, int cs, int w, int lr, int lg)
{
    const f4 a = *reinterpret_cast<const f4 *>(a16 + lr * 20 + 4 * lg);
#pragma unroll
    for (int nb = 0; nb < C::NBW; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            out[nb] = mma(a[r], ys[(4 * lg + r) * C::LD + ncol<C>(cs, w, nb) + lr], out[nb]);
}

// out[nb] += A16^T . Y (contraction over the row index of A16)
template <class C>
__device__ __forceinline__ void small_apply_t(f4 (&out)[C::NBW], const float *a16,
                                              const float *ys, int cs, int w, int lr, int lg)
{
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float a = a16[(4 * lg + r) * 20 + lr];
#pragma unroll
        for (int nb = 0; nb < C::NBW; ++nb)
            out[nb] = mma(a, ys[(4 * lg + r) * C::LD + ncol<C>(cs, w, nb) + lr], out[nb]);
    }
}

// sum over the ROWS staged rows of column c
template <class C, int ROWS>
__device__ __forceinline__ float col_sum(const float *xs, int c)
{
    float s = 0.f;
#pragma unroll 4
    for (int i = 0; i < ROWS; ++i)
        s += xs[i * C::LD + c];
    return s;
}

// sum over the ROWS staged rows of wt[i] * xs[i][c]
template <class C, int ROWS>
__device__ __forceinline__ float col_wsum(const float *xs, const float *wt, int c)
{
    float s = 0.f;
#pragma unroll 4
    for (int i = 0; i < ROWS; ++i)
        s += wt[i] * xs[i * C::LD + c];
    return s;
}

// outv[i] = x_i . vec for ROWS staged rows, one wave per row
template <class C, int ROWS>
__device__ __forceinline__ void row_dots(float *outv, const float *xs, const float *vec,
                                         int w, int lane)
{
    for (int i = w; i < ROWS; i += C::NW) {
        float s = 0.f;
        for (int d = lane; d < C::D; d += 64)
            s += xs[i * C::LD + d] * vec[d];
        s = wave_sum(s);
        if (lane == 0)
            outv[i] = s;
    }
}

// W = mask(1 + sum of the wave partials) into w16 (row stride 20); causal
// mask keeps j <= i.  Also returns nothing; all threads take part.
template <class C>
__device__ __forceinline__ void build_w(float *w16, const float *part, int tid)
{
    for (int x = tid; x < 256; x += C::NT) {
        const int i = x >> 4, j = x & 15;
        float p = 0.f;
        for (int ww = 0; ww < C::NW; ++ww)
            p += part[ww * 256 + x];
        w16[i * 20 + j] = (j <= i) ? 1.f + p : 0.f;
    }
}

struct Where {
    int64_t bh;
    int seg, cs;
};

template <int CS>
__device__ __forceinline__ Where decode(int nseg)
{
    Where g;
    int64_t b = blockIdx.x;
    g.cs = (int)(b % CS);
    b /= CS;
    g.seg = (int)(b % nseg);
    g.bh = b / nseg;
    return g;
}

// ============================================================ kernels

// Segment-local forward state: Mat = K^T V over the segment's rows and the
// column sums z = sum k, u = sum v.  Record: Mat[D][D] row-major, z[D], u[D].
template <class ST, int D>
__global__ __launch_bounds__(threads_for<D>()) void k_state_local(
    const typename ST::T *__restrict__ Kp, const typename ST::T *__restrict__ Vp,
    float *__restrict__ part, int64_t N, int64_t seg_len, int nseg, int dl)
{
    typedef Cfg<D, DefCS<D>::value> C;
    constexpr int R = C::RN;
    __shared__ __attribute__((aligned(16))) float xs[R * C::LD];
    __shared__ __attribute__((aligned(16))) float ys[R * C::LD];
    const Where g = decode<C::CS>(nseg);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15,
              lg = lane >> 4;
    const int64_t beg = g.seg * seg_len;
    const int64_t end = (beg + seg_len < N) ? beg + seg_len : N;
    const typename ST::T *xh = Kp + g.bh * N * dl;
    const typename ST::T *yh = Vp + g.bh * N * dl;

    Acc<C> acc;
    acc.zero();
    float csum = 0.f;

    Tile<ST, C, R> tx, ty;
    tx.fetch(xh, beg, end, dl);
    ty.fetch(yh, beg, end, dl);
    for (int64_t c0 = beg; c0 < end; c0 += R) {
        __syncthreads();
        tx.commit(xs);
        ty.commit(ys);
        if (c0 + R < end) {
            tx.fetch(xh, c0 + R, end, dl);
            ty.fetch(yh, c0 + R, end, dl);
        }
        __syncthreads();
        reduce_rows<C, R>(acc, xs, ys, g.cs, w, lr, lg);
        if (tid < 2 * D)
            csum += (tid < D) ? col_sum<C, R>(xs, tid) : col_sum<C, R>(ys, tid - D);
    }
    float *out = part + (g.bh * nseg + g.seg) * (int64_t)C::PS;
    acc.store(out, g.cs, w, lr, lg);
    if (g.cs == 0 && tid < 2 * D)
        out[D * D + tid] = csum;
}

// Combine the per-segment records of every head in a fixed order, starting
// from init[bh] (a record carried in from outside the call; zero when init
// is null):
//   mode 0: out[bh] = init[bh] + sum_s part[bh][s]
//   mode 1: part[bh][s] <- init[bh] + sum_{s' < s} part[bh][s']   (in place)
//   mode 2: part[bh][s] <- init[bh] + sum_{s' > s} part[bh][s']   (in place)
// and, when total is not null, total[bh] = init[bh] + sum_s part[bh][s]
// (the record carried out of the call).
// Each thread takes 4 consecutive floats of the record (records are PS =
// D^2 + 2D floats, a multiple of 4, and 16-byte aligned); the segments'
// loads of a batch are issued before any of them is added, in order.
__global__ __launch_bounds__(256) void k_state_scan(float *__restrict__ part,
                                                    float *__restrict__ out, int nseg,
                                                    int64_t PS, int64_t blocks_per_head,
                                                    int mode, const float *__restrict__ init,
                                                    float *__restrict__ total)
{
    constexpr int BATCH = 8;
    const int64_t bh = blockIdx.x / blocks_per_head;
    const int64_t e = 4 * ((blockIdx.x % blocks_per_head) * 256 + threadIdx.x);
    if (e >= PS)
        return;
    f4 *p = reinterpret_cast<f4 *>(part + bh * nseg * PS + e);
    const int64_t ps4 = PS / 4;
    f4 run = {0.f, 0.f, 0.f, 0.f};
    if (init)
        run = *reinterpret_cast<const f4 *>(init + bh * PS + e);
    if (mode == 0) {
        for (int s0 = 0; s0 < nseg; s0 += BATCH) {
            f4 v[BATCH];
#pragma unroll
            for (int b = 0; b < BATCH; ++b)
                if (s0 + b < nseg)
                    v[b] = p[(s0 + b) * ps4];
#pragma unroll
            for (int b = 0; b < BATCH; ++b)
                if (s0 + b < nseg)
                    run += v[b];
        }
        *reinterpret_cast<f4 *>(out + bh * PS + e) = run;
    } else if (mode == 1) {
        for (int s = 0; s < nseg; ++s) {
            const f4 v = p[s * ps4];
            p[s * ps4] = run;
            run += v;
        }
    } else {
        for (int s = nseg - 1; s >= 0; --s) {
            const f4 v = p[s * ps4];
            p[s * ps4] = run;
            run += v;
        }
    }
    if (total)
        *reinterpret_cast<f4 *>(total + bh * PS + e) = run;
}

// Forward.  state: CAUSAL ? exclusive-prefix record per (head, segment)
//                         : total record per head.
template <class ST, int D, bool CAUSAL>
__global__ __launch_bounds__(threads_for<D>()) void k_forward(
    const typename ST::T *__restrict__ Q, const typename ST::T *__restrict__ Kp,
    const typename ST::T *__restrict__ Vp, typename ST::T *__restrict__ O,
    float *__restrict__ den_out, const float *__restrict__ state, int64_t N,
    int64_t seg_len, int nseg, float n0, OutLay ol, int dl)
{
    typedef Cfg<D, DefCS<D>::value> C;
    constexpr int R = CAUSAL ? C::RC : C::RN;
    constexpr int TB = R / 16;
    constexpr int RK = CAUSAL ? R : 1;
    __shared__ __attribute__((aligned(16))) float qs[R * C::LD];
    __shared__ __attribute__((aligned(16))) float ks[RK * C::LD];
    __shared__ __attribute__((aligned(16))) float vs[RK * C::LD];
    __shared__ __attribute__((aligned(16))) float pp[CAUSAL ? C::NW * 256 : 1];
    __shared__ __attribute__((aligned(16))) float wl[CAUSAL ? 16 * 20 : 1];
    __shared__ float zl[2][D], ul[2][D];
    __shared__ float rowv[R], denl[R];

    const Where g = decode<C::CS>(nseg);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15,
              lg = lane >> 4;
    const int64_t beg = g.seg * seg_len;
    const int64_t end = (beg + seg_len < N) ? beg + seg_len : N;
    const int64_t hoff = g.bh * N * dl;
    const float *st = state + (CAUSAL ? (g.bh * nseg + g.seg) : g.bh) * (int64_t)C::PS;

    Acc<C> S;  // Mat[k=d][n=e] = S
    S.load(st, g.cs, w, lr, lg);
    if (tid < D) {
        zl[0][tid] = st[D * D + tid];
        ul[0][tid] = st[D * D + D + tid];
    }
    int cur = 0;

    Tile<ST, C, R> tq;
    Tile<ST, C, RK> tk, tv;
    tq.fetch(Q + hoff, beg, end, dl);
    if constexpr (CAUSAL) {
        tk.fetch(Kp + hoff, beg, end, dl);
        tv.fetch(Vp + hoff, beg, end, dl);
    }
    for (int64_t c0 = beg; c0 < end; c0 += R) {
        __syncthreads();
        tq.commit(qs);
        if constexpr (CAUSAL) {
            tk.commit(ks);
            tv.commit(vs);
        }
        if (c0 + R < end) {
            tq.fetch(Q + hoff, c0 + R, end, dl);
            if constexpr (CAUSAL) {
                tk.fetch(Kp + hoff, c0 + R, end, dl);
                tv.fetch(Vp + hoff, c0 + R, end, dl);
            }
        }
        __syncthreads();
        row_dots<C, R>(rowv, qs, zl[cur], w, lane);
        if constexpr (CAUSAL)
            pair_partial<C>(pp, qs, ks, w, lr, lg);
        __syncthreads();
        if constexpr (CAUSAL) {
            build_w<C>(wl, pp, tid);
            if (tid < R) {
                float s = (n0 + (float)c0) + rowv[tid];
                for (int j = 0; j <= tid; ++j) {
                    float p = 0.f;
                    for (int ww = 0; ww < C::NW; ++ww)
                        p += pp[ww * 256 + tid * 16 + j];
                    s += 1.f + p;
                }
                denl[tid] = s;
            }
        } else {
            for (int i = tid; i < R; i += C::NT)
                denl[i] = (n0 + (float)N) + rowv[i];
        }
        __syncthreads();

        f4 out[TB][C::NBW];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int nb = 0; nb < C::NBW; ++nb) {
                const float u = ul[cur][ncol<C>(g.cs, w, nb) + lr];
                out[tb][nb] = f4{u, u, u, u};
            }
        apply_rows<C, TB>(out, qs, S, lr, lg);
        if constexpr (CAUSAL)
            small_apply<C>(out[0], wl, vs, g.cs, w, lr, lg);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int nb = 0; nb < C::NBW; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = tb * 16 + 4 * lg + r;
                    const int col = ncol<C>(g.cs, w, nb) + lr;
                    if (c0 + row < end && col < dl)
                        O[ol.head(g.bh) + (c0 + row) * ol.sn + col] =
                            ST::narrow(out[tb][nb][r] / denl[row]);
                }
        if (den_out != nullptr && g.cs == 0)
            for (int i = tid; i < R; i += C::NT)
                if (c0 + i < end)
                    den_out[g.bh * N + c0 + i] = denl[i];
        if constexpr (CAUSAL) {
            reduce_rows<C, RK>(S, ks, vs, g.cs, w, lr, lg);
            if (tid < D)
                zl[cur ^ 1][tid] = zl[cur][tid] + col_sum<C, RK>(ks, tid);
            else if (tid < 2 * D)
                ul[cur ^ 1][tid - D] = ul[cur][tid - D] + col_sum<C, RK>(vs, tid - D);
            cur ^= 1;
        }
    }
}

// Backward, query side: dQ, and the segment-local gradient record (dS =
// Q^T A, r = sum c q, t = sum a) into gpart.  Stores (c_i, den_i) per token
// into cbuf when CAUSAL.  The workgroup holds all of S (one column slice),
// since c_i needs q_i.(S a_i) in full.
template <class ST, int D, bool CAUSAL>
__global__ __launch_bounds__(threads_for<D>()) void k_bwd_q(
    const typename ST::T *__restrict__ Q, const typename ST::T *__restrict__ Kp,
    const typename ST::T *__restrict__ Vp, const typename ST::T *__restrict__ G,
    typename ST::T *__restrict__ dQ, const float *__restrict__ state,
    float *__restrict__ gpart, float *__restrict__ cbuf, int64_t N, int64_t seg_len,
    int nseg, float n0, OutLay ol, int dl)
{
    typedef Cfg<D, 1> C;
    constexpr int R = CAUSAL ? C::RC : C::RN;
    constexpr int TB = R / 16;
    constexpr int RK = CAUSAL ? R : 1;
    __shared__ __attribute__((aligned(16))) float qs[R * C::LD];
    __shared__ __attribute__((aligned(16))) float gs[R * C::LD];  // dO, then A
    __shared__ __attribute__((aligned(16))) float ks[RK * C::LD];
    __shared__ __attribute__((aligned(16))) float vs[RK * C::LD];
    __shared__ __attribute__((aligned(16))) float pp[CAUSAL ? C::NW * 256 : 1];
    __shared__ __attribute__((aligned(16))) float ep[CAUSAL ? C::NW * 256 : 1];
    __shared__ __attribute__((aligned(16))) float wl[CAUSAL ? 16 * 20 : 1];
    __shared__ __attribute__((aligned(16))) float pml[CAUSAL ? 16 * 20 : 1];
    __shared__ float zl[2][D], ul[2][D];
    __shared__ float rowqz[R], rowau[R], denl[R], cl[R];
    __shared__ float qyp[C::NW][R];

    const Where g = decode<1>(nseg);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15,
              lg = lane >> 4;
    const int64_t beg = g.seg * seg_len;
    const int64_t end = (beg + seg_len < N) ? beg + seg_len : N;
    const int64_t hoff = g.bh * N * dl;
    const float *st = state + (CAUSAL ? (g.bh * nseg + g.seg) : g.bh) * (int64_t)C::PS;

    Acc<C> ST_;  // Mat[k=e][n=d] = S^T
    ST_.load_t(st, 0, w, lr, lg);
    Acc<C> dS;   // Mat[k=d][n=e] = sum q a^T over the segment
    dS.zero();
    if (tid < D) {
        zl[0][tid] = st[D * D + tid];
        ul[0][tid] = st[D * D + D + tid];
    }
    int cur = 0;
    float colacc = 0.f;  // tid < D: r[tid]; D <= tid < 2D: t[tid - D]

    Tile<ST, C, R> tq, tg;
    Tile<ST, C, RK> tk, tv;
    tq.fetch(Q + hoff, beg, end, dl);
    tg.fetch(G + hoff, beg, end, dl);
    if constexpr (CAUSAL) {
        tk.fetch(Kp + hoff, beg, end, dl);
        tv.fetch(Vp + hoff, beg, end, dl);
    }
    for (int64_t c0 = beg; c0 < end; c0 += R) {
        __syncthreads();
        tq.commit(qs);
        tg.commit(gs);
        if constexpr (CAUSAL) {
            tk.commit(ks);
            tv.commit(vs);
        }
        if (c0 + R < end) {
            tq.fetch(Q + hoff, c0 + R, end, dl);
            tg.fetch(G + hoff, c0 + R, end, dl);
            if constexpr (CAUSAL) {
                tk.fetch(Kp + hoff, c0 + R, end, dl);
                tv.fetch(Vp + hoff, c0 + R, end, dl);
            }
        }
        __syncthreads();
        row_dots<C, R>(rowqz, qs, zl[cur], w, lane);
        if constexpr (CAUSAL)
            pair_partial<C>(pp, qs, ks, w, lr, lg);
        __syncthreads();
        if constexpr (CAUSAL) {
            build_w<C>(wl, pp, tid);
            if (tid < R) {
                float s = (n0 + (float)c0) + rowqz[tid];
                for (int j = 0; j <= tid; ++j) {
                    float p = 0.f;
                    for (int ww = 0; ww < C::NW; ++ww)
                        p += pp[ww * 256 + tid * 16 + j];
                    s += 1.f + p;
                }
                denl[tid] = s;
            }
        } else {
            for (int i = tid; i < R; i += C::NT)
                denl[i] = (n0 + (float)N) + rowqz[i];
        }
        __syncthreads();
        // A = dO / den (rows past the end are zero)
        for (int x = tid; x < R * D; x += C::NT) {
            const int i = x / D, d = x % D;
            gs[i * C::LD + d] = (c0 + i < end) ? gs[i * C::LD + d] / denl[i] : 0.f;
        }
        __syncthreads();
        // Y = A S^T (row i is S a_i), accumulator layout
        f4 y[TB][C::NBW];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int nb = 0; nb < C::NBW; ++nb)
                y[tb][nb] = f4{0.f, 0.f, 0.f, 0.f};
        apply_rows<C, TB>(y, gs, ST_, lr, lg);
        // q_i . y_i over this wave's columns
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = tb * 16 + 4 * lg + r;
                float s = 0.f;
#pragma unroll
                for (int nb = 0; nb < C::NBW; ++nb)
                    s += qs[row * C::LD + ncol<C>(0, w, nb) + lr] * y[tb][nb][r];
                s = group16_sum(s);
                if (lr == 0)
                    qyp[w][row] = s;
            }
        row_dots<C, R>(rowau, gs, ul[cur], w, lane);
        if constexpr (CAUSAL)
            pair_partial<C>(ep, gs, vs, w, lr, lg);  // E = A V^T
        __syncthreads();
        // c_i den_i = a_i.u + q_i.(S a_i) (+ sum_j W_ij a_i.v_j in the chunk)
        if (tid < R) {
            const int i = tid;
            float s = rowau[i];
            for (int ww = 0; ww < C::NW; ++ww)
                s += qyp[ww][i];
            if constexpr (CAUSAL) {
                for (int j = 0; j <= i; ++j) {
                    float e = 0.f;
                    for (int ww = 0; ww < C::NW; ++ww)
                        e += ep[ww * 256 + i * 16 + j];
                    s += wl[i * 20 + j] * e;
                }
            }
            cl[i] = s / denl[i];
        }
        __syncthreads();
        if constexpr (CAUSAL) {
            for (int x = tid; x < 256; x += C::NT) {
                const int i = x >> 4, j = x & 15;
                float e = 0.f;
                for (int ww = 0; ww < C::NW; ++ww)
                    e += ep[ww * 256 + x];
                pml[i * 20 + j] = (j <= i) ? e - cl[i] : 0.f;
            }
        }
        if constexpr (CAUSAL) {
            for (int i = tid; i < R; i += C::NT)
                if (c0 + i < end) {
                    cbuf[(g.bh * N + c0 + i) * 2 + 0] = cl[i];
                    cbuf[(g.bh * N + c0 + i) * 2 + 1] = denl[i];
                }
        }
        if constexpr (CAUSAL)
            __syncthreads();
        // dQ = Y - c z^T (+ Pm K in the chunk)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int nb = 0; nb < C::NBW; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = tb * 16 + 4 * lg + r;
                    y[tb][nb][r] -= cl[row] * zl[cur][ncol<C>(0, w, nb) + lr];
                }
        if constexpr (CAUSAL)
            small_apply<C>(y[0], pml, ks, 0, w, lr, lg);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int nb = 0; nb < C::NBW; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = tb * 16 + 4 * lg + r;
                    const int col = ncol<C>(0, w, nb) + lr;
                    if (c0 + row < end && col < dl)
                        dQ[ol.head(g.bh) + (c0 + row) * ol.sn + col] = ST::narrow(y[tb][nb][r]);
                }
        reduce_rows<C, R>(dS, qs, gs, 0, w, lr, lg);
        if (tid < D)
            colacc += col_wsum<C, R>(qs, cl, tid);
        else if (tid < 2 * D)
            colacc += col_sum<C, R>(gs, tid - D);
        if constexpr (CAUSAL) {
            // S^T += V^T K ; z += sum k ; u += sum v
            reduce_rows<C, RK>(ST_, vs, ks, 0, w, lr, lg);
            if (tid < D)
                zl[cur ^ 1][tid] = zl[cur][tid] + col_sum<C, RK>(ks, tid);
            else if (tid < 2 * D)
                ul[cur ^ 1][tid - D] = ul[cur][tid - D] + col_sum<C, RK>(vs, tid - D);
            cur ^= 1;
        }
    }
    float *out = gpart + (g.bh * nseg + g.seg) * (int64_t)C::PS;
    dS.store(out, 0, w, lr, lg);
    if (tid < 2 * D)
        out[D * D + tid] = colacc;
}

// Backward, key/value side: dK = V dS^T - r (+ Pm^T Q), dV = K dS + t
// (+ W^T A).  gstate: CAUSAL ? exclusive-suffix record per (head, segment)
//                            : total record per head.
template <class ST, int D, bool CAUSAL>
__global__ __launch_bounds__(threads_for<D>()) void k_bwd_kv(
    const typename ST::T *__restrict__ Q, const typename ST::T *__restrict__ Kp,
    const typename ST::T *__restrict__ Vp, const typename ST::T *__restrict__ G,
    typename ST::T *__restrict__ dK, typename ST::T *__restrict__ dV,
    const float *__restrict__ gstate, const float *__restrict__ cbuf, int64_t N,
    int64_t seg_len, int nseg, OutLay ol, int dl)
{
    typedef Cfg<D, DefCS<D>::value> C;
    constexpr int R = CAUSAL ? C::RC : C::RN;
    constexpr int TB = R / 16;
    constexpr int RQ = CAUSAL ? R : 1;
    __shared__ __attribute__((aligned(16))) float ks[R * C::LD];
    __shared__ __attribute__((aligned(16))) float vs[R * C::LD];
    __shared__ __attribute__((aligned(16))) float qs[RQ * C::LD];
    __shared__ __attribute__((aligned(16))) float gs[RQ * C::LD];  // dO, then A
    __shared__ __attribute__((aligned(16))) float pp[CAUSAL ? C::NW * 256 : 1];
    __shared__ __attribute__((aligned(16))) float wl[CAUSAL ? 16 * 20 : 1];
    __shared__ __attribute__((aligned(16))) float pml[CAUSAL ? 16 * 20 : 1];
    __shared__ float rl[2][D], tl[2][D];
    __shared__ float cl[RQ], denl[RQ];

    const Where g = decode<C::CS>(nseg);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15,
              lg = lane >> 4;
    const int64_t beg = g.seg * seg_len;
    const int64_t end = (beg + seg_len < N) ? beg + seg_len : N;
    const int64_t hoff = g.bh * N * dl;
    const float *st = gstate + (CAUSAL ? (g.bh * nseg + g.seg) : g.bh) * (int64_t)C::PS;

    Acc<C> dST, dSN;  // Mat[k=e][n=d] = dS^T (for dK);  Mat[k=d][n=e] = dS (for dV)
    dST.load_t(st, g.cs, w, lr, lg);
    dSN.load(st, g.cs, w, lr, lg);
    if (tid < D) {
        rl[0][tid] = st[D * D + tid];
        tl[0][tid] = st[D * D + D + tid];
    }
    int cur = 0;

    // chunk order: forward when non-causal; backward (growing suffix) when causal
    const int64_t nch = (end - beg + R - 1) / R;
    Tile<ST, C, R> tk, tv;
    Tile<ST, C, RQ> tq, tg;
    {
        const int64_t c = CAUSAL ? beg + (nch - 1) * R : beg;
        tk.fetch(Kp + hoff, c, end, dl);
        tv.fetch(Vp + hoff, c, end, dl);
        if constexpr (CAUSAL) {
            tq.fetch(Q + hoff, c, end, dl);
            tg.fetch(G + hoff, c, end, dl);
        }
    }
    for (int64_t ci = 0; ci < nch; ++ci) {
        const int64_t c0 = CAUSAL ? beg + (nch - 1 - ci) * R : beg + ci * R;
        __syncthreads();
        tk.commit(ks);
        tv.commit(vs);
        if constexpr (CAUSAL) {
            tq.commit(qs);
            tg.commit(gs);
        }
        if (ci + 1 < nch) {
            const int64_t c1 = CAUSAL ? c0 - R : c0 + R;
            tk.fetch(Kp + hoff, c1, end, dl);
            tv.fetch(Vp + hoff, c1, end, dl);
            if constexpr (CAUSAL) {
                tq.fetch(Q + hoff, c1, end, dl);
                tg.fetch(G + hoff, c1, end, dl);
            }
        }
        if constexpr (CAUSAL) {
            if (tid < R) {
                const bool ok = c0 + tid < end;
                cl[tid] = ok ? cbuf[(g.bh * N + c0 + tid) * 2 + 0] : 0.f;
                denl[tid] = ok ? cbuf[(g.bh * N + c0 + tid) * 2 + 1] : 1.f;
            }
        }
        __syncthreads();
        if constexpr (CAUSAL) {
            pair_partial<C>(pp, qs, ks, w, lr, lg);  // P = Q K^T
            __syncthreads();
            build_w<C>(wl, pp, tid);
            for (int x = tid; x < R * D; x += C::NT) {
                const int i = x / D, d = x % D;
                gs[i * C::LD + d] = (c0 + i < end) ? gs[i * C::LD + d] / denl[i] : 0.f;
            }
            __syncthreads();
            pair_partial<C>(pp, gs, vs, w, lr, lg);  // E = A V^T
            __syncthreads();
            for (int x = tid; x < 256; x += C::NT) {
                const int i = x >> 4, j = x & 15;
                float e = 0.f;
                for (int ww = 0; ww < C::NW; ++ww)
                    e += pp[ww * 256 + x];
                pml[i * 20 + j] = (j <= i) ? e - cl[i] : 0.f;
            }
            __syncthreads();
        }
        f4 dk[TB][C::NBW], dv[TB][C::NBW];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int nb = 0; nb < C::NBW; ++nb) {
                const int col = ncol<C>(g.cs, w, nb) + lr;
                const float rr = -rl[cur][col], tt = tl[cur][col];
                dk[tb][nb] = f4{rr, rr, rr, rr};
                dv[tb][nb] = f4{tt, tt, tt, tt};
            }
        apply_rows<C, TB>(dk, vs, dST, lr, lg);
        apply_rows<C, TB>(dv, ks, dSN, lr, lg);
        if constexpr (CAUSAL) {
            small_apply_t<C>(dk[0], pml, qs, g.cs, w, lr, lg);
            small_apply_t<C>(dv[0], wl, gs, g.cs, w, lr, lg);
        }
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int nb = 0; nb < C::NBW; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = tb * 16 + 4 * lg + r;
                    const int col = ncol<C>(g.cs, w, nb) + lr;
                    if (c0 + row < end && col < dl) {
                        const int64_t o = ol.head(g.bh) + (c0 + row) * ol.sn + col;
                        dK[o] = ST::narrow(dk[tb][nb][r]);
                        dV[o] = ST::narrow(dv[tb][nb][r]);
                    }
                }
        if constexpr (CAUSAL) {
            // the suffix state takes this chunk in: dS^T += A^T Q, dS += Q^T A
            reduce_rows<C, RQ>(dST, gs, qs, g.cs, w, lr, lg);
            reduce_rows<C, RQ>(dSN, qs, gs, g.cs, w, lr, lg);
            if (tid < D)
                rl[cur ^ 1][tid] = rl[cur][tid] + col_wsum<C, RQ>(qs, cl, tid);
            else if (tid < 2 * D)
                tl[cur ^ 1][tid - D] = tl[cur][tid - D] + col_sum<C, RQ>(gs, tid - D);
            cur ^= 1;
        }
    }
}

}  // namespace la
