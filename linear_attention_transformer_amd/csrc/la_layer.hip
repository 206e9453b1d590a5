// la_layer.hip -- one linear-attention layer around the head-batch passes:
// the input rows go through a linear map to queries, keys and values, linear
// attention gives the context rows, and a second linear map gives the output
// (the technical-framework paragraph, 技术框架, of the shd-paper.top digest
// of "Transformer Based Linear Attention with Optimized GPU Kernel
// Implementation").  Per sequence b, with X_b [N, C], Wqkv [C, 3 H D] and
// Wo [H D, C]:
//
//     [Q | K | V] = X Wqkv        (columns: H heads of D for each of Q, K, V)
//     O_h = LA(Q_h, K_h, V_h)     (la_forward, every head h)
//     Y = [O_1 .. O_H] Wo
//
// The projections are plain GEMMs and run on rocBLAS (gemm_ex, fp32
// accumulation, storage-type inputs and outputs); the head split and merge
// between the row layout [B, N, T, H, D] and the head layout [B, H, N, D] of
// the attention passes is a kernel of this file; the attention is the
// library's own la_forward / la_backward.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "la.h"

namespace {

constexpr int kThreads = 256;
constexpr size_t kBlasWorkspace = (size_t)64 << 20;   // rocBLAS scratch, from the caller's workspace

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

size_t esize(int dtype) { return dtype == LA_FP32 ? 4 : 2; }

// Rows of the [B, N, T*H*D] row layout <-> T tensors [B, H, N, D].  A
// workgroup walks whole rows (b, n); its threads take consecutive chunks of
// the row (16 bytes when D allows, else one element), so both sides move
// contiguous runs.
template <class E, bool TO_HEADS>
__global__ __launch_bounds__(kThreads) void k_heads(E *__restrict__ rows_, E *__restrict__ t0,
                                                    E *__restrict__ t1, E *__restrict__ t2,
                                                    int64_t BN, int64_t N, int T, int H, int D)
{
    constexpr int V = 16 / sizeof(E);
    const bool vec = D % V == 0;
    const int W = vec ? V : 1;                       // elements per chunk
    const int row_len = T * H * D;
    const int chunks = row_len / W;
    for (int64_t r = blockIdx.x; r < BN; r += gridDim.x) {
        const int64_t b = r / N, n = r - b * N;
        E *row = rows_ + r * row_len;
        for (int ch = threadIdx.x; ch < chunks; ch += kThreads) {
            const int e = ch * W;
            const int c = e % D, th = e / D;
            const int h = th % H, t = th / H;
            E *tens = t == 0 ? t0 : (t == 1 ? t1 : t2);
            E *hp = tens + ((b * H + h) * N + n) * (int64_t)D + c;
            E *rp = row + e;
            if (vec) {
                if (TO_HEADS)
                    *reinterpret_cast<uint4 *>(hp) = *reinterpret_cast<const uint4 *>(rp);
                else
                    *reinterpret_cast<uint4 *>(rp) = *reinterpret_cast<const uint4 *>(hp);
            } else {
                if (TO_HEADS)
                    *hp = *rp;
                else
                    *rp = *hp;
            }
        }
    }
}

int heads(bool to_heads, void *rows_, void *t0, void *t1, void *t2, int64_t BN, int64_t N,
          int T, int64_t H, int64_t D, int dtype, hipStream_t s)
{
    const dim3 grid((unsigned)std::min<int64_t>(BN, 8192)), blk(kThreads);
    if (dtype == LA_FP32) {
        if (to_heads)
            k_heads<float, true><<<grid, blk, 0, s>>>(
                static_cast<float *>(rows_), static_cast<float *>(t0), static_cast<float *>(t1),
                static_cast<float *>(t2), BN, N, T, (int)H, (int)D);
        else
            k_heads<float, false><<<grid, blk, 0, s>>>(
                static_cast<float *>(rows_), static_cast<float *>(t0), static_cast<float *>(t1),
                static_cast<float *>(t2), BN, N, T, (int)H, (int)D);
    } else {
        if (to_heads)
            k_heads<uint16_t, true><<<grid, blk, 0, s>>>(
                static_cast<uint16_t *>(rows_), static_cast<uint16_t *>(t0),
                static_cast<uint16_t *>(t1), static_cast<uint16_t *>(t2), BN, N, T, (int)H,
                (int)D);
        else
            k_heads<uint16_t, false><<<grid, blk, 0, s>>>(
                static_cast<uint16_t *>(rows_), static_cast<uint16_t *>(t0),
                static_cast<uint16_t *>(t1), static_cast<uint16_t *>(t2), BN, N, T, (int)H,
                (int)D);
    }
    return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

// An error that earlier HIP calls on this thread left pending is not this
// call's: it launches nothing and leaves the error pending (as the head-batch
// calls do; hipErrorNotReady, a query's answer, is cleared).
int pending_error()
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

// ------------------------------------------------------------ rocBLAS
// One handle per device, created on first use; a call holds the device's
// lock while it sets the stream and workspace and enqueues its GEMMs.
struct Blas {
    rocblas_handle h = nullptr;
    std::mutex m;
};

Blas g_blas[64];
std::mutex g_blas_init;

Blas *blas_for_current_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return nullptr;
    std::lock_guard<std::mutex> lk(g_blas_init);
    if (g_blas[dev].h == nullptr && rocblas_create_handle(&g_blas[dev].h) != rocblas_status_success)
        return nullptr;
    return &g_blas[dev];
}

rocblas_datatype blas_type(int dtype)
{
    return dtype == LA_FP32 ? rocblas_datatype_f32_r
                            : (dtype == LA_BF16 ? rocblas_datatype_bf16_r : rocblas_datatype_f16_r);
}

// Row-major C[M, Nc] = op(A) op(B) (+ beta C), op(A) [M, K], op(B) [K, Nc];
// lda, ldb, ldc are the row lengths of A, B, C as stored.  rocBLAS is
// column-major, so this is C^T = op(B)^T op(A)^T there.
int gemm(rocblas_handle h, bool ta, bool tb, int64_t M, int64_t Nc, int64_t K, const void *A,
         int64_t lda, const void *B, int64_t ldb, void *C, int64_t ldc, int dtype)
{
    const float one = 1.f, zero = 0.f;
    const rocblas_datatype t = blas_type(dtype);
    const rocblas_status st = rocblas_gemm_ex(
        h, tb ? rocblas_operation_transpose : rocblas_operation_none,
        ta ? rocblas_operation_transpose : rocblas_operation_none, (rocblas_int)Nc,
        (rocblas_int)M, (rocblas_int)K, &one, B, t, (rocblas_int)ldb, A, t, (rocblas_int)lda,
        &zero, C, t, (rocblas_int)ldc, C, t, (rocblas_int)ldc, rocblas_datatype_f32_r,
        rocblas_gemm_algo_standard, 0, 0);
    return st == rocblas_status_success ? LA_OK : LA_ERR_HIP;
}

// ------------------------------------------------------------ layout
// saved (forward -> backward): Q, K, V [B,H,N,D], O in rows [B,N,H*D], the
// attention state.  Forward workspace: QKV rows [B,N,3HD], O [B,H,N,D], the
// attention workspace, rocBLAS scratch (+ the saved tensors when no saved
// buffer is given).  Backward workspace: dO rows, dO, dQ, dK, dV, dQKV rows,
// the attention workspace, rocBLAS scratch.
struct Sizes {
    size_t head, rows1, rows3, state, la_ws;
    size_t saved;        // Q K V O-rows state
    size_t fwd, bwd;     // workspace of each pass (forward without a saved buffer)
};

Sizes sizes(int64_t B, int64_t N, int64_t C, int64_t H, int64_t D, int causal, int dtype)
{
    Sizes z{};
    const size_t s = esize(dtype);
    z.head = up256((size_t)(B * H * N * D) * s);
    z.rows1 = up256((size_t)(B * N * H * D) * s);
    z.rows3 = up256((size_t)(B * N * 3 * H * D) * s);
    z.state = up256(la_state_size(B, H, N, D, causal));
    z.la_ws = up256(la_workspace_size_for(B, H, N, D, causal, dtype));
    z.saved = 3 * z.head + z.rows1 + z.state;
    z.fwd = z.rows3 + z.head + z.la_ws + kBlasWorkspace + z.saved;
    z.bwd = z.rows1 + 4 * z.head + z.rows3 + z.la_ws + kBlasWorkspace;
    (void)C;
    return z;
}

int check(int64_t B, int64_t N, int64_t C, int64_t H, int64_t D, int causal, int dtype)
{
    if (dtype != LA_FP32 && dtype != LA_BF16 && dtype != LA_FP16)
        return LA_ERR_DTYPE;
    if ((causal != 0 && causal != 1) || D < 1 || D > 256)
        return LA_ERR_UNSUPPORTED;
    if (B < 0 || N < 0 || C < 0 || H < 0)
        return LA_ERR_SHAPE;
    // GEMM sizes are 32-bit in rocBLAS
    const int64_t lim = ((int64_t)1 << 31) - 1;
    int64_t t;
    if (__builtin_mul_overflow(B, N, &t) || t > lim || C > lim ||
        __builtin_mul_overflow(3 * H, D, &t) || t > lim ||
        __builtin_mul_overflow(B * N, std::max<int64_t>(C, 3 * H * D), &t) ||
        la_workspace_size(std::max<int64_t>(B, 1), std::max<int64_t>(H, 1),
                          std::max<int64_t>(N, 1), D, causal) == 0)
        return LA_ERR_SHAPE;
    return LA_OK;
}

bool misaligned(const void *p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u); }

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

}  // namespace

extern "C" {

size_t la_layer_saved_size(int64_t B, int64_t N, int64_t C, int64_t H, int64_t D, int causal,
                           int dtype)
{
    if (check(B, N, C, H, D, causal, dtype) != LA_OK || B * N * H == 0)
        return 0;
    return sizes(B, N, C, H, D, causal, dtype).saved;
}

size_t la_layer_workspace_size(int64_t B, int64_t N, int64_t C, int64_t H, int64_t D,
                               int causal, int dtype)
{
    if (check(B, N, C, H, D, causal, dtype) != LA_OK || B * N * H == 0)
        return 0;
    const Sizes z = sizes(B, N, C, H, D, causal, dtype);
    return std::max(z.fwd, z.bwd);
}

int la_layer_forward(const void *X, const void *Wqkv, const void *Wo, void *Y, int64_t B,
                     int64_t N, int64_t C, int64_t H, int64_t D, int causal, int dtype,
                     void *saved, void *ws, size_t ws_bytes, void *stream)
{
    int rc = check(B, N, C, H, D, causal, dtype);
    if (rc != LA_OK)
        return rc;
    if (B * N == 0 || C == 0)
        return LA_OK;
    if (H == 0)
        return LA_ERR_SHAPE;   // Y would be X . (empty) : not a layer
    if (!X || !Wqkv || !Wo || !Y || !ws)
        return LA_ERR_NULL;
    const Sizes z = sizes(B, N, C, H, D, causal, dtype);
    const size_t need = saved ? z.fwd - z.saved : z.fwd;
    if (ws_bytes < need)
        return LA_ERR_WORKSPACE;
    if (misaligned(X) || misaligned(Wqkv) || misaligned(Wo) || misaligned(Y) ||
        misaligned(saved) || misaligned(ws))
        return LA_ERR_ALIGN;
    const size_t s = esize(dtype), HD = (size_t)(H * D);
    const Range ins[3] = {{(const char *)X, (size_t)(B * N * C) * s},
                          {(const char *)Wqkv, (size_t)C * 3 * HD * s},
                          {(const char *)Wo, HD * (size_t)C * s}};
    const Range outs[3] = {{(const char *)Y, (size_t)(B * N * C) * s},
                           {(const char *)saved, saved ? z.saved : 0},
                           {(const char *)ws, need}};
    if (aliased(outs, 3, ins, 3))
        return LA_ERR_ALIAS;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *w = static_cast<char *>(ws);
    char *sv = saved ? static_cast<char *>(saved) : w + (z.fwd - z.saved);
    void *q = sv, *k = sv + z.head, *v = sv + 2 * z.head, *orows = sv + 3 * z.head;
    void *state = sv + 3 * z.head + z.rows1;
    void *qkv = w, *o = w + z.rows3, *law = w + z.rows3 + z.head;
    void *bw = w + z.rows3 + z.head + z.la_ws;
    const int64_t BN = B * N;

    if ((rc = pending_error()) != LA_OK)
        return rc;
    Blas *bl = blas_for_current_device();
    if (!bl)
        return LA_ERR_HIP;
    {
        std::lock_guard<std::mutex> lk(bl->m);
        if (rocblas_set_stream(bl->h, st) != rocblas_status_success ||
            rocblas_set_workspace(bl->h, bw, kBlasWorkspace) != rocblas_status_success)
            return LA_ERR_HIP;
        if ((rc = gemm(bl->h, false, false, BN, 3 * H * D, C, X, C, Wqkv, 3 * H * D, qkv,
                       3 * H * D, dtype)) != LA_OK)
            return rc;
    }
    if ((rc = heads(true, qkv, q, k, v, BN, N, 3, H, D, dtype, st)) != LA_OK)
        return rc;
    if ((rc = la_forward(q, k, v, o, B, H, N, D, causal, dtype, nullptr, state, law, z.la_ws,
                         stream)) != LA_OK)
        return rc;
    if ((rc = heads(false, orows, o, nullptr, nullptr, BN, N, 1, H, D, dtype, st)) != LA_OK)
        return rc;
    std::lock_guard<std::mutex> lk(bl->m);
    if (rocblas_set_stream(bl->h, st) != rocblas_status_success ||
        rocblas_set_workspace(bl->h, bw, kBlasWorkspace) != rocblas_status_success)
        return LA_ERR_HIP;
    return gemm(bl->h, false, false, BN, C, H * D, orows, H * D, Wo, C, Y, C, dtype);
}

int la_layer_backward(const void *X, const void *Wqkv, const void *Wo, const void *dY,
                      void *dX, void *dWqkv, void *dWo, int64_t B, int64_t N, int64_t C,
                      int64_t H, int64_t D, int causal, int dtype, const void *saved, void *ws,
                      size_t ws_bytes, void *stream)
{
    int rc = check(B, N, C, H, D, causal, dtype);
    if (rc != LA_OK)
        return rc;
    if (B * N == 0 || C == 0)
        return LA_OK;
    if (H == 0)
        return LA_ERR_SHAPE;
    if (!X || !Wqkv || !Wo || !dY || !dX || !dWqkv || !dWo || !saved || !ws)
        return LA_ERR_NULL;
    const Sizes z = sizes(B, N, C, H, D, causal, dtype);
    if (ws_bytes < z.bwd)
        return LA_ERR_WORKSPACE;
    if (misaligned(X) || misaligned(Wqkv) || misaligned(Wo) || misaligned(dY) ||
        misaligned(dX) || misaligned(dWqkv) || misaligned(dWo) || misaligned(saved) ||
        misaligned(ws))
        return LA_ERR_ALIGN;
    const size_t s = esize(dtype), HD = (size_t)(H * D);
    const Range ins[5] = {{(const char *)X, (size_t)(B * N * C) * s},
                          {(const char *)Wqkv, (size_t)C * 3 * HD * s},
                          {(const char *)Wo, HD * (size_t)C * s},
                          {(const char *)dY, (size_t)(B * N * C) * s},
                          {(const char *)saved, z.saved}};
    const Range outs[4] = {{(const char *)dX, (size_t)(B * N * C) * s},
                           {(const char *)dWqkv, (size_t)C * 3 * HD * s},
                           {(const char *)dWo, HD * (size_t)C * s},
                           {(const char *)ws, z.bwd}};
    if (aliased(outs, 4, ins, 5))
        return LA_ERR_ALIAS;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const char *sv = static_cast<const char *>(saved);
    const void *q = sv, *k = sv + z.head, *v = sv + 2 * z.head, *orows = sv + 3 * z.head;
    const void *state = sv + 3 * z.head + z.rows1;
    char *w = static_cast<char *>(ws);
    void *dorows = w, *dO = w + z.rows1, *dq = w + z.rows1 + z.head,
         *dk = w + z.rows1 + 2 * z.head, *dv = w + z.rows1 + 3 * z.head,
         *dqkv = w + z.rows1 + 4 * z.head, *law = w + z.rows1 + 4 * z.head + z.rows3;
    void *bw = w + z.rows1 + 4 * z.head + z.rows3 + z.la_ws;
    const int64_t BN = B * N;

    if ((rc = pending_error()) != LA_OK)
        return rc;
    Blas *bl = blas_for_current_device();
    if (!bl)
        return LA_ERR_HIP;
    {
        std::lock_guard<std::mutex> lk(bl->m);
        if (rocblas_set_stream(bl->h, st) != rocblas_status_success ||
            rocblas_set_workspace(bl->h, bw, kBlasWorkspace) != rocblas_status_success)
            return LA_ERR_HIP;
        // dWo = O_rows^T dY ; dO_rows = dY Wo^T
        if ((rc = gemm(bl->h, true, false, H * D, C, BN, orows, H * D, dY, C, dWo, C, dtype)) !=
                LA_OK ||
            (rc = gemm(bl->h, false, true, BN, H * D, C, dY, C, Wo, C, dorows, H * D, dtype)) !=
                LA_OK)
            return rc;
    }
    if ((rc = heads(true, dorows, dO, nullptr, nullptr, BN, N, 1, H, D, dtype, st)) != LA_OK)
        return rc;
    if ((rc = la_backward(q, k, v, dO, dq, dk, dv, B, H, N, D, causal, dtype, state, law,
                          z.la_ws, stream)) != LA_OK)
        return rc;
    if ((rc = heads(false, dqkv, dq, dk, dv, BN, N, 3, H, D, dtype, st)) != LA_OK)
        return rc;
    std::lock_guard<std::mutex> lk(bl->m);
    if (rocblas_set_stream(bl->h, st) != rocblas_status_success ||
        rocblas_set_workspace(bl->h, bw, kBlasWorkspace) != rocblas_status_success)
        return LA_ERR_HIP;
    // dWqkv = X^T dQKV ; dX = dQKV Wqkv^T
    if ((rc = gemm(bl->h, true, false, C, 3 * H * D, BN, X, C, dqkv, 3 * H * D, dWqkv,
                   3 * H * D, dtype)) != LA_OK)
        return rc;
    return gemm(bl->h, false, true, BN, C, 3 * H * D, dqkv, 3 * H * D, Wqkv, 3 * H * D, dX, C,
                dtype);
}

}  // extern "C"
