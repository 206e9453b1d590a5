// la_layer.hip -- one linear-attention layer around the head-batch passes:
// the input rows go through a linear map to queries, keys and values, linear
// attention gives the context rows, and a second linear map gives the output
// (the technical-framework paragraph, 技术框架, of the shd-paper.top digest
// of "Transformer Based Linear Attention with Optimized GPU Kernel
// Implementation").  Per sequence b, with X_b [N, C], Wqkv [C, 3 H D] and
// Wo [H D, C]:
//
//     [Q | K | V] = X Wqkv        (columns: H heads of D for each of Q, K, V)
//     O_h = LA(Q_h, K_h, V_h)     (the library's attention, every head h)
//     Y = [O_1 .. O_H] Wo
//
// The projections are GEMMs on rocBLAS (fp32 accumulation, storage-type
// inputs and outputs) arranged so that no pass moves rows between layouts:
//   - the QKV projection is one strided-batched GEMM per (sequence, Q|K|V)
//     over the heads, writing each head's [N, D] block straight into the
//     [B, H, N, D] tensors the attention reads;
//   - the attention writes O in the row layout [B, N, H, D], which the output
//     projection and its weight gradient take as a plain [B N, H D] matrix;
//   - backward, dO is formed per (sequence) by one strided-batched GEMM over
//     the heads in the [B, H, N, D] layout, and the attention writes dQ, dK,
//     dV side by side in the row layout [B, N, 3, H, D], which the two
//     gradient GEMMs of the projection take as a plain [B N, 3 H D] matrix.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "la.h"
#include "la_internal.hpp"

namespace {

constexpr size_t kBlasWorkspace = (size_t)64 << 20;   // rocBLAS scratch, from the caller's workspace

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

size_t esize(int dtype) { return dtype == LA_FP32 ? 4 : 2; }

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

// The same for `count` products C_i = op(A_i) op(B_i), A_i = A + i * sa,
// B_i = B + i * sb, C_i = C + i * sc (elements; a stride of 0 reuses one
// matrix for every product).
int gemm_batched(rocblas_handle h, bool ta, bool tb, int64_t M, int64_t Nc, int64_t K,
                 const void *A, int64_t lda, int64_t sa, const void *B, int64_t ldb, int64_t sb,
                 void *C, int64_t ldc, int64_t sc, int64_t count, int dtype)
{
    const float one = 1.f, zero = 0.f;
    const rocblas_datatype t = blas_type(dtype);
    const rocblas_status st = rocblas_gemm_strided_batched_ex(
        h, tb ? rocblas_operation_transpose : rocblas_operation_none,
        ta ? rocblas_operation_transpose : rocblas_operation_none, (rocblas_int)Nc,
        (rocblas_int)M, (rocblas_int)K, &one, B, t, (rocblas_int)ldb, (rocblas_stride)sb, A, t,
        (rocblas_int)lda, (rocblas_stride)sa, &zero, C, t, (rocblas_int)ldc, (rocblas_stride)sc,
        C, t, (rocblas_int)ldc, (rocblas_stride)sc, (rocblas_int)count, rocblas_datatype_f32_r,
        rocblas_gemm_algo_standard, 0, 0);
    return st == rocblas_status_success ? LA_OK : LA_ERR_HIP;
}

// ------------------------------------------------------------ layout
// saved (forward -> backward): Q, K, V [B,H,N,D], O in rows [B,N,H*D], the
// attention state.  Forward workspace: the attention workspace and rocBLAS
// scratch (+ the saved tensors when no saved buffer is given).  Backward
// workspace: dO [B,H,N,D], dQKV rows [B,N,3HD], the attention workspace,
// rocBLAS scratch.
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
    z.fwd = z.la_ws + kBlasWorkspace + z.saved;
    z.bwd = z.head + z.rows3 + z.la_ws + kBlasWorkspace;
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
    const size_t s = esize(dtype), hd = (size_t)(H * D);
    const Range ins[3] = {{(const char *)X, (size_t)(B * N * C) * s},
                          {(const char *)Wqkv, (size_t)C * 3 * hd * s},
                          {(const char *)Wo, hd * (size_t)C * s}};
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
    void *law = w, *bw = w + z.la_ws;
    const int64_t BN = B * N, HD = H * D;
    const size_t es = esize(dtype);

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
        // head h of Q (j = 0), K (1), V (2) of sequence b:
        // X_b [N, C] . Wqkv[:, j HD + h D ..] [C, D] -> [N, D] at (b H + h) N D
        void *dst[3] = {q, k, v};
        for (int64_t b = 0; b < B; ++b)
            for (int j = 0; j < 3; ++j)
                if ((rc = gemm_batched(bl->h, false, false, N, D, C,
                                       static_cast<const char *>(X) + (size_t)(b * N * C) * es, C,
                                       0, static_cast<const char *>(Wqkv) + (size_t)(j * HD) * es,
                                       3 * HD, D,
                                       static_cast<char *>(dst[j]) + (size_t)(b * H * N * D) * es,
                                       D, N * D, H, dtype)) != LA_OK)
                    return rc;
    }
    // O straight into the rows [B, N, H, D]
    if ((rc = la_internal::forward_to(q, k, v, orows, B, H, N, D, causal, dtype, state, law,
                                      z.la_ws, stream, {N * HD, D, HD})) != LA_OK)
        return rc;
    std::lock_guard<std::mutex> lk(bl->m);
    if (rocblas_set_stream(bl->h, st) != rocblas_status_success ||
        rocblas_set_workspace(bl->h, bw, kBlasWorkspace) != rocblas_status_success)
        return LA_ERR_HIP;
    return gemm(bl->h, false, false, BN, C, HD, orows, HD, Wo, C, Y, C, dtype);
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
    const size_t s = esize(dtype), hd = (size_t)(H * D);
    const Range ins[5] = {{(const char *)X, (size_t)(B * N * C) * s},
                          {(const char *)Wqkv, (size_t)C * 3 * hd * s},
                          {(const char *)Wo, hd * (size_t)C * s},
                          {(const char *)dY, (size_t)(B * N * C) * s},
                          {(const char *)saved, z.saved}};
    const Range outs[4] = {{(const char *)dX, (size_t)(B * N * C) * s},
                           {(const char *)dWqkv, (size_t)C * 3 * hd * s},
                           {(const char *)dWo, hd * (size_t)C * s},
                           {(const char *)ws, z.bwd}};
    if (aliased(outs, 4, ins, 5))
        return LA_ERR_ALIAS;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const char *sv = static_cast<const char *>(saved);
    const void *q = sv, *k = sv + z.head, *v = sv + 2 * z.head, *orows = sv + 3 * z.head;
    const void *state = sv + 3 * z.head + z.rows1;
    char *w = static_cast<char *>(ws);
    void *dO = w, *dqkv = w + z.head, *law = w + z.head + z.rows3;
    void *bw = w + z.head + z.rows3 + z.la_ws;
    const int64_t BN = B * N, HD = H * D;
    const size_t es = esize(dtype);

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
        // dWo = O_rows^T dY
        if ((rc = gemm(bl->h, true, false, HD, C, BN, orows, HD, dY, C, dWo, C, dtype)) != LA_OK)
            return rc;
        // head h of dO of sequence b: dY_b [N, C] . (rows h D .. of Wo)^T [C, D]
        for (int64_t b = 0; b < B; ++b)
            if ((rc = gemm_batched(bl->h, false, true, N, D, C,
                                   static_cast<const char *>(dY) + (size_t)(b * N * C) * es, C, 0,
                                   Wo, C, D * C,
                                   static_cast<char *>(dO) + (size_t)(b * H * N * D) * es, D,
                                   N * D, H, dtype)) != LA_OK)
                return rc;
    }
    // dQ, dK, dV side by side in the rows [B, N, 3, H, D]
    char *dq = static_cast<char *>(dqkv);
    if ((rc = la_internal::backward_to(q, k, v, dO, dq, dq + (size_t)HD * es,
                                       dq + (size_t)(2 * HD) * es, B, H, N, D, causal, dtype,
                                       state, law, z.la_ws, stream, {N * 3 * HD, D, 3 * HD})) !=
        LA_OK)
        return rc;
    std::lock_guard<std::mutex> lk(bl->m);
    if (rocblas_set_stream(bl->h, st) != rocblas_status_success ||
        rocblas_set_workspace(bl->h, bw, kBlasWorkspace) != rocblas_status_success)
        return LA_ERR_HIP;
    // dWqkv = X^T dQKV ; dX = dQKV Wqkv^T
    if ((rc = gemm(bl->h, true, false, C, 3 * HD, BN, X, C, dqkv, 3 * HD, dWqkv, 3 * HD,
                   dtype)) != LA_OK)
        return rc;
    return gemm(bl->h, false, true, BN, C, 3 * HD, dqkv, 3 * HD, Wqkv, 3 * HD, dX, C, dtype);
}

}  // extern "C"
