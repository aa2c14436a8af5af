// linear.cpp -- the step's QKV projection: one bf16 GEMM over the whole mixed token array.
//
// bowenzhou.top "Sarathi：让解码搭上 prefill 的顺风车", section "Decode-maximal batching：顺车的账本":
// in a mixed batch the linear layers of the decode tokens and of the prefill chunk run as one
// matrix product, so every weight is read from memory once for all of them (attention stays
// separate).  The product here is out[T][N] = x[T][K] . w[N][K]^T with bf16 operands and fp32
// accumulation -- a plain library GEMM, done by hipBLASLt (up to 16 tokens the weight-streaming
// kernel of linear_skinny.hip runs instead).  hipBLASLt is column-major: with the
// row-major arrays read as their transposes this is D(N x T) = op_T(w as K x N) . x(K x T), the
// "TN" form.  Layouts and the chosen algorithm are cached per token count (the serving loop sees
// a few distinct T again and again).  The first call for a token count times up to kCandidates
// of the algorithms hipBLASLt proposes (on the caller's buffers, synchronising the stream) and
// keeps the fastest; the output is then written by that algorithm.

#include <hipblaslt/hipblaslt.h>

#include <map>
#include <string>

#include "internal.h"

namespace ca {

struct Linear {
    hipblasLtHandle_t handle = nullptr;
    hipblasLtMatmulDesc_t desc = nullptr;
    int64_t K = -1, N = -1;
    struct Shape {
        hipblasLtMatrixLayout_t a = nullptr, b = nullptr, d = nullptr;
        hipblasLtMatmulAlgo_t algo{};
        size_t ws = 0;
    };
    std::map<int64_t, Shape> shapes;  // by T
    void* ws = nullptr;
    size_t ws_bytes = 0;
};

namespace {

constexpr size_t kWorkspace = size_t(32) << 20;
constexpr int kCandidates = 16;

std::string blas_error(const char* what, hipblasStatus_t st) {
    return std::string(what) + ": hipBLASLt status " + std::to_string(static_cast<int>(st));
}

void clear_shapes(Linear* L) {
    for (auto& kv : L->shapes) {
        hipblasLtMatrixLayoutDestroy(kv.second.a);
        hipblasLtMatrixLayoutDestroy(kv.second.b);
        hipblasLtMatrixLayoutDestroy(kv.second.d);
    }
    L->shapes.clear();
}

}  // namespace

void linear_release(Linear* L) {
    if (!L) return;
    clear_shapes(L);
    if (L->desc) hipblasLtMatmulDescDestroy(L->desc);
    if (L->handle) hipblasLtDestroy(L->handle);
    if (L->ws) (void)hipFree(L->ws);
    delete L;
}

// out[T][N] = x[T][K] . w[N][K]^T (bf16, fp32 accumulation).  Returns false with *err set on a
// library or runtime error.
bool linear_bf16(Linear*& L, int64_t T, int64_t K, int64_t N, const void* x, const void* w,
                 void* out, hipStream_t stream, std::string* err) {
    if (!L) {
        L = new Linear();
        hipblasStatus_t st = hipblasLtCreate(&L->handle);
        if (st != HIPBLAS_STATUS_SUCCESS) { *err = blas_error("hipblasLtCreate", st); linear_release(L); L = nullptr; return false; }
        st = hipblasLtMatmulDescCreate(&L->desc, HIPBLAS_COMPUTE_32F, HIP_R_32F);
        if (st != HIPBLAS_STATUS_SUCCESS) { *err = blas_error("hipblasLtMatmulDescCreate", st); linear_release(L); L = nullptr; return false; }
        const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
        hipblasLtMatmulDescSetAttribute(L->desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta));
        hipblasLtMatmulDescSetAttribute(L->desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb));
        hipError_t e = hipMalloc(&L->ws, kWorkspace);
        if (e != hipSuccess) { *err = std::string("workspace: ") + hipGetErrorString(e); L->ws = nullptr; linear_release(L); L = nullptr; return false; }
        L->ws_bytes = kWorkspace;
    }
    if (K != L->K || N != L->N) {
        clear_shapes(L);
        L->K = K;
        L->N = N;
    }
    auto it = L->shapes.find(T);
    if (it == L->shapes.end()) {
        Linear::Shape s;
        hipblasStatus_t st = hipblasLtMatrixLayoutCreate(&s.a, HIP_R_16BF, K, N, K);
        if (st == HIPBLAS_STATUS_SUCCESS) st = hipblasLtMatrixLayoutCreate(&s.b, HIP_R_16BF, K, T, K);
        if (st == HIPBLAS_STATUS_SUCCESS) st = hipblasLtMatrixLayoutCreate(&s.d, HIP_R_16BF, N, T, N);
        hipblasLtMatmulPreference_t pref = nullptr;
        if (st == HIPBLAS_STATUS_SUCCESS) st = hipblasLtMatmulPreferenceCreate(&pref);
        const uint64_t cap = L->ws_bytes;
        if (st == HIPBLAS_STATUS_SUCCESS)
            st = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &cap, sizeof(cap));
        hipblasLtMatmulHeuristicResult_t res[kCandidates];
        int got = 0;
        if (st == HIPBLAS_STATUS_SUCCESS)
            st = hipblasLtMatmulAlgoGetHeuristic(L->handle, L->desc, s.a, s.b, s.d, s.d, pref, kCandidates, res, &got);
        if (pref) hipblasLtMatmulPreferenceDestroy(pref);
        if (st != HIPBLAS_STATUS_SUCCESS || got < 1) {
            *err = st != HIPBLAS_STATUS_SUCCESS ? blas_error("hipBLASLt plan", st)
                                                : std::string("hipBLASLt: no algorithm for this shape");
            if (s.a) hipblasLtMatrixLayoutDestroy(s.a);
            if (s.b) hipblasLtMatrixLayoutDestroy(s.b);
            if (s.d) hipblasLtMatrixLayoutDestroy(s.d);
            return false;
        }
        s.algo = res[0].algo;
        s.ws = res[0].workspaceSize;
        if (got > 1) {
            hipEvent_t e0 = nullptr, e1 = nullptr;
            if (hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess) {
                const float alpha = 1.0f, beta = 0.0f;
                float best = 1e30f;
                for (int i = 0; i < got; ++i) {
                    if (res[i].state != HIPBLAS_STATUS_SUCCESS || res[i].workspaceSize > L->ws_bytes) continue;
                    bool ok = true;
                    for (int r = 0; r < 2 && ok; ++r)  // warm-up
                        ok = hipblasLtMatmul(L->handle, L->desc, &alpha, w, s.a, x, s.b, &beta, out, s.d, out, s.d,
                                             &res[i].algo, L->ws, res[i].workspaceSize, stream) == HIPBLAS_STATUS_SUCCESS;
                    if (!ok) continue;
                    (void)hipEventRecord(e0, stream);
                    for (int r = 0; r < 5 && ok; ++r)
                        ok = hipblasLtMatmul(L->handle, L->desc, &alpha, w, s.a, x, s.b, &beta, out, s.d, out, s.d,
                                             &res[i].algo, L->ws, res[i].workspaceSize, stream) == HIPBLAS_STATUS_SUCCESS;
                    (void)hipEventRecord(e1, stream);
                    float ms = 0.0f;
                    if (!ok || hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&ms, e0, e1) != hipSuccess) continue;
                    if (ms < best) {
                        best = ms;
                        s.algo = res[i].algo;
                        s.ws = res[i].workspaceSize;
                    }
                }
            }
            if (e0) (void)hipEventDestroy(e0);
            if (e1) (void)hipEventDestroy(e1);
        }
        it = L->shapes.emplace(T, s).first;
    }
    const float alpha = 1.0f, beta = 0.0f;
    const Linear::Shape& s = it->second;
    const hipblasStatus_t st = hipblasLtMatmul(L->handle, L->desc, &alpha, w, s.a, x, s.b, &beta, out, s.d,
                                               out, s.d, &s.algo, L->ws, s.ws, stream);
    if (st != HIPBLAS_STATUS_SUCCESS) {
        *err = blas_error("hipblasLtMatmul", st);
        return false;
    }
    return true;
}

}  // namespace ca
