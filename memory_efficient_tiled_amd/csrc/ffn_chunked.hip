// ffn_chunked.hip -- the transformer feed-forward block over chunks of token
// rows, y = W2 gelu(W1 x + b1) + b2 (FFN chunking: the English
// noflash-attention post, section "The DIY approach", lists it with a
// runtime safety check as its second memory saver).  Per chunk of C rows:
//   H = X_c W1^T          hipBLASLt GEMM into a C x F workspace (fp32 acc.)
//   H = gelu(H + b1)      this file's kernel, in place, 8 elements a thread
//   Y_c = H W2^T          hipBLASLt GEMM into the output rows
//   Y_c += b2             this file's kernel
// so the N x F activation never exists.  Both products are plain GEMMs, the
// library's job on the matrix cores; the elementwise steps are HBM-bound
// passes over the chunk.

#include "attn_common.h"
#include "ffn.h"

#include <hipblaslt/hipblaslt.h>

#include <mutex>

namespace {

constexpr size_t kGemmWorkspace = 128u << 20;  // hipBLASLt workspace per call
constexpr int kAlgos = 16;                      // heuristic candidates examined
// Default chunk: the rows whose hidden activation fits 96 MiB, rounded down
// to a multiple of 1024 rows (at width 5120 / hidden 13824 that is 3072
// rows, where hipBLASLt's products ran at 51% of the bf16 peak against 42%
// at 4864 rows).
constexpr size_t kHiddenBudget = 96u << 20;

__device__ __forceinline__ float gelu_tanh(float a) {
  return 0.5f * a * (1.f + tanhf(0.7978845608028654f * (a + 0.044715f * a * a * a)));
}

// h = gelu(h + b1) over a [rows, F] matrix, 8 elements per thread.
template <class Tag>
__global__ __launch_bounds__(256) void ffn_bias_gelu(uint16_t* h, const uint16_t* b1, size_t n8,
                                                     int f8) {
  using N = Num<Tag>;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  u32x4 v = ((const u32x4*)h)[i];
  u32x4 b = {0u, 0u, 0u, 0u};
  if (b1) b = ((const u32x4*)b1)[i % f8];
#pragma unroll
  for (int w = 0; w < 4; ++w)
    v[w] = N::pack2(gelu_tanh(lo_f32<Tag>(v[w]) + lo_f32<Tag>(b[w])),
                    gelu_tanh(hi_f32<Tag>(v[w]) + hi_f32<Tag>(b[w])));
  ((u32x4*)h)[i] = v;
}

// y += b2 over a [rows, Dm] matrix, 8 elements per thread.
template <class Tag>
__global__ __launch_bounds__(256) void ffn_bias_add(uint16_t* y, const uint16_t* b2, size_t n8,
                                                    int d8) {
  using N = Num<Tag>;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  u32x4 v = ((const u32x4*)y)[i];
  const u32x4 b = ((const u32x4*)b2)[i % d8];
#pragma unroll
  for (int w = 0; w < 4; ++w)
    v[w] = N::pack2(lo_f32<Tag>(v[w]) + lo_f32<Tag>(b[w]), hi_f32<Tag>(v[w]) + hi_f32<Tag>(b[w]));
  ((u32x4*)y)[i] = v;
}

// Per workgroup: max |a - b| and max |b| over its slice of n values, into
// part[2 * blockIdx.x + {0, 1}] (no atomics); ffn_max_final folds them.  A
// NaN difference or output counts as +inf (fmaxf alone would drop it), so
// any non-finite value in either evaluation makes a result infinite.
__device__ __forceinline__ float max_keep_nan(float acc, float x) {
  return x == x ? fmaxf(acc, x) : INFINITY;
}

template <class Tag>
__global__ __launch_bounds__(256) void ffn_max_diff(const uint16_t* a, const uint16_t* b, size_t n,
                                                    float* part) {
  __shared__ float sd[256], sr[256];
  float d = 0.f, r = 0.f;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const uint32_t x = a[i], y = b[i];
    const float fx = lo_f32<Tag>(x), fy = lo_f32<Tag>(y);
    d = max_keep_nan(d, fabsf(fx - fy));
    r = max_keep_nan(r, fabsf(fy));
  }
  sd[threadIdx.x] = d;
  sr[threadIdx.x] = r;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
      sd[threadIdx.x] = fmaxf(sd[threadIdx.x], sd[threadIdx.x + s]);
      sr[threadIdx.x] = fmaxf(sr[threadIdx.x], sr[threadIdx.x + s]);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    part[2 * blockIdx.x] = sd[0];
    part[2 * blockIdx.x + 1] = sr[0];
  }
}

__global__ __launch_bounds__(256) void ffn_max_final(const float* part, int nparts, float* out) {
  __shared__ float sd[256], sr[256];
  float d = 0.f, r = 0.f;
  for (int i = threadIdx.x; i < nparts; i += 256) {
    d = fmaxf(d, part[2 * i]);
    r = fmaxf(r, part[2 * i + 1]);
  }
  sd[threadIdx.x] = d;
  sr[threadIdx.x] = r;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
      sd[threadIdx.x] = fmaxf(sd[threadIdx.x], sd[threadIdx.x + s]);
      sr[threadIdx.x] = fmaxf(sr[threadIdx.x], sr[threadIdx.x + s]);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    out[0] = sd[0];
    out[1] = sr[0];
  }
}

// One hipBLASLt handle per device, created on first use.
std::mutex g_lt_mu;
hipblasLtHandle_t g_lt[64] = {};

int lt_handle(hipblasLtHandle_t* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return ATTN_EHIP;
  std::lock_guard<std::mutex> lk(g_lt_mu);
  if (!g_lt[dev] && hipblasLtCreate(&g_lt[dev]) != HIPBLAS_STATUS_SUCCESS) {
    g_lt[dev] = nullptr;
    return ATTN_EHIP;
  }
  *out = g_lt[dev];
  return ATTN_OK;
}

// out [rows, M] = epi(x [rows, K] w [M, K]^T), all row-major 16-bit.  In
// hipBLASLt's column-major terms: out^T (M x rows) = op(W^T) X^T with the
// weight as a K x M matrix read transposed.  epi adds `bias` ([M], the
// input type; NULL for none) and, with `gelu`, applies hipBLASLt's GELU to
// the fp32 accumulator before the single rounding to 16 bits.  With
// `fused_only` the call returns ATTN_EUNSUPPORTED when hipBLASLt offers no
// algorithm for that epilogue (the caller then runs the plain product and
// its own elementwise kernel).
int gemm_xwt(hipblasLtHandle_t h, void* out, const void* x, const void* w, int rows, int M, int K,
             hipDataType t, void* ws, hipStream_t st, const void* bias = nullptr,
             bool gelu = false, bool fused_only = false) {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
  hipblasLtMatmulPreference_t pref = nullptr;
  int rc = ATTN_EHIP;
  const hipblasOperation_t opT = HIPBLAS_OP_T, opN = HIPBLAS_OP_N;
  const uint64_t wsb = kGemmWorkspace;
  hipblasLtMatmulHeuristicResult_t res[kAlgos];
  int got = 0, pick = -1;
  const float alpha = 1.f, beta = 0.f;
  if (hipblasLtMatmulDescCreate(&desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS)
    goto done;
  if (hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opT, sizeof(opT)) !=
          HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opN, sizeof(opN)) !=
          HIPBLAS_STATUS_SUCCESS)
    goto done;
  if (bias || gelu) {
    const uint32_t epi = gelu ? (bias ? HIPBLASLT_EPILOGUE_GELU_BIAS : HIPBLASLT_EPILOGUE_GELU)
                              : HIPBLASLT_EPILOGUE_BIAS;
    const int32_t bt = (int32_t)t;
    if (hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_EPILOGUE, &epi, sizeof(epi)) !=
        HIPBLAS_STATUS_SUCCESS)
      goto done;
    if (bias && (hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias,
                                                 sizeof(bias)) != HIPBLAS_STATUS_SUCCESS ||
                 hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_BIAS_DATA_TYPE, &bt,
                                                 sizeof(bt)) != HIPBLAS_STATUS_SUCCESS))
      goto done;
  }
  if (hipblasLtMatrixLayoutCreate(&la, t, K, M, K) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&lb, t, K, rows, K) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&lc, t, M, rows, M) != HIPBLAS_STATUS_SUCCESS)
    goto done;
  if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb,
                                            sizeof(wsb)) != HIPBLAS_STATUS_SUCCESS)
    goto done;
  if (hipblasLtMatmulAlgoGetHeuristic(h, desc, la, lb, lc, lc, pref, kAlgos, res, &got) !=
      HIPBLAS_STATUS_SUCCESS)
    got = 0;
  // the first candidate whose own workspace requirement fits the buffer,
  // run with exactly that workspace size
  for (int i = 0; i < got && i < kAlgos && pick < 0; ++i)
    if (res[i].state == HIPBLAS_STATUS_SUCCESS && res[i].workspaceSize <= kGemmWorkspace) pick = i;
  if (pick < 0) {
    if (fused_only) rc = ATTN_EUNSUPPORTED;
    goto done;
  }
  if (hipblasLtMatmul(h, desc, &alpha, w, la, x, lb, &beta, out, lc, out, lc, &res[pick].algo,
                      res[pick].workspaceSize ? ws : nullptr, res[pick].workspaceSize,
                      st) != HIPBLAS_STATUS_SUCCESS)
    goto done;
  rc = ATTN_OK;
done:
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (lc) hipblasLtMatrixLayoutDestroy(lc);
  if (lb) hipblasLtMatrixLayoutDestroy(lb);
  if (la) hipblasLtMatrixLayoutDestroy(la);
  if (desc) hipblasLtMatmulDescDestroy(desc);
  return rc;
}

bool overlaps_ffn(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

int validate_ffn(const void* x, const void* w1, const void* b1, const void* w2, const void* b2,
                 const void* y, int N, int Dm, int F, int act, int chunk_rows, int dtype) {
  if (N <= 0 || Dm <= 0 || F <= 0 || chunk_rows < 0) return ATTN_EINVAL;
  if ((Dm & 7) || (F & 7)) return ATTN_EINVAL;
  if (act != FFN_GELU_TANH) return ATTN_EINVAL;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_EINVAL;
  if (!x || !w1 || !w2) return ATTN_EINVAL;
  if (((uintptr_t)x | (uintptr_t)w1 | (uintptr_t)w2 | (uintptr_t)b1 | (uintptr_t)b2 |
       (uintptr_t)y) & 15)
    return ATTN_EINVAL;
  if ((long long)N * Dm > (1LL << 40) || (long long)Dm * F > (1LL << 40)) return ATTN_EINVAL;
  if (y) {
    const size_t yb = (size_t)N * Dm * 2, xb = yb, wb = (size_t)F * Dm * 2;
    if (overlaps_ffn(y, yb, x, xb) || overlaps_ffn(y, yb, w1, wb) || overlaps_ffn(y, yb, w2, wb) ||
        (b1 && overlaps_ffn(y, yb, b1, (size_t)F * 2)) ||
        (b2 && overlaps_ffn(y, yb, b2, (size_t)Dm * 2)))
      return ATTN_EINVAL;
  }
  return ATTN_OK;
}

int default_chunk(int N, int F) {
  long long c = (long long)(kHiddenBudget / ((size_t)F * 2)) / 1024 * 1024;
  if (c < 1024) c = 1024;
  return (int)(c < N ? c : N);
}

size_t hidden_bytes(int chunk, int F) { return ((size_t)chunk * F * 2 + 255) / 256 * 256; }

// The block on rows [0, N) of x into y, chunk rows at a time, using the
// workspace ws (hidden_bytes(chunk, F) + kGemmWorkspace bytes).
int run_chunks(hipblasLtHandle_t h, const void* x, const void* w1, const void* b1, const void* w2,
               const void* b2, void* y, int N, int Dm, int F, int chunk, bool bf16, void* ws,
               hipStream_t st) {
  const hipDataType t = bf16 ? HIP_R_16BF : HIP_R_16F;
  uint16_t* hid = (uint16_t*)ws;
  void* gws = (char*)ws + hidden_bytes(chunk, F);
  for (int r0 = 0; r0 < N; r0 += chunk) {
    const int rows = N - r0 < chunk ? N - r0 : chunk;
    const uint16_t* xc = (const uint16_t*)x + (size_t)r0 * Dm;
    uint16_t* yc = (uint16_t*)y + (size_t)r0 * Dm;
    // H = gelu(X W1^T + b1): in the product's epilogue where hipBLASLt
    // offers one for the shape, else the product and this file's kernel
    int rc = gemm_xwt(h, hid, xc, w1, rows, F, Dm, t, gws, st, b1, true, true);
    if (rc == ATTN_EUNSUPPORTED) {
      rc = gemm_xwt(h, hid, xc, w1, rows, F, Dm, t, gws, st);
      if (rc != ATTN_OK) return rc;
      const size_t n8 = (size_t)rows * F / 8;
      const unsigned g1 = (unsigned)((n8 + 255) / 256);
      if (bf16)
        hipLaunchKernelGGL(ffn_bias_gelu<TagBF16>, dim3(g1), dim3(256), 0, st, hid,
                           (const uint16_t*)b1, n8, F / 8);
      else
        hipLaunchKernelGGL(ffn_bias_gelu<TagF16>, dim3(g1), dim3(256), 0, st, hid,
                           (const uint16_t*)b1, n8, F / 8);
      if (hipGetLastError() != hipSuccess) return ATTN_EHIP;
    } else if (rc != ATTN_OK) {
      return rc;
    }
    // Y = H W2^T + b2, likewise
    rc = b2 ? gemm_xwt(h, yc, hid, w2, rows, Dm, F, t, gws, st, b2, false, true)
            : ATTN_EUNSUPPORTED;
    if (rc == ATTN_OK) continue;
    if (rc != ATTN_EUNSUPPORTED) return rc;
    rc = gemm_xwt(h, yc, hid, w2, rows, Dm, F, t, gws, st);
    if (rc != ATTN_OK) return rc;
    if (b2) {
      const size_t m8 = (size_t)rows * Dm / 8;
      const unsigned g2 = (unsigned)((m8 + 255) / 256);
      if (bf16)
        hipLaunchKernelGGL(ffn_bias_add<TagBF16>, dim3(g2), dim3(256), 0, st, yc,
                           (const uint16_t*)b2, m8, Dm / 8);
      else
        hipLaunchKernelGGL(ffn_bias_add<TagF16>, dim3(g2), dim3(256), 0, st, yc,
                           (const uint16_t*)b2, m8, Dm / 8);
      if (hipGetLastError() != hipSuccess) return ATTN_EHIP;
    }
  }
  return ATTN_OK;
}

}  // namespace

extern "C" {

int ffn_chunked_check(const void* x, const void* w1, const void* b1, const void* w2,
                      const void* b2, const void* y, int N, int Dm, int F, int act,
                      int chunk_rows, int dtype) {
  if (!y) return ATTN_EINVAL;
  return validate_ffn(x, w1, b1, w2, b2, y, N, Dm, F, act, chunk_rows, dtype);
}

size_t ffn_workspace_bytes(int chunk_rows, int F, int Dm, int dtype) {
  (void)Dm;
  if (chunk_rows <= 0 || F <= 0 || (dtype != ATTN_F16 && dtype != ATTN_BF16)) return 0;
  return hidden_bytes(chunk_rows, F) + kGemmWorkspace;
}

int ffn_chunked(const void* x, const void* w1, const void* b1, const void* w2, const void* b2,
                void* y, int N, int Dm, int F, int act, int chunk_rows, int dtype,
                void* stream) {
  int rc = ffn_chunked_check(x, w1, b1, w2, b2, y, N, Dm, F, act, chunk_rows, dtype);
  if (rc != ATTN_OK) return rc;
  rc = attn_host::check_device(nullptr);
  if (rc != ATTN_OK) return rc;
  hipblasLtHandle_t h;
  rc = lt_handle(&h);
  if (rc != ATTN_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  const int chunk = chunk_rows > 0 ? (chunk_rows < N ? chunk_rows : N) : default_chunk(N, F);
  void* ws = nullptr;
  hipError_t e = attn_host::workspace_alloc(&ws, hidden_bytes(chunk, F) + kGemmWorkspace, st);
  if (e != hipSuccess || !ws) {
    attn_host::set_last_hip_error((int)e);
    (void)hipGetLastError();
    return ATTN_ENOMEM;
  }
  rc = run_chunks(h, x, w1, b1, w2, b2, y, N, Dm, F, chunk, dtype == ATTN_BF16, ws, st);
  const hipError_t ef = hipFreeAsync(ws, st);
  if (rc == ATTN_OK && ef != hipSuccess) {
    attn_host::set_last_hip_error((int)ef);
    rc = ATTN_EHIP;
  }
  return rc;
}

int ffn_verify(const void* x, const void* w1, const void* b1, const void* w2, const void* b2,
               int N, int Dm, int F, int act, int chunk_rows, int dtype, float* max_abs_diff,
               float* max_abs_ref, void* stream) {
  if (!max_abs_diff || !max_abs_ref) return ATTN_EINVAL;
  int rc = validate_ffn(x, w1, b1, w2, b2, nullptr, N, Dm, F, act, chunk_rows, dtype);
  if (rc != ATTN_OK) return rc;
  rc = attn_host::check_device(nullptr);
  if (rc != ATTN_OK) return rc;
  hipblasLtHandle_t h;
  rc = lt_handle(&h);
  if (rc != ATTN_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  const int chunk = chunk_rows > 0 ? (chunk_rows < N ? chunk_rows : N) : default_chunk(N, F);
  const long long r_ll = 2LL * chunk + 1 < N ? 2LL * chunk + 1 : N;
  const int R = (int)r_ll;
  const size_t yb = ((size_t)R * Dm * 2 + 255) / 256 * 256;
  constexpr int kParts = 256;
  const size_t wsb = hidden_bytes(R, F) + kGemmWorkspace;  // enough for either chunking
  void* ws = nullptr;
  hipError_t e = attn_host::workspace_alloc(&ws, wsb + 2 * yb + (2 * kParts + 2) * sizeof(float), st);
  if (e != hipSuccess || !ws) {
    attn_host::set_last_hip_error((int)e);
    (void)hipGetLastError();
    return ATTN_ENOMEM;
  }
  uint16_t* ya = (uint16_t*)((char*)ws + wsb);
  uint16_t* yr = (uint16_t*)((char*)ya + yb);
  float* part = (float*)((char*)yr + yb);
  float* res = part + 2 * kParts;
  const bool bf16 = dtype == ATTN_BF16;
  rc = run_chunks(h, x, w1, b1, w2, b2, ya, R, Dm, F, chunk, bf16, ws, st);
  if (rc == ATTN_OK) rc = run_chunks(h, x, w1, b1, w2, b2, yr, R, Dm, F, R, bf16, ws, st);
  float hres[2] = {0.f, 0.f};
  if (rc == ATTN_OK) {
    const size_t n = (size_t)R * Dm;
    if (bf16)
      hipLaunchKernelGGL(ffn_max_diff<TagBF16>, dim3(kParts), dim3(256), 0, st, ya, yr, n, part);
    else
      hipLaunchKernelGGL(ffn_max_diff<TagF16>, dim3(kParts), dim3(256), 0, st, ya, yr, n, part);
    hipLaunchKernelGGL(ffn_max_final, dim3(1), dim3(256), 0, st, part, kParts, res);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpyAsync(hres, res, sizeof(hres), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
      attn_host::set_last_hip_error((int)e);
      rc = ATTN_EHIP;
    }
  }
  const hipError_t ef = hipFreeAsync(ws, st);
  if (rc == ATTN_OK && ef != hipSuccess) {
    attn_host::set_last_hip_error((int)ef);
    rc = ATTN_EHIP;
  }
  *max_abs_diff = hres[0];
  *max_abs_ref = hres[1];
  return rc;
}

}  // extern "C"
