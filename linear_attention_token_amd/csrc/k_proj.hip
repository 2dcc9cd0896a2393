// The layer's projections around the mixer: input projection (q | k | v and the gate logits from
// one fused input matrix), the data-dependent decay and write gates, and the output projection.
//
// The paper reading "Qwen3.8-Flash-Next" (方法) sends the normalised residual stream through learned
// projections before the short conv, with a data-dependent decay gate and a write gate; the analysis
// notes "Qwen3.8-Flash-Next：架构、效率与技术谱系" (§07 optimizer table) describe the GDN input as one
// fused matrix of independent operators, 2-D input/output weights, and per-head alpha / beta
// vectors. The gate formula is not on the pages; the reading used here is
//     alpha = exp(-exp(A_h) softplus(a + delta_h)),   beta = sigmoid(b),
// with [a | b] = x W_ab and per-head vectors A, delta.
//
// The plain products (q | k | v, gate logits, output projection) are library GEMMs (hipBLASLt, bf16
// in, fp32 accumulate, bf16 out). The gate pre-activations must stay fp32 (alpha is steep in a), so
// they come from a kernel of their own that multiplies on bf16 MFMA with fp32 accumulation and
// applies the gate formula in the epilogue.
//
// Weights are in the linear-layer layout [out features][in features], row-major: every MFMA operand
// piece is then 16 consecutive bytes of a row.
#include <hipblaslt/hipblaslt.h>

#include <mutex>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kGateTok = 16;   // tokens per block of the gate kernel
constexpr int kGateWaves = 8;  // waves per block, each a slice of the k-steps
constexpr int kGateBatch = 5;  // k-steps whose operands a wave loads before multiplying any

// [a | b] = x W_ab^T for 16 tokens on 16x16x32 bf16 MFMA, NT column tiles of 16 (2 HV <= 16 NT).
// Wave w takes k-steps w, w + 8, ...; it loads kGateBatch steps of operands (its x piece and the NT
// weight pieces of each) before multiplying, so a block's whole reduction costs about two memory
// round trips; the eight partial tiles are summed in LDS, then the gates.
template <int NT>
__global__ void __launch_bounds__(64 * kGateWaves) k_gates(const uint16_t* __restrict__ x, int64_t ld_x, int64_t T,
                                                          int H, const uint16_t* __restrict__ w_ab, int hv,
                                                          const float* __restrict__ a_log,
                                                          const float* __restrict__ dt_bias,
                                                          float* __restrict__ alpha, float* __restrict__ beta) {
  __shared__ float part[kGateWaves][NT][16][16];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, li = lane & 15, lq = lane >> 4;
  const int64_t t0 = int64_t(blockIdx.x) * kGateTok;
  const int ncol = 2 * hv, nks = H / 32;
  const int64_t row = min(t0 + li, T - 1);  // rows past the end read the last row, not stored
  const uint16_t* xr = x + row * ld_x + 8 * lq;
  const uint16_t* wr[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) wr[j] = w_ab + int64_t(min(16 * j + li, ncol - 1)) * H + 8 * lq;
  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = w; s0 < nks; s0 += kGateWaves * kGateBatch) {
    short8 av[kGateBatch], bv[kGateBatch][NT];
#pragma unroll
    for (int u = 0; u < kGateBatch; ++u) {
      const int s = min(s0 + kGateWaves * u, nks - 1);  // clamped steps are loaded and not used
      av[u] = ld_short8(xr + 32 * s);
#pragma unroll
      for (int j = 0; j < NT; ++j) bv[u][j] = ld_short8(wr[j] + 32 * s);
    }
#pragma unroll
    for (int u = 0; u < kGateBatch; ++u)
      if (s0 + kGateWaves * u < nks) {
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j] = mfma16x16x32(av[u], bv[u][j], acc[j]);
      }
  }
  // acc[j][r]: token 4lq + r, column 16j + li
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) part[w][j][4 * lq + r][li] = acc[j][r];
  __syncthreads();
  for (int i = t; i < kGateTok * ncol; i += 64 * kGateWaves) {
    const int tok = i / ncol, col = i - tok * ncol;
    if (t0 + tok >= T) continue;
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < kGateWaves; ++ww) v += part[ww][col >> 4][tok][col & 15];
    if (col < hv) {
      const float u = v + dt_bias[col];
      const float sp = fmaxf(u, 0.f) + log1pf(__expf(-fabsf(u)));  // softplus without overflow
      alpha[(t0 + tok) * hv + col] = __expf(-__expf(a_log[col]) * sp);
    } else {
      beta[(t0 + tok) * hv + (col - hv)] = sigmoidf_(v);
    }
  }
}

// ---- hipBLASLt: D (M x N, column-major, ld ldd) = A^T B, A (K x M, ld lda), B (K x N, ld ldb); bf16
// in and out, fp32 accumulate. A row-major [rows][K] matrix is a column-major K x rows one, so with
// A = a weight [out][in] and B = activations [T][in] this is activations x weight^T, row-major
// [T][out]. One handle per device, and the heuristic's first algorithm cached per shape. ----
namespace {
struct GemmKey {
  int dev;
  int64_t M, N, K, lda, ldb, ldd;
  bool operator==(const GemmKey& o) const {
    return dev == o.dev && M == o.M && N == o.N && K == o.K && lda == o.lda && ldb == o.ldb && ldd == o.ldd;
  }
};
struct GemmEntry {
  GemmKey key;
  hipblasLtMatmulAlgo_t algo;
  size_t ws;
};
std::mutex g_mu;
hipblasLtHandle_t g_handle[64] = {};
GemmEntry g_cache[64];
int g_ncache = 0;
}  // namespace

hipError_t gemm_bf16_tn(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                        void* D, int64_t ldd, void* ws, size_t ws_bytes, hipStream_t s, const char** why) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) { *why = "device index out of range"; return hipErrorInvalidDevice; }
  hipblasLtMatmulDesc_t op = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
  hipblasLtMatmulAlgo_t algo;
  bool have = false;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_handle[dev] && hipblasLtCreate(&g_handle[dev]) != HIPBLAS_STATUS_SUCCESS) {
    g_handle[dev] = nullptr;
    *why = "hipblasLtCreate failed";
    return hipErrorUnknown;
  }
  const hipblasLtHandle_t h = g_handle[dev];
  const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
  hipblasStatus_t st = hipblasLtMatmulDescCreate(&op, HIPBLAS_COMPUTE_32F, HIP_R_32F);
  if (st == HIPBLAS_STATUS_SUCCESS)
    st = hipblasLtMatmulDescSetAttribute(op, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta));
  if (st == HIPBLAS_STATUS_SUCCESS)
    st = hipblasLtMatmulDescSetAttribute(op, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb));
  if (st == HIPBLAS_STATUS_SUCCESS) st = hipblasLtMatrixLayoutCreate(&la, HIP_R_16BF, K, M, lda);
  if (st == HIPBLAS_STATUS_SUCCESS) st = hipblasLtMatrixLayoutCreate(&lb, HIP_R_16BF, K, N, ldb);
  if (st == HIPBLAS_STATUS_SUCCESS) st = hipblasLtMatrixLayoutCreate(&ld, HIP_R_16BF, M, N, ldd);
  const GemmKey key{dev, M, N, K, lda, ldb, ldd};
  if (st == HIPBLAS_STATUS_SUCCESS) {
    for (int i = 0; i < g_ncache; ++i)
      if (g_cache[i].key == key && g_cache[i].ws <= ws_bytes) {
        algo = g_cache[i].algo;
        have = true;
      }
    if (!have) {
      hipblasLtMatmulPreference_t pref = nullptr;
      uint64_t cap = ws_bytes;
      constexpr int kCand = 8;
      hipblasLtMatmulHeuristicResult_t res[kCand];
      int n = 0;
      st = hipblasLtMatmulPreferenceCreate(&pref);
      if (st == HIPBLAS_STATUS_SUCCESS)
        st = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &cap, sizeof(cap));
      if (st == HIPBLAS_STATUS_SUCCESS)
        st = hipblasLtMatmulAlgoGetHeuristic(h, op, la, lb, ld, ld, pref, kCand, res, &n);
      if (pref) hipblasLtMatmulPreferenceDestroy(pref);
      // a returned entry is usable only if its own state is success (its other fields are
      // undefined otherwise) and its workspace fits the caller's
      int pick = -1;
      for (int i = 0; st == HIPBLAS_STATUS_SUCCESS && i < n && i < kCand && pick < 0; ++i)
        if (res[i].state == HIPBLAS_STATUS_SUCCESS && res[i].workspaceSize <= ws_bytes) pick = i;
      if (st == HIPBLAS_STATUS_SUCCESS && pick < 0) st = HIPBLAS_STATUS_NOT_SUPPORTED;
      if (st == HIPBLAS_STATUS_SUCCESS) {
        algo = res[pick].algo;
        have = true;
        if (g_ncache < 64) g_cache[g_ncache++] = GemmEntry{key, algo, res[pick].workspaceSize};
      }
    }
  }
  const float one = 1.f, zero = 0.f;
  if (st == HIPBLAS_STATUS_SUCCESS && have)
    st = hipblasLtMatmul(h, op, &one, A, la, B, lb, &zero, D, ld, D, ld, &algo, ws, ws_bytes, s);
  if (ld) hipblasLtMatrixLayoutDestroy(ld);
  if (lb) hipblasLtMatrixLayoutDestroy(lb);
  if (la) hipblasLtMatrixLayoutDestroy(la);
  if (op) hipblasLtMatmulDescDestroy(op);
  if (st != HIPBLAS_STATUS_SUCCESS) {
    *why = "hipBLASLt matmul failed";
    return hipErrorUnknown;
  }
  return hipGetLastError();
}

hipError_t launch_gates(const void* x, int64_t ld_x, int64_t T, int H, const void* w_ab, int hv, const float* a_log,
                        const float* dt_bias, float* alpha, float* beta, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid(unsigned((T + kGateTok - 1) / kGateTok)), block(64 * kGateWaves);
  const auto* xp = static_cast<const uint16_t*>(x);
  const auto* wp = static_cast<const uint16_t*>(w_ab);
  switch ((2 * hv + 15) / 16) {  // column tiles; hv <= 64 is checked by the caller
#define GDN_GATES(NT) \
  case NT: hipLaunchKernelGGL(k_gates<NT>, grid, block, 0, s, xp, ld_x, T, H, wp, hv, a_log, dt_bias, alpha, beta); break;
    GDN_GATES(1) GDN_GATES(2) GDN_GATES(3) GDN_GATES(4) GDN_GATES(5) GDN_GATES(6) GDN_GATES(7) GDN_GATES(8)
#undef GDN_GATES
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gdn
