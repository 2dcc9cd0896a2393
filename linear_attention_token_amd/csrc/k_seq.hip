// Token-sequential gated delta rule in fp32, fused with RMSNorm and the sigmoid gate.
//
// Serves every call the chunked bf16 MFMA path does not: fp32 io (which must stay within fp32
// accuracy) and head dims other than 128. One block per (sequence, value head); the fp32 state
// lives in registers for the whole sequence.
//
// Per token (analysis notes "Qwen3.8-Flash-Next：架构、效率与技术谱系" §03 update equations), in one
// pass over the old state S:
//   a = S^T k,  b = S^T q,  e = v - alpha a,  y = alpha b + beta (q.k) e,  S <- alpha S + beta k e^T
// which is S~ = alpha S; e = v - S~^T k; S = S~ + beta k e^T; y = S^T q rewritten so S is read once.
// Then zero-centred RMSNorm and the sigmoid gate (analysis notes §03; paper summary, Method).
//
// Thread layout: thread (rg, cg) owns columns 4cg..4cg+3 of the rows rg, rg + NRG, ... (NRG =
// 256 / (d_v / 4) row groups); partial column sums are combined through LDS.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kSeqThreads = 256;
constexpr int kSeqMaxRows = 16;  // rows of S per thread: d_k * d_v / 1024 <= 16 for d <= 128

struct SeqArgs {
  const int32_t* cu;
  int n_seqs;
  int64_t T;
  int hk, hv, dk, dv;
  const float *qhat, *khat, *vhat;  // fp32 work arrays [T][hk][dk], [T][hv][dv]
  const float *alpha, *beta;        // [T][hv]
  const void* gate;                 // io [T][hv][dv]
  const float* norm_w;
  int norm_stride;
  const float* state_in;
  float* state_out;
  void* out;                        // io [T][hv][dv]
  uint32_t flags;
  float scale, norm_eps;
};

template <typename IO>
__global__ void __launch_bounds__(kSeqThreads) k_sequential(SeqArgs a) {
  const int n = blockIdx.x, h = blockIdx.y;
  const int g = (h * a.hk) / a.hv;
  const int tid = threadIdx.x;
  const int ncg = a.dv / 4;           // column groups
  const int nrg = kSeqThreads / ncg;  // row groups
  const int cg = tid % ncg, rg = tid / ncg;
  const int col = 4 * cg;

  __shared__ float qs[128], ks[128], vs[128];
  __shared__ float red_a[kSeqThreads * 4], red_b[kSeqThreads * 4];
  __shared__ float qk_s;

  const int64_t s0 = min<int64_t>(max<int64_t>(a.cu[n], 0), a.T);
  const int64_t s1 = min<int64_t>(max<int64_t>(a.cu[n + 1], s0), a.T);
  const size_t sbase = (size_t(n) * a.hv + h) * size_t(a.dk) * a.dv;

  float S[kSeqMaxRows][4];
#pragma unroll
  for (int j = 0; j < kSeqMaxRows; ++j) {
    const int i = rg + j * nrg;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < a.dk && a.state_in != nullptr) v = *reinterpret_cast<const float4*>(a.state_in + sbase + size_t(i) * a.dv + col);
    S[j][0] = v.x; S[j][1] = v.y; S[j][2] = v.z; S[j][3] = v.w;
  }
  float w1[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    w1[e] = 1.0f + ((a.flags & GDN_NORM) ? a.norm_w[size_t(h) * a.norm_stride + col + e] : 0.f);

  for (int64_t t = s0; t < s1; ++t) {
    // stage q, k, v of this token
    if (tid < a.dk) {
      qs[tid] = a.qhat[(t * a.hk + g) * a.dk + tid];
      ks[tid] = a.khat[(t * a.hk + g) * a.dk + tid];
    }
    if (tid < a.dv) vs[tid] = a.vhat[(t * a.hv + h) * a.dv + tid];
    __syncthreads();
    if (tid < 64) {  // q . k by wave 0
      float p = 0.f;
      for (int i = tid; i < a.dk; i += 64) p += qs[i] * ks[i];
      p = group_sum<64>(p);
      if (tid == 0) qk_s = p;
    }
    float pa[4] = {0.f, 0.f, 0.f, 0.f}, pb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kSeqMaxRows; ++j) {
      const int i = rg + j * nrg;
      if (i < a.dk) {
        const float ki = ks[i], qi = qs[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) { pa[e] += S[j][e] * ki; pb[e] += S[j][e] * qi; }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) { red_a[rg * a.dv + col + e] = pa[e]; red_b[rg * a.dv + col + e] = pb[e]; }
    __syncthreads();
    const int nr = min(nrg, a.dk);
    float av[4] = {0.f, 0.f, 0.f, 0.f}, bv[4] = {0.f, 0.f, 0.f, 0.f};
    for (int r = 0; r < nr; ++r) {
#pragma unroll
      for (int e = 0; e < 4; ++e) { av[e] += red_a[r * a.dv + col + e]; bv[e] += red_b[r * a.dv + col + e]; }
    }
    const float al = a.alpha[t * a.hv + h], be = a.beta[t * a.hv + h];
    const float qk = qk_s;
    float ev[4], y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ev[e] = vs[col + e] - al * av[e];
      y[e] = a.scale * (al * bv[e] + be * qk * ev[e]);
    }
#pragma unroll
    for (int j = 0; j < kSeqMaxRows; ++j) {
      const int i = rg + j * nrg;
      if (i < a.dk) {
        const float bk = be * ks[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) S[j][e] = al * S[j][e] + bk * ev[e];
      }
    }
    // RMSNorm over d_v: every group of ncg consecutive lanes covers all d_v columns once
    float ss = y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3];
    for (int o = ncg >> 1; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
    if (rg == 0) {
      float o4[4];
      const float rs = (a.flags & GDN_NORM) ? 1.0f / sqrtf(ss / float(a.dv) + a.norm_eps) : 1.0f;
      const IO* gp = static_cast<const IO*>(a.gate) + (t * a.hv + h) * a.dv + col;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float o = y[e];
        if (a.flags & GDN_NORM) o = o * rs * w1[e];
        if (a.flags & GDN_GATE) o *= sigmoidf_(io<IO>::ld(gp + e));
        o4[e] = o;
      }
      IO* op = static_cast<IO*>(a.out) + (t * a.hv + h) * a.dv + col;
#pragma unroll
      for (int e = 0; e < 4; ++e) io<IO>::st(op + e, o4[e]);
    }
    __syncthreads();
  }
  if (a.state_out != nullptr) {
#pragma unroll
    for (int j = 0; j < kSeqMaxRows; ++j) {
      const int i = rg + j * nrg;
      if (i < a.dk)
        *reinterpret_cast<float4*>(a.state_out + sbase + size_t(i) * a.dv + col) = make_float4(S[j][0], S[j][1], S[j][2], S[j][3]);
    }
  }
}

hipError_t launch_sequential(const Problem& p, const int32_t* cu, const Workspace& ws,
                             const float* alpha, const float* beta, const void* gate,
                             const float* norm_w, const float* state_in, float* state_out, void* out,
                             hipStream_t s) {
  if (p.n_seqs == 0) return hipSuccess;
  SeqArgs a{cu, p.n_seqs, p.T, p.hk, p.hv, p.dk, p.dv,
            static_cast<const float*>(ws.qhat), static_cast<const float*>(ws.khat),
            static_cast<const float*>(ws.vhat), alpha, beta, gate, norm_w, p.norm_stride,
            state_in, state_out, out, p.flags, p.scale, p.norm_eps};
  dim3 grid(unsigned(p.n_seqs), unsigned(p.hv));
  if (p.bf16) hipLaunchKernelGGL(k_sequential<bf16>, grid, dim3(kSeqThreads), 0, s, a);
  else hipLaunchKernelGGL(k_sequential<float>, grid, dim3(kSeqThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace gdn
