// Backward of the gated delta rule recurrence (fp32, d_k = d_v = 128): given dL/dy_t and dL/dS_final,
// the derivatives for q, k, v, alpha, beta and the initial state. The update statements are those of
// the analysis notes "Qwen3.8-Flash-Next：架构、效率与技术谱系" (§03 update equations); the reverse pass
// applies the chain rule to them last to first:
//   y_t = scale S_t^T q_t      ->  dS += scale q_t dy_t^T,  dq_t = scale S_t dy_t
//   S_t = S~ + beta k e^T      ->  dbeta = k^T dS e,  dk = beta dS e,  de = beta dS^T k
//   e = v - S~^T k             ->  dv = de,  dS~ = dS - k de^T,  dk -= S~ de
//   S~ = alpha S_{t-1}         ->  dalpha = <S_{t-1}, dS~>,  dS_{t-1} = alpha dS~
//
// One workgroup per (sequence, value head), 256 threads, each holding an 8x8 tile of the 128x128
// state: rows 8 ti .. 8 ti + 7, columns 8 tj .. 8 tj + 7 with ti = thread / 16, tj = thread % 16.
// Row sums (over a row's columns) are 16-lane shuffles; column sums (over a column's rows) are
// shuffles across the 4 row groups of a wave plus one LDS exchange across the 4 waves. A forward pass
// stores every state S_t (fp32, each thread's tile contiguous) and every error e_t in the workspace;
// the reverse pass reads them back, so every state it uses is the forward's own, with no inversion
// of the update.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kBD = 128;
constexpr int kBT = 256;  // threads per workgroup
constexpr int kTile = 64; // state entries per thread

struct BwdLds {
  float col[2][4][kBD];   // column-sum exchange, double-buffered by token parity
  float dal[2][4];        // per-wave dalpha partials, written one token and read at the next
};

// Column sums: part[c] is this thread's sum over its 8 rows for column 8 tj + c; returns the sum over
// all 128 rows in every thread of the column. One barrier.
__device__ __forceinline__ void col_sum(float (&part)[8], float (&full)[8], BwdLds& L, int buf) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, tj = t & 15;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    part[c] += __shfl_xor(part[c], 16, kWave);
    part[c] += __shfl_xor(part[c], 32, kWave);
  }
  if (lane < 16)
#pragma unroll
    for (int c = 0; c < 8; ++c) L.col[buf][w][8 * tj + c] = part[c];
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 8; ++c)
    full[c] = L.col[buf][0][8 * tj + c] + L.col[buf][1][8 * tj + c] + L.col[buf][2][8 * tj + c] +
              L.col[buf][3][8 * tj + c];
}

// Row sums over the 16 column tiles (16 consecutive lanes).
__device__ __forceinline__ float row_sum(float x) {
  x += __shfl_xor(x, 1, kWave);
  x += __shfl_xor(x, 2, kWave);
  x += __shfl_xor(x, 4, kWave);
  x += __shfl_xor(x, 8, kWave);
  return x;
}

__device__ __forceinline__ void ld8f(const float* p, float (&o)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

__device__ __forceinline__ void st8f(float* p, const float (&o)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(o[0], o[1], o[2], o[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(o[4], o[5], o[6], o[7]);
}

// A 128x128 fp32 matrix [row][col] <-> this thread's tile.
__device__ __forceinline__ void ld_tile_mat(const float* m, float (&s)[8][8], int ti, int tj) {
#pragma unroll
  for (int r = 0; r < 8; ++r) ld8f(m + (8 * ti + r) * kBD + 8 * tj, s[r]);
}
__device__ __forceinline__ void st_tile_mat(float* m, const float (&s)[8][8], int ti, int tj) {
#pragma unroll
  for (int r = 0; r < 8; ++r) st8f(m + (8 * ti + r) * kBD + 8 * tj, s[r]);
}
// Workspace copy of a state: each thread's 64 entries contiguous.
__device__ __forceinline__ void st_tile_ws(float* p, const float (&s)[8][8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) st8f(p + 8 * r, s[r]);
}
__device__ __forceinline__ void ld_tile_ws(const float* p, float (&s)[8][8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) ld8f(p + 8 * r, s[r]);
}

}  // namespace

__global__ void __launch_bounds__(kBT) k_bwd_d128(BwdArgs a) {
  __shared__ BwdLds L;
  const int t = threadIdx.x, ti = t >> 4, tj = t & 15;
  const int n = blockIdx.x / a.hv, h = blockIdx.x - n * a.hv, g = h * a.hk / a.hv;
  const int64_t s0 = min(max(int64_t(a.cu[n]), int64_t(0)), a.T);
  const int64_t s1 = min(max(int64_t(a.cu[n + 1]), s0), a.T);
  const int64_t HV = a.hv, HK = a.hk;

  float S[8][8];
  if (a.s0)
    ld_tile_mat(a.s0 + (int64_t(n) * HV + h) * kBD * kBD, S, ti, tj);
  else
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) S[r][c] = 0.f;

  // ---- forward: store S_t and e_t ----
  int buf = 0;
  for (int64_t tok = s0; tok < s1; ++tok, buf ^= 1) {
    float kr[8], vc[8], part[8], full[8];
    ld8f(a.k + (tok * HK + g) * kBD + 8 * ti, kr);
    ld8f(a.v + (tok * HV + h) * kBD + 8 * tj, vc);
    const float al = a.alpha[tok * HV + h], be = a.beta[tok * HV + h];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float acc = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r) acc = fmaf(S[r][c], kr[r], acc);
      part[c] = al * acc;  // (S~^T k) partial, S~ = alpha S
    }
    col_sum(part, full, L, buf);
    float e[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) e[c] = vc[c] - full[c];
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) S[r][c] = fmaf(be * kr[r], e[c], al * S[r][c]);
    st_tile_ws(a.states + ((tok * HV + h) * kBT + t) * kTile, S);
    if (ti == 0) st8f(a.errs + (tok * HV + h) * kBD + 8 * tj, e);
  }
  __threadfence();
  __syncthreads();

  // ---- reverse ----
  float dS[8][8];
  if (a.dsf)
    ld_tile_mat(a.dsf + (int64_t(n) * HV + h) * kBD * kBD, dS, ti, tj);
  else
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) dS[r][c] = 0.f;
  // S holds S_{s1-1} (the final state)
  int64_t pending = -1;  // token whose dalpha partials wait in L.dal[pbuf]
  int pbuf = 0;
  for (int64_t tok = s1 - 1; tok >= s0; --tok, buf ^= 1) {
    float P[8][8];  // S_{t-1}
    if (tok > s0)
      ld_tile_ws(a.states + (((tok - 1) * HV + h) * kBT + t) * kTile, P);
    else if (a.s0)
      ld_tile_mat(a.s0 + (int64_t(n) * HV + h) * kBD * kBD, P, ti, tj);
    else
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) P[r][c] = 0.f;
    float qr[8], kr[8], dyc[8], ec[8];
    ld8f(a.q + (tok * HK + g) * kBD + 8 * ti, qr);
    ld8f(a.k + (tok * HK + g) * kBD + 8 * ti, kr);
    ld8f(a.dy + (tok * HV + h) * kBD + 8 * tj, dyc);
    ld8f(a.errs + (tok * HV + h) * kBD + 8 * tj, ec);
    const float al = a.alpha[tok * HV + h], be = a.beta[tok * HV + h];
    // y_t = scale S_t^T q_t
    float dq[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        acc = fmaf(S[r][c], dyc[c], acc);
        dS[r][c] = fmaf(a.scale * qr[r], dyc[c], dS[r][c]);
      }
      dq[r] = a.scale * acc;
    }
    // de = beta dS^T k (column sums)
    float part[8], dsk[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float acc = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r) acc = fmaf(dS[r][c], kr[r], acc);
      part[c] = acc;
    }
    col_sum(part, dsk, L, buf);
    if (t == 0 && pending >= 0)
      a.dalpha[pending * HV + h] = L.dal[pbuf][0] + L.dal[pbuf][1] + L.dal[pbuf][2] + L.dal[pbuf][3];
    float de[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) de[c] = be * dsk[c];
    if (ti == 0) {
      float db = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) db = fmaf(dsk[c], ec[c], db);
      db = row_sum(db);
      if (t == 0) a.dbeta[tok * HV + h] = db;
      st8f(a.dv + (tok * HV + h) * kBD + 8 * tj, de);
    }
    // dk = beta dS e - alpha S_{t-1} de;  dS~ = dS - k de^T;  dalpha = <S_{t-1}, dS~>;  dS = alpha dS~
    float dk[8], dal = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float x = 0.f, y = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        x = fmaf(dS[r][c], ec[c], x);
        y = fmaf(P[r][c], de[c], y);
        const float dst = fmaf(-kr[r], de[c], dS[r][c]);
        dal = fmaf(P[r][c], dst, dal);
        dS[r][c] = al * dst;
      }
      dk[r] = be * x - al * y;
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      dq[r] = row_sum(dq[r]);
      dk[r] = row_sum(dk[r]);
    }
    if (tj == 0) {
      st8f(a.dqv + (tok * HV + h) * kBD + 8 * ti, dq);
      st8f(a.dkv + (tok * HV + h) * kBD + 8 * ti, dk);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) dal += __shfl_xor(dal, o, kWave);
    if ((t & 63) == 0) L.dal[buf][t >> 6] = dal;
    pending = tok;
    pbuf = buf;
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) S[r][c] = P[r][c];
  }
  __syncthreads();
  if (t == 0 && pending >= 0)
    a.dalpha[pending * HV + h] = L.dal[pbuf][0] + L.dal[pbuf][1] + L.dal[pbuf][2] + L.dal[pbuf][3];
  if (a.ds0) st_tile_mat(a.ds0 + (int64_t(n) * HV + h) * kBD * kBD, dS, ti, tj);
}

// dq, dk per QK head: the sum over the value heads that read it.
__global__ void __launch_bounds__(256) k_bwd_group_sum(int64_t T, int hk, int hv, const float* __restrict__ dqv,
                                                       const float* __restrict__ dkv, float* __restrict__ dq,
                                                       float* __restrict__ dk) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;  // over T * hk * 128
  if (i >= T * hk * kBD) return;
  const int64_t tok = i / (int64_t(hk) * kBD);
  const int rem = int(i - tok * hk * kBD), gq = rem / kBD, d = rem - gq * kBD;
  const int per = hv / hk;
  float sq = 0.f, sk = 0.f;
  for (int u = 0; u < per; ++u) {
    const int64_t j = (tok * hv + gq * per + u) * kBD + d;
    sq += dqv[j];
    sk += dkv[j];
  }
  dq[i] = sq;
  dk[i] = sk;
}

hipError_t launch_bwd(const BwdArgs& a, float* dq, float* dk, hipStream_t s) {
  if (a.n_seqs == 0) return hipSuccess;
  hipLaunchKernelGGL(k_bwd_d128, dim3(static_cast<unsigned>(a.n_seqs * a.hv)), dim3(kBT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.hv == a.hk || a.T == 0) return e;
  const int64_t n = a.T * a.hk * kBD;
  hipLaunchKernelGGL(k_bwd_group_sum, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, a.T, a.hk, a.hv,
                     a.dqv, a.dkv, dq, dk);
  return hipGetLastError();
}

}  // namespace gdn
