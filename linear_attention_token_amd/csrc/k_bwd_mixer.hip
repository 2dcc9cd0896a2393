// Backward of the mixer's steps around the recurrence (fp32, d = 128), for gdn_backward:
//   k_norm_gate_bwd   o = n * sigmoid(z), n = y / r * (1 + w), r = sqrt(mean(y^2) + eps):
//                     dz = do * n * s (1 - s);  dn = do * s;  dw = sum of dn * y / r (per-block parts, then
//                     k_sum_parts);
//                     dy = (1 + w) dn / r - y <(1 + w) dn, y> / (128 r^3)
//   k_l2silu_bwd      a = a0 / sqrt(|a0|^2 + eps) (q, k heads), a0 = silu(u), u the conv output:
//                     da0 = (da - a <a, da>) / sqrt(|a0|^2 + eps);  du = da0 sigmoid(u) (1 + u (1 - sigmoid(u)))
//   k_conv_bwd        u[t] = sum_j w[j] x[t - 3 + j]:  dx[t] = sum_j w[j] du[t + 3 - j] (inside the sequence),
//                     dw[j] = sum_t du[t] x[t - 3 + j] (x[-3..-1] = the conv history; per 64-token block
//                     parts, then k_conv_w_sum)
//   k_conv_in_bwd     d history[r] = sum_j w[j] du[r - j] (r = 0..2 for positions -3..-1)
// (the steps of the paper reading "On the Design of Qwen3.8-Next Architecture … 精读" §四 4.1 and the
// analysis notes "Qwen3.8-Flash-Next：架构、效率与技术谱系" §03, differentiated).
#include "gdn_device.h"
#include "ext_internal.h"

namespace gdn {

namespace {
constexpr int kD = 128;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

// Sequence of packed row `row`: the largest n with cu[n] <= row.
__device__ __forceinline__ int seq_of(const int32_t* cu, int n_seqs, int64_t row) {
  int lo = 0, hi = n_seqs;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (int64_t(cu[mid]) <= row) lo = mid; else hi = mid;
  }
  return lo;
}
}  // namespace

__global__ void __launch_bounds__(256) k_zero(float* __restrict__ p, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// One wave per (token, value head) row, lanes holding channels lane and lane + 64; 16 rows per wave.
__global__ void __launch_bounds__(256) k_norm_gate_bwd(int64_t rows, const float* __restrict__ y,
                                                       const float* __restrict__ z, const float* __restrict__ dout,
                                                       const float* __restrict__ norm_w, float eps,
                                                       float* __restrict__ dy, float* __restrict__ dz,
                                                       float* __restrict__ dw_part) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const float w0 = 1.f + norm_w[lane], w1 = 1.f + norm_w[lane + 64];
  float dw0 = 0.f, dw1 = 0.f;
  for (int i = 0; i < 16; ++i) {
    const int64_t row = (int64_t(blockIdx.x) * 4 + w) * 16 + i;
    if (row >= rows) break;
    const int64_t b = row * kD;
    const float y0 = y[b + lane], y1 = y[b + lane + 64];
    const float r = sqrtf(wave_sum(y0 * y0 + y1 * y1) * (1.f / kD) + eps), ir = 1.f / r;
    const float s0 = 1.f / (1.f + __expf(-z[b + lane])), s1 = 1.f / (1.f + __expf(-z[b + lane + 64]));
    const float do0 = dout[b + lane], do1 = dout[b + lane + 64];
    const float n0 = y0 * ir * w0, n1 = y1 * ir * w1;
    dz[b + lane] = do0 * n0 * s0 * (1.f - s0);
    dz[b + lane + 64] = do1 * n1 * s1 * (1.f - s1);
    const float dn0 = do0 * s0, dn1 = do1 * s1;
    dw0 = fmaf(dn0 * y0, ir, dw0);
    dw1 = fmaf(dn1 * y1, ir, dw1);
    const float g0 = w0 * dn0, g1 = w1 * dn1;
    const float dot = wave_sum(g0 * y0 + g1 * y1) * ir * ir * ir * (1.f / kD);
    dy[b + lane] = g0 * ir - y0 * dot;
    dy[b + lane + 64] = g1 * ir - y1 * dot;
  }
  // this block's part of the norm gain's derivative: the waves' sums, then one row of dw_part
  __shared__ float red[4][kD];
  red[w][lane] = dw0;
  red[w][lane + 64] = dw1;
  __syncthreads();
  if (threadIdx.x < kD)
    dw_part[int64_t(blockIdx.x) * kD + threadIdx.x] =
        red[0][threadIdx.x] + red[1][threadIdx.x] + red[2][threadIdx.x] + red[3][threadIdx.x];
}

// dnorm_w[c] = sum over the blocks' rows of dw_part: 8 groups of 128 threads take every eighth row, then
// the 8 group sums are added in a fixed order (reproducible).
__global__ void __launch_bounds__(1024) k_sum_parts(const float* __restrict__ part, int64_t nblocks,
                                                    float* __restrict__ out) {
  __shared__ float red[8][kD];
  const int c = threadIdx.x & (kD - 1), grp = threadIdx.x >> 7;
  float acc = 0.f;
#pragma unroll 8
  for (int64_t b = grp; b < nblocks; b += 8) acc += part[b * kD + c];
  red[grp][c] = acc;
  __syncthreads();
  if (threadIdx.x < kD) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += red[i][c];
    out[c] = s;
  }
}

// Conv output of channel c at packed token t (sequence n starting at s0): sum_j w[j] x[t - 3 + j] with the
// history for positions before s0.
__device__ __forceinline__ float conv_at(const float* x, int64_t ld_x, int64_t col, const float* w4, int64_t t,
                                         int64_t s0, const float* hist, int64_t C, int64_t c) {
  float u = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t p = t - 3 + j;
    const float xv = p >= s0 ? x[p * ld_x + col] : (hist ? hist[(p - s0 + 3) * C + c] : 0.f);
    u = fmaf(w4[j], xv, u);
  }
  return u;
}

// One wave per (token, head) of q, k (L2 and SiLU) or v (SiLU): du into [T][C].
__global__ void __launch_bounds__(256) k_l2silu_bwd(BwdMixArgs m) {
  const int lane = threadIdx.x & 63;
  const int64_t item = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int heads = 2 * m.hk + m.hv;
  if (item >= m.T * heads) return;
  const int64_t t = item / heads;
  const int hd = int(item - t * heads);
  const int n = seq_of(m.cu, m.n_seqs, t);
  const int64_t s0 = m.cu[n];
  const float* hist = m.conv_in ? m.conv_in + int64_t(n) * 3 * m.C : nullptr;
  const float* x;
  int64_t ld, col0;
  const float* da;
  bool l2 = true;
  if (hd < m.hk) {
    x = m.q; ld = int64_t(m.hk) * kD; col0 = int64_t(hd) * kD;
    da = m.dqa + (t * m.hk + hd) * kD;
  } else if (hd < 2 * m.hk) {
    x = m.k; ld = int64_t(m.hk) * kD; col0 = int64_t(hd - m.hk) * kD;
    da = m.dka + (t * m.hk + hd - m.hk) * kD;
  } else {
    x = m.v; ld = int64_t(m.hv) * kD; col0 = int64_t(hd - 2 * m.hk) * kD;
    da = m.dva + (t * m.hv + hd - 2 * m.hk) * kD;
    l2 = false;
  }
  const int64_t cbase = int64_t(hd) * kD;  // conv channel of the head's first dim (q | k | v order)
  float u[2], a0[2], g[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int d = lane + 64 * i;
    const int64_t c = cbase + d;
    u[i] = conv_at(x, ld, col0 + d, m.conv_w + c * 4, t, s0, hist, m.C, c);
    const float sg = 1.f / (1.f + __expf(-u[i]));
    a0[i] = u[i] * sg;
    g[i] = da[d];
    u[i] = sg * (1.f + u[i] * (1.f - sg));  // silu'(u), kept in u
  }
  if (l2) {
    const float inv = 1.f / sqrtf(wave_sum(a0[0] * a0[0] + a0[1] * a0[1]) + m.l2_eps);
    const float adot = wave_sum(a0[0] * g[0] + a0[1] * g[1]) * inv;  // <a, da> with a = a0 inv
#pragma unroll
    for (int i = 0; i < 2; ++i) g[i] = (g[i] - a0[i] * inv * adot) * inv;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) m.du[t * m.C + cbase + lane + 64 * i] = g[i] * u[i];
}

// Thread per channel, 64 packed tokens per block row: dx for those tokens and this block's part of dw.
__global__ void __launch_bounds__(256) k_conv_bwd(BwdMixArgs m) {
  const int64_t c = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (c >= m.C) return;
  const int64_t t0 = int64_t(blockIdx.y) * 64, t1 = min(t0 + 64, m.T);
  // channel -> (input tensor, column, output tensor)
  const float* x;
  float* dx;
  int64_t ld, col;
  const int64_t qk = int64_t(m.hk) * kD;
  if (c < qk) { x = m.q; dx = m.dq; ld = qk; col = c; }
  else if (c < 2 * qk) { x = m.k; dx = m.dk; ld = qk; col = c - qk; }
  else { x = m.v; dx = m.dv; ld = int64_t(m.hv) * kD; col = c - 2 * qk; }
  float w4[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) w4[j] = m.conv_w[c * 4 + j];
  float dw[4] = {0.f, 0.f, 0.f, 0.f};
  int n = seq_of(m.cu, m.n_seqs, t0);
  for (int64_t t = t0; t < t1; ++t) {
    while (n + 1 < m.n_seqs && int64_t(m.cu[n + 1]) <= t) ++n;
    const int64_t s0 = m.cu[n], s1 = m.cu[n + 1];
    const float* hist = m.conv_in ? m.conv_in + int64_t(n) * 3 * m.C : nullptr;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t tu = t + 3 - j;  // the conv output that reads x[t] through tap j
      if (tu < s1) acc = fmaf(w4[j], m.du[tu * m.C + c], acc);
    }
    dx[t * ld + col] = acc;
    const float dut = m.du[t * m.C + c];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t p = t - 3 + j;
      const float xv = p >= s0 ? x[p * ld + col] : (hist ? hist[(p - s0 + 3) * m.C + c] : 0.f);
      dw[j] = fmaf(dut, xv, dw[j]);
    }
  }
  *reinterpret_cast<float4*>(m.dw_part + (int64_t(blockIdx.y) * m.C + c) * 4) = make_float4(dw[0], dw[1], dw[2], dw[3]);
}

// dconv_w = the sum of the token blocks' parts, in block order (reproducible).
__global__ void __launch_bounds__(256) k_conv_w_sum(BwdMixArgs m, int64_t nblocks) {
  const int64_t c = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (c >= m.C) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t b = 0; b < nblocks; ++b) {
    const float4 v = *reinterpret_cast<const float4*>(m.dw_part + (b * m.C + c) * 4);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  *reinterpret_cast<float4*>(m.dconv_w + c * 4) = acc;
}

// d conv_in[n][r][c] = sum_j w[c][j] du[s0 + r - j] for s0 + r - j in [s0, s1).
__global__ void __launch_bounds__(256) k_conv_in_bwd(BwdMixArgs m) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;  // over n_seqs * 3 * C
  if (i >= int64_t(m.n_seqs) * 3 * m.C) return;
  const int64_t n = i / (3 * m.C), r = (i / m.C) % 3, c = i % m.C;
  const int64_t s0 = m.cu[n], s1 = m.cu[n + 1];
  float acc = 0.f;
  for (int j = 0; j < 4; ++j) {
    const int64_t tu = s0 + r - j;
    if (j <= r && tu < s1) acc = fmaf(m.conv_w[c * 4 + j], m.du[tu * m.C + c], acc);
  }
  m.dconv_in[i] = acc;
}

hipError_t launch_norm_gate_bwd(int64_t rows, const float* y, const float* z, const float* dout, const float* norm_w,
                                float eps, float* dy, float* dz, float* dnorm_w, float* dw_part, hipStream_t s) {
  if (rows == 0) {
    hipLaunchKernelGGL(k_zero, dim3(1), dim3(256), 0, s, dnorm_w, int64_t(kD));
    return hipGetLastError();
  }
  const int64_t nb = (rows + 63) / 64;
  hipLaunchKernelGGL(k_norm_gate_bwd, dim3(static_cast<unsigned>(nb)), dim3(256), 0, s, rows, y, z, dout, norm_w, eps,
                     dy, dz, dw_part);
  hipLaunchKernelGGL(k_sum_parts, dim3(1), dim3(1024), 0, s, dw_part, nb, dnorm_w);
  return hipGetLastError();
}

hipError_t launch_mixer_input_bwd(const BwdMixArgs& m, hipStream_t s) {
  if (m.T > 0) {
    const int64_t items = m.T * (2 * m.hk + m.hv), nb = (m.T + 63) / 64;
    hipLaunchKernelGGL(k_l2silu_bwd, dim3(static_cast<unsigned>((items + 3) / 4)), dim3(256), 0, s, m);
    hipLaunchKernelGGL(k_conv_bwd, dim3(static_cast<unsigned>((m.C + 255) / 256), static_cast<unsigned>(nb)),
                       dim3(256), 0, s, m);
    hipLaunchKernelGGL(k_conv_w_sum, dim3(static_cast<unsigned>((m.C + 255) / 256)), dim3(256), 0, s, m, nb);
  } else {
    hipLaunchKernelGGL(k_zero, dim3(static_cast<unsigned>((m.C * 4 + 255) / 256)), dim3(256), 0, s, m.dconv_w, m.C * 4);
  }
  if (m.dconv_in && m.n_seqs > 0)
    hipLaunchKernelGGL(k_conv_in_bwd, dim3(static_cast<unsigned>((int64_t(m.n_seqs) * 3 * m.C + 255) / 256)),
                       dim3(256), 0, s, m);
  return hipGetLastError();
}

}  // namespace gdn
