// Backward of the mixer's steps around the recurrence (fp32, d = 128), for gdn_backward:
//   k_norm_gate_bwd   o = n * sigmoid(z), n = y / r * (1 + w), r = sqrt(mean(y^2) + eps):
//                     dz = do * n * s (1 - s);  dn = do * s;  dw = sum of dn * y / r (per-block parts, then
//                     k_sum_parts);
//                     dy = (1 + w) dn / r - y <(1 + w) dn, y> / (128 r^3)
//   k_l2silu_bwd      a = a0 / sqrt(|a0|^2 + eps) (q, k heads), a0 = silu(u), u the conv output:
//                     da0 = (da - a <a, da>) / sqrt(|a0|^2 + eps);  du = da0 sigmoid(u) (1 + u (1 - sigmoid(u)))
//   k_conv_bwd        u[t] = sum_j w[j] x[t - 3 + j]:  dx[t] = sum_j w[j] du[t + 3 - j] (inside the sequence),
//                     dw[j] = sum_t du[t] x[t - 3 + j] (x[-3..-1] = the conv history; per 16-token block
//                     parts, then k_conv_w_sum)
//   k_conv_in_bwd     d history[r] = sum_j w[j] du[r - j] (r = 0..2 for positions -3..-1)
// (the steps of the paper reading "On the Design of Qwen3.8-Next Architecture … 精读" §四 4.1 and the
// analysis notes "Qwen3.8-Flash-Next：架构、效率与技术谱系" §03, differentiated).
#include <algorithm>

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

// Half a wave per (token, value head) row, four channels per lane; block b takes rows 8b + i, 8b + i +
// 8 gridDim.x, ... (i its half-wave), so its part of dw is the sum over a fixed set of rows.
__global__ void __launch_bounds__(256) k_norm_gate_bwd(int64_t rows, const float* __restrict__ y,
                                                       const float* __restrict__ z, const float* __restrict__ dout,
                                                       const float* __restrict__ norm_w, float eps,
                                                       float* __restrict__ dy, float* __restrict__ dz,
                                                       float* __restrict__ dw_part) {
  const int l = threadIdx.x & 31, hw = threadIdx.x >> 5, d0 = 4 * l;
  const float4 nw = *reinterpret_cast<const float4*>(norm_w + d0);
  const float wg[4] = {1.f + nw.x, 1.f + nw.y, 1.f + nw.z, 1.f + nw.w};
  float dwa[4] = {0.f, 0.f, 0.f, 0.f};
  constexpr int kBatch = 4;  // rows whose loads are issued together
  const int64_t stride = int64_t(gridDim.x) * 8;
  for (int64_t row0 = int64_t(blockIdx.x) * 8 + hw; row0 < rows; row0 += kBatch * stride) {
  float4 y4s[kBatch], z4s[kBatch], o4s[kBatch];
#pragma unroll
  for (int k = 0; k < kBatch; ++k) {
    const int64_t row = min(row0 + k * stride, rows - 1);
    const int64_t b = row * kD + d0;
    y4s[k] = *reinterpret_cast<const float4*>(y + b);
    z4s[k] = *reinterpret_cast<const float4*>(z + b);
    o4s[k] = *reinterpret_cast<const float4*>(dout + b);
  }
#pragma unroll
  for (int k = 0; k < kBatch; ++k) {
    const int64_t row = row0 + k * stride;
    if (row >= rows) break;  // uniform over the half-wave
    const int64_t b = row * kD + d0;
    const float4 y4 = y4s[k], z4 = z4s[k], o4 = o4s[k];
    const float yv[4] = {y4.x, y4.y, y4.z, y4.w}, zv[4] = {z4.x, z4.y, z4.z, z4.w};
    const float ov[4] = {o4.x, o4.y, o4.z, o4.w};
    const float r = sqrtf(group_sum<32>(yv[0] * yv[0] + yv[1] * yv[1] + yv[2] * yv[2] + yv[3] * yv[3]) * (1.f / kD) + eps);
    const float ir = 1.f / r;
    float dzv[4], g[4], gy = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float sg = 1.f / (1.f + __expf(-zv[e]));
      const float nv = yv[e] * ir * wg[e];
      dzv[e] = ov[e] * nv * sg * (1.f - sg);
      const float dn = ov[e] * sg;
      dwa[e] = fmaf(dn * yv[e], ir, dwa[e]);
      g[e] = wg[e] * dn;
      gy += g[e] * yv[e];
    }
    const float dot = group_sum<32>(gy) * ir * ir * ir * (1.f / kD);
    *reinterpret_cast<float4*>(dz + b) = make_float4(dzv[0], dzv[1], dzv[2], dzv[3]);
    *reinterpret_cast<float4*>(dy + b) =
        make_float4(g[0] * ir - yv[0] * dot, g[1] * ir - yv[1] * dot, g[2] * ir - yv[2] * dot, g[3] * ir - yv[3] * dot);
  }
  }
  // this block's part of the norm gain's derivative: the half-waves' sums in a fixed order
  __shared__ float red[8][kD];
#pragma unroll
  for (int e = 0; e < 4; ++e) red[hw][d0 + e] = dwa[e];
  __syncthreads();
  if (threadIdx.x < kD) {
    float sacc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) sacc += red[i][threadIdx.x];
    dw_part[int64_t(blockIdx.x) * kD + threadIdx.x] = sacc;
  }
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

// Half a wave per (token, head) of q, k (L2 and SiLU) or v (SiLU), four channels per lane: du into
// [T][C]. Eight rows per block.
__global__ void __launch_bounds__(256) k_l2silu_bwd(BwdMixArgs m) {
  const int l = threadIdx.x & 31;
  const int64_t item = int64_t(blockIdx.x) * 8 + (threadIdx.x >> 5);
  const int heads = 2 * m.hk + m.hv;
  const bool live = item < m.T * heads;  // the shuffles below run in every lane
  const int64_t it = live ? item : 0;
  const int64_t t = it / heads;
  const int hd = int(it - t * heads);
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
  const int d0 = 4 * l;
  const int64_t c0 = int64_t(hd) * kD + d0;  // conv channel of this lane's first dim (q | k | v order)
  // the four taps' inputs (history before the sequence start) and the weights, as float4s
  float4 xs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t p = t - 3 + j;
    xs[j] = p >= s0 ? *reinterpret_cast<const float4*>(x + p * ld + col0 + d0)
                    : (hist ? *reinterpret_cast<const float4*>(hist + (p - s0 + 3) * m.C + c0) : make_float4(0.f, 0.f, 0.f, 0.f));
  }
  float4 w4[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) w4[e] = *reinterpret_cast<const float4*>(m.conv_w + (c0 + e) * 4);
  const float4 g4 = *reinterpret_cast<const float4*>(da + d0);
  float u[4], a0[4], g[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float wv[4] = {w4[e].x, w4[e].y, w4[e].z, w4[e].w};
    float uu = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float xv = e == 0 ? xs[j].x : e == 1 ? xs[j].y : e == 2 ? xs[j].z : xs[j].w;
      uu = fmaf(wv[j], xv, uu);
    }
    const float sg = 1.f / (1.f + __expf(-uu));
    a0[e] = uu * sg;
    u[e] = sg * (1.f + uu * (1.f - sg));  // silu'(u)
  }
  if (l2) {  // uniform over the half-wave (one head)
    const float inv = 1.f / sqrtf(group_sum<32>(a0[0] * a0[0] + a0[1] * a0[1] + a0[2] * a0[2] + a0[3] * a0[3]) + m.l2_eps);
    const float adot = group_sum<32>(a0[0] * g[0] + a0[1] * g[1] + a0[2] * g[2] + a0[3] * g[3]) * inv;
#pragma unroll
    for (int e = 0; e < 4; ++e) g[e] = (g[e] - a0[e] * inv * adot) * inv;
  }
  if (live)
    *reinterpret_cast<float4*>(m.du + t * m.C + c0) = make_float4(g[0] * u[0], g[1] * u[1], g[2] * u[2], g[3] * u[3]);
}

// Four channels per thread (16-byte loads and stores), windows of kConvBwdRows packed tokens per
// block row, walked in register halves of kConvBwdHalf tokens: dx for those tokens and this block's
// part of dw. The du rows t .. t + 3 and x rows t - 3 .. t that a half reads are loaded once each,
// all before use (history rows of a sequence start are read where needed).
constexpr int kConvBwdRows = 16;
constexpr int kConvBwdHalf = 8;
__global__ void __launch_bounds__(256) k_conv_bwd(BwdMixArgs m) {
  constexpr int R = kConvBwdHalf;
  const int64_t c = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;  // first of the thread's channels
  if (c >= m.C) return;
  // channel -> (input tensor, column, output tensor); the tensor boundaries are multiples of 128
  const float* x;
  float* dx;
  int64_t ld, col;
  const int64_t qk = int64_t(m.hk) * kD;
  if (c < qk) { x = m.q; dx = m.dq; ld = qk; col = c; }
  else if (c < 2 * qk) { x = m.k; dx = m.dk; ld = qk; col = c - qk; }
  else { x = m.v; dx = m.dv; ld = int64_t(m.hv) * kD; col = c - 2 * qk; }
  float4 w4[4];  // w4[e] = taps of channel c + e
#pragma unroll
  for (int e = 0; e < 4; ++e) w4[e] = *reinterpret_cast<const float4*>(m.conv_w + (c + e) * 4);
  float dw[4][4] = {};  // dw[e][j]
  // windows blockIdx.y, + gridDim.y, ...: this block's part of dw sums a fixed set of tokens
  for (int64_t t00 = int64_t(blockIdx.y) * kConvBwdRows; t00 < m.T; t00 += int64_t(gridDim.y) * kConvBwdRows) {
  for (int64_t t0 = t00; t0 < min(t00 + kConvBwdRows, m.T); t0 += R) {
  const int64_t t1 = min(t0 + R, m.T);
  float4 duw[R + 3], xw[R + 3];  // du[t0 + i], x[t0 - 3 + i]
#pragma unroll
  for (int i = 0; i < R + 3; ++i) {
    const int64_t tu = t0 + i, p = t0 - 3 + i;
    duw[i] = tu < m.T ? *reinterpret_cast<const float4*>(m.du + tu * m.C + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    xw[i] = (p >= 0 && p < m.T) ? *reinterpret_cast<const float4*>(x + p * ld + col) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  int n = seq_of(m.cu, m.n_seqs, t0);
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int64_t t = t0 + i;
    if (t >= t1) break;
    while (n + 1 < m.n_seqs && int64_t(m.cu[n + 1]) <= t) ++n;
    const int64_t s0 = m.cu[n], s1 = m.cu[n + 1];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t tu = t + 3 - j;  // the conv output that reads x[t] through tap j
      if (tu < s1) {
        const float4 d = duw[i + 3 - j];
        acc.x = fmaf(w4[0][j], d.x, acc.x);
        acc.y = fmaf(w4[1][j], d.y, acc.y);
        acc.z = fmaf(w4[2][j], d.z, acc.z);
        acc.w = fmaf(w4[3][j], d.w, acc.w);
      }
    }
    *reinterpret_cast<float4*>(dx + t * ld + col) = acc;
    const float4 dut = duw[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t p = t - 3 + j;
      float4 xv;
      if (p >= s0) xv = xw[i + j];
      else xv = m.conv_in ? *reinterpret_cast<const float4*>(m.conv_in + (int64_t(n) * 3 + (p - s0 + 3)) * m.C + c)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
      dw[0][j] = fmaf(dut.x, xv.x, dw[0][j]);
      dw[1][j] = fmaf(dut.y, xv.y, dw[1][j]);
      dw[2][j] = fmaf(dut.z, xv.z, dw[2][j]);
      dw[3][j] = fmaf(dut.w, xv.w, dw[3][j]);
    }
  }
  }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
    *reinterpret_cast<float4*>(m.dw_part + (int64_t(blockIdx.y) * m.C + c + e) * 4) =
        make_float4(dw[e][0], dw[e][1], dw[e][2], dw[e][3]);
}

// dconv_w = the sum of the token-window groups' parts: thread (channel, q) adds parts q, q + 4, ..., then
// the four sums are added in order (reproducible). 64 channels per block.
__global__ void __launch_bounds__(256) k_conv_w_sum(BwdMixArgs m, int64_t nblocks) {
  __shared__ float4 red[4][64];
  const int cl = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int64_t c = int64_t(blockIdx.x) * 64 + cl;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (c < m.C) {
#pragma unroll 4
    for (int64_t b = q; b < nblocks; b += 4) {
      const float4 v = *reinterpret_cast<const float4*>(m.dw_part + (b * m.C + c) * 4);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
  }
  red[q][cl] = acc;
  __syncthreads();
  if (q == 0 && c < m.C) {
    float4 t = red[0][cl];
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      t.x += red[i][cl].x; t.y += red[i][cl].y; t.z += red[i][cl].z; t.w += red[i][cl].w;
    }
    *reinterpret_cast<float4*>(m.dconv_w + c * 4) = t;
  }
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
  const int64_t nb = std::min<int64_t>((rows + 7) / 8, kNormGateParts);
  hipLaunchKernelGGL(k_norm_gate_bwd, dim3(static_cast<unsigned>(nb)), dim3(256), 0, s, rows, y, z, dout, norm_w, eps,
                     dy, dz, dw_part);
  hipLaunchKernelGGL(k_sum_parts, dim3(1), dim3(1024), 0, s, dw_part, nb, dnorm_w);
  return hipGetLastError();
}

hipError_t launch_mixer_input_bwd(const BwdMixArgs& m, hipStream_t s) {
  if (m.T > 0) {
    const int64_t items = m.T * (2 * m.hk + m.hv);
    const int64_t nb = std::min<int64_t>((m.T + kConvBwdRows - 1) / kConvBwdRows, kConvWeightParts);
    hipLaunchKernelGGL(k_l2silu_bwd, dim3(static_cast<unsigned>((items + 7) / 8)), dim3(256), 0, s, m);
    hipLaunchKernelGGL(k_conv_bwd, dim3(static_cast<unsigned>((m.C / 4 + 255) / 256), static_cast<unsigned>(nb)),
                       dim3(256), 0, s, m);
    hipLaunchKernelGGL(k_conv_w_sum, dim3(static_cast<unsigned>((m.C + 63) / 64)), dim3(256), 0, s, m, nb);
  } else {
    hipLaunchKernelGGL(k_zero, dim3(static_cast<unsigned>((m.C * 4 + 255) / 256)), dim3(256), 0, s, m.dconv_w, m.C * 4);
  }
  if (m.dconv_in && m.n_seqs > 0)
    hipLaunchKernelGGL(k_conv_in_bwd, dim3(static_cast<unsigned>((int64_t(m.n_seqs) * 3 * m.C + 255) / 256)),
                       dim3(256), 0, s, m);
  return hipGetLastError();
}

}  // namespace gdn
