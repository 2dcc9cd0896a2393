// Output of the chunked prefill, one block per (64-token chunk, value head), all chunks in parallel.
//
// From the chunk-start state S and the chunk's writes W (state kernel), the readout y_t = S_t^T q_t
// of the analysis notes "Qwen3.8-Flash-Next：架构、效率与技术谱系" (§03) over a chunk is
//     Y = diag(exp(G)) Q S + (L o E o Q K^T) W,   E[t,i] = exp(G_t - G_i),  L = lower incl. diagonal,
// then zero-centred RMSNorm over the 128 channels of the head, gain (1 + w), and the sigmoid output
// gate (analysis notes §03 changes made to GDN; paper summary "Qwen3.8-Flash-Next", Method: head
// outputs are normalised, then gated).
//
// Wave w computes columns 32w..32w+31 of Y for all 64 rows (its own slice of the chunk state and
// of W); RMSNorm row sums are combined across the four waves in LDS. bf16 MFMA, fp32 accumulate.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

struct OutArgs {
  const int4* tab;
  int n_units;                   // chunks x QK heads
  int hk, hv, R;
  const uint16_t *qhat, *khat;   // bf16 [T][hk][128]
  const float* G;                // [nc][hv][64]
  const uint16_t *ST, *WT;       // [nc][hv] operand pieces of 1 KB (see the state pass)
  const uint16_t* gate;          // bf16 [T][hv][128]
  const float* norm_w;
  int norm_stride;
  uint16_t* out;                 // bf16 [T][hv][128]
  uint32_t flags;
  float scale, norm_eps;
};

__global__ void __launch_bounds__(256) k_out(OutArgs a) {
  // the R value heads of a QK head read the same q^ / k^ tiles: keep them on one XCD
  int u, hr;
  xcd_item(int(blockIdx.x), a.R, u, hr);
  if (u >= a.n_units) return;
  const int c = u / a.hk, g = u - c * a.hk, h = g * a.R + hr;
  const int4 ct = a.tab[c];
  const int len = ct.y;
  if (len <= 0) return;
  const int64_t start = ct.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, lq = lane >> 4;
  constexpr int kLd = 136;
  constexpr int kPLd = 72;
  constexpr int kYLd = 132;  // fp32 row stride of the staged Y tile (64 x 132 x 4 B fits Qs + Ks)
  // one buffer for the Q and K tiles, reused afterwards for the fp32 Y tile
  __shared__ __attribute__((aligned(16))) uint16_t QKs[2 * 64 * kLd];
  static_assert(64 * kYLd * 4 <= 2 * 64 * kLd * 2, "Y tile must fit the Q/K buffer");
  uint16_t* Qs = QKs;
  uint16_t* Ks = QKs + 64 * kLd;
  __shared__ __attribute__((aligned(16))) uint16_t Ps[64 * kPLd];
  __shared__ float Gs[64];
  __shared__ float red[4][64];

  // B operands of this wave's columns (chunk state and W), issued first so they overlap the rest;
  // the state pass stores them as these operand pieces, 1 KB of consecutive bytes per load
  const uint16_t* st = a.ST + (int64_t(c) * a.hv + h) * 128 * 128;
  const uint16_t* wt = a.WT + (int64_t(c) * a.hv + h) * 128 * 64;
  short8 bs[2][4], bw[2][2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
    for (int s = 0; s < 4; ++s) bs[nt][s] = ld_short8(st + (((w * 2 + nt) * 4 + s) * 64 + lane) * 8);
#pragma unroll
    for (int s = 0; s < 2; ++s) bw[nt][s] = ld_short8(wt + (((w * 2 + nt) * 2 + s) * 64 + lane) * 8);
  }
  // gate tile of this chunk and head, 16 bytes per thread and piece: piece p = tid + 256 * it covers
  // row p / 16, columns 8 * (p % 16) .. +8 (fully coalesced 256-byte rows)
  const int64_t orow = int64_t(a.hv) * 128;
  uint4 gv[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int pidx = tid + it * 256, t = pidx >> 4, sg = pidx & 15;
    gv[it] = make_uint4(0, 0, 0, 0);
    if ((a.flags & GDN_GATE) && t < len)
      gv[it] = *reinterpret_cast<const uint4*>(a.gate + (start + t) * orow + h * 128 + sg * 8);
  }
  // zero-centred gain (1 + w) of this thread's 8 epilogue columns (the same for all its pieces)
  float gain[8];
  {
    const int sg = tid & 15;
    float4 g0 = make_float4(0.f, 0.f, 0.f, 0.f), g1 = g0;
    if (a.flags & GDN_NORM) {
      const float4* wp = reinterpret_cast<const float4*>(a.norm_w + int64_t(h) * a.norm_stride + sg * 8);
      g0 = wp[0];
      g1 = wp[1];
    }
    gain[0] = 1.f + g0.x; gain[1] = 1.f + g0.y; gain[2] = 1.f + g0.z; gain[3] = 1.f + g0.w;
    gain[4] = 1.f + g1.x; gain[5] = 1.f + g1.y; gain[6] = 1.f + g1.z; gain[7] = 1.f + g1.w;
  }
  const int64_t krow = int64_t(a.hk) * 128;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int idx = tid + it * 256;
    const int t = idx >> 4, sg = idx & 15;
    uint4 qv = make_uint4(0, 0, 0, 0), kv = make_uint4(0, 0, 0, 0);
    if (t < len) {
      qv = *reinterpret_cast<const uint4*>(a.qhat + (start + t) * krow + g * 128 + sg * 8);
      kv = *reinterpret_cast<const uint4*>(a.khat + (start + t) * krow + g * 128 + sg * 8);
    }
    *reinterpret_cast<uint4*>(&Qs[t * kLd + sg * 8]) = qv;
    *reinterpret_cast<uint4*>(&Ks[t * kLd + sg * 8]) = kv;
  }
  if (tid < 64) Gs[tid] = a.G[(int64_t(c) * a.hv + h) * 64 + tid];
  __syncthreads();

  // P = L o E o (Q K^T) in bf16
  for (int nt = 0; nt < 4; ++nt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (nt <= w) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc = mfma16x16x32(ld_short8(&Qs[(16 * w + li) * kLd + 32 * s + 8 * lq]),
                           ld_short8(&Ks[(16 * nt + li) * kLd + 32 * s + 8 * lq]), acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * w + 4 * lq + r, i = 16 * nt + li;
      Ps[t * kPLd + i] = f2bf(i <= t ? acc[r] * __expf(Gs[t] - Gs[i]) : 0.f);
    }
  }
  __syncthreads();

  // Y: wave w owns columns 32w..32w+31 (two 16-column tiles) for all 64 rows, so it reads only its
  // own columns of the chunk state and of W; the RMSNorm row sums are combined across waves in LDS.
  f32x4 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const short8 qa = ld_short8(&Qs[(16 * mt + li) * kLd + 32 * s + 8 * lq]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mfma16x16x32(qa, bs[nt][s], acc[mt][nt]);
    }
    float gam[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) gam[r] = __expf(Gs[16 * mt + 4 * lq + r]);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[mt][nt][r] *= gam[r];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const short8 pa = ld_short8(&Ps[(16 * mt + li) * kPLd + 32 * s + 8 * lq]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mfma16x16x32(pa, bw[nt][s], acc[mt][nt]);
    }
  }

  // scale and RMSNorm row sums; Y (fp32) staged in LDS over the Q/K tiles for a coalesced epilogue
  __syncthreads();  // every wave is done reading Qs / Ks / Ps
  float* Ys = reinterpret_cast<float*>(QKs);  // [64][kYLd] fp32 over the Q/K buffer
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float ss = 0.f;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float y = acc[mt][nt][r] * a.scale;
        ss += y * y;
        Ys[(16 * mt + 4 * lq + r) * kYLd + 32 * w + 16 * nt + li] = y;
      }
      ss = group_sum<16>(ss);
      if (li == 0) red[w][16 * mt + 4 * lq + r] = ss;
    }
  }
  __syncthreads();
  // epilogue: piece p = tid + 256 * it -> row p / 16, columns 8 * (p % 16) .. +8
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int pidx = tid + it * 256, t = pidx >> 4, sg = pidx & 15;
    if (t >= len) continue;
    const float tot = red[0][t] + red[1][t] + red[2][t] + red[3][t];
    const float rs = (a.flags & GDN_NORM) ? 1.0f / sqrtf(tot * (1.0f / 128.0f) + a.norm_eps) : 1.0f;
    float gl[8], o[8];
    vec16<bf16>::cvt(gv[it], gl);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = Ys[t * kYLd + sg * 8 + e] * rs;
      if (a.flags & GDN_NORM) v *= gain[e];
      if (a.flags & GDN_GATE) v *= sigmoidf_(gl[e]);
      o[e] = v;
    }
    vec16<bf16>::st(reinterpret_cast<bf16*>(a.out + (start + t) * orow + h * 128 + sg * 8), o);
  }
}

hipError_t launch_output(const Problem& p, const Workspace& ws, const void* gate, const float* norm_w,
                         void* out, hipStream_t s) {
  if (p.nc_max == 0) return hipSuccess;
  const int R = p.hv / p.hk;
  const int64_t units = p.nc_max * p.hk;
  OutArgs a{ws.chunk_tab, int(units), p.hk, p.hv, R, static_cast<const uint16_t*>(ws.qhat),
            static_cast<const uint16_t*>(ws.khat), ws.G, ws.ST, ws.WT,
            static_cast<const uint16_t*>(gate), norm_w, p.norm_stride, static_cast<uint16_t*>(out),
            p.flags, p.scale, p.norm_eps};
  hipLaunchKernelGGL(k_out, dim3(unsigned(xcd_blocks(units, R))), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace gdn
