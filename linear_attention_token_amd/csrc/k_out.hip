// Output of the chunked prefill, one block per (64-token chunk, value head), all chunks in parallel.
//
// From the chunk-start state S and the chunk's writes W (state kernel), the readout y_t = S_t^T q_t
// of the analysis notes "Qwen3.8-Flash-Next：架构、效率与技术谱系" (§03) over a chunk is
//     Y = diag(exp(G)) Q S + (L o E o Q K^T) W,   E[t,i] = exp(G_t - G_i),  L = lower incl. diagonal,
// then zero-centred RMSNorm over the 128 channels of the head, gain (1 + w), and the sigmoid output
// gate (analysis notes §03 changes made to GDN; paper summary "Qwen3.8-Flash-Next", Method: head
// outputs are normalised, then gated).
//
// Wave w computes channels 32w..32w+31 of Y for all 64 tokens (its own slice of the chunk state and
// of W), as Y^T = S^T Q^T + W^T P^T: the chunk-state and W pieces are then A operands as loaded, and
// each lane ends with 4 consecutive channels of a token, so RMSNorm, gain and gate run on registers.
// Per-token sums of squares are combined across the four waves in LDS. The gate tile is loaded and
// the output tile stored as whole 256-byte token rows (16 bytes per lane), passing through LDS in
// between. bf16 MFMA, fp32 accumulate.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

struct OutArgs {
  const int4* tab;
  int n_units;                   // chunks x QK heads
  int n_main;                    // blocks of the output proper; the rest write the conv tail
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

__global__ void __launch_bounds__(256, 4) k_out(OutArgs a, ConvTailArgs tail) {
  if (int(blockIdx.x) >= a.n_main) {  // conv-cache tail (no barrier below is reached)
    const int b = int(blockIdx.x) - a.n_main, n = b / tail.cblk;
    conv_tail_piece<bf16>(tail, n, int64_t(b - n * tail.cblk) * 256 + threadIdx.x);
    return;
  }
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
  __shared__ __attribute__((aligned(16))) uint16_t QKs[2 * 64 * kLd];  // Q and K tiles
  uint16_t* Qs = QKs;
  uint16_t* Ks = QKs + 64 * kLd;
  uint16_t* Ps = Ks;  // P [64][kPLd] over the K tile once every wave is done with K
  __shared__ float Gs[64];
  __shared__ float red[4][64];

  // B operands of this wave's columns (chunk state and W), issued first so they overlap the rest;
  // the state pass stores them as these operand pieces, 1 KB of consecutive bytes per load. They,
  // the gate and the output are touched once, so they go non-temporal, leaving the caches to q^ and
  // k^, which the value heads of a QK head share.
  const uint16_t* st = a.ST + (int64_t(c) * a.hv + h) * 128 * 128;
  const uint16_t* wt = a.WT + (int64_t(c) * a.hv + h) * 128 * 64;
  short8 bs[2][4], bw[2][2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      bs[nt][s] = __builtin_nontemporal_load(reinterpret_cast<const short8*>(st + (((w * 2 + nt) * 4 + s) * 64 + lane) * 8));
#pragma unroll
    for (int s = 0; s < 2; ++s)
      bw[nt][s] = __builtin_nontemporal_load(reinterpret_cast<const short8*>(wt + (((w * 2 + nt) * 2 + s) * 64 + lane) * 8));
  }
  // gate logits as whole token rows: piece idx = tid + 256 it is token idx / 16, channels
  // 8 (idx % 16) .. +7 (rows past the chunk end read the last row; their outputs are not stored)
  const int64_t orow = int64_t(a.hv) * 128;
  uint4 gq[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int idx = tid + it * 256;
    gq[it] = make_uint4(0u, 0u, 0u, 0u);
    if (a.flags & GDN_GATE)
      gq[it] = ldnt16(a.gate + (start + min(idx >> 4, len - 1)) * orow + h * 128 + (idx & 15) * 8);
  }
  // zero-centred gain (1 + w) of this lane's 8 channels
  float gain[2][4];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float4 g4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.flags & GDN_NORM)
      g4 = *reinterpret_cast<const float4*>(a.norm_w + int64_t(h) * a.norm_stride + 32 * w + 16 * nt + 4 * lq);
    gain[nt][0] = 1.f + g4.x; gain[nt][1] = 1.f + g4.y; gain[nt][2] = 1.f + g4.z; gain[nt][3] = 1.f + g4.w;
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

  // P = L o E o (Q K^T) in bf16, written over K once all waves are done reading it
  f32x4 pacc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    pacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (nt <= w) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        pacc[nt] = mfma16x16x32(ld_short8(&Qs[(16 * w + li) * kLd + 32 * s + 8 * lq]),
                                ld_short8(&Ks[(16 * nt + li) * kLd + 32 * s + 8 * lq]), pacc[nt]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * w + 4 * lq + r, i = 16 * nt + li;
      Ps[t * kPLd + i] = f2bf(i <= t ? pacc[nt][r] * __expf(Gs[t] - Gs[i]) : 0.f);
    }
  __syncthreads();

  // Y^T: acc[tt][nt][r] is channel 32w + 16nt + 4lq + r of token 16tt + li
  f32x4 acc[4][2];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[tt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const short8 qb = ld_short8(&Qs[(16 * tt + li) * kLd + 32 * s + 8 * lq]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[tt][nt] = mfma16x16x32(bs[nt][s], qb, acc[tt][nt]);
    }
    const float gam = __expf(Gs[16 * tt + li]);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[tt][nt] *= gam;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (32 * s > 16 * tt + 15) continue;  // P is zero above the diagonal
      const short8 pb = ld_short8(&Ps[(16 * tt + li) * kPLd + 32 * s + 8 * lq]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[tt][nt] = mfma16x16x32(bw[nt][s], pb, acc[tt][nt]);
    }
  }

  // scale, and each token's sum of squares over this wave's 32 channels
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    float ss = 0.f;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        acc[tt][nt][r] *= a.scale;
        ss += acc[tt][nt][r] * acc[tt][nt][r];
      }
    ss = half_pair_sum(row_pair_sum(ss));
    if (lq == 0) red[w][16 * tt + li] = ss;
  }
  __syncthreads();  // every wave is past its last read of Q and P
  // the gate tile [64][kLd] over Q; each lane then replaces the 8 bytes of logits it reads with the
  // 8 bytes of output it computes from them, so the output tile needs no further barrier to form
  uint16_t* Os = Qs;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int idx = tid + it * 256;
    *reinterpret_cast<uint4*>(&Os[(idx >> 4) * kLd + (idx & 15) * 8]) = gq[it];
  }
  __syncthreads();
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int t = 16 * tt + li;
    const float tot = red[0][t] + red[1][t] + red[2][t] + red[3][t];
    const float rs = (a.flags & GDN_NORM) ? 1.0f / sqrtf(tot * (1.0f / 128.0f) + a.norm_eps) : 1.0f;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      uint2* slot = reinterpret_cast<uint2*>(&Os[t * kLd + 32 * w + 16 * nt + 4 * lq]);
      const uint2 gg = *slot;
      const float gl[4] = {__uint_as_float(gg.x << 16), __uint_as_float(gg.x & 0xffff0000u),
                           __uint_as_float(gg.y << 16), __uint_as_float(gg.y & 0xffff0000u)};
      float o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = acc[tt][nt][r] * rs;
        if (a.flags & GDN_NORM) v *= gain[nt][r];
        if (a.flags & GDN_GATE) v *= sigmoidf_(gl[r]);
        o[r] = v;
      }
      *slot = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
    }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int idx = tid + it * 256, t = idx >> 4;
    if (t < len)
      stnt16(a.out + (start + t) * orow + h * 128 + (idx & 15) * 8, *reinterpret_cast<const uint4*>(&Os[t * kLd + (idx & 15) * 8]));
  }
}

hipError_t launch_output(const Problem& p, const Workspace& ws, const void* gate, const float* norm_w,
                         void* out, const ConvTailArgs& tail, hipStream_t s) {
  if (p.nc_max == 0) return hipSuccess;
  const int R = p.hv / p.hk;
  const int64_t units = p.nc_max * p.hk;
  const int64_t n_main = xcd_blocks(units, R);
  const int64_t n_tail = tail.conv_out != nullptr ? int64_t(tail.n_seqs) * tail.cblk : 0;
  OutArgs a{ws.chunk_tab, int(units), int(n_main), p.hk, p.hv, R, static_cast<const uint16_t*>(ws.qhat),
            static_cast<const uint16_t*>(ws.khat), ws.G, ws.ST, ws.WT,
            static_cast<const uint16_t*>(gate), norm_w, p.norm_stride, static_cast<uint16_t*>(out),
            p.flags, p.scale, p.norm_eps};
  hipLaunchKernelGGL(k_out, dim3(unsigned(n_main + n_tail)), dim3(256), 0, s, a, tail);
  return hipGetLastError();
}

}  // namespace gdn
