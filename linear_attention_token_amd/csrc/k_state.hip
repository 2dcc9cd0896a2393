// Inter-chunk state propagation: the only sequential part of the chunked prefill.
//
// For each chunk of a sequence, from the chunk-start state S (fp32, kept in registers):
//     W  = U - Wk S                               (the chunk's effective writes beta_t e_t)
//     S <- exp(G_C) S + K^T diag(exp(G_C - G_i)) W  (state after the chunk)
// which is the update equations of the analysis notes "Qwen3.8-Flash-Next：架构、效率与技术谱系"
// (§03) applied to 64 tokens at once (U, Wk, G from the WY kernel). The chunk-start state and W are
// stored (bf16) for the output kernel, which then runs chunk-parallel.
//
// The d_v columns of S are independent in these products, so a chain is split into 4 slices of
// 32 columns: one block of 4 waves per (sequence, value head, slice). Wave w owns state rows
// 32w..32w+31 (two 16-row MFMA tiles) and W rows 16w..16w+15; S and W cross waves through LDS in
// bf16 as the B operand of the bf16 MFMAs, accumulation stays fp32.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kSlice = 32;
constexpr int kSlices = 128 / kSlice;

struct StateArgs {
  const int32_t* seq_off;
  int hk, hv, R;
  const float* G;
  const uint16_t *Wk, *U, *KT;
  uint16_t *ST, *WT;
  const float* state_in;
  float* state_out;
};

struct ChunkOperands {
  short8 wk[4];        // A operand of Wk S: Wk rows 16w + li, k = 32s + 8lq .. +8
  short8 kt[2][2];     // A operand of K^T W~: K^T rows 32w + 16m + li, tokens 32s + 8lq .. +8
  uint16_t u[2][4];    // U rows 16w + 4lq + r, columns 16nt + li of this slice (raw bf16)
  float gr[4];         // G of rows 16w + 4lq + r
  float gc;            // G of the last row (decay over the whole chunk)
};

__device__ __forceinline__ void load_chunk(const StateArgs& a, int64_t c, int h, int g, int sl, int w,
                                           int li, int lq, ChunkOperands& o) {
  const uint16_t* wk = a.Wk + (c * a.hv + h) * 64 * 128;
#pragma unroll
  for (int s = 0; s < 4; ++s) o.wk[s] = ld_short8(wk + (16 * w + li) * 128 + 32 * s + 8 * lq);
  const uint16_t* kt = a.KT + (c * a.hk + g) * 128 * 64;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int s = 0; s < 2; ++s) o.kt[m][s] = ld_short8(kt + (32 * w + 16 * m + li) * 64 + 32 * s + 8 * lq);
  const uint16_t* u = a.U + (c * a.hv + h) * 64 * 128;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) o.u[nt][r] = u[(16 * w + 4 * lq + r) * 128 + kSlice * sl + 16 * nt + li];
  const float* G = a.G + (c * a.hv + h) * 64;
#pragma unroll
  for (int r = 0; r < 4; ++r) o.gr[r] = G[16 * w + 4 * lq + r];
  o.gc = G[63];
}

__global__ void __launch_bounds__(256) k_state(StateArgs a) {
  const int n = blockIdx.x, h = blockIdx.y, sl = blockIdx.z;
  const int g = h / a.R;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, lq = lane >> 4;
  constexpr int kStLd = 136;  // bf16 row stride of S^T [32 cols][128 k]
  constexpr int kWtLd = 72;   // bf16 row stride of W~^T [32 cols][64 tokens]
  __shared__ __attribute__((aligned(16))) uint16_t STs[kSlice * kStLd];
  __shared__ __attribute__((aligned(16))) uint16_t WTs[kSlice * kWtLd];

  // state rows 32w + 16m + 4lq + r, columns 32sl + 16nt + li
  f32x4 S[2][2];
  const size_t sbase = (size_t(n) * a.hv + h) * 128 * 128;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S[m][nt][r] = a.state_in ? a.state_in[sbase + size_t(32 * w + 16 * m + 4 * lq + r) * 128 + kSlice * sl + 16 * nt + li] : 0.f;

  const int64_t c0 = a.seq_off[n], c1 = a.seq_off[n + 1];

  // One chunk step from the operands in `cur` (loaded one step ahead, so their latency hides
  // behind the previous step).
  auto chunk_step = [&](const ChunkOperands& cur, int64_t c) {
    // S (bf16) -> LDS as S^T, and to the chunk-state output
    uint16_t* stg = a.ST + (size_t(c) * a.hv + h) * 128 * 128;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int col = 16 * nt + li, k0 = 32 * w + 16 * m + 4 * lq;
        const uint32_t lo = pack_bf16x2(S[m][nt][0], S[m][nt][1]);
        const uint32_t hi = pack_bf16x2(S[m][nt][2], S[m][nt][3]);
        *reinterpret_cast<uint2*>(&STs[col * kStLd + k0]) = make_uint2(lo, hi);
        *reinterpret_cast<uint2*>(stg + size_t(kSlice * sl + col) * 128 + k0) = make_uint2(lo, hi);
      }
    __syncthreads();

    // W = U - Wk S   (rows 16w + 4lq + r, columns 16nt + li)
    f32x4 Wt[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc = mfma16x16x32(cur.wk[s], ld_short8(&STs[(16 * nt + li) * kStLd + 32 * s + 8 * lq]), acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) Wt[nt][r] = bf2f(cur.u[nt][r]) - acc[r];
    }
    // W^T to the output kernel; W~ = diag(exp(G_C - G_i)) W to LDS as the B operand of K^T W~
    uint16_t* wtg = a.WT + (size_t(c) * a.hv + h) * 128 * 64;
    float dec[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) dec[r] = __expf(cur.gc - cur.gr[r]);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int col = 16 * nt + li, t0 = 16 * w + 4 * lq;
      const uint32_t lo = pack_bf16x2(Wt[nt][0], Wt[nt][1]);
      const uint32_t hi = pack_bf16x2(Wt[nt][2], Wt[nt][3]);
      *reinterpret_cast<uint2*>(wtg + size_t(kSlice * sl + col) * 64 + t0) = make_uint2(lo, hi);
      const uint32_t lo2 = pack_bf16x2(Wt[nt][0] * dec[0], Wt[nt][1] * dec[1]);
      const uint32_t hi2 = pack_bf16x2(Wt[nt][2] * dec[2], Wt[nt][3] * dec[3]);
      *reinterpret_cast<uint2*>(&WTs[col * kWtLd + t0]) = make_uint2(lo2, hi2);
    }
    __syncthreads();

    // S <- exp(G_C) S + K^T W~
    const float gC = __expf(cur.gc);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        f32x4 acc = S[m][nt] * gC;
#pragma unroll
        for (int s = 0; s < 2; ++s)
          acc = mfma16x16x32(cur.kt[m][s], ld_short8(&WTs[(16 * nt + li) * kWtLd + 32 * s + 8 * lq]), acc);
        S[m][nt] = acc;
      }
  };

  // ping-pong operand buffers: step c uses one while the loads for step c + 1 fill the other
  ChunkOperands bufA, bufB;
  if (c0 < c1) load_chunk(a, c0, h, g, sl, w, li, lq, bufA);
  for (int64_t c = c0; c < c1; c += 2) {
    if (c + 1 < c1) load_chunk(a, c + 1, h, g, sl, w, li, lq, bufB);
    chunk_step(bufA, c);
    if (c + 1 >= c1) break;
    if (c + 2 < c1) load_chunk(a, c + 2, h, g, sl, w, li, lq, bufA);
    chunk_step(bufB, c + 1);
  }

  if (a.state_out) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          a.state_out[sbase + size_t(32 * w + 16 * m + 4 * lq + r) * 128 + kSlice * sl + 16 * nt + li] = S[m][nt][r];
  }
}

hipError_t launch_state(const Problem& p, const Workspace& ws, const float* state_in, float* state_out,
                        hipStream_t s) {
  if (p.n_seqs == 0) return hipSuccess;
  StateArgs a{ws.seq_chunk_off, p.hk, p.hv, p.hv / p.hk, ws.G, ws.Wk, ws.U, ws.KT, ws.ST, ws.WT,
              state_in, state_out};
  hipLaunchKernelGGL(k_state, dim3(unsigned(p.n_seqs), unsigned(p.hv), unsigned(kSlices)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace gdn
