// Chunk WY/UT transform of the gated delta rule, one block per (64-token chunk, QK head, batch of
// value heads): the value heads of a QK head share its k^ tile, loaded and transposed once.
//
// Unrolling the update equations of the analysis notes "Qwen3.8-Flash-Next：架构、效率与技术谱系"
// (§03) over a chunk that starts from state S, with G_t = sum_{s<=t} ln alpha_s and
// gamma_t = exp(G_t), the effective writes w_t = beta_t e_t satisfy
//     (I + A) W = diag(beta) V - diag(beta gamma) K S,   A[t,i] = beta_t exp(G_t - G_i) k_t.k_i (i < t)
// so with T = (I + A)^-1:  W = U - Wk S,  U = T diag(beta) V,  Wk = T diag(beta gamma) K.
// U and Wk depend only on the chunk, so every chunk is transformed in parallel here; the state
// pass then needs only two products per chunk.
//
// Steps: k^ k^T on bf16 MFMA (fp32 accumulate) -> A in fp32 -> T by blocked forward substitution
// in fp32 (16x16 diagonal blocks inverted per column, off-diagonal blocks merged with fp32 MFMA)
// -> T diag(beta), T diag(beta gamma) rounded to bf16 -> U, Wk on bf16 MFMA.
// Rows past the end of a partial chunk carry beta = 0 and ln alpha = 0, so their U and Wk rows are
// zero and G stays at the last real token.
//
// A block holds TEAMS teams of 4 waves, one per value head of its batch; all teams run the same
// steps in lockstep (block-wide barriers), each on its own LDS region.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

struct WyArgs {
  const int4* tab;
  int n_units;                    // chunks x QK heads
  int hk, hv, R;
  const uint16_t *khat, *vhat;    // bf16 [T][hk][128], [T][hv][128]
  const float *alpha, *beta;      // [T][hv]
  float* G;                       // [nc][hv][64]
  uint16_t *Wk;                   // [nc][hv][64][128]
  uint16_t *U;                    // [nc][hv][4 waves][8 tiles][64 lanes][4 rows]
  uint16_t* KT;                   // [nc][hk][128][64]
};

constexpr int kKsLd = 144;   // bf16 row stride of the 64x128 k^ tile (and of T' / T'' later)
constexpr int kKTLd = 72;    // bf16 row stride of the transposed 128x64 tiles
constexpr int kFLd = 72;     // fp32 row stride of the 64x64 A and T matrices

// T_ij = -D_i * sum_{k=j}^{i-1} A_ik T_kj for block row i > j (16x16 blocks), by one wave.
__device__ __forceinline__ void wy_offdiag(const float* Am, float* Tm, float* X, int i, int j, int lane) {
  const int li = lane & 15, lq = lane >> 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int kb = j; kb < i; ++kb) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const float av = Am[(16 * i + li) * kFLd + 16 * kb + 4 * kk + lq];
      const float bv = Tm[(16 * kb + 4 * kk + lq) * kFLd + 16 * j + li];
      acc = mfma16x16x4f32(av, bv, acc);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) X[(4 * lq + r) * 16 + li] = acc[r];
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const float av = Tm[(16 * i + li) * kFLd + 16 * i + 4 * kk + lq];
    const float bv = X[(4 * kk + lq) * 16 + li];
    acc2 = mfma16x16x4f32(av, bv, acc2);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) Tm[(16 * i + 4 * lq + r) * kFLd + 16 * j + li] = -acc2[r];
}

template <int TEAMS>
__global__ void __launch_bounds__(256 * TEAMS) k_wy(WyArgs a) {
  // block -> (chunk, QK head) unit and batch of TEAMS value heads; the batches of one unit run on
  // one XCD, back to back
  int u, hb;
  xcd_item(int(blockIdx.x), a.R / TEAMS, u, hb);
  if (u >= a.n_units) return;
  const int c = u / a.hk, g = u - c * a.hk;
  const int4 ct = a.tab[c];
  const int len = ct.y;
  if (len <= 0) return;
  const int64_t start = ct.x;
  const int tid = threadIdx.x, lane = tid & 63, team = tid >> 8, w = (tid >> 6) & 3;
  const int ttid = tid & 255;  // thread index inside the team
  const int li = lane & 15, lq = lane >> 4;
  const int hr = hb * TEAMS + team, h = g * a.R + hr;

  __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * kKsLd];    // k^ rows
  __shared__ __attribute__((aligned(16))) uint16_t KTs[128 * kKTLd];  // k^ transposed
  __shared__ __attribute__((aligned(16))) float Am_[TEAMS][64 * kFLd];  // A; later T', T''; Wk staging
  __shared__ __attribute__((aligned(16))) float Tm_[TEAMS][64 * kFLd];  // T; later V^ transposed
  __shared__ float Xs_[TEAMS][4][256];
  __shared__ float Gs_[TEAMS][64], Bs_[TEAMS][64];
  float* Am = Am_[team];
  float* Tm = Tm_[team];
  float (*Xs)[256] = Xs_[team];
  float* Gs = Gs_[team];
  float* Bs = Bs_[team];

  // ---- load k^ (row-major and transposed; all teams) and prefetch v^; alpha/beta -> G ----
  // piece (t = idx % 64, sg = idx / 64) of idx = tid + 256 TEAMS it: a wave handles one column
  // segment of all 64 rows, so its transposed 2-byte LDS writes cover 128 contiguous bytes.
  const int64_t krow = int64_t(a.hk) * 128;
  const int64_t vrow = int64_t(a.hv) * 128;
  // decay and write strength of this chunk (wave 0 of the team scans them), issued with the loads
  float la_raw = 1.f, be_raw = 0.f;
  if (w == 0 && lane < len) {
    la_raw = a.alpha[(start + lane) * a.hv + h];
    be_raw = a.beta[(start + lane) * a.hv + h];
  }
  uint4 vv[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int t = lane, sg = w + 4 * it;
    vv[it] = make_uint4(0, 0, 0, 0);
    if (t < len) vv[it] = *reinterpret_cast<const uint4*>(a.vhat + (start + t) * vrow + h * 128 + sg * 8);
  }
#pragma unroll
  for (int it = 0; it < (1024 + 256 * TEAMS - 1) / (256 * TEAMS); ++it) {
    const int idx = tid + 256 * TEAMS * it;
    if (idx >= 1024) break;
    const int t = idx & 63, sg = idx >> 6;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (t < len) v = *reinterpret_cast<const uint4*>(a.khat + (start + t) * krow + g * 128 + sg * 8);
    *reinterpret_cast<uint4*>(&Ks[t * kKsLd + sg * 8]) = v;
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      KTs[(sg * 8 + 2 * e) * kKTLd + t] = uint16_t(wv[e] & 0xffffu);
      KTs[(sg * 8 + 2 * e + 1) * kKTLd + t] = uint16_t(wv[e] >> 16);
    }
  }
  if (w == 0) {
    float la = lane < len ? logf(la_raw) : 0.f;
    const float be = be_raw;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(la, o, 64);
      if (lane >= o) la += y;
    }
    Gs[lane] = la;
    Bs[lane] = be;
    a.G[(int64_t(c) * a.hv + h) * 64 + lane] = la;
  }
  __syncthreads();

  // K^T of the chunk for the state pass, written once per QK head
  if (hr == 0) {
    uint16_t* dst = a.KT + (int64_t(c) * a.hk + g) * 128 * 64;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = ttid + it * 256;  // 128 rows x 8 segments
      const int r = idx >> 3, sg = idx & 7;
      *reinterpret_cast<uint4*>(dst + r * 64 + sg * 8) = *reinterpret_cast<const uint4*>(&KTs[r * kKTLd + sg * 8]);
    }
  }

  // ---- Gram k^ k^T (lower block triangle) on MFMA -> A[t,i] = beta_t exp(G_t - G_i) k_t.k_i, i < t
  for (int nt = 0; nt < 4; ++nt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (nt <= w) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const short8 av = ld_short8(&Ks[(16 * w + li) * kKsLd + 32 * s + 8 * lq]);
        const short8 bv = ld_short8(&Ks[(16 * nt + li) * kKsLd + 32 * s + 8 * lq]);
        acc = mfma16x16x32(av, bv, acc);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * w + 4 * lq + r, i = 16 * nt + li;
      Am[t * kFLd + i] = (i < t) ? Bs[t] * __expf(Gs[t] - Gs[i]) * acc[r] : 0.f;
    }
  }

  __syncthreads();

  // ---- diagonal 16x16 blocks: D_w = (I + A_ww)^-1 by forward substitution, lane = column ----
  {
    const int b0 = 16 * w;
    if (lane < 16) {
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = (r == lane) ? 1.f : 0.f;
#pragma unroll
        for (int s = 0; s < r; ++s) v -= Am[(b0 + r) * kFLd + b0 + s] * x[s];
        x[r] = v;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) Tm[(b0 + r) * kFLd + b0 + lane] = x[r];
    }
    // zero the blocks above the diagonal in this block row
    for (int idx = lane; idx < 16 * 64; idx += 64) {
      const int r = idx >> 6, col = idx & 63;
      if (col >= b0 + 16) Tm[(b0 + r) * kFLd + col] = 0.f;
    }
  }
  __syncthreads();
  // ---- off-diagonal blocks, level by level ----
  if (w < 3) wy_offdiag(Am, Tm, Xs[w], w + 1, w, lane);         // T10, T21, T32
  __syncthreads();
  if (w < 2) wy_offdiag(Am, Tm, Xs[w], w + 2, w, lane);         // T20, T31
  __syncthreads();
  if (w == 0) wy_offdiag(Am, Tm, Xs[w], 3, 0, lane);            // T30
  __syncthreads();

  // ---- T' = T diag(beta), T'' = T diag(beta gamma) in bf16 over A; then V^ transposed over T ----
  uint16_t* T1 = reinterpret_cast<uint16_t*>(Am);  // [64][72]
  uint16_t* T2 = T1 + 64 * kKTLd;                  // [64][72]
  for (int idx = ttid; idx < 64 * 64; idx += 256) {
    const int t = idx >> 6, i = idx & 63;
    const float tv = Tm[t * kFLd + i];
    const float b = Bs[i];
    T1[t * kKTLd + i] = f2bf(tv * b);
    T2[t * kKTLd + i] = f2bf(tv * b * __expf(Gs[i]));
  }
  __syncthreads();  // T is read completely
  uint16_t* VTs = reinterpret_cast<uint16_t*>(Tm);  // [128][72]
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int t = lane, sg = w + 4 * it;
    const uint32_t wv[4] = {vv[it].x, vv[it].y, vv[it].z, vv[it].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      VTs[(sg * 8 + 2 * e) * kKTLd + t] = uint16_t(wv[e] & 0xffffu);
      VTs[(sg * 8 + 2 * e + 1) * kKTLd + t] = uint16_t(wv[e] >> 16);
    }
  }
  __syncthreads();

  // ---- U = T' V^, Wk = T'' K^  (rows 16w.., all 128 columns) ----
  f32x4 accU[8], accW[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    accU[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    accW[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const short8 a1 = ld_short8(&T1[(16 * w + li) * kKTLd + 32 * s + 8 * lq]);
    const short8 a2 = ld_short8(&T2[(16 * w + li) * kKTLd + 32 * s + 8 * lq]);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const short8 bv = ld_short8(&VTs[(16 * nt + li) * kKTLd + 32 * s + 8 * lq]);
      const short8 bk = ld_short8(&KTs[(16 * nt + li) * kKTLd + 32 * s + 8 * lq]);
      accU[nt] = mfma16x16x32(a1, bv, accU[nt]);
      accW[nt] = mfma16x16x32(a2, bk, accW[nt]);
    }
  }
  // U goes out in this accumulator layout, [wave][16-col tile][lane][4 rows], which is exactly how
  // the state pass consumes it (8 contiguous bytes per lane).
  uint16_t* Ug = a.U + (int64_t(c) * a.hv + h) * 64 * 128;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt)
    *reinterpret_cast<uint2*>(Ug + ((w * 8 + nt) * 64 + lane) * 4) =
        make_uint2(pack_bf16x2(accU[nt][0], accU[nt][1]), pack_bf16x2(accU[nt][2], accU[nt][3]));
  // T', T'' are dead once every wave of the team is done with them: stage Wk over them
  __syncthreads();
  uint16_t* Ws = reinterpret_cast<uint16_t*>(Am);  // [64][136]
  constexpr int kOLd = 136;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * w + 4 * lq + r, col = 16 * nt + li;
      Ws[t * kOLd + col] = f2bf(accW[nt][r]);
    }
  }
  __syncthreads();
  uint16_t* Wg = a.Wk + (int64_t(c) * a.hv + h) * 64 * 128;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int idx = ttid + it * 256;
    const int t = idx >> 4, sg = idx & 15;
    *reinterpret_cast<uint4*>(Wg + t * 128 + sg * 8) = *reinterpret_cast<const uint4*>(&Ws[t * kOLd + sg * 8]);
  }
}

hipError_t launch_wy(const Problem& p, const Workspace& ws, const float* alpha, const float* beta,
                     hipStream_t s) {
  if (p.nc_max == 0) return hipSuccess;
  const int R = p.hv / p.hk;
  const int64_t units = p.nc_max * p.hk;
  WyArgs a{ws.chunk_tab, int(units), p.hk, p.hv, R, static_cast<const uint16_t*>(ws.khat),
           static_cast<const uint16_t*>(ws.vhat), alpha, beta, ws.G, ws.Wk, ws.U, ws.KT};
  // value heads per block: three teams fill the LDS of a CU
  if (R % 3 == 0) hipLaunchKernelGGL(k_wy<3>, dim3(unsigned(xcd_blocks(units, R / 3))), dim3(768), 0, s, a);
  else if (R % 2 == 0) hipLaunchKernelGGL(k_wy<2>, dim3(unsigned(xcd_blocks(units, R / 2))), dim3(512), 0, s, a);
  else hipLaunchKernelGGL(k_wy<1>, dim3(unsigned(xcd_blocks(units, R))), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace gdn
