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
#include <algorithm>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

struct WyArgs {
  int n_units;                    // chunks x QK heads
  int hk, hv, R;
  const uint16_t *khat, *vhat;    // bf16 [T][hk][128], [T][hv][128]
  const float *alpha, *beta;      // [T][hv]
  float* G;                       // [nc][hv][64]
  uint16_t *Wk;                   // [nc][hv][64][128]
  uint16_t *U;                    // [nc][hv][4 waves][4 tile pairs][64 lanes][2 tiles][4 rows]
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

// Block b works through the items b, b + gridDim.x, ... (one item = chunk, QK head and batch of
// TEAMS value heads) with one block per CU; the raw inputs of its next item are loaded into
// registers while the current one is transformed, so loads overlap compute.
template <int TEAMS>
__global__ void __launch_bounds__(256 * TEAMS) k_wy(WyArgs a, const int4* __restrict__ tab) {
  constexpr int kKIt = (1024 + 256 * TEAMS - 1) / (256 * TEAMS);  // k^ pieces per thread
  const int tid = threadIdx.x, lane = tid & 63, team = tid >> 8, w = (tid >> 6) & 3;
  const int ttid = tid & 255;  // thread index inside the team
  const int li = lane & 15, lq = lane >> 4;
  const int nb = a.R / TEAMS;  // batches of value heads per QK head
  const int n_items = a.n_units * nb;
  const int64_t krow = int64_t(a.hk) * 128;
  const int64_t vrow = int64_t(a.hv) * 128;

  __shared__ __attribute__((aligned(16))) uint16_t Ks_[64 * kKsLd];    // k^ rows
  __shared__ __attribute__((aligned(16))) uint16_t KTs_[128 * kKTLd];  // k^ transposed
  __shared__ __attribute__((aligned(16))) float Am_[TEAMS][64 * kFLd];  // A; later T', T''; Wk staging
  __shared__ __attribute__((aligned(16))) float Tm_[TEAMS][64 * kFLd];  // T; later V^ transposed
  __shared__ float Xs_[TEAMS][4][256];
  __shared__ __attribute__((aligned(16))) float Gs_[TEAMS][64], Bs_[TEAMS][64], Cs_[TEAMS][64];

  // item -> chunk c, QK head g, this thread's value head h; chunk start and length
  struct Item { int c, g, hr, h, len; int64_t start; };
  auto decode = [&](int item) {
    Item it;
    const int u = item / nb, hb = item - u * nb;
    it.c = u / a.hk;
    it.g = u - it.c * a.hk;
    it.hr = hb * TEAMS + team;
    it.h = it.g * a.R + it.hr;
    const int4 ct = tab[it.c];  // wave-uniform address: a scalar load
    it.start = ct.x;
    it.len = ct.y;
    return it;
  };
  // raw inputs of an item: k^ pieces (t = idx % 64, segment idx / 64 of idx = tid + 256 TEAMS j; a
  // wave covers one column segment of all 64 rows, so its transposed LDS writes are contiguous),
  // v^ pieces (t = lane, segment w + 4j of this team's head), alpha and beta (wave 0 of a team)
  uint4 kv[kKIt], vv[4];
  float la_raw = 1.f, be_raw = 0.f;
  auto fetch_k = [&](int item) {
    if (item >= n_items) return;
    const Item it = decode(item);
#pragma unroll
    for (int j = 0; j < kKIt; ++j) {
      const int idx = tid + 256 * TEAMS * j, t = idx & 63, sg = idx >> 6;
      kv[j] = make_uint4(0, 0, 0, 0);
      if (idx < 1024 && t < it.len)
        kv[j] = *reinterpret_cast<const uint4*>(a.khat + (it.start + t) * krow + it.g * 128 + sg * 8);
    }
  };
  auto fetch_v = [&](int item) {
    if (item >= n_items) return;
    const Item it = decode(item);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vv[j] = make_uint4(0, 0, 0, 0);
      if (lane < it.len)
        vv[j] = *reinterpret_cast<const uint4*>(a.vhat + (it.start + lane) * vrow + it.h * 128 + (w + 4 * j) * 8);
    }
    la_raw = 1.f;
    be_raw = 0.f;
    if (w == 0 && lane < it.len) {
      la_raw = a.alpha[(it.start + lane) * a.hv + it.h];
      be_raw = a.beta[(it.start + lane) * a.hv + it.h];
    }
  };

  int item = blockIdx.x;
  fetch_k(item);
  fetch_v(item);
  for (; item < n_items; item += gridDim.x) {
    const Item it = decode(item);
    const int c = it.c, g = it.g, hr = it.hr, h = it.h, len = it.len;
    const int64_t start = it.start;
    // Thread indices and LDS views are rebuilt from an opaque zero in each item, so that the
    // compiler recomputes their many per-lane derivatives instead of keeping them all live across
    // the item loop (more registers than the three-team block has).
    int z;
    asm volatile("s_mov_b32 %0, 0" : "=s"(z));
    const int tid = int(threadIdx.x) + z, lane = tid & 63, w = (tid >> 6) & 3, ttid = tid & 255;
    const int li = lane & 15, lq = lane >> 4;
    uint16_t* const Ks = Ks_ + z;
    uint16_t* const KTs = KTs_ + z;
    float* const Am = Am_[team] + z;
    float* const Tm = Tm_[team] + z;
    float (*const Xs)[256] = reinterpret_cast<float (*)[256]>(&Xs_[team][0][0] + z);
    float* const Gs = Gs_[team] + z;
    float* const Bs = Bs_[team] + z;
    float* const Cs = Cs_[team] + z;  // beta exp(G)
    if (len <= 0) {  // past the last chunk (uniform over the block)
      fetch_k(item + gridDim.x);
      fetch_v(item + gridDim.x);
      continue;
    }

  // ---- k^ into LDS (row-major and transposed; all teams); alpha/beta -> G ----
#pragma unroll
  for (int j = 0; j < kKIt; ++j) {
    const int idx = tid + 256 * TEAMS * j;
    if (idx >= 1024) break;
    const int t = idx & 63, sg = idx >> 6;
    const uint4 v = kv[j];
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
    Cs[lane] = be * __expf(la);
    a.G[(int64_t(c) * a.hv + h) * 64 + lane] = la;
  }
  __syncthreads();
  fetch_k(item + gridDim.x);  // the next item's k^ flies while this one is transformed

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
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // 4 consecutive columns per thread and pass
    const int idx = ttid + 256 * j, t = idx >> 4, i0 = (idx & 15) * 4;
    const float4 tv = *reinterpret_cast<const float4*>(&Tm[t * kFLd + i0]);
    const float4 b = *reinterpret_cast<const float4*>(&Bs[i0]);
    const float4 cg = *reinterpret_cast<const float4*>(&Cs[i0]);
    *reinterpret_cast<uint2*>(&T1[t * kKTLd + i0]) =
        make_uint2(pack_bf16x2(tv.x * b.x, tv.y * b.y), pack_bf16x2(tv.z * b.z, tv.w * b.w));
    *reinterpret_cast<uint2*>(&T2[t * kKTLd + i0]) =
        make_uint2(pack_bf16x2(tv.x * cg.x, tv.y * cg.y), pack_bf16x2(tv.z * cg.z, tv.w * cg.w));
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

  // ---- U = T' V^, then Wk = T'' K^  (rows 16w.., all 128 columns), one accumulator set at a time
  f32x4 acc[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const short8 a1 = ld_short8(&T1[(16 * w + li) * kKTLd + 32 * s + 8 * lq]);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
      acc[nt] = mfma16x16x32(a1, ld_short8(&VTs[(16 * nt + li) * kKTLd + 32 * s + 8 * lq]), acc[nt]);
  }
  fetch_v(item + gridDim.x);  // V^ of this item is in LDS; the next item's flies meanwhile
  // U goes out in this accumulator layout, tiles paired: [wave][tile pair][lane][2 tiles][4 rows],
  // which is how the state pass consumes it (16 contiguous bytes per lane)
  uint16_t* Ug = a.U + (int64_t(c) * a.hv + h) * 64 * 128;
#pragma unroll
  for (int p = 0; p < 4; ++p)
    *reinterpret_cast<uint4*>(Ug + ((w * 4 + p) * 64 + lane) * 8) =
        make_uint4(pack_bf16x2(acc[2 * p][0], acc[2 * p][1]), pack_bf16x2(acc[2 * p][2], acc[2 * p][3]),
                   pack_bf16x2(acc[2 * p + 1][0], acc[2 * p + 1][1]),
                   pack_bf16x2(acc[2 * p + 1][2], acc[2 * p + 1][3]));
  // Wk^T = K^T T''^T with the rows of K^T (channels) in the order pi: accumulator tiles 2s, 2s + 1
  // of lane (token 16w + li, lq) hold Wk[token][32s + 8lq .. +7], stored as one 16-byte piece
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const short8 b2 = ld_short8(&T2[(16 * w + li) * kKTLd + 32 * s + 8 * lq]);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
      acc[nt] = mfma16x16x32(ld_short8(&KTs[pi32(16 * nt + li) * kKTLd + 32 * s + 8 * lq]), b2, acc[nt]);
  }
  uint16_t* Wg = a.Wk + (int64_t(c) * a.hv + h) * 64 * 128 + (16 * w + li) * 128 + 8 * lq;
#pragma unroll
  for (int s = 0; s < 4; ++s) *reinterpret_cast<short8*>(Wg + 32 * s) = pack8(acc[2 * s], acc[2 * s + 1]);
  __syncthreads();  // every read of this item's LDS is done before the next item overwrites it
  }  // items
}

static int cu_count() {
  // one entry per device; hipDeviceGetAttribute is cheap, so a race only repeats the query
  static int counts[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (counts[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    counts[dev] = n;
  }
  return counts[dev];
}

hipError_t launch_wy(const Problem& p, const Workspace& ws, const float* alpha, const float* beta,
                     hipStream_t s) {
  if (p.nc_max == 0) return hipSuccess;
  const int R = p.hv / p.hk;
  const int64_t units = p.nc_max * p.hk;
  WyArgs a{int(units), p.hk, p.hv, R, static_cast<const uint16_t*>(ws.khat),
           static_cast<const uint16_t*>(ws.vhat), alpha, beta, ws.G, ws.Wk, ws.U, ws.KT};
  // value heads per block: three teams fill the LDS of a CU, so one block per CU (two with one
  // team), each working through its share of the items
  const int teams = R % 3 == 0 ? 3 : (R % 2 == 0 ? 2 : 1);
  const int64_t items = units * (R / teams);
  const unsigned grid = unsigned(std::min<int64_t>(items, int64_t(cu_count()) * (teams == 1 ? 2 : 1)));
  if (teams == 3) hipLaunchKernelGGL(k_wy<3>, dim3(grid), dim3(768), 0, s, a, ws.chunk_tab);
  else if (teams == 2) hipLaunchKernelGGL(k_wy<2>, dim3(grid), dim3(512), 0, s, a, ws.chunk_tab);
  else hipLaunchKernelGGL(k_wy<1>, dim3(grid), dim3(256), 0, s, a, ws.chunk_tab);
  return hipGetLastError();
}

}  // namespace gdn
