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
// Steps: k^ k^T on bf16 MFMA (fp32 accumulate) -> A; the 16x16 diagonal blocks of I + A inverted
// in fp32 by forward substitution (D_i); then [U | Wk] solves (I + A) X = [diag(beta) V | diag(beta
// gamma) K] by block forward substitution over the four 16-token blocks,
//     X_i = D_i (B_i - sum_{k<i} A_ik X_k),
// on bf16 MFMA (fp32 accumulate), each wave owning four of the sixteen 16-column tiles of X, so
// the blocks X_k it needs stay in its registers.
// Rows past the end of a partial chunk carry beta = 0 and ln alpha = 0, so their U and Wk rows are
// zero and G stays at the last real token.
//
// A block holds TEAMS teams of 4 waves, one per value head of its batch; all teams run the same
// steps in lockstep (block-wide barriers), each on its own LDS region. k^ and v^ are loaded as
// whole token rows and kept row-major in LDS; the substitution reads them as transposed MFMA
// operands with LDS transpose reads.
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
  uint16_t *U;                    // [nc][hv][8 column tiles][2 token slabs][64 lanes][8 tokens]
  uint16_t* KT;                   // [nc][hk][128][64]
};

constexpr int kKsLd = 144;   // bf16 row stride of the 64x128 k^ and v^ tiles
constexpr int kKTLd = 72;    // bf16 row stride of the transposed 128x64 k^ tile and of -A

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
  // per team: -A in bf16 with D_i on the diagonal blocks; A's diagonal blocks in fp32; v^ rows
  // (later the Wk staging)
  __shared__ __attribute__((aligned(16))) uint16_t Ab_[TEAMS][64 * kKTLd];
  __shared__ __attribute__((aligned(16))) float Df_[TEAMS][4][16][16];
  __shared__ __attribute__((aligned(16))) uint16_t Vs_[TEAMS][64 * kKsLd];
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
  // raw inputs of an item, as 16-byte pieces of whole token rows (a wave load covers four 256-byte
  // rows): k^ pieces idx = tid + 256 TEAMS j, v^ pieces idx = ttid + 256 j of this team's head, each
  // token idx / 16, segment idx % 16; alpha and beta (wave 0 of a team)
  uint4 kv[kKIt], vv[4];
  float la_raw = 1.f, be_raw = 0.f;
  auto fetch_k = [&](int item) {
    if (item >= n_items) return;
    const Item it = decode(item);
#pragma unroll
    for (int j = 0; j < kKIt; ++j) {
      const int idx = tid + 256 * TEAMS * j, t = idx >> 4, sg = idx & 15;
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
      const int idx = ttid + 256 * j, t = idx >> 4, sg = idx & 15;
      vv[j] = make_uint4(0, 0, 0, 0);
      if (t < it.len)
        vv[j] = *reinterpret_cast<const uint4*>(a.vhat + (it.start + t) * vrow + it.h * 128 + sg * 8);
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
    uint16_t* const Ab = Ab_[team] + z;
    float (*const Df)[16][16] = reinterpret_cast<float (*)[16][16]>(&Df_[team][0][0][0] + z);
    uint16_t* const Vs = Vs_[team] + z;
    float* const Gs = Gs_[team] + z;
    float* const Bs = Bs_[team] + z;
    float* const Cs = Cs_[team] + z;  // beta exp(G)
    if (len <= 0) {  // past the last chunk (uniform over the block)
      fetch_k(item + gridDim.x);
      fetch_v(item + gridDim.x);
      continue;
    }

  // ---- k^ and v^ rows into LDS; alpha/beta -> G ----
#pragma unroll
  for (int j = 0; j < kKIt; ++j) {
    const int idx = tid + 256 * TEAMS * j;
    if (idx >= 1024) break;
    *reinterpret_cast<uint4*>(&Ks[(idx >> 4) * kKsLd + (idx & 15) * 8]) = kv[j];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int idx = ttid + 256 * j;
    *reinterpret_cast<uint4*>(&Vs[(idx >> 4) * kKsLd + (idx & 15) * 8]) = vv[j];
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
  fetch_k(item + gridDim.x);  // the next item's inputs fly while this one is transformed
  fetch_v(item + gridDim.x);

  // K^T of the chunk for the state pass, formed by transpose reads of the k^ rows: read q of the
  // 32 (16 channels x 16 tokens) covers channels 16 (q % 8) .., tokens 16 (q / 8) + 4 lq .. +3
  for (int q = tid >> 6; q < 32; q += 4 * TEAMS) {
    const int cb = q & 7, tb = q >> 3;
    const short4v v = ld_tr16(&Ks[(16 * tb + 4 * lq + (li >> 2)) * kKsLd + 16 * cb + 4 * (li & 3)]);
    *reinterpret_cast<short4v*>(&KTs[(16 * cb + li) * kKTLd + 16 * tb + 4 * lq]) = v;
  }

  // ---- Gram k^ k^T (lower block triangle) on MFMA; A[t,i] = beta_t exp(G_t - G_i) k_t.k_i, i < t:
  // -A in bf16 for the off-diagonal blocks, A in fp32 for the diagonal ones
  for (int nt = 0; nt < 4; ++nt) {
    if (nt > w) break;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const short8 av = ld_short8(&Ks[(16 * w + li) * kKsLd + 32 * s + 8 * lq]);
      const short8 bv = ld_short8(&Ks[(16 * nt + li) * kKsLd + 32 * s + 8 * lq]);
      acc = mfma16x16x32(av, bv, acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * w + 4 * lq + r, i = 16 * nt + li;
      const float av = (i < t) ? Bs[t] * __expf(Gs[t] - Gs[i]) * acc[r] : 0.f;
      if (nt < w) Ab[t * kKTLd + i] = f2bf(-av);
      else Df[w][4 * lq + r][li] = av;
    }
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

  // ---- D_w = (I + A_ww)^-1 by forward substitution, lane = column; into Ab's diagonal block ----
  if (lane < 16) {
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v = (r == lane) ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < r; ++s) v -= Df[w][r][s] * x[s];
      x[r] = v;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Ab[(16 * w + r) * kKTLd + 16 * w + lane] = f2bf(x[r]);
  }
  __syncthreads();

  // ---- X = [U | Wk] by block forward substitution. Wave w owns column tiles 4w .. 4w+3 of the 16:
  // tiles 0-7 of U (source V^, row scale beta), tiles 8-15 of Wk (source K^, row scale beta gamma).
  // A tile (rows 16i.., 16 columns) is kept as the bf16 MFMA operand xb[i][j]: lane (c, q) holds
  // rows 16i + 4q .. +3 of column c, which is both the accumulator layout and the B-operand layout
  // of the 16x16x16 MFMA.
  const bool wk_tiles = w >= 2;
  const uint16_t* src = wk_tiles ? Ks : Vs;  // sources [token][column]
  const float* rs = wk_tiles ? Cs : Bs;
  const int col0 = 16 * (4 * w - (wk_tiles ? 8 : 0));  // first source column of this wave
  short4v xb[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 sc = *reinterpret_cast<const float4*>(&rs[16 * i + 4 * lq]);
    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // column col0 + 16j + li, tokens 16i + 4lq .. +3
      const short4v sv = ld_tr16(&src[(16 * i + 4 * lq + (li >> 2)) * kKsLd + col0 + 16 * j + 4 * (li & 3)]);
      acc[j] = f32x4{bf2f(sv[0]) * sc.x, bf2f(sv[1]) * sc.y, bf2f(sv[2]) * sc.z, bf2f(sv[3]) * sc.w};
    }
#pragma unroll
    for (int k = 0; k < i; ++k) {  // acc -= A_ik X_k  (Ab holds -A)
      const short4v af = ld_short4(&Ab[(16 * i + li) * kKTLd + 16 * k + 4 * lq]);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = mfma16x16x16(af, xb[k][j], acc[j]);
    }
    const short4v df = ld_short4(&Ab[(16 * i + li) * kKTLd + 16 * i + 4 * lq]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 x = mfma16x16x16(df, pack4(acc[j]), f32x4{0.f, 0.f, 0.f, 0.f});
      xb[i][j] = pack4(x);
    }
  }

  // U goes out as the state pass's 16-byte pieces: piece (column tile j, token slab s), lane
  // (i, q) holds tokens 32s + 8q .. +7 of column 16j + i. This lane's rows 16ib + 4lq .. +3 are
  // the half 4 (lq % 2) .. +3 of the piece of lane (li, 2 (ib % 2) + lq / 2) in slab ib / 2.
  if (!wk_tiles) {
    uint16_t* Ug = a.U + (int64_t(c) * a.hv + h) * 64 * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int sl = i >> 1, q = 2 * (i & 1) + (lq >> 1);
        *reinterpret_cast<short4v*>(Ug + (((4 * w + j) * 2 + sl) * 64 + q * 16 + li) * 8 + 4 * (lq & 1)) = xb[i][j];
      }
  }
  __syncthreads();  // the v^ rows are dead: stage Wk over them
  uint16_t* Ws = Vs;  // [64][136]
  constexpr int kOLd = 136;
  if (wk_tiles) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          Ws[(16 * i + 4 * lq + r) * kOLd + col0 + 16 * j + li] = uint16_t(xb[i][j][r]);
  }
  __syncthreads();
  uint16_t* Wg = a.Wk + (int64_t(c) * a.hv + h) * 64 * 128;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int idx = ttid + it * 256;
    const int t = idx >> 4, sg = idx & 15;
    *reinterpret_cast<uint4*>(Wg + t * 128 + sg * 8) = *reinterpret_cast<const uint4*>(&Ws[t * kOLd + sg * 8]);
  }
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
