// Chunked backward of the gated delta rule (fp32, d_k = d_v = 128, 64-token chunks).
//
// The forward recurrence of the analysis notes "Qwen3.8-Flash-Next：架构、效率与技术谱系" (§03 update
// equations) re-associates, per chunk with chunk-start state S, G_t = sum_{s<=t} ln alpha_s, g = exp(G),
// E[t,i] = exp(G_t - G_i), kd_i = exp(G_C - G_i) (C the chunk's last row), into
//     A  = strict_lower(beta_t E[t,i] k_t.k_i),  T = (I + A)^-1,  U = T diag(beta) V,  Wk = T diag(beta g) K,
//     W  = U - Wk S,   P = lower(E o Q K^T),   Y = scale (diag(g) Q S + P W),   S' = g_C S + K^T diag(kd) W.
// Reverse mode takes these statements last to first. With dY scaled by `scale` and dS' the derivative of
// the state after the chunk, the only sequential part is
//     dW = diag(kd) K dS' + P^T dY,        dS = g_C dS' + Q^T diag(g) dY - Wk^T dW,
// a pass over the chunks in reverse, independent per value column like the forward. Everything else is
// chunk-parallel products of 64 x 64 and 64 x 128 tiles:
//     dK~ = W dS'^T, dQ = diag(g) dY S^T + (dP o E) K, dP = lower(dY W^T), dWk = -dW S^T,
//     dT = dW (beta V)^T + dWk (beta g K)^T, d(beta V) = T^T dW, d(beta g K) = T^T dWk,
//     dA = -strict_lower(T^T dT T^T), and the rows' k, beta and G terms of A, E, g, kd;
// then d ln alpha_s = sum_{t >= s} dG_t within the chunk (G is a within-chunk prefix sum).
//
// Only chunk-level states are kept (S and dS' per chunk and value head, O(chunks x heads x 128^2)); the
// forward's own chunk quantities (T, U, Wk, W, P) are reused by the backward. Each product runs as one
// launch of a batched kernel over all (chunk, value head) items, one block per item with both operands
// staged in LDS; the two chunk passes run one block per (sequence, value head, 16-column slice).
#include <atomic>
#include <initializer_list>

#include "ext_internal.h"
#include "gdn_device.h"

namespace gdn {

namespace {

constexpr int kC = 64, kD = 128, kSl = 32;  // chunk, head dim, value columns per slice of the chunk passes
constexpr int kCT = kSl / 16;                // 16-column tiles of a slice
constexpr int kSlices = kD / kSl;

// ---- chunk table: seq_off[n] = first chunk of sequence n; tab[c] = (start token, length, sequence) ----
// Offsets stop at nc_max, so boundaries that break the contract (decreasing, overlapping) drop chunks
// rather than index past the table.
__global__ void __launch_bounds__(64) k_cb_offsets(const int32_t* __restrict__ cu, int n_seqs, int64_t T,
                                                   int64_t nc_max, int32_t* __restrict__ seq_off) {
  if (threadIdx.x != 0) return;
  int64_t off = 0;
  for (int n = 0; n < n_seqs; ++n) {
    const int64_t s0 = min<int64_t>(max<int64_t>(cu[n], 0), T), s1 = min<int64_t>(max<int64_t>(cu[n + 1], s0), T);
    seq_off[n] = int32_t(off);
    off = min<int64_t>(off + (s1 - s0 + kC - 1) / kC, nc_max);
  }
  seq_off[n_seqs] = int32_t(off);
}

// one block per sequence, and block n_seqs marks the unused slots
__global__ void __launch_bounds__(256) k_cb_table(const int32_t* __restrict__ cu, int n_seqs, int64_t T,
                                                  int64_t nc_max, const int32_t* __restrict__ seq_off,
                                                  int4* __restrict__ tab) {
  const int n = blockIdx.x;
  if (n == n_seqs) {
    for (int64_t c = seq_off[n_seqs] + threadIdx.x; c < nc_max; c += blockDim.x) tab[c] = make_int4(0, 0, -1, 0);
    return;
  }
  const int64_t s0 = min<int64_t>(max<int64_t>(cu[n], 0), T), s1 = min<int64_t>(max<int64_t>(cu[n + 1], s0), T);
  const int64_t c0 = seq_off[n], nch = seq_off[n + 1] - c0;
  for (int64_t j = threadIdx.x; j < nch; j += blockDim.x)
    tab[c0 + j] = make_int4(int(s0 + j * kC), int(min<int64_t>(kC, s1 - s0 - j * kC)), n, 0);
}

// ---- gather: per item (chunk c, value head h), zero-padded 64-row tiles and the decay prefix ----
// what: 1 = the forward's inputs (Q, K, V, G, beta), 2 = dY
__global__ void __launch_bounds__(256) k_cb_gather(CBwdArgs a, int what) {
  const int64_t item = blockIdx.x;
  const int c = int(item / a.hv), h = int(item - int64_t(c) * a.hv), g = h / a.R;
  const int4 ct = a.tab[c];
  const int len = ct.y;
  if (len <= 0) return;
  const int64_t s = ct.x;
  const int tid = threadIdx.x;
  const int64_t qrow = int64_t(a.hk) * kD, vrow = int64_t(a.hv) * kD;
  for (int idx = tid; idx < kC * kD / 4; idx += 256) {
    const int t = idx / (kD / 4), c4 = (idx % (kD / 4)) * 4;
    const int64_t o = item * (kC * kD) + t * kD + c4;
    if (what & 1) {
      float4 qv = make_float4(0.f, 0.f, 0.f, 0.f), kv = qv, vv = qv;
      if (t < len) {
        qv = *reinterpret_cast<const float4*>(a.q + (s + t) * qrow + g * kD + c4);
        kv = *reinterpret_cast<const float4*>(a.k + (s + t) * qrow + g * kD + c4);
        vv = *reinterpret_cast<const float4*>(a.v + (s + t) * vrow + h * kD + c4);
      }
      *reinterpret_cast<float4*>(a.Qi + o) = qv;
      *reinterpret_cast<float4*>(a.Ki + o) = kv;
      *reinterpret_cast<float4*>(a.Vi + o) = vv;
    }
    if (what & 2) {
      float4 dv = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t < len) {
        dv = *reinterpret_cast<const float4*>(a.dy + (s + t) * vrow + h * kD + c4);
        dv.x *= a.scale; dv.y *= a.scale; dv.z *= a.scale; dv.w *= a.scale;
      }
      *reinterpret_cast<float4*>(a.dYi + o) = dv;
    }
  }
  if ((what & 1) && tid < 64) {  // padded rows: ln alpha = 0 (G stays), beta = 0
    float la = 0.f, be = 0.f;
    if (tid < len) {
      la = logf(a.alpha[(s + tid) * a.hv + h]);
      be = a.beta[(s + tid) * a.hv + h];
    }
    float G = la;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(G, o, 64);
      if (tid >= o) G += y;
    }
    a.G[item * kC + tid] = G;
    a.bt[item * kC + tid] = be;
  }
}

// ---- batched products: per item, up to three jobs C (64 x N) = alpha op(A) op(B) (+ C) ----
// A job with `chain` set adds its product to the previous job's instead of storing its own; the last
// job of a chain stores the sum with the first job's C, alpha, mask and accumulate settings.
struct MmJob {
  const float* A;
  const float* B;
  float* C;
  float* C2;           // optional transposed copy of C, stored [N][64]
  int64_t sA, sB, sC;  // per-item strides (floats); C2 uses sC
  int lda, ldb, ldc;   // row strides of the stored matrices
  float alpha;
  int accumulate;      // add C's previous contents
  int mask;            // 0: none; 1: keep m >= n; 2: keep m > n
  int chain;
  int reuse_b;         // same B as the previous job: not staged again
};
struct MmJobs {
  MmJob j[3];
  int n;
};

// One block per (item, NB-column block of C), four waves; wave w computes rows 16w .. 16w + 15 of C over the
// block's NB columns on 16x16x4 fp32 MFMAs. The N / NB blocks of an item are numbered onto one XCD, so the
// op(A) rows they all read come from HBM once; narrow blocks keep the LDS tile and the accumulators small,
// so more blocks share a CU and one block's loads overlap another's products. op(B) is staged in LDS as [K][N + 4] (the four lane groups of an operand read hit distinct
// banks); each wave reads its own rows of op(A) straight into registers. At step (p, c) lane group q contributes contraction index 16p + 4q + c, so a
// row-major A gives each lane float4 runs.
template <int N, int NB, int K, bool TA, bool TB>
__global__ void __launch_bounds__(256) k_cb_mm(MmJobs jobs, const int4* __restrict__ tab, int hv, int64_t items) {
  constexpr int kLd = NB + 4;
  extern __shared__ __attribute__((aligned(16))) float Bs[];  // [K][kLd]: Bs[k][n] = op(B)[k][n0 + n]
  int unit, half;
  xcd_item(int(blockIdx.x), N / NB, unit, half);
  const int64_t item = unit;
  if (item >= items || tab[item / hv].y <= 0) return;
  const int n0 = NB * half;  // first column of C in this block
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lm = lane & 15, lg = lane >> 4;
  // this wave's A operands: op(A)[16w + lm][16p + 4lg + c]
  auto load_a = [&](const MmJob& jb, float (&av)[K / 16][4]) {
    const float* A = jb.A + item * jb.sA;
#pragma unroll
    for (int p = 0; p < K / 16; ++p) {
      if (!TA) {
        const float4 v = *reinterpret_cast<const float4*>(A + int64_t(16 * w + lm) * jb.lda + 16 * p + 4 * lg);
        av[p][0] = v.x; av[p][1] = v.y; av[p][2] = v.z; av[p][3] = v.w;
      } else {  // A stored [K][64]
#pragma unroll
        for (int c = 0; c < 4; ++c) av[p][c] = A[int64_t(16 * p + 4 * lg + c) * jb.lda + 16 * w + lm];
      }
    }
  };
  auto stage_b = [&](const MmJob& jb) {
    const float* B = jb.B + item * jb.sB;
    if (!TB) {  // B stored [K][N]
#pragma unroll
      for (int r = 0; r < K * NB / 1024; ++r) {
        const int idx = tid + 256 * r, k = idx / (NB / 4), n4 = (idx % (NB / 4)) * 4;
        *reinterpret_cast<float4*>(Bs + k * kLd + n4) = *reinterpret_cast<const float4*>(B + int64_t(k) * jb.ldb + n0 + n4);
      }
    } else {  // B stored [N][K]: a wave reads 64 contiguous bytes of each of 16 rows n, and its transposed
              // LDS writes (rows k, 16 consecutive n per row) hit distinct banks
#pragma unroll
      for (int r = 0; r < K * NB / 1024; ++r) {
        const int f = tid + 256 * r, rest = f >> 6;
        const int n = 16 * (rest % (NB / 16)) + (f & 15), k4 = 16 * (rest / (NB / 16)) + 4 * ((f >> 4) & 3);
        const float4 v = *reinterpret_cast<const float4*>(B + int64_t(n0 + n) * jb.ldb + k4);
        Bs[(k4 + 0) * kLd + n] = v.x; Bs[(k4 + 1) * kLd + n] = v.y;
        Bs[(k4 + 2) * kLd + n] = v.z; Bs[(k4 + 3) * kLd + n] = v.w;
      }
    }
  };
  f32x4 acc[NB / 16];
  int head = 0;  // first job of the current chain
#pragma unroll 1
  for (int jj = 0; jj < jobs.n; ++jj) {
    const MmJob& jb = jobs.j[jj];
    float av[K / 16][4];
    load_a(jb, av);  // in flight with the B staging
    if (!jb.reuse_b) {
      if (jj > 0) __syncthreads();  // every wave is done with the previous B
      stage_b(jb);
      __syncthreads();
    }
    if (!jb.chain) {
      head = jj;
#pragma unroll
      for (int j = 0; j < NB / 16; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // B operands of step p + 1 are read from LDS while step p's MFMAs run (the scheduling barriers keep
    // the compiler from sinking the reads next to their uses)
    float bop[2][4][NB / 16];
    auto read_b = [&](int p, float (&dst)[4][NB / 16]) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int j = 0; j < NB / 16; ++j) dst[c][j] = Bs[(16 * p + 4 * lg + c) * kLd + 16 * j + lm];
    };
    read_b(0, bop[0]);
#pragma unroll
    for (int p = 0; p < K / 16; ++p) {
      if (p + 1 < K / 16) read_b(p + 1, bop[(p + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int j = 0; j < NB / 16; ++j) acc[j] = mfma16x16x4f32(av[p][c], bop[p & 1][c][j], acc[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (jj + 1 < jobs.n && jobs.j[jj + 1].chain) continue;
    // store the chain's sum with its first job's settings
    const MmJob& hb = jobs.j[head];
    float* C = hb.C + item * hb.sC;
    float* C2 = hb.C2 ? hb.C2 + item * hb.sC : nullptr;
#pragma unroll
    for (int j = 0; j < NB / 16; ++j) {
      const int n = n0 + 16 * j + lm;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * w + 4 * lg + e;
        v[e] = hb.alpha * acc[j][e];
        if ((hb.mask == 1 && n > m) || (hb.mask == 2 && n >= m)) v[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float* cp = C + int64_t(16 * w + 4 * lg + e) * hb.ldc + n;
        *cp = hb.accumulate ? *cp + v[e] : v[e];
      }
      if (C2)  // [N][64]: the lane's four rows are contiguous
        *reinterpret_cast<float4*>(C2 + int64_t(n) * kC + 16 * w + 4 * lg) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

// ---- A = strict_lower(beta_t E KK), P = lower(E QK) ----
__global__ void __launch_bounds__(256) k_cb_ap(CBwdArgs a) {
  const int64_t item = blockIdx.x;
  if (a.tab[item / a.hv].y <= 0) return;
  __shared__ float Gs[kC], Bs[kC];
  if (threadIdx.x < kC) {
    Gs[threadIdx.x] = a.G[item * kC + threadIdx.x];
    Bs[threadIdx.x] = a.bt[item * kC + threadIdx.x];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < kC * kC / 4; idx += 256) {
    const int t = idx / (kC / 4), i0 = (idx % (kC / 4)) * 4;
    const int64_t o = item * kC * kC + t * kC + i0;
    const float4 kk = *reinterpret_cast<const float4*>(a.KK + o), qk = *reinterpret_cast<const float4*>(a.QK + o);
    const float kkv[4] = {kk.x, kk.y, kk.z, kk.w}, qkv[4] = {qk.x, qk.y, qk.z, qk.w};
    float av[4], pv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = i0 + e;
      const float ex = __expf(fminf(Gs[t] - Gs[i], 0.f));
      av[e] = i < t ? Bs[t] * ex * kkv[e] : 0.f;
      pv[e] = i <= t ? ex * qkv[e] : 0.f;
    }
    *reinterpret_cast<float4*>(a.Am + o) = make_float4(av[0], av[1], av[2], av[3]);
    *reinterpret_cast<float4*>(a.Pm + o) = make_float4(pv[0], pv[1], pv[2], pv[3]);
  }
}

// ---- T = (I + A)^-1, A strictly lower, by 16 x 16 blocks ----
// The diagonal blocks D_i = (I + A_ii)^-1 by forward substitution (wave i, lane = column), then block
// row by block row T_ij = -D_i sum_{k=j}^{i-1} A_ik T_kj (j < i).
__global__ void __launch_bounds__(256) k_cb_inv(CBwdArgs a) {
  __shared__ float As[kC][kC + 1];
  __shared__ float Ts[kC][kC + 1];
  __shared__ float Rs[3][16][17];
  const int64_t item = blockIdx.x;
  if (a.tab[item / a.hv].y <= 0) return;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const float* A = a.Am + item * kC * kC;
  for (int idx = tid; idx < kC * kC / 4; idx += 256) {
    const int r = idx / (kC / 4), c4 = (idx % (kC / 4)) * 4;
    const float4 v = *reinterpret_cast<const float4*>(A + r * kC + c4);
    As[r][c4] = v.x; As[r][c4 + 1] = v.y; As[r][c4 + 2] = v.z; As[r][c4 + 3] = v.w;
    Ts[r][c4] = 0.f; Ts[r][c4 + 1] = 0.f; Ts[r][c4 + 2] = 0.f; Ts[r][c4 + 3] = 0.f;
  }
  __syncthreads();
  if (lane < 16) {  // D_w, column `lane`
    const int o = 16 * w;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v = (r == lane) ? 1.f : 0.f;
#pragma unroll
      for (int q = 0; q < r; ++q) v -= As[o + r][o + q] * x[q];
      x[r] = v;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Ts[o + r][o + lane] = x[r];
  }
  __syncthreads();
  const int r = tid >> 4, c = tid & 15;
  for (int i = 1; i < 4; ++i) {
    // R_ij (j < i), element (r, c), into Rs[j]
    for (int j = 0; j < i; ++j) {
      float acc = 0.f;
      for (int k = j; k < i; ++k)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc += As[16 * i + r][16 * k + q] * Ts[16 * k + q][16 * j + c];
      Rs[j][r][c] = acc;
    }
    __syncthreads();
    for (int j = 0; j < i; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int q = 0; q < 16; ++q) acc += Ts[16 * i + r][16 * i + q] * Rs[j][q][c];
      Ts[16 * i + r][16 * j + c] = -acc;
    }
    __syncthreads();
  }
  float* T = a.Tm + item * kC * kC;
  for (int idx = tid; idx < kC * kC / 4; idx += 256) {
    const int rr = idx / (kC / 4), c4 = (idx % (kC / 4)) * 4;
    *reinterpret_cast<float4*>(T + rr * kC + c4) = make_float4(Ts[rr][c4], Ts[rr][c4 + 1], Ts[rr][c4 + 2], Ts[rr][c4 + 3]);
  }
}

// ---- bV = diag(beta) V, bgK = diag(beta g) K, Kt = diag(kd) K and its transpose, gQ = diag(g) Q ----
__global__ void __launch_bounds__(256) k_cb_prep(CBwdArgs a) {
  __shared__ float tile[kC][kC + 1];
  __shared__ float gs[kC], kds[kC], bs[kC];
  const int64_t item = blockIdx.x;
  if (a.tab[item / a.hv].y <= 0) return;
  if (threadIdx.x < kC) {
    const float* G = a.G + item * kC;
    const float Gt = G[threadIdx.x];
    gs[threadIdx.x] = __expf(Gt);
    kds[threadIdx.x] = __expf(G[kC - 1] - Gt);
    bs[threadIdx.x] = a.bt[item * kC + threadIdx.x];
  }
  __syncthreads();
  const int64_t b2 = item * kC * kD;
  for (int idx = threadIdx.x; idx < kC * kD / 4; idx += 256) {
    const int t = idx / (kD / 4);
    const int64_t o = b2 + 4 * idx;
    const float be = bs[t], g = gs[t], kd = kds[t], bg = be * g;
    const float4 kv = *reinterpret_cast<const float4*>(a.Ki + o);
    const float4 vv = *reinterpret_cast<const float4*>(a.Vi + o);
    const float4 qv = *reinterpret_cast<const float4*>(a.Qi + o);
    *reinterpret_cast<float4*>(a.bV + o) = make_float4(be * vv.x, be * vv.y, be * vv.z, be * vv.w);
    *reinterpret_cast<float4*>(a.bgK + o) = make_float4(bg * kv.x, bg * kv.y, bg * kv.z, bg * kv.w);
    *reinterpret_cast<float4*>(a.Kt + o) = make_float4(kd * kv.x, kd * kv.y, kd * kv.z, kd * kv.w);
    *reinterpret_cast<float4*>(a.gQ + o) = make_float4(g * qv.x, g * qv.y, g * qv.z, g * qv.w);
  }
  // KtT [128][64], through LDS in two 64-column halves
  for (int half = 0; half < 2; ++half) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < kC * kC / 4; idx += 256) {
      const int t = idx / (kC / 4), r4 = (idx % (kC / 4)) * 4;
      const float4 kv = *reinterpret_cast<const float4*>(a.Ki + b2 + t * kD + 64 * half + r4);
      const float kd = kds[t];
      tile[t][r4] = kd * kv.x; tile[t][r4 + 1] = kd * kv.y; tile[t][r4 + 2] = kd * kv.z; tile[t][r4 + 3] = kd * kv.w;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < kC * kC / 4; idx += 256) {
      const int r = idx / (kC / 4), t4 = (idx % (kC / 4)) * 4;
      *reinterpret_cast<float4*>(a.KtT + b2 + (64 * half + r) * kC + t4) =
          make_float4(tile[t4][r], tile[t4 + 1][r], tile[t4 + 2][r], tile[t4 + 3][r]);
    }
  }
}

// ---- the chunk passes: the only sequential part, one block per (sequence, value head, 16-column slice) ----
// Both passes carry a 128 x 16 slice X of a state-sized matrix across the sequence's chunks:
//     Z = B + s1 A1 X   (64 x 16),      X <- g_C X + H + s2 A2^T Z   (128 x 16),
// forward (chunks in order):  X = S,   A1 = Wk, s1 = -1, B = U,       Z = W,  A2 = Kt, s2 = +1, H = 0;
// backward (in reverse):      X = dS', A1 = Kt, s1 = +1, B = P^T dY,  Z = dW, A2 = Wk, s2 = -1, H = gQ^T dY.
// The products run on 16x16x4 fp32 MFMAs; wave w computes rows 16w.. of Z and rows 32w.. of X over the
// slice's kCT 16-column tiles (each A operand read feeds every tile), and X stays in registers in the
// accumulator layout (lane l: rows 4 (l / 16) + e of each 16-row tile, column l % 16 of each column tile).
// The contraction order is chosen so that each lane's A operands are float4 runs of one row: at step
// (p, c) lane group q contributes index 16p + 4q + c. A block is one chain's slice and runs alone on its
// CU (four waves, one per SIMD), so every operand of the next chunk -- A1, A2^T, B, G and (backward) H
// and S -- is requested before the current chunk's products, into the other of two register sets.
// A wave's rows of B, H and S arrive as 16-byte pieces and reach the accumulator layout through a
// per-wave LDS area, and its rows of X and Z leave as 16-byte pieces from the LDS tiles the products
// read: few memory instructions per chunk, so every wait for this chunk's operands can leave the next
// chunk's requests in flight (a wave tracks at most 63).
constexpr int kXLd = kSl + 4;  // LDS row stride of X, Z and the staging areas (floats): the four lane groups
                               // of an accumulator-layout access hit distinct banks

struct PassLoads {
  float4 a1[8];   // A1 row 16w + l % 16, columns 4 (l / 16 + 4p) ..
  f32x4 a2[8];    // A2^T rows 32w + 16i + l % 16, columns 4 (l / 16 + 4p) .. (piece 4i + p)
  float4 b[2];    // B: piece l + 64k of the wave's 16 x kSl rows (row (l + 64k) / 8, columns 4 ((l + 64k) % 8) ..)
  float4 h[4];    // backward: H and S, piece l + 64k of the wave's 32 x kSl rows (same mapping)
  float4 sp[4];
  float Gc;       // G at the chunk's last row (exponentiated at use: a wait here would stall the loads)
};
// per wave: B [16][kXLd], H [32][kXLd], S [32][kXLd]
constexpr int kStageB = 0, kStageH = 16 * kXLd, kStageS = 48 * kXLd, kStageW = 80 * kXLd;

template <bool kBwd>
__device__ __forceinline__ void pass_load(const CBwdArgs& a, int64_t item, int w, int lane, int lm, int lg,
                                          int c0, PassLoads& L) {
  const float* A1 = (kBwd ? a.Kt : a.Wk) + item * kC * kD;
  const float* A2T = (kBwd ? a.WkT : a.KtT) + item * kD * kC;
  const float* B = (kBwd ? a.dW : a.U) + item * kC * kD;
#pragma unroll
  for (int p = 0; p < 8; ++p) L.a1[p] = *reinterpret_cast<const float4*>(A1 + (16 * w + lm) * kD + 4 * (lg + 4 * p));
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int p = 0; p < 4; ++p)
      L.a2[4 * i + p] = *reinterpret_cast<const f32x4*>(A2T + (32 * w + 16 * i + lm) * kC + 4 * (lg + 4 * p));
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int pc = lane + 64 * k;
    L.b[k] = *reinterpret_cast<const float4*>(B + (16 * w + pc / 8) * kD + c0 + 4 * (pc % 8));
  }
  if (kBwd) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int pc = lane + 64 * k;
      const int64_t o = item * kD * kD + (32 * w + pc / 8) * kD + c0 + 4 * (pc % 8);
      L.h[k] = *reinterpret_cast<const float4*>(a.dS + o);
      L.sp[k] = *reinterpret_cast<const float4*>(a.S + o);
    }
  }
  L.Gc = a.G[item * kC + kC - 1];
}

// One chunk of a pass: X (the state at the chunk's start; backward: dL/d state after it) is stored, Z
// computed and stored, and X advanced. c0 is the slice's first column; St is this wave's staging area.
template <bool kBwd>
__device__ __forceinline__ void pass_step(const CBwdArgs& a, int64_t item, const PassLoads& L, int64_t next_item,
                                          PassLoads& N, f32x4 (&X)[kCT][2], float* Xs, float* Zs, float* St, int w,
                                          int lane, int lm, int lg, int c0, int sl) {
  const float s1 = kBwd ? 1.f : -1.f, s2 = kBwd ? -1.f : 1.f;
  float* Zout = kBwd ? a.dW : a.W;
  float* Xout = kBwd ? a.dS : a.S;
  // The next chunk's operands are requested after this chunk's: memory counters drain in order, so a
  // wait for this chunk's operands then does not also wait for the next chunk's. (H lives in the dS
  // slot this chunk's X overwrites below; it was read a chunk ahead, before that store.)
  __builtin_amdgcn_sched_barrier(0);
  pass_load<kBwd>(a, next_item, w, lane, lm, lg, c0, N);
  __builtin_amdgcn_sched_barrier(0);
  // this chunk's B (and H, S) pieces into the wave's staging area
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int pc = lane + 64 * k;
    *reinterpret_cast<float4*>(St + kStageB + (pc / 8) * kXLd + 4 * (pc % 8)) = L.b[k];
  }
  if (kBwd) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int pc = lane + 64 * k;
      *reinterpret_cast<float4*>(St + kStageH + (pc / 8) * kXLd + 4 * (pc % 8)) = L.h[k];
      *reinterpret_cast<float4*>(St + kStageS + (pc / 8) * kXLd + 4 * (pc % 8)) = L.sp[k];
    }
  }
  // X into the LDS tile; the wave's own rows then leave as 16-byte pieces (a wave's LDS accesses
  // complete in order, so its own writes are visible to it without a barrier)
#pragma unroll
  for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) Xs[(32 * w + 16 * i + 4 * lg + e) * kXLd + 16 * ct + lm] = X[ct][i][e];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int pc = lane + 64 * k, row = 32 * w + pc / 8;
    *reinterpret_cast<float4*>(Xout + item * kD * kD + size_t(row) * kD + c0 + 4 * (pc % 8)) =
        *reinterpret_cast<const float4*>(Xs + row * kXLd + 4 * (pc % 8));
  }
  __syncthreads();
  // Z = B + s1 A1 X: rows 16w + 4 lg + e. B joins the accumulators only after the products.
#pragma unroll
  for (int ct = 0; ct < kCT; ++ct) {
    float xb[8][4];
#pragma unroll
    for (int p = 0; p < 8; ++p)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) xb[p][cc] = Xs[(16 * p + 4 * lg + cc) * kXLd + 16 * ct + lm];
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
    f32x4 z0 = {0.f, 0.f, 0.f, 0.f}, z1 = z0;
#pragma unroll
    for (int p = 0; p < 8; p += 2) {
      const float av0[4] = {L.a1[p].x, L.a1[p].y, L.a1[p].z, L.a1[p].w};
      const float av1[4] = {L.a1[p + 1].x, L.a1[p + 1].y, L.a1[p + 1].z, L.a1[p + 1].w};
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        z0 = mfma16x16x4f32(s1 * av0[cc], xb[p][cc], z0);
        z1 = mfma16x16x4f32(s1 * av1[cc], xb[p + 1][cc], z1);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 4 * lg + e;  // row of the wave's 16
      Zs[(16 * w + t) * kXLd + 16 * ct + lm] = z0[e] + z1[e] + St[kStageB + t * kXLd + 16 * ct + lm];
    }
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int pc = lane + 64 * k, row = 16 * w + pc / 8;
    *reinterpret_cast<float4*>(Zout + item * kC * kD + size_t(row) * kD + c0 + 4 * (pc % 8)) =
        *reinterpret_cast<const float4*>(Zs + row * kXLd + 4 * (pc % 8));
  }
  __syncthreads();
  // X <- g_C X + H + s2 A2^T Z
  const float gc = __expf(L.Gc);
  float part = 0.f;
#pragma unroll
  for (int ct = 0; ct < kCT; ++ct) {
    float zb[4][4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) zb[p][cc] = Zs[(16 * p + 4 * lg + cc) * kXLd + 16 * ct + lm];
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][e] = gc * X[ct][i][e];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const f32x4 av0 = L.a2[p], av1 = L.a2[4 + p];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        acc[0] = mfma16x16x4f32(s2 * av0[cc], zb[p][cc], acc[0]);
        acc[1] = mfma16x16x4f32(s2 * av1[cc], zb[p][cc], acc[1]);
      }
    }
    if (kBwd) {  // this wave's part of <S, dS'> (for dG), then X <- ... + H
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int o = (16 * i + 4 * lg + e) * kXLd + 16 * ct + lm;
          part += St[kStageS + o] * X[ct][i][e];
          acc[i][e] += St[kStageH + o];
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) X[ct][i] = acc[i];
  }
  if (kBwd) {
    part = group_sum<64>(part);
    if (lane == 0) a.dgc[(item * kSlices + sl) * 4 + w] = part;
  }
}

template <bool kBwd>
__global__ void __launch_bounds__(256, 1) k_cb_pass(CBwdArgs a) {
  __shared__ float Xs[kD * kXLd];
  __shared__ float Zs[kC * kXLd];
  __shared__ float Stage[4 * kStageW];
  // the slices of a chain read the same chunk operands: numbered to run on one XCD, so those come from
  // HBM once and from that XCD's L2 for the others
  int chain, sl;
  xcd_item(int(blockIdx.x), kSlices, chain, sl);
  if (chain >= a.n_seqs * a.hv) return;
  const int n = chain / a.hv, h = chain % a.hv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lm = lane & 15, lg = lane >> 4;
  const int cs0 = kSl * sl, col = cs0 + lm;  // the slice's first column; this lane's in column tile 0
  float* const St = Stage + w * kStageW;
  const float* x0 = kBwd ? a.dsf : a.s0;
  const size_t sb = (size_t(n) * a.hv + h) * kD * kD;
  f32x4 X[kCT][2];
#pragma unroll
  for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        X[ct][i][e] = x0 ? x0[sb + size_t(32 * w + 16 * i + 4 * lg + e) * kD + col + 16 * ct] : 0.f;
  const int c0 = a.seq_off[n], nch = a.seq_off[n + 1] - c0;
  // chunk of step it (the backward walks the chunks in reverse)
  auto item_of = [&](int it) { return int64_t(kBwd ? c0 + nch - 1 - it : c0 + it) * a.hv + h; };
  // two operand sets used in turn, so the next chunk's loads are in flight during this chunk's products
  // (no register copies between them that would wait for those loads). The loads are unconditional
  // (past the last chunk they repeat it), so every wait for them counts the same loads on every path.
  PassLoads L0, L1;
  if (nch > 0) {
    const int last = nch - 1;
    pass_load<kBwd>(a, item_of(0), w, lane, lm, lg, cs0, L0);
    for (int it = 0;; it += 2) {
      pass_step<kBwd>(a, item_of(it), L0, item_of(min(it + 1, last)), L1, X, Xs, Zs, St, w, lane, lm, lg, cs0, sl);
      if (it + 1 > last) break;
      pass_step<kBwd>(a, item_of(it + 1), L1, item_of(min(it + 2, last)), L0, X, Xs, Zs, St, w, lane, lm, lg, cs0, sl);
      if (it + 2 > last) break;
    }
  }
  if (kBwd && a.ds0) {
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          a.ds0[sb + size_t(32 * w + 16 * i + 4 * lg + e) * kD + col + 16 * ct] = X[ct][i][e];
  }
}

// ---- y = scale (gQ S + P W), gathered per item in X, scattered to the tokens ----
__global__ void __launch_bounds__(256) k_cb_scatter_y(CBwdArgs a) {
  const int64_t item = blockIdx.x;
  const int c = int(item / a.hv), h = int(item - int64_t(c) * a.hv);
  const int4 ct = a.tab[c];
  for (int idx = threadIdx.x; idx < ct.y * (kD / 4); idx += 256) {
    const int t = idx / (kD / 4), c4 = (idx % (kD / 4)) * 4;
    float4 v = *reinterpret_cast<const float4*>(a.X + item * kC * kD + t * kD + c4);
    v.x *= a.scale; v.y *= a.scale; v.z *= a.scale; v.w *= a.scale;
    *reinterpret_cast<float4*>(a.y + (ct.x + t) * int64_t(a.hv) * kD + h * kD + c4) = v;
  }
}

// ---- dQK = dP o E (into M1) and dE = dP o QK (in place of dP) ----
__global__ void __launch_bounds__(256) k_cb_ew1(CBwdArgs a) {
  const int64_t item = blockIdx.x;
  if (a.tab[item / a.hv].y <= 0) return;
  __shared__ float Gs[kC];
  if (threadIdx.x < kC) Gs[threadIdx.x] = a.G[item * kC + threadIdx.x];
  __syncthreads();
  for (int idx = threadIdx.x; idx < kC * kC / 4; idx += 256) {
    const int t = idx / (kC / 4), i0 = (idx % (kC / 4)) * 4;
    const int64_t o = item * kC * kC + t * kC + i0;
    const float4 dp = *reinterpret_cast<const float4*>(a.dP + o), qk = *reinterpret_cast<const float4*>(a.QK + o);
    const float dpv[4] = {dp.x, dp.y, dp.z, dp.w};
    float m1[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) m1[e] = dpv[e] * __expf(fminf(Gs[t] - Gs[i0 + e], 0.f));
    *reinterpret_cast<float4*>(a.M1 + o) = make_float4(m1[0], m1[1], m1[2], m1[3]);
    *reinterpret_cast<float4*>(a.dP + o) = make_float4(dp.x * qk.x, dp.y * qk.y, dp.z * qk.z, dp.w * qk.w);
  }
}

// ---- dAKK = dA o beta_t o E (into dT, free by now) ----
__global__ void __launch_bounds__(256) k_cb_ew2(CBwdArgs a) {
  const int64_t item = blockIdx.x;
  if (a.tab[item / a.hv].y <= 0) return;
  __shared__ float Gs[kC], Bs[kC];
  if (threadIdx.x < kC) {
    Gs[threadIdx.x] = a.G[item * kC + threadIdx.x];
    Bs[threadIdx.x] = a.bt[item * kC + threadIdx.x];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < kC * kC / 4; idx += 256) {
    const int t = idx / (kC / 4), i0 = (idx % (kC / 4)) * 4;
    const int64_t o = item * kC * kC + t * kC + i0;
    const float4 da = *reinterpret_cast<const float4*>(a.dA + o);
    const float dav[4] = {da.x, da.y, da.z, da.w};
    float r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = dav[e] * Bs[t] * __expf(fminf(Gs[t] - Gs[i0 + e], 0.f));
    *reinterpret_cast<float4*>(a.dT + o) = make_float4(r[0], r[1], r[2], r[3]);
  }
}

// ---- per item: the row terms, dG, d ln alpha, and the outputs of the chunk's tokens ----
__global__ void __launch_bounds__(256) k_cb_final(CBwdArgs a) {
  const int64_t item = blockIdx.x;
  const int c = int(item / a.hv), h = int(item - int64_t(c) * a.hv);
  const int4 ct = a.tab[c];
  if (ct.y <= 0) return;
  __shared__ float dG[kC], dbe[kC], dkd[kC], Gs[kC], bts[kC];
  __shared__ float dAs[kC][kC + 1], KKs[kC][kC + 1], dPs[kC][kC + 1];
  __shared__ float part[4][kC][2];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  if (tid < kC) Gs[tid] = a.G[item * kC + tid];
  __syncthreads();
  const float GC = Gs[kC - 1];
  const int64_t b2 = item * kC * kD, b1 = item * kC * kC;
  // rows: one wave per 16 rows, two rows at a time (a half-wave each, four columns per lane)
  const int hw = lane >> 5, c4 = 4 * (lane & 31);
  for (int r2 = 0; r2 < 8; ++r2) {
    const int t = 16 * w + 2 * r2 + hw;
    const float g = __expf(Gs[t]), kd = __expf(GC - Gs[t]), be = a.bt[item * kC + t];
    const int64_t o = b2 + t * kD + c4;
    const float4 X = *reinterpret_cast<const float4*>(a.X + o), Q = *reinterpret_cast<const float4*>(a.Qi + o);
    const float4 K = *reinterpret_cast<const float4*>(a.Ki + o), V = *reinterpret_cast<const float4*>(a.Vi + o);
    const float4 dbgk = *reinterpret_cast<const float4*>(a.dbgK + o);
    const float4 dbv = *reinterpret_cast<const float4*>(a.dbV + o);
    const float4 dkt = *reinterpret_cast<const float4*>(a.dKt + o);
    float sqx = Q.x * X.x + Q.y * X.y + Q.z * X.z + Q.w * X.w;
    float sbk = dbgk.x * K.x + dbgk.y * K.y + dbgk.z * K.z + dbgk.w * K.w;
    float sbv = dbv.x * V.x + dbv.y * V.y + dbv.z * V.z + dbv.w * V.w;
    float skt = dkt.x * K.x + dkt.y * K.y + dkt.z * K.z + dkt.w * K.w;
    if (t < ct.y) {
      const int64_t tok = (ct.x + t) * int64_t(a.hv) * kD + h * kD + c4;
      const float4 dQ = *reinterpret_cast<const float4*>(a.dQ + o), dK = *reinterpret_cast<const float4*>(a.dK + o);
      const float bg = be * g;
      *reinterpret_cast<float4*>(a.dqh + tok) =
          make_float4(dQ.x + g * X.x, dQ.y + g * X.y, dQ.z + g * X.z, dQ.w + g * X.w);
      *reinterpret_cast<float4*>(a.dkh + tok) =
          make_float4(dK.x + kd * dkt.x + bg * dbgk.x, dK.y + kd * dkt.y + bg * dbgk.y,
                      dK.z + kd * dkt.z + bg * dbgk.z, dK.w + kd * dkt.w + bg * dbgk.w);
      *reinterpret_cast<float4*>(a.dv + tok) = make_float4(be * dbv.x, be * dbv.y, be * dbv.z, be * dbv.w);
    }
    sqx = group_sum<32>(sqx);
    sbk = group_sum<32>(sbk);
    sbv = group_sum<32>(sbv);
    skt = group_sum<32>(skt);
    if ((lane & 31) == 0) {
      dG[t] = (sqx + be * sbk) * g;  // dg_t g_t
      dbe[t] = sbv + g * sbk;
      dkd[t] = skt * kd;              // dkd_t kd_t
    }
  }
  __syncthreads();
  // E terms: dE (from dP o QK, plus dA o beta o KK), dbeta from dA o E o KK. The three 64 x 64 tiles are
  // staged in LDS (stride 65: row and column walks are both conflict-free); thread (t, q) covers
  // i = 16q .. 16q + 15 of row t and of column t.
  for (int idx = tid; idx < kC * kC / 4; idx += 256) {
    const int r = idx / (kC / 4), c4 = (idx % (kC / 4)) * 4;
    const float4 da = *reinterpret_cast<const float4*>(a.dA + b1 + r * kC + c4);
    const float4 kk = *reinterpret_cast<const float4*>(a.KK + b1 + r * kC + c4);
    const float4 dp = *reinterpret_cast<const float4*>(a.dP + b1 + r * kC + c4);
    const float dav[4] = {da.x, da.y, da.z, da.w}, kkv[4] = {kk.x, kk.y, kk.z, kk.w}, dpv[4] = {dp.x, dp.y, dp.z, dp.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dAs[r][c4 + j] = dav[j];
      KKs[r][c4 + j] = kkv[j];
      dPs[r][c4 + j] = dpv[j];
    }
  }
  if (tid < kC) bts[tid] = a.bt[item * kC + tid];
  __syncthreads();
  {
    const int t = tid & 63, q = tid >> 6;
    const float be = bts[t];
    float rowsum = 0.f, colsum = 0.f, dbA = 0.f;
    for (int i = 16 * q; i < 16 * q + 16; ++i) {
      const float e_ti = __expf(fminf(Gs[t] - Gs[i], 0.f)), e_it = __expf(fminf(Gs[i] - Gs[t], 0.f));
      const float dA_ti = dAs[t][i], kk_ti = KKs[t][i];
      const float dE_ti = (i <= t ? dPs[t][i] : 0.f) + dA_ti * be * kk_ti;
      rowsum += dE_ti * e_ti;
      dbA += dA_ti * e_ti * kk_ti;
      const float dE_it = (t <= i ? dPs[i][t] : 0.f) + dAs[i][t] * bts[i] * KKs[i][t];
      colsum += dE_it * e_it;
    }
    part[q][t][0] = rowsum - colsum;
    part[q][t][1] = dbA;
  }
  __syncthreads();
  if (tid < kC) {
    const int t = tid;
    dG[t] += part[0][t][0] + part[1][t][0] + part[2][t][0] + part[3][t][0] - dkd[t];
    dbe[t] += part[0][t][1] + part[1][t][1] + part[2][t][1] + part[3][t][1];
  }
  __syncthreads();
  if (tid == 0) {
    float s = 0.f;
    for (int i = 0; i < kC; ++i) s += dkd[i];
    float dgc = 0.f;
    for (int k = 0; k < 4 * kSlices; ++k) dgc += a.dgc[item * kSlices * 4 + k];
    dG[kC - 1] += s + dgc * __expf(GC);
  }
  __syncthreads();
  if (tid < kC) {
    // d ln alpha_s = sum_{t >= s} dG_t (reverse prefix sum over the chunk)
    float v = dG[kC - 1 - tid];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(v, o, 64);
      if (tid >= o) v += y;
    }
    const int sidx = kC - 1 - tid;
    if (sidx < ct.y) {
      const int64_t ai = (ct.x + sidx) * int64_t(a.hv) + h;
      a.dalpha[ai] = v / a.alpha[ai];
      a.dbeta[ai] = dbe[sidx];
    }
  }
}

// ---- dq, dk: sums over the value heads that read each QK head (four channels per thread) ----
__global__ void __launch_bounds__(256) k_cb_group_sum(const float* __restrict__ dqh, const float* __restrict__ dkh,
                                                      int64_t T, int hk, int hv, float* __restrict__ dq,
                                                      float* __restrict__ dk) {
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;  // over T x hk x 32
  if (idx >= T * hk * (kD / 4)) return;
  const int64_t t = idx / (int64_t(hk) * (kD / 4));
  const int g = int((idx / (kD / 4)) % hk), c4 = int(idx % (kD / 4)) * 4, R = hv / hk;
  float4 sq = make_float4(0.f, 0.f, 0.f, 0.f), sk = sq;
  for (int r = 0; r < R; ++r) {
    const int64_t o = (t * hv + g * R + r) * kD + c4;
    const float4 a = *reinterpret_cast<const float4*>(dqh + o), b = *reinterpret_cast<const float4*>(dkh + o);
    sq.x += a.x; sq.y += a.y; sq.z += a.z; sq.w += a.w;
    sk.x += b.x; sk.y += b.y; sk.z += b.z; sk.w += b.w;
  }
  *reinterpret_cast<float4*>(dq + 4 * idx) = sq;
  *reinterpret_cast<float4*>(dk + 4 * idx) = sk;
}

}  // namespace

size_t cbwd_workspace_bytes(int n_seqs, int64_t T, int hv) {
  const size_t nc = size_t(T / kC + n_seqs), items = nc * hv;
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t f = sizeof(float);
  return al(sizeof(int32_t) * (n_seqs + 1)) + al(sizeof(int4) * nc) +
         21 * al(f * items * kC * kD) +           // the 64 x 128 tiles (KtT, WkT stored 128 x 64)
         2 * al(f * items * kD * kD) +            // S dS
         9 * al(f * items * kC * kC) +            // KK QK Am Pm Tm dP M1 dT dA
         2 * al(f * items * kC) + al(f * items * kSlices * 4) +  // G bt dgc
         2 * al(f * size_t(T) * hv * kD);          // dqh dkh
}

void cbwd_plan(CBwdArgs& a, void* base) {
  const size_t nc = size_t(a.T / kC + a.n_seqs), items = nc * a.hv;
  a.nc_max = int64_t(nc);
  char* p = static_cast<char*>(base);
  auto take = [&](size_t bytes) {
    void* r = p;
    p += (bytes + 255) & ~size_t(255);
    return r;
  };
  const size_t f = sizeof(float), big = f * items * kC * kD, st = f * items * kD * kD, sm = f * items * kC * kC;
  a.seq_off = static_cast<int32_t*>(take(sizeof(int32_t) * (a.n_seqs + 1)));
  a.tab = static_cast<int4*>(take(sizeof(int4) * nc));
  float** bigs[] = {&a.Qi, &a.Ki, &a.Vi, &a.dYi, &a.bV, &a.bgK, &a.U, &a.Wk, &a.W, &a.dW, &a.dKt, &a.X, &a.dWk,
                    &a.dQ, &a.dK, &a.dbV, &a.dbgK, &a.Kt, &a.KtT, &a.WkT, &a.gQ};
  for (float** q : bigs) *q = static_cast<float*>(take(big));
  a.S = static_cast<float*>(take(st));
  a.dS = static_cast<float*>(take(st));
  float** sms[] = {&a.KK, &a.QK, &a.Am, &a.Pm, &a.Tm, &a.dP, &a.M1, &a.dT, &a.dA};
  for (float** q : sms) *q = static_cast<float*>(take(sm));
  a.G = static_cast<float*>(take(f * items * kC));
  a.bt = static_cast<float*>(take(f * items * kC));
  a.dgc = static_cast<float*>(take(f * items * kSlices * 4));
  a.dqh = static_cast<float*>(take(f * size_t(a.T) * a.hv * kD));
  a.dkh = static_cast<float*>(take(f * size_t(a.T) * a.hv * kD));
}

namespace {
template <int N, int K, bool TA, bool TB>
hipError_t mm_launch(const MmJobs& jobs, const CBwdArgs& a, hipStream_t s) {
  constexpr int NB = N == 128 ? 64 : 32;  // columns of C per block (measured best per width)
  const void* f = reinterpret_cast<const void*>(k_cb_mm<N, NB, K, TA, TB>);
  const int smem = int(sizeof(float) * K * (NB + 4));
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  // this instance's LDS limit is raised once per device (an idempotent call, so a race only repeats it)
  static std::atomic<uint64_t> raised{0};
  const uint64_t bit = uint64_t(1) << (dev & 63);
  if (!(raised.load() & bit)) {
    if ((e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, smem)) != hipSuccess) return e;
    raised.fetch_or(bit);
  }
  const int64_t items = a.nc_max * a.hv;
  hipLaunchKernelGGL((k_cb_mm<N, NB, K, TA, TB>), dim3(unsigned(xcd_blocks(items, N / NB))), dim3(256), size_t(smem), s,
                     jobs, a.tab, a.hv, items);
  return hipGetLastError();
}

// One product job: C (64 x N) = alpha op(A) op(B) (+ C), op(A) 64 x K, op(B) K x N.
MmJob job(const float* A, int64_t sA, int lda, const float* B, int64_t sB, int ldb, float* C, int64_t sC, int ldc,
          float alpha = 1.f, int accumulate = 0, int mask = 0) {
  return MmJob{A, B, C, nullptr, sA, sB, sC, lda, ldb, ldc, alpha, accumulate, mask, 0, 0};
}
MmJob chained(MmJob j) {
  j.chain = 1;
  return j;
}

// Launches up to three jobs that share N, K and the transposition of A and B as one batched product.
hipError_t mm(const CBwdArgs& a, int N, int K, bool ta, bool tb, std::initializer_list<MmJob> list, hipStream_t s) {
  MmJobs jobs{};
  for (const MmJob& jb : list) {
    if (jobs.n == 3) return hipErrorInvalidValue;
    jobs.j[jobs.n] = jb;
    if (jobs.n > 0) {
      const MmJob& pr = jobs.j[jobs.n - 1];
      jobs.j[jobs.n].reuse_b = jb.B == pr.B && jb.sB == pr.sB && jb.ldb == pr.ldb;
    }
    ++jobs.n;
  }
  const int key = (N == 128) * 8 + (K == 128) * 4 + ta * 2 + tb;
  switch (key) {
    case 1: return mm_launch<64, 64, false, true>(jobs, a, s);
    case 2: return mm_launch<64, 64, true, false>(jobs, a, s);
    case 5: return mm_launch<64, 128, false, true>(jobs, a, s);
    case 8: return mm_launch<128, 64, false, false>(jobs, a, s);
    case 10: return mm_launch<128, 64, true, false>(jobs, a, s);
    case 12: return mm_launch<128, 128, false, false>(jobs, a, s);
    case 13: return mm_launch<128, 128, false, true>(jobs, a, s);
    default: return hipErrorInvalidValue;  // shapes the backward does not use
  }
}
}  // namespace

hipError_t launch_cbwd(const CBwdArgs& a, bool forward, bool backward, float* dq, float* dk, hipStream_t s) {
  hipError_t e = hipSuccess;
  const int64_t items = a.nc_max * a.hv;
  const unsigned nb = unsigned(items), chains = unsigned(xcd_blocks(int64_t(a.n_seqs) * a.hv, kSlices));
  const int64_t I2 = kC * kD, I1 = kC * kC, I3 = kD * kD;
  if (forward) {
    hipLaunchKernelGGL(k_cb_offsets, dim3(1), dim3(64), 0, s, a.cu, a.n_seqs, a.T, a.nc_max, a.seq_off);
    hipLaunchKernelGGL(k_cb_table, dim3(unsigned(a.n_seqs) + 1), dim3(256), 0, s, a.cu, a.n_seqs, a.T, a.nc_max,
                       a.seq_off, a.tab);
    hipLaunchKernelGGL(k_cb_gather, dim3(nb), dim3(256), 0, s, a, 1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // KK = K K^T, QK = Q K^T
    if ((e = mm(a, 64, 128, false, true, {job(a.Ki, I2, kD, a.Ki, I2, kD, a.KK, I1, kC),
                                          job(a.Qi, I2, kD, a.Ki, I2, kD, a.QK, I1, kC)}, s)) != hipSuccess)
      return e;
    hipLaunchKernelGGL(k_cb_ap, dim3(nb), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_cb_inv, dim3(nb), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_cb_prep, dim3(nb), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // U = T bV, Wk = T bgK (and Wk^T)
    {
      MmJob wk = job(a.Tm, I1, kC, a.bgK, I2, kD, a.Wk, I2, kD);
      wk.C2 = a.WkT;
      if ((e = mm(a, 128, 64, false, false, {job(a.Tm, I1, kC, a.bV, I2, kD, a.U, I2, kD), wk}, s)) != hipSuccess)
        return e;
    }
    hipLaunchKernelGGL(k_cb_pass<false>, dim3(chains), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.y) {  // y = scale (gQ S + P W), through X
      if ((e = mm(a, 128, 128, false, false, {job(a.gQ, I2, kD, a.S, I3, kD, a.X, I2, kD)}, s)) != hipSuccess) return e;
      if ((e = mm(a, 128, 64, false, false, {job(a.Pm, I1, kC, a.W, I2, kD, a.X, I2, kD, 1.f, 1)}, s)) != hipSuccess)
        return e;
      hipLaunchKernelGGL(k_cb_scatter_y, dim3(nb), dim3(256), 0, s, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  if (!backward) return hipSuccess;
  // dY is needed from here on: gathered (scaled) now, since the forward may run before dy exists
  hipLaunchKernelGGL(k_cb_gather, dim3(nb), dim3(256), 0, s, a, 2);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // the backward pass's addends: dW <- P^T dY; dS <- gQ^T dY (128 x 128, as two 64-row halves)
  if ((e = mm(a, 128, 64, true, false, {job(a.Pm, I1, kC, a.dYi, I2, kD, a.dW, I2, kD),
                                        job(a.gQ, I2, kD, a.dYi, I2, kD, a.dS, I3, kD),
                                        job(a.gQ + 64, I2, kD, a.dYi, I2, kD, a.dS + 64 * kD, I3, kD)}, s)) != hipSuccess)
    return e;
  hipLaunchKernelGGL(k_cb_pass<true>, dim3(chains), dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // X = dY S^T; dWk = -dW S^T; dK~ = W dS'^T
  if ((e = mm(a, 128, 128, false, true, {job(a.dYi, I2, kD, a.S, I3, kD, a.X, I2, kD),
                                         job(a.dW, I2, kD, a.S, I3, kD, a.dWk, I2, kD, -1.f),
                                         job(a.W, I2, kD, a.dS, I3, kD, a.dKt, I2, kD)}, s)) != hipSuccess)
    return e;
  // dP = lower(dY W^T); dT = dW bV^T + dWk bgK^T
  if ((e = mm(a, 64, 128, false, true, {job(a.dYi, I2, kD, a.W, I2, kD, a.dP, I1, kC, 1.f, 0, 1),
                                        job(a.dW, I2, kD, a.bV, I2, kD, a.dT, I1, kC),
                                        chained(job(a.dWk, I2, kD, a.bgK, I2, kD, nullptr, 0, 0))}, s)) != hipSuccess)
    return e;
  hipLaunchKernelGGL(k_cb_ew1, dim3(nb), dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // dQ = dQK K; dK = dQK^T Q; d(bV) = T^T dW; d(bgK) = T^T dWk
  if ((e = mm(a, 128, 64, false, false, {job(a.M1, I1, kC, a.Ki, I2, kD, a.dQ, I2, kD)}, s)) != hipSuccess) return e;
  if ((e = mm(a, 128, 64, true, false, {job(a.M1, I1, kC, a.Qi, I2, kD, a.dK, I2, kD),
                                        job(a.Tm, I1, kC, a.dW, I2, kD, a.dbV, I2, kD),
                                        job(a.Tm, I1, kC, a.dWk, I2, kD, a.dbgK, I2, kD)}, s)) != hipSuccess)
    return e;
  // dA = -strict_lower(T^T (dT T^T))
  if ((e = mm(a, 64, 64, false, true, {job(a.dT, I1, kC, a.Tm, I1, kC, a.M1, I1, kC)}, s)) != hipSuccess) return e;
  if ((e = mm(a, 64, 64, true, false, {job(a.Tm, I1, kC, a.M1, I1, kC, a.dA, I1, kC, -1.f, 0, 2)}, s)) != hipSuccess)
    return e;
  hipLaunchKernelGGL(k_cb_ew2, dim3(nb), dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // dK += dAKK K + dAKK^T K
  if ((e = mm(a, 128, 64, false, false, {job(a.dT, I1, kC, a.Ki, I2, kD, a.dK, I2, kD, 1.f, 1)}, s)) != hipSuccess)
    return e;
  if ((e = mm(a, 128, 64, true, false, {job(a.dT, I1, kC, a.Ki, I2, kD, a.dK, I2, kD, 1.f, 1)}, s)) != hipSuccess)
    return e;
  hipLaunchKernelGGL(k_cb_final, dim3(nb), dim3(256), 0, s, a);
  const int64_t nq = a.T * a.hk * (kD / 4);
  if (nq > 0)
    hipLaunchKernelGGL(k_cb_group_sum, dim3(unsigned((nq + 255) / 256)), dim3(256), 0, s, a.dqh, a.dkh, a.T, a.hk,
                       a.hv, dq, dk);
  return hipGetLastError();
}

}  // namespace gdn
