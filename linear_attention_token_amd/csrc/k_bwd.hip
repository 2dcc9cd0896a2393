// Backward of the gated delta rule recurrence (fp32, d_k = d_v = 128): given dL/dy_t and dL/dS_final,
// the derivatives for q, k, v, alpha, beta and the initial state. The update statements are those of
// the analysis notes "Qwen3.8-Flash-Next：架构、效率与技术谱系" (§03 update equations); the reverse pass
// applies the chain rule to them last to first:
//   y_t = scale S_t^T q_t      ->  dS += scale q_t dy_t^T,  dq_t = scale S_t dy_t
//   S_t = S~ + beta k e^T      ->  dbeta = k^T dS e,  dk = beta dS e,  de = beta dS^T k
//   e = v - S~^T k             ->  dv = de,  dS~ = dS - k de^T,  dk -= S~ de
//   S~ = alpha S_{t-1}         ->  dalpha = <S_{t-1}, dS~>,  dS_{t-1} = alpha dS~
//
// Each value column of the state evolves on its own (the columns share only k, alpha, beta), so a
// (sequence, value head) chain is split into 8 slices of 16 columns, one workgroup each: 256 threads,
// each holding a 2x4 tile (rows 2 ti, 2 ti + 1, slice columns 4 tj .. 4 tj + 3; ti = thread / 4,
// tj = thread % 4). Column sums are shuffles across a wave's 16 row groups plus one LDS exchange across
// the 4 waves; row sums are 4-lane shuffles and give per-slice partials of dq and dk (and of dalpha and
// dbeta), which k_bwd_reduce adds over the slices and over the value heads that share a QK head.
// A forward pass stores every state S_t (fp32, slot-major so that the stores coalesce) and every error
// e_t in the workspace; the reverse pass reads them back, so every state it uses is the forward's own,
// with no inversion of the update.
#include "gdn_device.h"
#include "ext_internal.h"

namespace gdn {

namespace {

constexpr int kBD = 128;
constexpr int kBT = 256;         // threads per workgroup
constexpr int kSC = 16;          // columns per slice
constexpr int kNS = kBD / kSC;   // slices per chain
constexpr int kR = 2, kC = 4;    // a thread's tile: kR rows x kC columns
constexpr int kTJ = kSC / kC;    // column tiles per slice (threads per row)
static_assert((kBD / kR) * kTJ == kBT, "the tiles must cover the slice with 256 threads");

struct BwdLds {
  float col[2][4][kSC];   // column-sum exchange, double-buffered by token parity
  float coly[2][4][kSC + 4];  // forward pass with y output: S~^T q per column, and k.q
  float dal[2][4];        // per-wave dalpha partials, written one token and read at the next
};

// Workgroup barrier that waits only for this thread's LDS accesses (lgkmcnt(0)), not for its global
// loads: __syncthreads would also drain the loads issued ahead for the next token (vmcnt(0)). The
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));  // vmcnt 63, expcnt 7, lgkmcnt 0
  asm volatile("s_barrier" ::: "memory");
}

// The forward pass with y output exchanges S~^T q and k.q along with S~^T k (one barrier): y_t =
// scale (S~^T q + beta e (k.q)) since S_t = S~ + beta k e^T.
__device__ __forceinline__ void col_sum3(float (&part)[kC], float (&full)[kC], float (&party)[kC], float (&fully)[kC],
                                         float& kq, BwdLds& L, int buf) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, tj = t % kTJ;
#pragma unroll
  for (int o = kTJ; o < 64; o <<= 1) {
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      part[c] += __shfl_xor(part[c], o, kWave);
      party[c] += __shfl_xor(party[c], o, kWave);
    }
    kq += __shfl_xor(kq, o, kWave);
  }
  if (lane < kTJ) {
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      L.col[buf][w][kC * tj + c] = part[c];
      L.coly[buf][w][kC * tj + c] = party[c];
    }
    if (tj == 0) L.coly[buf][w][kSC] = kq;
  }
  lds_barrier();
#pragma unroll
  for (int c = 0; c < kC; ++c) {
    full[c] = L.col[buf][0][kC * tj + c] + L.col[buf][1][kC * tj + c] + L.col[buf][2][kC * tj + c] +
              L.col[buf][3][kC * tj + c];
    fully[c] = L.coly[buf][0][kC * tj + c] + L.coly[buf][1][kC * tj + c] + L.coly[buf][2][kC * tj + c] +
               L.coly[buf][3][kC * tj + c];
  }
  kq = L.coly[buf][0][kSC] + L.coly[buf][1][kSC] + L.coly[buf][2][kSC] + L.coly[buf][3][kSC];
}

// Column sums: part[c] is this thread's sum over its rows for column c of its tile; returns the sum over
// all 128 rows in every thread of the column. One barrier.
__device__ __forceinline__ void col_sum(float (&part)[kC], float (&full)[kC], BwdLds& L, int buf) {
  float (*col)[4][kSC] = L.col;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, tj = t % kTJ;
#pragma unroll
  for (int c = 0; c < kC; ++c)
#pragma unroll
    for (int o = kTJ; o < 64; o <<= 1) part[c] += __shfl_xor(part[c], o, kWave);
  if (lane < kTJ)
#pragma unroll
    for (int c = 0; c < kC; ++c) col[buf][w][kC * tj + c] = part[c];
  lds_barrier();
#pragma unroll
  for (int c = 0; c < kC; ++c)
    full[c] = col[buf][0][kC * tj + c] + col[buf][1][kC * tj + c] + col[buf][2][kC * tj + c] + col[buf][3][kC * tj + c];
}

__device__ __forceinline__ float row_sum(float x) {  // over the column tiles of a slice
#pragma unroll
  for (int o = 1; o < kTJ; o <<= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

__device__ __forceinline__ void ld4f(const float* p, float (&o)[4]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
}
__device__ __forceinline__ void st4f(float* p, const float (&o)[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ void st2f(float* p, const float (&o)[kR]) {
  *reinterpret_cast<float2*>(p) = make_float2(o[0], o[1]);
}
__device__ __forceinline__ void ldr(const float* p, float (&o)[kR]) {  // kR = 2 consecutive floats
  const float2 a = *reinterpret_cast<const float2*>(p);
  o[0] = a.x; o[1] = a.y;
}

// A 128x128 fp32 matrix [row][col] <-> this thread's tile (rows kR ti .., columns col ..).
__device__ __forceinline__ void ld_tile_mat(const float* m, float (&s)[kR][kC], int ti, int col) {
#pragma unroll
  for (int r = 0; r < kR; ++r) ld4f(m + (kR * ti + r) * kBD + col, s[r]);
}
__device__ __forceinline__ void st_tile_mat(float* m, const float (&s)[kR][kC], int ti, int col) {
#pragma unroll
  for (int r = 0; r < kR; ++r) st4f(m + (kR * ti + r) * kBD + col, s[r]);
}
// Workspace copy of a slice state, slot-major: row r of thread t at (r * 256 + t) * 4, so each store or
// load instruction of a wave covers 1 KB of consecutive bytes.
// The kept states are written once and read back once, much later: non-temporal accesses keep them
// from displacing the inputs in the caches.
__device__ __forceinline__ void st_tile_ws(float* p, const float (&s)[kR][kC]) {
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    uint4 v;
    v.x = __float_as_uint(s[r][0]); v.y = __float_as_uint(s[r][1]);
    v.z = __float_as_uint(s[r][2]); v.w = __float_as_uint(s[r][3]);
    stnt16(p + (r * kBT + threadIdx.x) * kC, v);
  }
}
__device__ __forceinline__ void ld_tile_ws(const float* p, float (&s)[kR][kC]) {
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const uint4 v = ldnt16(p + (r * kBT + threadIdx.x) * kC);
    s[r][0] = __uint_as_float(v.x); s[r][1] = __uint_as_float(v.y);
    s[r][2] = __uint_as_float(v.z); s[r][3] = __uint_as_float(v.w);
  }
}

__device__ __forceinline__ void zero(float (&s)[kR][kC]) {
#pragma unroll
  for (int r = 0; r < kR; ++r)
#pragma unroll
    for (int c = 0; c < kC; ++c) s[r][c] = 0.f;
}

}  // namespace

// grid: n_seqs * HV * kNS workgroups; workgroup (n, h, slice).
__global__ void __launch_bounds__(kBT) k_bwd_d128(BwdArgs a) {
  __shared__ BwdLds L;
  const int t = threadIdx.x, ti = t / kTJ, tj = t % kTJ;
  const int sl = blockIdx.x % kNS, chain = blockIdx.x / kNS;
  const int n = chain / a.hv, h = chain - n * a.hv, g = h * a.hk / a.hv;
  const int col = sl * kSC + kC * tj;  // first value column of this thread
  const int64_t s0 = min(max(int64_t(a.cu[n]), int64_t(0)), a.T);
  const int64_t s1 = min(max(int64_t(a.cu[n + 1]), s0), a.T);
  const int64_t HV = a.hv, HK = a.hk;
  const int64_t chain_off = (int64_t(n) * HV + h) * kBD * kBD;
  auto ws_state = [&](int64_t tok) { return a.states + ((tok * HV + h) * kNS + sl) * (kBT * kR * kC); };

  float S[kR][kC];
  if (a.s0) ld_tile_mat(a.s0 + chain_off, S, ti, col); else zero(S);
  const bool fwd = a.mode & kBwdForward, rev = a.mode & kBwdReverse, want_y = a.mode & kBwdWriteY;
  int buf = 0;
  if (fwd) {

  // ---- forward: store S_t and e_t (and y_t); the next token's inputs load while this one is processed ----
  float kr[kR], vc[kC], al = 1.f, be = 0.f;
  if (s0 < s1) {
    ldr(a.k + (s0 * HK + g) * kBD + kR * ti, kr);
    ld4f(a.v + (s0 * HV + h) * kBD + col, vc);
    al = a.alpha[s0 * HV + h];
    be = a.beta[s0 * HV + h];
  }
  for (int64_t tok = s0; tok < s1; ++tok, buf ^= 1) {
    const int64_t nx = min(tok + 1, s1 - 1);
    float kn[kR], vn[kC];
    ldr(a.k + (nx * HK + g) * kBD + kR * ti, kn);
    ld4f(a.v + (nx * HV + h) * kBD + col, vn);
    const float aln = a.alpha[nx * HV + h], ben = a.beta[nx * HV + h];
    float part[kC], full[kC];
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      float acc = 0.f;
#pragma unroll
      for (int r = 0; r < kR; ++r) acc = fmaf(S[r][c], kr[r], acc);
      part[c] = al * acc;  // (S~^T k) partial, S~ = alpha S
    }
    float fy[kC];
    float kq = 0.f;
    if (want_y) {  // y_t = scale (S~^T q + beta e (k.q)), exchanged with S~^T k
      float qq[kR], py[kC];
      ldr(a.q + (tok * HK + g) * kBD + kR * ti, qq);
#pragma unroll
      for (int c = 0; c < kC; ++c) {
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < kR; ++r) acc = fmaf(S[r][c], qq[r], acc);
        py[c] = al * acc;
      }
#pragma unroll
      for (int r = 0; r < kR; ++r) kq = fmaf(kr[r], qq[r], kq);
      col_sum3(part, full, py, fy, kq, L, buf);
    } else {
      col_sum(part, full, L, buf);
    }
    float e[kC];
#pragma unroll
    for (int c = 0; c < kC; ++c) e[c] = vc[c] - full[c];
#pragma unroll
    for (int r = 0; r < kR; ++r)
#pragma unroll
      for (int c = 0; c < kC; ++c) S[r][c] = fmaf(be * kr[r], e[c], al * S[r][c]);
    st_tile_ws(ws_state(tok), S);
    if (ti == 0) {
      st4f(a.errs + (tok * HV + h) * kBD + col, e);
      if (want_y) {
#pragma unroll
        for (int c = 0; c < kC; ++c) fy[c] = a.scale * fmaf(be * kq, e[c], fy[c]);
        st4f(a.y + (tok * HV + h) * kBD + col, fy);
      }
    }
#pragma unroll
    for (int i = 0; i < kR; ++i) kr[i] = kn[i];
#pragma unroll
    for (int i = 0; i < kC; ++i) vc[i] = vn[i];
    al = aln;
    be = ben;
  }
  }  // forward
  if (!rev) return;
  __threadfence();
  __syncthreads();

  // ---- reverse ----
  // Iteration t holds P = S_{t-1} and works on token t; it also loads S_{t-2} and token t-1's inputs
  // for the next iteration, and computes token t-1's dq = scale S_{t-1} dy_{t-1} from the P it holds.
  // The last token's dq uses S itself.
  float dS[kR][kC];
  if (a.dsf) ld_tile_mat(a.dsf + chain_off, dS, ti, col); else zero(dS);
  int64_t pending = -1;  // token whose dalpha partials wait in L.dal[pbuf]
  int pbuf = 0;
  const int64_t part_stride = kNS;  // per-slice partials: [T][HV][kNS][...]
  if (s1 > s0) {
    struct TokIn {
      float q[kR], k[kR], dy[kC], e[kC], al, be;
    };
    auto load_in = [&](int64_t tk, TokIn& x) {
      ldr(a.q + (tk * HK + g) * kBD + kR * ti, x.q);
      ldr(a.k + (tk * HK + g) * kBD + kR * ti, x.k);
      ld4f(a.dy + (tk * HV + h) * kBD + col, x.dy);
      ld4f(a.errs + (tk * HV + h) * kBD + col, x.e);
      x.al = a.alpha[tk * HV + h];
      x.be = a.beta[tk * HV + h];
    };
    auto load_state = [&](int64_t tk, float (&st)[kR][kC]) {  // S_tk; tk = s0 - 1 is the initial state
      if (tk >= s0) ld_tile_ws(ws_state(tk), st);
      else if (a.s0) ld_tile_mat(a.s0 + chain_off, st, ti, col);
      else zero(st);
    };
    auto store_dq = [&](int64_t tk, const float (&src)[kR][kC], const float (&dy4)[kC]) {
      float dq[kR];
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < kC; ++c) acc = fmaf(src[r][c], dy4[c], acc);
        dq[r] = row_sum(a.scale * acc);
      }
      if (tj == 0) st2f(a.dqv + ((tk * HV + h) * part_stride + sl) * kBD + kR * ti, dq);
    };
    // One token: P = S_{tok-1}, x its inputs. Loads token tok-1's inputs, then S_{tok-2}, in that
    // order, so that the dq of token tok-1 at the end waits only for the inputs.
    auto step = [&](int64_t tok, float (&P)[kR][kC], float (&Pn)[kR][kC], const TokIn& x, TokIn& nx) {
      const bool more = tok > s0;
      if (more) {
        load_in(tok - 1, nx);
        load_state(tok - 2, Pn);
      }
#pragma unroll
      for (int r = 0; r < kR; ++r)
#pragma unroll
        for (int c = 0; c < kC; ++c) dS[r][c] = fmaf(a.scale * x.q[r], x.dy[c], dS[r][c]);
      float part[kC], dsk[kC];
#pragma unroll
      for (int c = 0; c < kC; ++c) {
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < kR; ++r) acc = fmaf(dS[r][c], x.k[r], acc);
        part[c] = acc;
      }
      col_sum(part, dsk, L, buf);
      if (t == 0 && pending >= 0)
        a.dalpha_part[(pending * HV + h) * kNS + sl] = L.dal[pbuf][0] + L.dal[pbuf][1] + L.dal[pbuf][2] + L.dal[pbuf][3];
      float de[kC];
#pragma unroll
      for (int c = 0; c < kC; ++c) de[c] = x.be * dsk[c];
      if (ti == 0) {
        float db = 0.f;
#pragma unroll
        for (int c = 0; c < kC; ++c) db = fmaf(dsk[c], x.e[c], db);
        db = row_sum(db);
        if (t == 0) a.dbeta_part[(tok * HV + h) * kNS + sl] = db;
        st4f(a.dv + (tok * HV + h) * kBD + col, de);
      }
      float dk[kR], dal = 0.f;
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        float u = 0.f, y = 0.f;
#pragma unroll
        for (int c = 0; c < kC; ++c) {
          u = fmaf(dS[r][c], x.e[c], u);
          y = fmaf(P[r][c], de[c], y);
          const float dst = fmaf(-x.k[r], de[c], dS[r][c]);
          dal = fmaf(P[r][c], dst, dal);
          dS[r][c] = x.al * dst;
        }
        dk[r] = row_sum(x.be * u - x.al * y);
      }
      if (tj == 0) st2f(a.dkv + ((tok * HV + h) * part_stride + sl) * kBD + kR * ti, dk);
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) dal += __shfl_xor(dal, o, kWave);
      if ((t & 63) == 0) L.dal[buf][t >> 6] = dal;
      pending = tok;
      pbuf = buf;
      buf ^= 1;
      if (more) store_dq(tok - 1, P, nx.dy);  // dq_{tok-1} = scale S_{tok-1} dy_{tok-1}
    };
    if (!fwd) load_state(s1 - 1, S);  // the final state, kept by an earlier forward launch
    TokIn A, B;
    float P0[kR][kC], P1[kR][kC];
    load_in(s1 - 1, A);
    store_dq(s1 - 1, S, A.dy);  // the last token's dq from the final state
    load_state(s1 - 2, P0);
    // two tokens per trip with the register sets swapped, so no copy waits on a load in flight
    for (int64_t tok = s1 - 1; tok >= s0; tok -= 2) {
      step(tok, P0, P1, A, B);
      if (tok - 1 >= s0) step(tok - 1, P1, P0, B, A);
    }
  }
  __syncthreads();
  if (t == 0 && pending >= 0)
    a.dalpha_part[(pending * HV + h) * kNS + sl] = L.dal[pbuf][0] + L.dal[pbuf][1] + L.dal[pbuf][2] + L.dal[pbuf][3];
  if (a.ds0) st_tile_mat(a.ds0 + chain_off, dS, ti, col);
}

// dq, dk per QK head: the sum over the slices and over the value heads that read it; dalpha, dbeta:
// the sum over the slices.
__global__ void __launch_bounds__(256) k_bwd_reduce(int64_t T, int hk, int hv, const float* __restrict__ dqv,
                                                    const float* __restrict__ dkv, const float* __restrict__ dap,
                                                    const float* __restrict__ dbp, float* __restrict__ dq,
                                                    float* __restrict__ dk, float* __restrict__ dalpha,
                                                    float* __restrict__ dbeta) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t nq = T * hk * kBD;
  if (i < nq) {
    const int64_t tok = i / (int64_t(hk) * kBD);
    const int rem = int(i - tok * hk * kBD), gq = rem / kBD, d = rem - gq * kBD;
    const int per = hv / hk;
    float sq = 0.f, sk = 0.f;
    for (int u = 0; u < per; ++u)
#pragma unroll
      for (int sl = 0; sl < kNS; ++sl) {
        const int64_t j = ((tok * hv + gq * per + u) * kNS + sl) * kBD + d;
        sq += dqv[j];
        sk += dkv[j];
      }
    dq[i] = sq;
    dk[i] = sk;
  } else if (i < nq + T * hv) {
    const int64_t j = i - nq;  // (tok, h)
    float sa = 0.f, sb = 0.f;
#pragma unroll
    for (int sl = 0; sl < kNS; ++sl) {
      sa += dap[j * kNS + sl];
      sb += dbp[j * kNS + sl];
    }
    dalpha[j] = sa;
    dbeta[j] = sb;
  }
}

hipError_t launch_bwd(const BwdArgs& a, float* dq, float* dk, float* dalpha, float* dbeta, hipStream_t s) {
  if (a.n_seqs == 0) return hipSuccess;
  hipLaunchKernelGGL(k_bwd_d128, dim3(static_cast<unsigned>(a.n_seqs * a.hv * kNS)), dim3(kBT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.T == 0 || !(a.mode & kBwdReverse)) return e;
  const int64_t n = a.T * a.hk * kBD + a.T * a.hv;
  hipLaunchKernelGGL(k_bwd_reduce, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, a.T, a.hk, a.hv,
                     a.dqv, a.dkv, a.dalpha_part, a.dbeta_part, dq, dk, dalpha, dbeta);
  return hipGetLastError();
}

}  // namespace gdn
