// Speculative (multi-token) decoding: verify a draft of K tokens per sequence, then commit the
// accepted prefix.
//
// The pages decode with four-step speculation from a one-layer multi-token-prediction (MTP) head
// (paper summary "Qwen3.8-Flash-Next", results; analysis notes "Qwen3.8-Flash-Next：架构、效率与
// 技术谱系" §01 MTP row and §04 results table): each step the main model checks a draft of several
// tokens in one pass and keeps the accepted prefix. For a GDN layer that splits into
//   verify: the K draft tokens of each sequence run through the mixer (conv + SiLU, L2 of q and k,
//           the gated delta rule of the analysis notes §03, zero-centred RMSNorm, sigmoid gate)
//           from the cached state and conv cache, which are read and not advanced;
//   commit: the cache is advanced by the first n accepted drafts (0 <= n <= K).
// Instead of a state checkpoint per draft token (64 KB per value head and token), verify logs the
// rank-1 factors of each token's update S <- alpha S + (beta k) e^T -- the normalised key of each
// QK head and the error e of each value head in fp32 (1 KB per token and head), alpha, beta, and
// the raw conv inputs -- and commit applies the first n of them, in order, to the stored state.
// Verify reads each state once and writes none; commit reads and writes it once.
//
// Both kernels run one 256-thread block per (sequence, value head) with the register layout of the
// decode step: thread (cg, rg) = (t % 32, t / 32) holds columns 4cg .. +3 of rows rg + 8j (j < 16)
// of the head's state.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kD = 128;

struct MtpArgs {
  int K, hk, hv, R;
  int64_t C;
  const void *q, *k, *v;          // io [B*K][..] token rows, strides ld_*
  int64_t ld_q, ld_k, ld_v;
  const float *alpha, *beta;      // [B*K][HV]
  const void* gate;               // io [B*K][HV][128]
  const float *conv_w, *norm_w;
  int norm_stride;
  const void* conv_in;            // verify: the conv cache it reads [B][3][C]
  void* conv_state;               // commit: the conv cache, advanced in place
  const float* state_in;          // verify: the states it reads [B][HV][128][128]
  float* state;                   // commit: the states, advanced in place
  void* out;                      // verify: io [B*K][HV][128]
  MtpLog log;
  const int32_t* n_accept;        // commit: [B]
  uint32_t flags;
  float scale, l2_eps, norm_eps;
};

// One rank-1 step on a 16-byte piece of state row i: S <- alpha S + (beta k_i) e^T.
__device__ __forceinline__ float4 rank1(const float4& s, float al, float bk, const float4& e) {
  return make_float4(fmaf(bk, e.x, al * s.x), fmaf(bk, e.y, al * s.y), fmaf(bk, e.z, al * s.z),
                     fmaf(bk, e.w, al * s.w));
}

// Conv channel of channel c of a block serving QK group g and value heads from h0 on: its q head,
// its k head, then its value heads.
__device__ __forceinline__ int64_t block_channel(int c, int g, int h0, int hk) {
  const int64_t qk_ch = int64_t(hk) * kD;
  if (c < kD) return int64_t(g) * kD + c;
  if (c < 2 * kD) return qk_ch + int64_t(g) * kD + (c - kD);
  return 2 * qk_ch + int64_t(h0) * kD + (c - 2 * kD);
}

// LDS layout of the verify kernel (offsets in floats, every region 16-byte aligned).
struct VerifyLds {
  int act, cst, gsh, nwsh, absh, Gh, cA, cB, dkk, dqk, red, ssr, total;
};
__host__ __device__ inline VerifyLds verify_lds(int K, int R) {
  auto pad = [](int n) { return (n + 3) & ~3; };
  VerifyLds L;
  L.act = 0;                                   // [K][(2 + R) 128]
  L.gsh = L.act + K * (2 + R) * kD;            // [K][R 128]
  L.nwsh = L.gsh + K * R * kD;                 // [R 128]
  L.absh = L.nwsh + R * kD;                    // [K][2R]
  L.Gh = L.absh + pad(2 * R * K);              // [R][K]
  L.cA = L.Gh + pad(R * K);                    // [R][K][K]
  L.cB = L.cA + pad(R * K * K);                // [R][K][K]
  L.dkk = L.cB + pad(R * K * K);               // [K][K]
  L.dqk = L.dkk + pad(K * K);                  // [K][K]
  L.red = L.dqk + pad(K * K);                  // [K][2][4][128]
  L.cst = L.red;                               // [3][(2 + R) 128], read only by the conv, before red is used
  L.ssr = L.red + (K * 2 * 4 * kD > 3 * (2 + R) * kD ? K * 2 * 4 * kD : 3 * (2 + R) * kD);  // [4][K]
  L.total = L.ssr + pad(4 * K);
  return L;
}
size_t verify_smem_floats(int K, int R) { return size_t(verify_lds(K, R).total); }
size_t commit_smem_floats(int K, int R) { return size_t(K) * kD + size_t(K) * R * kD + ((2 * R * K + 3) & ~3); }

// Verify needs no state after a draft token, only the outputs and the errors e, and over a draft of
// K tokens both follow from the cached state S0 in closed form (the update equations unrolled, as
// in the chunked prefill): with G_t the cumulative log decay of the draft, gamma_t = exp(G_t),
//   e_t = v_t - gamma_t S0^T k_t - sum_{i<t} exp(G_t - G_i) (k_t.k_i) beta_i e_i
//   y_t = gamma_t S0^T q_t + sum_{i<=t} exp(G_t - G_i) (q_t.k_i) beta_i e_i.
// So a head needs one pass over S0 for the 2K products S0^T k_t, S0^T q_t (one barrier), then a
// K-step recurrence that is independent per column, instead of K dependent steps.
//
// One block per (sequence, value head): the q | k prologue of a QK group is computed by each of its
// value heads' blocks, but no block carries a second state in registers (88 VGPRs, 31 KB of LDS at
// K = 5), so five blocks fit on a CU and their state loads overlap each other's prologues. (One
// block per QK group walking its three value heads with the next head's state prefetched held two
// states in registers, three blocks per CU: 210-215 us against 200 us at B = 256, K = 5.)
template <typename IO>
__global__ void __launch_bounds__(256, 5) k_verify_d128(MtpArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int b = int(blockIdx.x / unsigned(a.hv)), h0 = int(blockIdx.x - unsigned(b) * unsigned(a.hv));
  const int g = h0 / a.R;                  // QK group
  const bool lead = h0 % a.R == 0;         // the block that logs the group's k^ and raw q | k
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int cg = t & 31, rg = t >> 5, col = 4 * cg;
  constexpr int R = 1;                     // value heads of the block
  const int K = a.K, nch = (2 + R) * kD, nv = R * kD;
  const VerifyLds L = verify_lds(K, R);
  float* const act = smem + L.act;    // [K][nch]: q^ | k^ | v^ of each draft token
  float* const cst = smem + L.cst;    // [3][nch] conv cache rows
  float* const gsh = smem + L.gsh;    // [K][nv] gate logits
  float* const nwsh = smem + L.nwsh;  // [nv] gains (1 + w)
  float* const absh = smem + L.absh;  // [K][2R] alpha | beta
  float* const Gh = smem + L.Gh;      // [R][K] cumulative log decay over the draft
  float* const cA = smem + L.cA;      // [R][K][K] exp(G_t - G_i) (k_t.k_i) beta_i, i < t
  float* const cB = smem + L.cB;      // [R][K][K] exp(G_t - G_i) (q_t.k_i) beta_i, i <= t
  float* const dkk = smem + L.dkk;    // [K][K] k_t.k_i
  float* const dqk = smem + L.dqk;    // [K][K] q_t.k_i
  float* const red = smem + L.red;    // [K][a, b][4 waves][128] partial products
  float* const ssr = smem + L.ssr;    // [4 waves][K] partial sums of squares

  const size_t head = size_t(kD) * kD;
  const float* const S0 = a.state_in + (size_t(b) * a.hv + size_t(h0)) * head;
  const int soff = (rg * kD + col) * 4;  // row j of this thread: soff + 4096 j bytes into the head
  float4 S[16];

  // ---- inputs of the group, all requested together as 16-byte pieces: the drafts' raw q | k | v
  // rows (into act, and copied to the log for the commit), the conv cache rows, the gate logits;
  // conv weights, gains, alpha and beta alongside ----
  const bool conv = (a.flags & GDN_CONV) != 0, gate = (a.flags & GDN_GATE) != 0;
  const int64_t row0 = int64_t(b) * K;  // token row of draft 0
  constexpr int VEC = vec16<IO>::N;     // io elements per piece
  const int prow = nch / VEC, pv = nv / VEC;
  const int n_raw = K * prow, n_cache = conv ? 3 * prow : 0, n_all = n_raw + n_cache + (gate ? K * pv : 0);
  // Conv weights and gains come through buffer ranges that are empty when the flag is off (zeros,
  // no memory access), so every load is unconditional and none waits before the next is issued.
  float4 cw[3];
  {
    const auto rw = buf_rsrc(a.conv_w, conv ? int(a.C * 16) : 0);
#pragma unroll
    for (int u = 0; u < 3; ++u) cw[u] = buf_ld16(rw, int(block_channel(min(t + 256 * u, nch - 1), g, h0, a.hk)) * 16, 0);
  }
  const auto rn = buf_rsrc(a.norm_w, (a.flags & GDN_NORM) ? int((size_t(a.hv - 1) * a.norm_stride + kD) * 4) : 0);
  auto gain_off = [&](int i) { return int(size_t(h0 + (4 * i) / kD) * a.norm_stride + (4 * i) % kD) * 4; };
  auto ab_ix = [&](int i, bool& is_alpha) {
    const int tt = i / (2 * R), j = i - tt * 2 * R;
    is_alpha = j < R;
    return (row0 + tt) * a.hv + int64_t(h0) + (j < R ? j : j - R);
  };
  const int i_ab = min(t, 2 * R * K - 1);
  bool ab_alpha;
  const int64_t ix_ab = ab_ix(i_ab, ab_alpha);
  const float4 nw0 = buf_ld16(rn, gain_off(min(t, nv / 4 - 1)), 0);
  const float ab0 = (ab_alpha ? a.alpha : a.beta)[ix_ab];
  auto issue_pieces = [&](int base, uint4 (&pc)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {  // up to four pieces per thread are requested before any is used
      const int i = base + u * 256 + t;
      pc[u] = make_uint4(0u, 0u, 0u, 0u);
      if (i < n_raw) {
        const int tt = i / prow, c0 = (i - tt * prow) * VEC;
        const IO* src = c0 < kD ? static_cast<const IO*>(a.q) + (row0 + tt) * a.ld_q + int64_t(g) * kD + c0
                      : c0 < 2 * kD ? static_cast<const IO*>(a.k) + (row0 + tt) * a.ld_k + int64_t(g) * kD + (c0 - kD)
                                    : static_cast<const IO*>(a.v) + (row0 + tt) * a.ld_v + int64_t(h0) * kD + (c0 - 2 * kD);
        pc[u] = *reinterpret_cast<const uint4*>(src);
      } else if (i < n_raw + n_cache) {
        const int j = (i - n_raw) / prow, c0 = (i - n_raw - j * prow) * VEC;
        pc[u] = *reinterpret_cast<const uint4*>(static_cast<const IO*>(a.conv_in) + (int64_t(b) * 3 + j) * a.C +
                                                block_channel(c0, g, h0, a.hk));
      } else if (i < n_all) {
        const int i2 = i - n_raw - n_cache, tt = i2 / pv, c0 = (i2 - tt * pv) * VEC;
        pc[u] = *reinterpret_cast<const uint4*>(static_cast<const IO*>(a.gate) + ((row0 + tt) * a.hv + int64_t(h0)) * kD + c0);
      }
    }
  };
  auto place_pieces = [&](int base, const uint4 (&pc)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = base + u * 256 + t;
      if (i >= n_all) break;
      float f[VEC];
      vec16<IO>::cvt(pc[u], f);
      float* dst;
      if (i < n_raw) {
        const int tt = i / prow, c0 = (i - tt * prow) * VEC;
        dst = act + tt * nch + c0;
        if (conv && (lead || c0 >= 2 * kD)) *reinterpret_cast<uint4*>(static_cast<IO*>(a.log.raw) + (row0 + tt) * a.C + block_channel(c0, g, h0, a.hk)) = pc[u];
      } else if (i < n_raw + n_cache) {
        const int j = (i - n_raw) / prow, c0 = (i - n_raw - j * prow) * VEC;
        dst = cst + j * nch + c0;
      } else {
        const int i2 = i - n_raw - n_cache, tt = i2 / pv, c0 = (i2 - tt * pv) * VEC;
        dst = gsh + tt * nv + c0;
      }
#pragma unroll
      for (int e = 0; e < VEC; e += 4) *reinterpret_cast<float4*>(dst + e) = make_float4(f[e], f[e + 1], f[e + 2], f[e + 3]);
    }
  };
  // the first 1024 pieces in straight-line code, so their loads share one wait with the loads above
  {
    uint4 pc[4];
    issue_pieces(0, pc);
    place_pieces(0, pc);
  }
  for (int base = 4 * 256; base < n_all; base += 4 * 256) {
    uint4 pc[4];
    issue_pieces(base, pc);
    place_pieces(base, pc);
  }
  if (t < nv / 4) *reinterpret_cast<float4*>(nwsh + 4 * t) = make_float4(1.f + nw0.x, 1.f + nw0.y, 1.f + nw0.z, 1.f + nw0.w);
  if (t < 2 * R * K) {
    absh[t] = ab0;
    a.log.ab[ix_ab * 2 + (ab_alpha ? 0 : 1)] = ab0;
  }
  for (int i = t + 256; i < nv / 4; i += 256) {
    const float4 nw = buf_ld16(rn, gain_off(i), 0);
    *reinterpret_cast<float4*>(nwsh + 4 * i) = make_float4(1.f + nw.x, 1.f + nw.y, 1.f + nw.z, 1.f + nw.w);
  }
  for (int i = t + 256; i < 2 * R * K; i += 256) {
    bool al;
    const int64_t ix = ab_ix(i, al);
    const float val = (al ? a.alpha : a.beta)[ix];
    absh[i] = val;
    a.log.ab[ix * 2 + (al ? 0 : 1)] = val;
  }
  // The first head's state is requested only now: loads complete in order, so had it been
  // requested first, every input of the prologue would have waited for its 64 KB. The conv weights
  // are marked ready here (an empty asm that takes them), so that no later use of them waits on the
  // state.
#pragma unroll
  for (int u = 0; u < 3; ++u) asm volatile("" : "+v"(cw[u].x), "+v"(cw[u].y), "+v"(cw[u].z), "+v"(cw[u].w));
  {
    const auto rs = buf_rsrc(S0, int(head * 4));
#pragma unroll
    for (int j = 0; j < 16; ++j) S[j] = buf_ld16_nt(rs, soff, 4096 * j);
  }
  __syncthreads();
  // conv + SiLU in place, one channel column per thread (tap 3 on the current token)
  if (conv) {
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int c = t + 256 * u;
      if (c < nch) {
        float x[3 + kMaxDrafts];
#pragma unroll
        for (int j = 0; j < 3; ++j) x[j] = cst[j * nch + c];
#pragma unroll
        for (int tt = 0; tt < kMaxDrafts; ++tt) x[3 + tt] = tt < K ? act[tt * nch + c] : 0.f;
#pragma unroll
        for (int tt = 0; tt < kMaxDrafts; ++tt)
          if (tt < K)
            act[tt * nch + c] = siluf_(cw[u].x * x[tt] + cw[u].y * x[tt + 1] + cw[u].z * x[tt + 2] + cw[u].w * x[tt + 3]);
      }
    }
  }
  __syncthreads();

  // ---- L2 of q and k per draft token (wave w takes tokens w, w + 4), k^ to the log; cumulative
  // log decays of each head ----
  const bool l2 = (a.flags & GDN_L2QK) != 0;
  for (int tt = w; tt < K; tt += 4) {
    float* const aq = act + tt * nch;
    float* const ak = aq + kD;
    const float q0 = aq[2 * lane], q1 = aq[2 * lane + 1], k0 = ak[2 * lane], k1 = ak[2 * lane + 1];
    const float sq = wave_sum<64>(q0 * q0 + q1 * q1), sk = wave_sum<64>(k0 * k0 + k1 * k1);
    const float rq = l2 ? 1.0f / sqrtf(sq + a.l2_eps) : 1.0f, rk = l2 ? 1.0f / sqrtf(sk + a.l2_eps) : 1.0f;
    const float kh0 = k0 * rk, kh1 = k1 * rk;
    aq[2 * lane] = q0 * rq;
    aq[2 * lane + 1] = q1 * rq;
    ak[2 * lane] = kh0;
    ak[2 * lane + 1] = kh1;
    if (lead) *reinterpret_cast<float2*>(a.log.kh + ((row0 + tt) * a.hk + g) * kD + 2 * lane) = make_float2(kh0, kh1);
  }
  if (t < R) {
    float gsum = 0.f;
    for (int tt = 0; tt < K; ++tt) {
      gsum += logf(absh[tt * 2 * R + t]);
      Gh[t * K + tt] = gsum;
    }
  }
  __syncthreads();
  // ---- k_t.k_i (i < t) and q_t.k_i (i <= t) of the draft, one wave per pair ----
  for (int pidx = w; pidx < 2 * K * K; pidx += 4) {
    const int isq = pidx >= K * K, pr = isq ? pidx - K * K : pidx, tt = pr / K, i = pr - tt * K;
    if (i > tt || (!isq && i == tt)) continue;  // wave-uniform
    const float* const x = act + tt * nch + (isq ? 0 : kD);
    const float* const y = act + i * nch + kD;
    const float d = wave_sum<64>(x[2 * lane] * y[2 * lane] + x[2 * lane + 1] * y[2 * lane + 1]);
    if (lane == 0) (isq ? dqk : dkk)[tt * K + i] = d;
  }
  __syncthreads();
  for (int i3 = t; i3 < R * K * K; i3 += 256) {
    const int r = i3 / (K * K), pr = i3 - r * K * K, tt = pr / K, i = pr - tt * K;
    const float dec = i <= tt ? __expf(Gh[r * K + tt] - Gh[r * K + i]) * absh[i * 2 * R + R + r] : 0.f;
    cA[i3] = i < tt ? dec * dkk[tt * K + i] : 0.f;
    cB[i3] = i <= tt ? dec * dqk[tt * K + i] : 0.f;
  }
  __syncthreads();

  // ---- the value head ----
  const int c = t & (kD - 1);  // column of the per-column phase
  const bool store_e = t < kD;  // threads 0..127 log e, threads 128..255 store the outputs
  for (int r = 0; r < R; ++r) {
    const int h = h0 + r;
    // S0^T k_t and S0^T q_t of every draft token over this thread's rows, then over row-group pairs
    for (int tt = 0; tt < K; ++tt) {
      const float* const aq = act + tt * nch;
      const float* const ak = aq + kD;
      float4 pa = make_float4(0.f, 0.f, 0.f, 0.f), pb = pa;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float ki = ak[rg + 8 * j], qi = aq[rg + 8 * j];
        pa.x += S[j].x * ki; pa.y += S[j].y * ki; pa.z += S[j].z * ki; pa.w += S[j].w * ki;
        pb.x += S[j].x * qi; pb.y += S[j].y * qi; pb.z += S[j].z * qi; pb.w += S[j].w * qi;
      }
      pa.x = half_pair_sum(pa.x); pa.y = half_pair_sum(pa.y);
      pa.z = half_pair_sum(pa.z); pa.w = half_pair_sum(pa.w);
      pb.x = half_pair_sum(pb.x); pb.y = half_pair_sum(pb.y);
      pb.z = half_pair_sum(pb.z); pb.w = half_pair_sum(pb.w);
      if (lane < 32) {
        *reinterpret_cast<float4*>(&red[((tt * 2) * 4 + w) * kD + col]) = pa;
        *reinterpret_cast<float4*>(&red[((tt * 2 + 1) * 4 + w) * kD + col]) = pb;
      }
    }
    __syncthreads();
    // per column c (every thread; the two halves of the block compute the same values): e_t, y_t
    float e[kMaxDrafts], y[kMaxDrafts];
    const float* const cAr = cA + r * K * K;
    const float* const cBr = cB + r * K * K;
#pragma unroll
    for (int tt = 0; tt < kMaxDrafts; ++tt) {
      e[tt] = 0.f;
      y[tt] = 0.f;
      if (tt < K) {
        const float* const rt = red + (tt * 2) * 4 * kD + c;
        const float a0 = (rt[0] + rt[kD]) + (rt[2 * kD] + rt[3 * kD]);
        const float b0 = (rt[4 * kD] + rt[5 * kD]) + (rt[6 * kD] + rt[7 * kD]);
        const float gam = __expf(Gh[r * K + tt]);
        float ev = act[tt * nch + (2 + r) * kD + c] - gam * a0;
        float yv = gam * b0;
#pragma unroll
        for (int i = 0; i < kMaxDrafts; ++i)
          if (i < tt) {
            ev -= cAr[tt * K + i] * e[i];
            yv += cBr[tt * K + i] * e[i];
          }
        e[tt] = ev;
        y[tt] = a.scale * (yv + cBr[tt * K + tt] * ev);
      }
    }
    // RMSNorm sums per token over the 128 columns (waves 0-1 and 2-3 each cover all of them)
#pragma unroll
    for (int tt = 0; tt < kMaxDrafts; ++tt)
      if (tt < K) {
        const float ss = wave_sum<64>(y[tt] * y[tt]);
        if (lane == 0) ssr[w * K + tt] = ss;
      }
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < kMaxDrafts; ++tt)
      if (tt < K) {
        if (store_e) {
          a.log.e[((row0 + tt) * a.hv + h) * kD + c] = e[tt];
        } else {
          const float ss = ssr[2 * K + tt] + ssr[3 * K + tt];
          const float rsn = (a.flags & GDN_NORM) ? 1.0f / sqrtf(ss / float(kD) + a.norm_eps) : 1.0f;
          float o = y[tt] * rsn * nwsh[r * kD + c];
          if (gate) o *= sigmoidf_(gsh[tt * nv + r * kD + c]);
          io<IO>::st(static_cast<IO*>(a.out) + ((row0 + tt) * a.hv + h) * kD + c, o);
        }
      }
  }
}

// Commit: one block per (sequence, value head), like verify (one state in registers, five blocks per
// CU); the block of a group's first value head also rolls the group's q | k conv-cache channels, each
// block its own value head's channels (each cache channel has one writer).
template <typename IO>
__global__ void __launch_bounds__(256, 5) k_commit_d128(MtpArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  // each XCD walks its own contiguous run of (sequence, value head) items
  const unsigned item = xcd_range_item(blockIdx.x, gridDim.x);
  const int b = int(item / unsigned(a.hv)), h0 = int(item - unsigned(b) * unsigned(a.hv));
  const int g = h0 / a.R;
  const bool lead = h0 % a.R == 0;
  const int t = threadIdx.x, cg = t & 31, rg = t >> 5, col = 4 * cg;
  const int K = a.K;
  const int n = min(max(a.n_accept[b], 0), K);  // out-of-range counts are clamped
  if (n == 0) return;                           // nothing accepted: the cache stays as it is
  float* const kh = smem;                       // [n][128] k^ of the group's QK head
  float* const es = kh + K * kD;                // [n][128] e of the block's value head
  float* const ab = es + K * kD;                // [n][alpha, beta]
  const int64_t row0 = int64_t(b) * K;

  const size_t head = size_t(kD) * kD;
  float* const Sp = a.state + (size_t(b) * a.hv + size_t(h0)) * head;
  const int soff = (rg * kD + col) * 4;
  float4 S[16];
  {
    const auto rs = buf_rsrc(Sp, int(head * 4));
#pragma unroll
    for (int j = 0; j < 16; ++j) S[j] = buf_ld16_nt(rs, soff, 4096 * j);
  }
  for (int i = t; i < n * kD; i += 256) {
    const int tt = i / kD, c = i - tt * kD;
    kh[i] = a.log.kh[((row0 + tt) * a.hk + g) * kD + c];
    es[i] = a.log.e[((row0 + tt) * a.hv + h0) * kD + c];
  }
  for (int i = t; i < n * 2; i += 256) ab[i] = a.log.ab[((row0 + i / 2) * a.hv + h0) * 2 + (i & 1)];
  // conv cache: the last 3 of (cached inputs, accepted raw inputs), per channel; each thread reads
  // its channel's three new rows before writing any
  if (a.flags & GDN_CONV) {
    for (int c = lead ? t : 2 * kD + t; c < 3 * kD; c += 256) {
      const int64_t gc = block_channel(c, g, h0, a.hk);
      IO* const cs = static_cast<IO*>(a.conv_state) + int64_t(b) * 3 * a.C + gc;
      const IO* const rw = static_cast<const IO*>(a.log.raw) + row0 * a.C + gc;
      IO z[3];
#pragma unroll
      for (int j = 0; j < 3; ++j) z[j] = n + j < 3 ? cs[(n + j) * a.C] : rw[(n + j - 3) * a.C];
#pragma unroll
      for (int j = 0; j < 3; ++j) cs[j * a.C] = z[j];
    }
  }
  __syncthreads();

  for (int tt = 0; tt < n; ++tt) {
    const float al = ab[2 * tt], be = ab[2 * tt + 1];
    const float4 ev = *reinterpret_cast<const float4*>(&es[tt * kD + col]);
#pragma unroll
    for (int j = 0; j < 16; ++j) S[j] = rank1(S[j], al, be * kh[tt * kD + rg + 8 * j], ev);
  }
#pragma unroll
  for (int j = 0; j < 16; ++j)
    __builtin_nontemporal_store(__builtin_bit_cast(f32x4, S[j]), reinterpret_cast<f32x4*>(Sp + (rg + 8 * j) * kD + col));
}

MtpLog plan_mtp_log(const Problem& p, int batch, int n_tok, void* base) {
  MtpLog L;
  char* const bb = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* r = bb ? static_cast<void*>(bb + off) : nullptr;
    off += (bytes + 255) & ~size_t(255);
    return r;
  };
  const size_t rows = size_t(batch) * size_t(n_tok);
  L.kh = static_cast<float*>(take(4 * rows * size_t(p.hk) * p.dk));
  L.e = static_cast<float*>(take(4 * rows * size_t(p.hv) * p.dv));
  L.ab = static_cast<float*>(take(4 * rows * size_t(p.hv) * 2));
  L.raw = take(size_t(p.bf16 ? 2 : 4) * rows * size_t(p.C));
  L.bytes = off;
  return L;
}

hipError_t launch_verify(const Problem& p, int batch, int n_tok, const void* q, const void* k, const void* v,
                         int64_t ld_q, int64_t ld_k, int64_t ld_v, const float* alpha, const float* beta,
                         const void* gate, const float* conv_w, const float* norm_w, const void* conv_state,
                         const float* state, void* out, const MtpLog& log, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  const int R = p.hv / p.hk;
  MtpArgs a{n_tok, p.hk, p.hv, R, p.C, q, k, v, ld_q, ld_k, ld_v, alpha, beta, gate, conv_w, norm_w,
            p.norm_stride, conv_state, nullptr, state, nullptr, out, log, nullptr, p.flags, p.scale,
            p.l2_eps, p.norm_eps};
  const size_t smem = verify_smem_floats(n_tok, 1) * 4;
  const dim3 grid(unsigned(batch) * unsigned(p.hv));
  if (p.bf16) hipLaunchKernelGGL(k_verify_d128<bf16>, grid, dim3(256), smem, s, a);
  else hipLaunchKernelGGL(k_verify_d128<float>, grid, dim3(256), smem, s, a);
  return hipGetLastError();
}

hipError_t launch_commit(const Problem& p, int batch, int n_tok, const int32_t* n_accept, const MtpLog& log,
                         void* conv_state, float* state, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  const int R = p.hv / p.hk;
  MtpArgs a{n_tok, p.hk, p.hv, R, p.C, nullptr, nullptr, nullptr, 0, 0, 0, nullptr, nullptr, nullptr,
            nullptr, nullptr, p.norm_stride, nullptr, conv_state, nullptr, state, nullptr, log, n_accept,
            p.flags, p.scale, p.l2_eps, p.norm_eps};
  const size_t smem = commit_smem_floats(n_tok, 1) * 4;
  const dim3 grid(unsigned(batch) * unsigned(p.hv));
  if (p.bf16) hipLaunchKernelGGL(k_commit_d128<bf16>, grid, dim3(256), smem, s, a);
  else hipLaunchKernelGGL(k_commit_d128<float>, grid, dim3(256), smem, s, a);
  return hipGetLastError();
}

}  // namespace gdn
