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
// the raw conv inputs -- and commit replays the first n of them onto the stored state with the
// same fp32 operations verify used in registers, so the committed state is exactly verify's state
// after n tokens. Verify reads each state once and writes none; commit reads and writes it once.
//
// Both kernels run one 256-thread block per (sequence, QK group) with the register layout of the
// decode step: thread (cg, rg) = (t % 32, t / 32) holds columns 4cg .. +3 of rows rg + 8j (j < 16)
// of a head's state. The next head's state is prefetched (non-temporal) while the current one is
// worked on -- after the last head through an empty buffer range, which reads zeros without
// touching memory -- and every wave issues the same memory instructions per head, so the waits for
// the prefetch are exact counts that leave earlier stores in flight.
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

// One rank-1 step on a 16-byte piece of state row i: S <- alpha S + (beta k_i) e^T. Verify applies
// it in registers and commit replays it from the log; the explicit fused multiply-adds make both
// round alike.
__device__ __forceinline__ float4 rank1(const float4& s, float al, float bk, const float4& e) {
  return make_float4(fmaf(bk, e.x, al * s.x), fmaf(bk, e.y, al * s.y), fmaf(bk, e.z, al * s.z),
                     fmaf(bk, e.w, al * s.w));
}

// Conv channel index (q, then k, then v channels of all heads) of channel c of QK group g, where a
// group's channels are its q head, its k head and its R value heads.
__device__ __forceinline__ int64_t group_channel(int c, int g, int R, int hk) {
  const int64_t qk_ch = int64_t(hk) * kD;
  if (c < kD) return int64_t(g) * kD + c;
  if (c < 2 * kD) return qk_ch + int64_t(g) * kD + (c - kD);
  return 2 * qk_ch + int64_t(g) * R * kD + (c - 2 * kD);
}

size_t verify_smem_floats(int K, int R) {
  const int nch = (2 + R) * kD, nv = R * kD;
  return size_t(K) * nch + size_t(K) * nv + nv + ((2 * R * K + 3) & ~3) + ((K + 3) & ~3) + 2 * 8 * kD;
}
size_t commit_smem_floats(int K, int R) { return size_t(K) * kD + size_t(K) * R * kD + ((2 * R * K + 3) & ~3); }

// Two blocks per CU: at three, the token loop's registers push part of the next head's prefetch
// into scratch, whose spill stores wait for those loads at once.
template <typename IO>
__global__ void __launch_bounds__(256, 2) k_verify_d128(MtpArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int b = int(blockIdx.x / unsigned(a.hk)), g = int(blockIdx.x - unsigned(b) * unsigned(a.hk));
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int cg = t & 31, rg = t >> 5, col = 4 * cg;
  const int R = a.R, K = a.K, nch = (2 + R) * kD, nv = R * kD;
  float* const act = smem;                           // [K][nch]: q^ | k^ | v^ of each draft token
  float* const gsh = act + K * nch;                  // [K][nv] gate logits
  float* const nwsh = gsh + K * nv;                  // [nv] gains (1 + w)
  float* const absh = nwsh + nv;                     // [K][2R] alpha | beta
  float* const qks = absh + ((2 * R * K + 3) & ~3);  // [K] q^.k^
  float* const red = qks + ((K + 3) & ~3);           // [2 buffers][4 waves][a, b][128]

  const size_t head = size_t(kD) * kD;
  const float* const S0 = a.state_in + (size_t(b) * a.hv + size_t(g) * R) * head;
  const int soff = (rg * kD + col) * 4;  // row j of this thread: soff + 4096 j bytes into the head
  float4 S[16], N[16];
  {
    const auto rs = buf_rsrc(S0, int(head * 4));
#pragma unroll
    for (int j = 0; j < 16; ++j) S[j] = buf_ld16_nt(rs, soff, 4096 * j);
  }

  // ---- conv + SiLU of the group's channels for every draft token (3 passes of 256 channels cover
  // the 640-768 channels of a group); the raw inputs go to the log for the commit ----
  const bool conv = (a.flags & GDN_CONV) != 0, gate = (a.flags & GDN_GATE) != 0;
  const int64_t row0 = int64_t(b) * K;  // token row of draft 0
#pragma unroll 1
  for (int u = 0; u < 3; ++u) {  // (not unrolled: the first state is in flight meanwhile)
    const int c = min(t + 256 * u, nch - 1);  // threads past the end redo the last channel, unstored
    const int64_t gc = group_channel(c, g, R, a.hk);
    const IO* src;
    int64_t ld;
    if (c < kD) {
      src = static_cast<const IO*>(a.q) + int64_t(g) * kD + c; ld = a.ld_q;
    } else if (c < 2 * kD) {
      src = static_cast<const IO*>(a.k) + int64_t(g) * kD + (c - kD); ld = a.ld_k;
    } else {
      src = static_cast<const IO*>(a.v) + int64_t(g) * nv + (c - 2 * kD); ld = a.ld_v;
    }
    float x[3 + kMaxDrafts];  // the three cached inputs, then the drafts
#pragma unroll
    for (int j = 0; j < 3; ++j)
      x[j] = conv ? io<IO>::ld(static_cast<const IO*>(a.conv_in) + (int64_t(b) * 3 + j) * a.C + gc) : 0.f;
#pragma unroll
    for (int tt = 0; tt < kMaxDrafts; ++tt) x[3 + tt] = tt < K ? io<IO>::ld(src + (row0 + tt) * ld) : 0.f;
    const float4 cw = conv ? reinterpret_cast<const float4*>(a.conv_w)[gc] : make_float4(0.f, 0.f, 0.f, 1.f);
    if (t + 256 * u < nch) {
#pragma unroll
      for (int tt = 0; tt < kMaxDrafts; ++tt) {
        if (tt >= K) break;
        float val = x[3 + tt];
        if (conv) {
          val = siluf_(cw.x * x[tt] + cw.y * x[tt + 1] + cw.z * x[tt + 2] + cw.w * x[tt + 3]);
          io<IO>::st(static_cast<IO*>(a.log.raw) + (row0 + tt) * a.C + gc, x[3 + tt]);
        }
        act[tt * nch + c] = val;
      }
    }
  }
  // gate logits, gains, alpha and beta of the group's heads (alpha and beta also to the log)
  if (gate)
    for (int i = t; i < K * nv; i += 256) {
      const int tt = i / nv, j = i - tt * nv;
      gsh[i] = io<IO>::ld(static_cast<const IO*>(a.gate) + ((row0 + tt) * a.hv + int64_t(g) * R) * kD + j);
    }
  for (int i = t; i < nv; i += 256)
    nwsh[i] = 1.0f + ((a.flags & GDN_NORM) ? a.norm_w[size_t(g * R + i / kD) * a.norm_stride + i % kD] : 0.f);
  for (int i = t; i < 2 * R * K; i += 256) {
    const int tt = i / (2 * R), j = i - tt * 2 * R, r = j < R ? j : j - R;
    const int64_t ix = (row0 + tt) * a.hv + int64_t(g) * R + r;
    const float val = (j < R ? a.alpha : a.beta)[ix];
    absh[i] = val;
    a.log.ab[ix * 2 + (j < R ? 0 : 1)] = val;
  }
  __syncthreads();

  // ---- L2 of q and k per draft token (wave w takes tokens w, w + 4), q^.k^, k^ to the log ----
  const bool l2 = (a.flags & GDN_L2QK) != 0;
  for (int tt = w; tt < K; tt += 4) {
    float* const aq = act + tt * nch;
    float* const ak = aq + kD;
    const float q0 = aq[2 * lane], q1 = aq[2 * lane + 1], k0 = ak[2 * lane], k1 = ak[2 * lane + 1];
    const float sq = group_sum<64>(q0 * q0 + q1 * q1), sk = group_sum<64>(k0 * k0 + k1 * k1);
    const float d = group_sum<64>(q0 * k0 + q1 * k1);
    const float rq = l2 ? 1.0f / sqrtf(sq + a.l2_eps) : 1.0f, rk = l2 ? 1.0f / sqrtf(sk + a.l2_eps) : 1.0f;
    const float kh0 = k0 * rk, kh1 = k1 * rk;
    aq[2 * lane] = q0 * rq;
    aq[2 * lane + 1] = q1 * rq;
    ak[2 * lane] = kh0;
    ak[2 * lane + 1] = kh1;
    *reinterpret_cast<float2*>(a.log.kh + ((row0 + tt) * a.hk + g) * kD + 2 * lane) = make_float2(kh0, kh1);
    if (lane == 0) qks[tt] = d * rq * rk;
  }
  __syncthreads();

  // ---- value heads in turn, each through the K drafts with its state in registers ----
  int ph = 0;  // reduction buffer parity: one barrier per token step
  for (int r = 0; r < R; ++r) {
    const int h = g * R + r;
    {  // the next head's state; after the last head an empty range (zeros, no memory access)
      const auto rn = buf_rsrc(S0 + size_t(r + 1 < R ? r + 1 : r) * head, r + 1 < R ? int(head * 4) : 0);
#pragma unroll
      for (int j = 0; j < 16; ++j) N[j] = buf_ld16_nt(rn, soff, 4096 * j);
    }
    for (int tt = 0; tt < K; ++tt) {
      const float* const aq = act + tt * nch;
      const float* const ak = aq + kD;
      const float al = absh[tt * 2 * R + r], be = absh[tt * 2 * R + R + r];
      // a = S^T k^, b = S^T q^ over this thread's rows, then over the 8 row groups
      float4 pa = make_float4(0.f, 0.f, 0.f, 0.f), pb = pa;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float ki = ak[rg + 8 * j], qi = aq[rg + 8 * j];
        pa.x += S[j].x * ki; pa.y += S[j].y * ki; pa.z += S[j].z * ki; pa.w += S[j].w * ki;
        pb.x += S[j].x * qi; pb.y += S[j].y * qi; pb.z += S[j].z * qi; pb.w += S[j].w * qi;
      }
      pa.x += __shfl_xor(pa.x, 32, 64); pa.y += __shfl_xor(pa.y, 32, 64);
      pa.z += __shfl_xor(pa.z, 32, 64); pa.w += __shfl_xor(pa.w, 32, 64);
      pb.x += __shfl_xor(pb.x, 32, 64); pb.y += __shfl_xor(pb.y, 32, 64);
      pb.z += __shfl_xor(pb.z, 32, 64); pb.w += __shfl_xor(pb.w, 32, 64);
      float* const rb = red + (ph & 1) * (8 * kD);
      ++ph;
      if (lane < 32) {
        *reinterpret_cast<float4*>(&rb[(2 * w) * kD + col]) = pa;
        *reinterpret_cast<float4*>(&rb[(2 * w + 1) * kD + col]) = pb;
      }
      __syncthreads();
      float4 av = make_float4(0.f, 0.f, 0.f, 0.f), bv = av;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float4 x = *reinterpret_cast<const float4*>(&rb[(2 * ww) * kD + col]);
        const float4 y = *reinterpret_cast<const float4*>(&rb[(2 * ww + 1) * kD + col]);
        av.x += x.x; av.y += x.y; av.z += x.z; av.w += x.w;
        bv.x += y.x; bv.y += y.y; bv.z += y.z; bv.w += y.w;
      }
      // e = v^ - alpha a (S~ = alpha S);  y = S_t^T q^ = alpha b + beta (q^.k^) e
      const float4 vv = *reinterpret_cast<const float4*>(aq + (2 + r) * kD + col);
      const float4 ev = make_float4(vv.x - al * av.x, vv.y - al * av.y, vv.z - al * av.z, vv.w - al * av.w);
      const float bq = be * qks[tt];
      const float y[4] = {a.scale * (al * bv.x + bq * ev.x), a.scale * (al * bv.y + bq * ev.y),
                          a.scale * (al * bv.z + bq * ev.z), a.scale * (al * bv.w + bq * ev.w)};
      // e to the log: wave w stores columns 32w .. 32w + 31 (lanes 8w .. 8w + 7 of its row group)
      if ((lane >> 3) == w)
        *reinterpret_cast<float4*>(a.log.e + ((row0 + tt) * a.hv + h) * kD + col) = ev;
#pragma unroll
      for (int j = 0; j < 16; ++j) S[j] = rank1(S[j], al, be * ak[rg + 8 * j], ev);
      // RMSNorm over the head's 128 outputs (every row group holds them all), gain, gate; wave w
      // stores channel col + w of each column group (its two row groups write the same values)
      const float ss = group_sum<32>(y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3]);
      const float rsn = (a.flags & GDN_NORM) ? 1.0f / sqrtf(ss / float(kD) + a.norm_eps) : 1.0f;
      const float yw = w == 0 ? y[0] : w == 1 ? y[1] : w == 2 ? y[2] : y[3];
      float o = yw * rsn * nwsh[r * kD + col + w];
      if (gate) o *= sigmoidf_(gsh[tt * nv + r * kD + col + w]);
      io<IO>::st(static_cast<IO*>(a.out) + ((row0 + tt) * a.hv + h) * kD + col + w, o);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) S[j] = N[j];
  }
}

template <typename IO>
__global__ void __launch_bounds__(256, 3) k_commit_d128(MtpArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int b = int(blockIdx.x / unsigned(a.hk)), g = int(blockIdx.x - unsigned(b) * unsigned(a.hk));
  const int t = threadIdx.x, cg = t & 31, rg = t >> 5, col = 4 * cg;
  const int R = a.R, K = a.K, nch = (2 + R) * kD;
  const int n = min(max(a.n_accept[b], 0), K);  // out-of-range counts are clamped
  if (n == 0) return;                           // nothing accepted: the cache stays as it is
  float* const kh = smem;                       // [n][128] k^ of the group's QK head
  float* const es = kh + K * kD;                // [n][R][128] e of the group's value heads
  float* const ab = es + K * R * kD;            // [n][R][alpha, beta]
  const int64_t row0 = int64_t(b) * K;

  const size_t head = size_t(kD) * kD;
  float* const S0 = a.state + (size_t(b) * a.hv + size_t(g) * R) * head;
  const int soff = (rg * kD + col) * 4;
  float4 S[16], N[16];
  {
    const auto rs = buf_rsrc(S0, int(head * 4));
#pragma unroll
    for (int j = 0; j < 16; ++j) S[j] = buf_ld16_nt(rs, soff, 4096 * j);
  }
  for (int i = t; i < n * kD; i += 256) {
    const int tt = i / kD;
    kh[i] = a.log.kh[((row0 + tt) * a.hk + g) * kD + (i - tt * kD)];
  }
  for (int i = t; i < n * R * kD; i += 256) {
    const int tt = i / (R * kD);
    es[i] = a.log.e[((row0 + tt) * a.hv + int64_t(g) * R) * kD + (i - tt * R * kD)];
  }
  for (int i = t; i < n * 2 * R; i += 256) {
    const int tt = i / (2 * R);
    ab[i] = a.log.ab[((row0 + tt) * a.hv + int64_t(g) * R) * 2 + (i - tt * 2 * R)];
  }
  // conv cache: the last 3 of (cached inputs, accepted raw inputs), per channel of the group; each
  // thread reads its channel's three new rows before writing any
  if (a.flags & GDN_CONV) {
    for (int c = t; c < nch; c += 256) {
      const int64_t gc = group_channel(c, g, R, a.hk);
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

  for (int r = 0; r < R; ++r) {
    {  // the next head's state; after the last head an empty range (zeros, no memory access)
      const auto rn = buf_rsrc(S0 + size_t(r + 1 < R ? r + 1 : r) * head, r + 1 < R ? int(head * 4) : 0);
#pragma unroll
      for (int j = 0; j < 16; ++j) N[j] = buf_ld16_nt(rn, soff, 4096 * j);
    }
    for (int tt = 0; tt < n; ++tt) {
      const float al = ab[tt * 2 * R + 2 * r], be = ab[tt * 2 * R + 2 * r + 1];
      const float4 ev = *reinterpret_cast<const float4*>(&es[(tt * R + r) * kD + col]);
#pragma unroll
      for (int j = 0; j < 16; ++j) S[j] = rank1(S[j], al, be * kh[tt * kD + rg + 8 * j], ev);
    }
    float* const Sp = S0 + size_t(r) * head;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      __builtin_nontemporal_store(__builtin_bit_cast(f32x4, S[j]), reinterpret_cast<f32x4*>(Sp + (rg + 8 * j) * kD + col));
#pragma unroll
    for (int j = 0; j < 16; ++j) S[j] = N[j];
  }
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
  const size_t smem = verify_smem_floats(n_tok, R) * 4;
  const dim3 grid(unsigned(batch) * unsigned(p.hk));
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
  const size_t smem = commit_smem_floats(n_tok, R) * 4;
  const dim3 grid(unsigned(batch) * unsigned(p.hk));
  if (p.bf16) hipLaunchKernelGGL(k_commit_d128<bf16>, grid, dim3(256), smem, s, a);
  else hipLaunchKernelGGL(k_commit_d128<float>, grid, dim3(256), smem, s, a);
  return hipGetLastError();
}

}  // namespace gdn
