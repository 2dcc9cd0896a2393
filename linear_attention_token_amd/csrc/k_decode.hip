// Decode step: one new token for each of B sequences, conv cache and fp32 state updated in place.
//
// The mixer with a sequence length of one (analysis notes "Qwen3.8-Flash-Next：架构、效率与技术谱系"
// §02 GDN row and §03 update equations; paper reading §四 4.1; paper summary, Method):
//   conv with the cached 3 inputs + SiLU, L2(q, k), then per value head, in one pass over S:
//   a = S^T k, b = S^T q, e = v - alpha a, y = alpha b + beta (q.k) e, S <- alpha S + beta k e^T,
//   then RMSNorm and the sigmoid gate.
//
// One block per (sequence, QK group). The block owns every conv channel of its group (q and k of
// the QK head, v of its HV/HK value heads), so the in-place cache update has a single writer and
// the value heads that share q/k read them from LDS. Each value head is handled by a team of 256
// threads that streams the 128x128 fp32 state from HBM once with 16-byte loads, all of a thread's
// loads in flight at once, and writes it back once. The kernel is bound by HBM bandwidth.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kTeam = 256;
constexpr int kDecMaxRows = 16;

struct DecodeArgs {
  int B, hk, hv, dk, dv, R, teams;
  int64_t C;
  const void *q, *k, *v;
  int64_t ld_q, ld_k, ld_v;
  const float *alpha, *beta;
  const void* gate;
  const float *conv_w, *norm_w;
  int norm_stride;
  void* conv_state;
  float* state;
  void* out;
  uint32_t flags;
  float scale, l2_eps, norm_eps;
};

template <typename IO>
__global__ void __launch_bounds__(768) k_decode(DecodeArgs a) {
  extern __shared__ float smem[];
  const int b = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int nch = 2 * a.dk + a.R * a.dv;
  float* act = smem;                  // [nch]: q | k | v of the group's heads, after conv + SiLU
  float* red = smem + ((nch + 3) & ~3);  // per team: red_a[256*4], red_b[256*4]
  __shared__ float scal[4];           // 1/|q|, 1/|k|, q.k (normalised)

  // ---- conv + SiLU for the group's channels; single-writer cache shift ----
  const int64_t qk_ch = int64_t(a.hk) * a.dk;
  for (int c = tid; c < nch; c += nthreads) {
    int64_t gc;          // global channel index
    const IO* src;
    if (c < a.dk) { gc = int64_t(g) * a.dk + c; src = static_cast<const IO*>(a.q) + int64_t(b) * a.ld_q + (gc); }
    else if (c < 2 * a.dk) { gc = qk_ch + int64_t(g) * a.dk + (c - a.dk); src = static_cast<const IO*>(a.k) + int64_t(b) * a.ld_k + (gc - qk_ch); }
    else { gc = 2 * qk_ch + int64_t(g) * a.R * a.dv + (c - 2 * a.dk); src = static_cast<const IO*>(a.v) + int64_t(b) * a.ld_v + (gc - 2 * qk_ch); }
    const float x = io<IO>::ld(src);
    float u = x;
    if (a.flags & GDN_CONV) {
      IO* cs = static_cast<IO*>(a.conv_state) + int64_t(b) * 3 * a.C + gc;
      const float h0 = io<IO>::ld(cs), h1 = io<IO>::ld(cs + a.C), h2 = io<IO>::ld(cs + 2 * a.C);
      const float4 w = reinterpret_cast<const float4*>(a.conv_w)[gc];
      u = w.x * h0 + w.y * h1 + w.z * h2 + w.w * x;
      u = siluf_(u);
      io<IO>::st(cs, h1);
      io<IO>::st(cs + a.C, h2);
      io<IO>::st(cs + 2 * a.C, x);
    }
    act[c] = u;
  }
  __syncthreads();
  if (tid < 64) {
    float sq = 0.f, sk = 0.f;
    for (int i = tid; i < a.dk; i += 64) { sq += act[i] * act[i]; sk += act[a.dk + i] * act[a.dk + i]; }
    sq = group_sum<64>(sq);
    sk = group_sum<64>(sk);
    const bool l2 = (a.flags & GDN_L2QK) != 0;
    const float rq = l2 ? 1.0f / sqrtf(sq + a.l2_eps) : 1.0f;
    const float rk = l2 ? 1.0f / sqrtf(sk + a.l2_eps) : 1.0f;
    float d = 0.f;
    for (int i = tid; i < a.dk; i += 64) d += act[i] * act[a.dk + i];
    d = group_sum<64>(d);
    if (tid == 0) { scal[0] = rq; scal[1] = rk; scal[2] = d * rq * rk; }
  }
  __syncthreads();
  const float rq = scal[0], rk = scal[1], qk = scal[2];

  // ---- state update, one team per value head ----
  const int team = tid / kTeam, lt = tid % kTeam;
  const int ncg = a.dv / 4, nrg = kTeam / ncg;
  const int cg = lt % ncg, rg = lt / ncg, col = 4 * cg;
  float* red_a = red + team * (2 * kTeam * 4);
  float* red_b = red_a + kTeam * 4;
  const int iters = (a.R + a.teams - 1) / a.teams;
  for (int it = 0; it < iters; ++it) {
    const int r = team + it * a.teams;
    const bool live = r < a.R;
    const int h = g * a.R + (live ? r : 0);
    float* Sp = a.state + (size_t(b) * a.hv + h) * size_t(a.dk) * a.dv;
    float S[kDecMaxRows][4];
#pragma unroll
    for (int j = 0; j < kDecMaxRows; ++j) {
      const int i = rg + j * nrg;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (live && i < a.dk) v = *reinterpret_cast<const float4*>(Sp + size_t(i) * a.dv + col);
      S[j][0] = v.x; S[j][1] = v.y; S[j][2] = v.z; S[j][3] = v.w;
    }
    float pa[4] = {0.f, 0.f, 0.f, 0.f}, pb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kDecMaxRows; ++j) {
      const int i = rg + j * nrg;
      if (i < a.dk) {
        const float qi = act[i] * rq, ki = act[a.dk + i] * rk;
#pragma unroll
        for (int e = 0; e < 4; ++e) { pa[e] += S[j][e] * ki; pb[e] += S[j][e] * qi; }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) { red_a[rg * a.dv + col + e] = pa[e]; red_b[rg * a.dv + col + e] = pb[e]; }
    __syncthreads();
    float av[4] = {0.f, 0.f, 0.f, 0.f}, bv[4] = {0.f, 0.f, 0.f, 0.f};
    const int nr = min(nrg, a.dk);
    for (int rr = 0; rr < nr; ++rr) {
#pragma unroll
      for (int e = 0; e < 4; ++e) { av[e] += red_a[rr * a.dv + col + e]; bv[e] += red_b[rr * a.dv + col + e]; }
    }
    const float al = live ? a.alpha[size_t(b) * a.hv + h] : 0.f;
    const float be = live ? a.beta[size_t(b) * a.hv + h] : 0.f;
    float ev[4], y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float vv = act[2 * a.dk + (live ? r : 0) * a.dv + col + e];
      ev[e] = vv - al * av[e];
      y[e] = a.scale * (al * bv[e] + be * qk * ev[e]);
    }
    if (live) {
#pragma unroll
      for (int j = 0; j < kDecMaxRows; ++j) {
        const int i = rg + j * nrg;
        if (i < a.dk) {
          const float bk = be * act[a.dk + i] * rk;
          float4 o;
          o.x = al * S[j][0] + bk * ev[0];
          o.y = al * S[j][1] + bk * ev[1];
          o.z = al * S[j][2] + bk * ev[2];
          o.w = al * S[j][3] + bk * ev[3];
          *reinterpret_cast<float4*>(Sp + size_t(i) * a.dv + col) = o;
        }
      }
    }
    float ss = y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3];
    for (int o = ncg >> 1; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
    if (live && rg == 0) {
      const float rs = (a.flags & GDN_NORM) ? 1.0f / sqrtf(ss / float(a.dv) + a.norm_eps) : 1.0f;
      const IO* gp = static_cast<const IO*>(a.gate) + (size_t(b) * a.hv + h) * a.dv + col;
      IO* op = static_cast<IO*>(a.out) + (size_t(b) * a.hv + h) * a.dv + col;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float o = y[e];
        if (a.flags & GDN_NORM) o = o * rs * (1.0f + a.norm_w[size_t(h) * a.norm_stride + col + e]);
        if (a.flags & GDN_GATE) o *= sigmoidf_(io<IO>::ld(gp + e));
        io<IO>::st(op + e, o);
      }
    }
    __syncthreads();
  }
}

// Head size 128 (the model's): one block of 256 threads per (sequence, QK group), which walks the
// group's value heads one after another. Thread (cg, rg) = (t % 32, t / 32) holds columns 4cg .. +3
// of rows rg + 8j (j < 16) of a head's state, so one load instruction of a wave reads two adjacent
// 512-byte rows. The first head's state is requested before the conv runs and each next head's
// before the current one is reduced, so a block always has a state in flight; three blocks share
// a CU (167 VGPRs, no spills: the staging below keeps the per-head registers to the two states). State is read with plain loads and written with non-temporal stores (each byte is touched once per step).
// Everything else a head needs (alpha, beta, gain, gate logits) is staged in LDS up front, and every
// wave issues the same memory instructions in every head (the last head's prefetch goes through an
// empty buffer range, which reads zeros without touching memory), so the compiler's waits for the
// prefetched state are exact counts that let the previous head's stores stay in flight.
constexpr int kD = 128;

template <typename IO>
__global__ void __launch_bounds__(256, 3) k_decode_d128(DecodeArgs a) {
  extern __shared__ float smem[];
  // item = b * hk + g; each XCD walks its own contiguous run of items, and so of the state (with
  // plain, cached state loads: 294 -> 285 us at B = 256 against non-temporal loads in block order)
  const unsigned item = xcd_range_item(blockIdx.x, gridDim.x);
  const int b = int(item / unsigned(a.hk)), g = int(item - unsigned(b) * unsigned(a.hk));
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int cg = t & 31, rg = t >> 5, col = 4 * cg;
  const int R = a.R;
  float* act = smem;                    // [(2 + R) * 128]: q | k | v of the group's heads, after conv + SiLU
  float* red = smem + (2 + 2 * R) * kD;  // [2 buffers][4 waves][a, b][128]
  float* nwsh = red + 8 * kD * 2;        // [R * 128] zero-centred gains (1 + w)
  float* absh = nwsh + R * kD;           // [2 R] alpha, beta of the group's heads
  __shared__ float nrm[8];

  const size_t head = size_t(kD) * kD;
  float* const S0 = a.state + (size_t(b) * a.hv + size_t(g) * R) * head;
  const int soff = (rg * kD + col) * 4;  // row j of this thread: soff + 4096 j bytes into the head
  float4 S[16], N[16];  // this head's state and the next head's, in flight meanwhile

  // ---- conv + SiLU of the group's channels (single writer of their cache) and the group's gate
  // logits. A pass covers 768 channels (all of them for up to 4 value heads per group) and issues
  // every load before the first use, so the pass costs one memory round trip ----
  const int nch = (2 + R) * kD, nv = R * kD;
  float* const gsh = act + nch;  // [R * 128] gate logits
  const int64_t qk_ch = int64_t(a.hk) * kD;
  const bool conv = (a.flags & GDN_CONV) != 0, gate = (a.flags & GDN_GATE) != 0;
  // [R * 128]; without the gate the logits may be absent: the group's v row (also R * 128 values)
  // stands in, and its values are discarded
  const IO* const gsrc = gate ? static_cast<const IO*>(a.gate) + (size_t(b) * a.hv + size_t(g) * R) * kD
                              : static_cast<const IO*>(a.v) + int64_t(b) * a.ld_v + int64_t(g) * nv;
  // Loads are issued unconditionally from clamped (always valid) addresses and converted only after
  // the whole pass is in flight; lanes past the end discard their values.
  float gv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) gv[u] = io<IO>::ld(gsrc + min(t + 256 * u, nv - 1));
  // gains (through a buffer range that is empty without the norm: zeros, no memory access) and
  // alpha | beta of the group, requested with the conv pass
  const auto rnw = buf_rsrc(a.norm_w, (a.flags & GDN_NORM) ? int((size_t(a.hv - 1) * a.norm_stride + kD) * 4) : 0);
  auto gain_off = [&](int c) { return int(size_t(g * R + c / kD) * a.norm_stride + c % kD) * 4; };
  float nwv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
    nwv[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rnw, gain_off(min(t + 256 * u, nv - 1)), 0, 0));
  const int iab = min(t, 2 * R - 1);
  const float abv = (iab < R ? a.alpha : a.beta)[size_t(b) * a.hv + g * R + (iab < R ? iab : iab - R)];
  float u_qk = 0.f;  // this thread's q (t < 128) or k channel after conv + SiLU
  for (int c0 = 0; c0 < nch; c0 += 768) {
    float x[3], h[3][3];
    float4 cw[3];
    int64_t gcs[3];
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int c = min(c0 + t + 256 * u, nch - 1);
      const bool isq = c < kD, isk = !isq && c < 2 * kD;
      const int cc = isq ? c : isk ? c - kD : c - 2 * kD;
      gcs[u] = (isq ? int64_t(0) : isk ? qk_ch : 2 * qk_ch) + int64_t(g) * (isq || isk ? kD : nv) + cc;
      const IO* src = isq ? static_cast<const IO*>(a.q) + int64_t(b) * a.ld_q + g * kD
                    : isk ? static_cast<const IO*>(a.k) + int64_t(b) * a.ld_k + g * kD
                          : static_cast<const IO*>(a.v) + int64_t(b) * a.ld_v + int64_t(g) * nv;
      x[u] = io<IO>::ld(src + cc);
      // without the conv the cache and weights may be absent: read valid stand-ins instead
      const IO* cs = conv ? static_cast<const IO*>(a.conv_state) + int64_t(b) * 3 * a.C + gcs[u] : src + cc;
      const int64_t cstep = conv ? a.C : 0;
      h[u][0] = io<IO>::ld(cs);
      h[u][1] = io<IO>::ld(cs + cstep);
      h[u][2] = io<IO>::ld(cs + 2 * cstep);
      cw[u] = conv ? reinterpret_cast<const float4*>(a.conv_w)[gcs[u]] : *reinterpret_cast<const float4*>(S0);
    }
    asm volatile("" ::: "memory");  // keeps the loads above from being sunk into the branches below
    if (c0 == 0) {  // the first head's state, requested after the first pass's inputs: loads complete
                    // in order, so requested first it would hold up every input of the prologue
      const auto rs = buf_rsrc(S0, int(head * 4));
#pragma unroll
      for (int j = 0; j < 16; ++j) S[j] = buf_ld16(rs, soff, 4096 * j);
    }
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int c = c0 + t + 256 * u;
      if (c < nch) {
        float val = x[u];
        if (conv) {
          IO* cs = static_cast<IO*>(a.conv_state) + int64_t(b) * 3 * a.C + gcs[u];
          io<IO>::st(cs, h[u][1]);
          io<IO>::st(cs + a.C, h[u][2]);
          io<IO>::st(cs + 2 * a.C, x[u]);
          val = siluf_(cw[u].x * h[u][0] + cw[u].y * h[u][1] + cw[u].z * h[u][2] + cw[u].w * x[u]);
        }
        act[c] = val;
        if (c0 == 0 && u == 0) u_qk = val;
      }
    }
  }
  if (gate) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (t + 256 * u < nv) gsh[t + 256 * u] = gv[u];
    for (int c = t + 512; c < nv; c += 256) gsh[c] = io<IO>::ld(gsrc + c);
  }
#pragma unroll
  for (int u = 0; u < 2; ++u)
    if (t + 256 * u < nv) nwsh[t + 256 * u] = 1.0f + nwv[u];
  for (int c = t + 512; c < nv; c += 256)
    nwsh[c] = 1.0f + __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rnw, gain_off(c), 0, 0));
  if (t < 2 * R) absh[t] = abv;
  const float u = u_qk;
  // |q|^2 (waves 0, 1) and |k|^2 (waves 2, 3), then q.k
  {
    const float ss = wave_sum<64>(u * u);
    if (lane == 0) nrm[w] = ss;
  }
  __syncthreads();
  if (t < kD) {
    const float d = wave_sum<64>(u * act[kD + t]);
    if (lane == 0) nrm[4 + w] = d;
  }
  __syncthreads();
  const bool l2 = (a.flags & GDN_L2QK) != 0;
  const float rq = l2 ? 1.0f / sqrtf(nrm[0] + nrm[1] + a.l2_eps) : 1.0f;
  const float rk = l2 ? 1.0f / sqrtf(nrm[2] + nrm[3] + a.l2_eps) : 1.0f;
  const float qk = (nrm[4] + nrm[5]) * rq * rk;

  for (int r = 0; r < R; ++r) {
    const int h = g * R + r;
    const float al = absh[r], be = absh[R + r];
    {  // the next head's state; after the last head an empty range (zeros, no memory access)
      const auto rn = buf_rsrc(S0 + size_t(r + 1 < R ? r + 1 : r) * head, r + 1 < R ? int(head * 4) : 0);
#pragma unroll
      for (int j = 0; j < 16; ++j) N[j] = buf_ld16(rn, soff, 4096 * j);
    }
    // a = S^T k^, b = S^T q^ over this thread's rows, then over the 8 row groups
    float4 pa = make_float4(0.f, 0.f, 0.f, 0.f), pb = pa;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float qi = act[rg + 8 * j], ki = act[kD + rg + 8 * j];
      pa.x += S[j].x * ki; pa.y += S[j].y * ki; pa.z += S[j].z * ki; pa.w += S[j].w * ki;
      pb.x += S[j].x * qi; pb.y += S[j].y * qi; pb.z += S[j].z * qi; pb.w += S[j].w * qi;
    }
    pa.x = half_pair_sum(pa.x); pa.y = half_pair_sum(pa.y);
    pa.z = half_pair_sum(pa.z); pa.w = half_pair_sum(pa.w);
    pb.x = half_pair_sum(pb.x); pb.y = half_pair_sum(pb.y);
    pb.z = half_pair_sum(pb.z); pb.w = half_pair_sum(pb.w);
    float* const rb = red + (r & 1) * (8 * kD);  // two buffers: one barrier per head suffices
    if (lane < 32) {
      *reinterpret_cast<float4*>(&rb[(2 * w) * kD + col]) = pa;
      *reinterpret_cast<float4*>(&rb[(2 * w + 1) * kD + col]) = pb;
    }
    __syncthreads();
    float av[4] = {0.f, 0.f, 0.f, 0.f}, bv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float4 x = *reinterpret_cast<const float4*>(&rb[(2 * ww) * kD + col]);
      const float4 y = *reinterpret_cast<const float4*>(&rb[(2 * ww + 1) * kD + col]);
      av[0] += x.x; av[1] += x.y; av[2] += x.z; av[3] += x.w;
      bv[0] += y.x; bv[1] += y.y; bv[2] += y.z; bv[3] += y.w;
    }
    float ev[4], y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ev[e] = act[(2 + r) * kD + col + e] - al * (av[e] * rk);
      y[e] = a.scale * (al * (bv[e] * rq) + be * qk * ev[e]);
    }
    // S <- alpha S + beta k^ e^T. Written with global stores: buffer stores whose data registers
    // the compiler refills right after issue were seen to lose single dwords on gfx950.
    float* const Sp = S0 + size_t(r) * head;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float bk = be * rk * act[kD + rg + 8 * j];
      float4 o;
      o.x = al * S[j].x + bk * ev[0];
      o.y = al * S[j].y + bk * ev[1];
      o.z = al * S[j].z + bk * ev[2];
      o.w = al * S[j].w + bk * ev[3];
      __builtin_nontemporal_store(__builtin_bit_cast(f32x4, o), reinterpret_cast<f32x4*>(Sp + (rg + 8 * j) * kD + col));
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) S[j] = N[j];
    // RMSNorm over the head's 128 outputs (every row group holds them all), gain, gate; wave w
    // stores channel col + w of each column group (its two row groups write the same values)
    const float ss = wave_sum<32>(y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3]);
    const float rs = (a.flags & GDN_NORM) ? 1.0f / sqrtf(ss / float(kD) + a.norm_eps) : 1.0f;
    const float yw = w == 0 ? y[0] : w == 1 ? y[1] : w == 2 ? y[2] : y[3];
    float o = yw * rs * nwsh[r * kD + col + w];
    if (gate) o *= sigmoidf_(gsh[r * kD + col + w]);
    io<IO>::st(static_cast<IO*>(a.out) + (size_t(b) * a.hv + h) * kD + col + w, o);
  }
}

size_t decode_smem_bytes(const Problem& p, int teams) {
  const int R = p.hv / p.hk;
  const int nch = 2 * p.dk + R * p.dv;
  return size_t((nch + 3) & ~3) * 4 + size_t(teams) * 2 * kTeam * 4 * 4;
}

hipError_t launch_decode(const Problem& p, int batch, const void* q, const void* k, const void* v,
                         int64_t ld_q, int64_t ld_k, int64_t ld_v, const float* alpha, const float* beta,
                         const void* gate, const float* conv_w, const float* norm_w, void* conv_state,
                         float* state, void* out, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  const int R = p.hv / p.hk;
  const int teams = R < 3 ? R : 3;
  DecodeArgs a{batch, p.hk, p.hv, p.dk, p.dv, R, teams, p.C, q, k, v, ld_q, ld_k, ld_v, alpha, beta,
               gate, conv_w, norm_w, p.norm_stride, conv_state, state, out, p.flags, p.scale,
               p.l2_eps, p.norm_eps};
  dim3 grid(unsigned(batch), unsigned(p.hk));
  if (p.dk == kD && p.dv == kD) {
    const size_t smem = size_t(2 + 2 * R) * kD * 4 + 8 * kD * 4 * 2 + size_t(R) * kD * 4 + size_t(2 * R) * 4;
    const dim3 grid1(unsigned(batch) * unsigned(p.hk));
    if (p.bf16) hipLaunchKernelGGL(k_decode_d128<bf16>, grid1, dim3(256), smem, s, a);
    else hipLaunchKernelGGL(k_decode_d128<float>, grid1, dim3(256), smem, s, a);
    return hipGetLastError();
  }
  const size_t smem = decode_smem_bytes(p, teams);
  if (p.bf16) hipLaunchKernelGGL(k_decode<bf16>, grid, dim3(kTeam * teams), smem, s, a);
  else hipLaunchKernelGGL(k_decode<float>, grid, dim3(kTeam * teams), smem, s, a);
  return hipGetLastError();
}

}  // namespace gdn
