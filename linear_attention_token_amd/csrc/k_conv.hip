// Chunk table, fused short-conv + SiLU + L2 (q, k) kernel, and the conv-cache tail.
//
// Short causal depthwise conv of width 4 on every q/k/v channel, then SiLU ("Qwen3.8-Flash-Next：
// 架构、效率与技术谱系" §02 configuration table, GDN row; paper reading §四 4.1), then L2
// normalisation of each q and k head (paper summary "Qwen3.8-Flash-Next", Method).
//
// Layout: one thread owns 16 contiguous bytes of channels (8 bf16 or 4 fp32) and walks a strip of
// tokens, keeping the 3-token conv window in registers, so every raw element is read once per strip
// with fully coalesced 16-byte loads. The lanes of one head (d_k / VEC consecutive lanes) reduce
// sum(a^2) with cross-lane shuffles.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

// ------------------------------------------------------------------------------------------------
// Chunk table: sequence n owns chunks [off[n], off[n+1]); chunk c covers tokens
// [start, start + len), len <= 64. Entries past the last chunk get len = 0.
// One block; sequences are scanned 1024 at a time.
// Runs on one block of up to 1024 threads.
__device__ void build_chunk_table(const int32_t* __restrict__ cu, int n_seqs, int64_t T, int64_t nc_max,
                                  int32_t* __restrict__ seq_off, int4* __restrict__ tab) {
  __shared__ int32_t wave_tot[16];
  __shared__ int32_t carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < n_seqs; base += blockDim.x) {
    const int n = base + tid;
    int64_t s0 = 0, s1 = 0;
    int cnt = 0;
    if (n < n_seqs) {
      s0 = min<int64_t>(max<int64_t>(cu[n], 0), T);
      s1 = min<int64_t>(max<int64_t>(cu[n + 1], s0), T);
      cnt = int((s1 - s0 + kChunk - 1) / kChunk);
    }
    // inclusive scan inside the wave
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wave_tot[wid] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wid; ++w) before += wave_tot[w];
    const int carry = carry_s;
    const int64_t off = int64_t(carry) + before + incl - cnt;
    if (n < n_seqs) {
      seq_off[n] = int32_t(min<int64_t>(off, nc_max));
      for (int j = 0; j < cnt; ++j) {
        const int64_t c = off + j;
        if (c >= nc_max) break;
        tab[c] = make_int4(int(s0 + int64_t(j) * kChunk), int(min<int64_t>(kChunk, s1 - s0 - int64_t(j) * kChunk)), n, 0);
      }
    }
    __syncthreads();
    if (tid == int(blockDim.x) - 1) carry_s = int32_t(min<int64_t>(off + cnt, nc_max));
    __syncthreads();
  }
  const int total = carry_s;
  if (tid == 0) seq_off[n_seqs] = total;
  for (int64_t c = int64_t(total) + tid; c < nc_max; c += blockDim.x) tab[c] = make_int4(0, 0, -1, 0);
}


// ------------------------------------------------------------------------------------------------
// Sequence containing token t: largest n with cu[n] <= t (binary search over cu[0..N]).
__device__ __forceinline__ int find_seq(const int32_t* cu, int n_seqs, int64_t t) {
  int lo = 0, hi = n_seqs;  // answer in [0, n_seqs - 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (int64_t(cu[mid]) <= t) lo = mid; else hi = mid;
  }
  return lo;
}

struct ConvArgs {
  const int32_t* cu;
  int n_seqs;
  int64_t T, C;
  int hk, hv, dk, dv;
  const void *q, *k, *v;
  int64_t ld_q, ld_k, ld_v;
  const float* conv_w;
  const void* conv_in;
  void *qhat, *khat, *vhat;
  uint32_t flags;
  float l2_eps;
  // block numbering: strips of kConvStrip tokens x blocks of 256 channel groups
  int64_t n_strips, strips_per_xcd;
  int n_cblk;
  // chunk table (chunked path only): built by the extra last block
  int64_t nc_max;
  int32_t* seq_off;
  int4* tab;
};

// IO: input/history type; WT: type of the normalised outputs.
template <typename IO, typename WT>
__global__ void __launch_bounds__(256) k_conv(ConvArgs a) {
  if (blockIdx.x == gridDim.x - 1) {  // the extra last block builds the chunk table
    if (a.tab != nullptr) build_chunk_table(a.cu, a.n_seqs, a.T, a.nc_max, a.seq_off, a.tab);
    return;
  }
  // Block b runs on XCD b % 8 (blocks are dealt round-robin over the XCDs). Each XCD walks its own
  // run of consecutive strips, all channel blocks of a strip before the next strip, so the 3 halo
  // rows a strip reads were fetched into the same XCD's L2 by the strip just before it.
  const int xcd = int(blockIdx.x & 7), kx = int(blockIdx.x >> 3);
  const int64_t strip = int64_t(xcd) * a.strips_per_xcd + kx / a.n_cblk;
  const int cblk = kx % a.n_cblk;
  if (strip >= a.n_strips) return;
  constexpr int VEC = vec16<IO>::N;
  const int64_t cg = int64_t(cblk) * blockDim.x + threadIdx.x;
  const int64_t c0 = cg * VEC;
  const bool active = c0 < a.C;
  const int64_t qk_ch = int64_t(a.hk) * a.dk;
  // which stream this thread's channels belong to
  const IO* src;
  int64_t ld;
  WT* dst;
  int64_t dld;
  bool isqk;
  if (c0 < qk_ch) {
    src = static_cast<const IO*>(a.q) + c0; ld = a.ld_q;
    dst = static_cast<WT*>(a.qhat) + c0; dld = qk_ch; isqk = true;
  } else if (c0 < 2 * qk_ch) {
    src = static_cast<const IO*>(a.k) + (c0 - qk_ch); ld = a.ld_k;
    dst = static_cast<WT*>(a.khat) + (c0 - qk_ch); dld = qk_ch; isqk = true;
  } else {
    src = static_cast<const IO*>(a.v) + (c0 - 2 * qk_ch); ld = a.ld_v;
    dst = static_cast<WT*>(a.vhat) + (c0 - 2 * qk_ch); dld = int64_t(a.hv) * a.dv; isqk = false;
  }
  const bool do_conv = (a.flags & GDN_CONV) != 0;
  const bool do_l2 = (a.flags & GDN_L2QK) != 0;
  const int width = a.dk / VEC;  // lanes per q/k head

  // raw rows t0-3 .. t0+15 of this thread's channels, all loads in flight together
  const int64_t t0 = strip * kConvStrip;
  uint4 xr[kConvStrip + 3];
#pragma unroll
  for (int j = 0; j < kConvStrip + 3; ++j) {
    const int64_t pos = t0 - 3 + j;
    xr[j] = make_uint4(0, 0, 0, 0);
    if (active && pos >= 0 && pos < a.T && (j >= 3 || do_conv))
      xr[j] = *reinterpret_cast<const uint4*>(src + pos * ld);
  }
  float w[4][VEC];
  if (active && do_conv) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const float4 t = reinterpret_cast<const float4*>(a.conv_w)[c0 + e];
      w[0][e] = t.x; w[1][e] = t.y; w[2][e] = t.z; w[3][e] = t.w;
    }
  }

  int n = find_seq(a.cu, a.n_seqs, t0);
  // clamped bounds: garbage cu_seqlens give meaningless results but no out-of-bounds access
  auto bounds = [&](int nn, int64_t& b0, int64_t& b1) {
    b0 = min<int64_t>(max<int64_t>(a.cu[nn], 0), a.T);
    b1 = min<int64_t>(max<int64_t>(a.cu[nn + 1], b0), a.T);
  };
  int64_t s0, s1;
  bounds(n, s0, s1);

#pragma unroll
  for (int j = 0; j < kConvStrip; ++j) {
    const int64_t t = t0 + j;
    if (t >= a.T) break;  // uniform across the block
    if (t >= s1) {        // uniform: a new sequence starts at t
      while (n + 1 < a.n_seqs && t >= int64_t(a.cu[n + 1])) ++n;
      bounds(n, s0, s1);
    }
    float x[VEC], y[VEC];
    vec16<IO>::cvt(xr[j + 3], x);
#pragma unroll
    for (int e = 0; e < VEC; ++e) y[e] = x[e];
    if (do_conv) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) y[e] = w[3][e] * x[e];
#pragma unroll
      for (int tap = 0; tap < 3; ++tap) {
        const int64_t pos = t - 3 + tap;
        float hv[VEC];
        if (pos >= s0) {
          vec16<IO>::cvt(xr[j + tap], hv);
        } else if (a.conv_in != nullptr && active && pos >= s0 - 3) {
          vec16<IO>::ld(static_cast<const IO*>(a.conv_in) + (int64_t(n) * 3 + (3 + (pos - s0))) * a.C + c0, hv);
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) hv[e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) y[e] += w[tap][e] * hv[e];
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) y[e] = siluf_(y[e]);
    }
    if (do_l2) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) ss += y[e] * y[e];
      if (width == 16) {  // a q/k head of 128 channels in one DPP row (bf16 pieces)
        ss = wave_sum<16>(ss);
      } else if (width == 32) {  // fp32 pieces: two rows
        ss = wave_sum<32>(ss);
      } else {
        for (int o = width >> 1; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
      }
      if (isqk) {
        const float r = 1.0f / sqrtf(ss + a.l2_eps);
#pragma unroll
        for (int e = 0; e < VEC; ++e) y[e] *= r;
      }
    }
    if (active) {
      if constexpr (sizeof(WT) == sizeof(IO)) {
        vec16<WT>::st(dst + t * dld, y);
      } else {
        // bf16 io with fp32 work type: two 16-byte stores
        vec16<WT>::st(dst + t * dld, y);
        vec16<WT>::st(dst + t * dld + 4, y + 4);
      }
    }
  }
}

hipError_t launch_conv(const Problem& p, const int32_t* cu, const void* q, const void* k, const void* v,
                       int64_t ld_q, int64_t ld_k, int64_t ld_v, const float* conv_w,
                       const void* conv_in, const Workspace& ws, bool work_bf16, hipStream_t s) {
  const bool table = work_bf16 && ws.chunk_tab != nullptr;
  if (p.T == 0 && !table) return hipSuccess;
  const int vec = p.bf16 ? 8 : 4;
  const int64_t groups = (p.C + vec - 1) / vec;
  const int n_cblk = int((groups + 255) / 256);
  const int64_t n_strips = (p.T + kConvStrip - 1) / kConvStrip;
  const int64_t per_xcd = (n_strips + kXcds - 1) / kXcds;
  ConvArgs a{cu, p.n_seqs, p.T, p.C, p.hk, p.hv, p.dk, p.dv, q, k, v, ld_q, ld_k, ld_v,
             conv_w, conv_in, ws.qhat, ws.khat, ws.vhat, p.flags, p.l2_eps,
             n_strips, per_xcd, n_cblk,
             p.nc_max, table ? ws.seq_chunk_off : nullptr, table ? ws.chunk_tab : nullptr};
  // kXcds x per_xcd x n_cblk strip blocks, then one block for the chunk table
  const dim3 grid(unsigned(int64_t(kXcds) * per_xcd * n_cblk + 1));
  if (p.bf16) {
    if (work_bf16) hipLaunchKernelGGL((k_conv<bf16, bf16>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_conv<bf16, float>), grid, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_conv<float, float>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Standalone conv-cache tail (the chunked path folds the same work into the output kernel).
template <typename IO>
__global__ void __launch_bounds__(256) k_conv_tail(ConvTailArgs a) {
  conv_tail_piece<IO>(a, blockIdx.x, int64_t(blockIdx.y) * blockDim.x + threadIdx.x);
}

hipError_t launch_conv_tail(const Problem& p, const int32_t* cu, const void* q, const void* k,
                            const void* v, int64_t ld_q, int64_t ld_k, int64_t ld_v,
                            const void* conv_in, void* conv_out, hipStream_t s) {
  if (p.n_seqs == 0) return hipSuccess;
  const ConvTailArgs a = conv_tail_args(p, cu, q, k, v, ld_q, ld_k, ld_v, conv_in, conv_out);
  const dim3 grid(unsigned(p.n_seqs), unsigned(a.cblk));
  if (p.bf16) hipLaunchKernelGGL(k_conv_tail<bf16>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_conv_tail<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace gdn
