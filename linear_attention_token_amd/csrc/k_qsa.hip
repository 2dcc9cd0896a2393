// Compressed block indexer of Qwen Sparse Attention (analysis notes "Qwen3.8-Flash-Next：架构、效率与
// 技术谱系" §04 indexer data flow; paper reading "On the Design of Qwen3.8-Next Architecture … 精读"
// §四 4.2): keys pooled over 4-token micro-blocks, RMS-normalised and rotated to the block's first
// position; each query's 4 heads score every complete block by a sum of ReLU'd dot products; the
// top-k blocks are kept.
//
// Kernels:
//   k_qsa_compress  one 16-lane group per block: pool, RMSNorm, partial RoPE, store (HBM-bound);
//   k_qsa_qprep     one row per query: find its sequence and position, rotate its 4 heads (fp32); in
//                   decode, also the new key joins its sequence's pending block, or completes it;
//   k_qsa_score     a row's compressed keys streamed by 16-lane groups, 16 B per lane (HBM-bound
//                   in decode, where the cache is read once per step);
//   k_qsa_score_mfma  bf16 prefill: 2 x 16 query rows x 16 compressed keys per bf16 MFMA step;
//   k_qsa_select    one block per row and segment, up to 16 consecutive scores per thread (1024
//                   threads: 16384 scores; 256 or 512 threads for short rows): exact top-k by a
//                   radix select on the score bits held in registers, then an ordered compaction
//                   by one block scan of per-thread counts;
//   k_qsa_merge     rows longer than one segment: the same select over the segments' candidates
//                   (every global top-k block is in its own segment's top-k).
//
// Lane layout shared by the vector kernels: lane m of a 16-lane group holds dims 8m .. 8m+7.
// Rotation pairs dim d with d + rope_dims/2 (d < rope_dims/2) at angle pos * base^(-2d/rope_dims);
// the angle is formed and reduced mod 2 pi in fp64, so positions near 2^20 keep fp32 accuracy.
#include <math.h>

#include <type_traits>

#include "gdn_device.h"
#include "ext_internal.h"

namespace gdn {

constexpr int kQsaD = 128;       // head dim of indexer queries and keys
constexpr int kQsaHeads = 4;     // query heads
constexpr int kScoreChunk = 1024;  // blocks per workgroup of the score kernel
constexpr int kScoreUnroll = 8;    // blocks per 16-lane group in flight
constexpr int kMfmaChunk = 1024;   // blocks per workgroup of the MFMA score kernel
constexpr int kSelPer = 16;        // scores per thread of the select

// ---- rotation -------------------------------------------------------------------------------
struct RopeLane {
  double theta[8];  // angle per position of each of the lane's dims (0 for unrotated lanes)
  int partner;      // lane (within the group) holding the other member of each pair
  int kind;         // 0 not rotated, 1 first member (x c - y s), 2 second member (y s + x c)
};

__device__ __forceinline__ RopeLane rope_lane(int m, const QsaShape& sh) {
  RopeLane r;
  const int h8 = sh.half / 8;
  int first = 0;
  if (m < h8) {
    r.kind = 1; r.partner = m + h8; first = 8 * m;
  } else if (m < 2 * h8) {
    r.kind = 2; r.partner = m - h8; first = 8 * (m - h8);
  } else {
    r.kind = 0; r.partner = m;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
    r.theta[i] = r.kind ? sh.theta[first + i] : 0.0;
  return r;
}

__device__ __forceinline__ void rope8(float (&y)[8], const RopeLane& rl, double pos, int lane) {
  const int src = (lane & 0x30) | rl.partner;
  float yp[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) yp[i] = __shfl(y[i], src, kWave);
  if (rl.kind == 0) return;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double a = pos * rl.theta[i];
    const double n = rint(a * (0.5 / M_PI));
    float s, c;
    sincosf(float(fma(-n, 2.0 * M_PI, a)), &s, &c);
    y[i] = rl.kind == 1 ? y[i] * c - yp[i] * s : yp[i] * s + y[i] * c;
  }
}

template <typename IO>
__device__ __forceinline__ void ld8(const IO* p, float (&o)[8]) {
  constexpr int N = vec16<IO>::N;
#pragma unroll
  for (int i = 0; i < 8; i += N) vec16<IO>::ld(p + i, o + i);
}

template <typename IO>
__device__ __forceinline__ void st8(IO* p, const float (&o)[8]) {
  constexpr int N = vec16<IO>::N;
#pragma unroll
  for (int i = 0; i < 8; i += N) vec16<IO>::st(p + i, o + i);
}

// Pooled block sum (4 keys added) -> RMSNorm with gain -> rotation to pos0 -> store. The 16 lanes of
// a group call it together.
template <typename IO>
__device__ __forceinline__ void finish_block(float (&y)[8], const float (&w)[8], const RopeLane& rl, int64_t pos0,
                                             float eps, int lane, IO* out) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    y[i] *= 0.25f;
    ss += y[i] * y[i];
  }
  ss = wave_sum<16>(ss);
  const float r = 1.0f / sqrtf(ss * (1.0f / kQsaD) + eps);
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] *= r * w[i];
  rope8(y, rl, double(pos0), lane);
  st8(out, y);
}

// ---- compression of a prefill: grid (block groups of 64, sequences), 16 groups per workgroup ----
template <typename IO>
__global__ void __launch_bounds__(256) k_qsa_compress(QsaShape sh, const IO* __restrict__ k, int64_t ld_k,
                                                      const int32_t* __restrict__ cu, int64_t T,
                                                      const float* __restrict__ norm_w, IO* __restrict__ kbar,
                                                      IO* __restrict__ pending) {
  const int t = threadIdx.x, lane = t & 63, g = t >> 4, m = t & 15;
  const int n = blockIdx.y;
  const int64_t s0 = min(max(int64_t(cu[n]), int64_t(0)), T);
  const int64_t s1 = min(max(int64_t(cu[n + 1]), s0), T);
  const int64_t len = s1 - s0, nb = min(len / 4, sh.cap);
  float w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = norm_w[8 * m + i];
  const RopeLane rl = rope_lane(m, sh);
  for (int i = 0; i < 4; ++i) {
    const int64_t b = int64_t(blockIdx.x) * 64 + g + 16 * i;
    if (b >= nb) break;
    float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float x[8];
      ld8(k + (s0 + 4 * b + j) * ld_k + 8 * m, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] += x[e];
    }
    finish_block(y, w, rl, 4 * b, sh.eps, lane, kbar + (int64_t(n) * sh.cap + b) * kQsaD + 8 * m);
  }
  if (pending && blockIdx.x == 0 && g < int(len & 3)) {
    float x[8];
    ld8(k + (s0 + (len & ~int64_t(3)) + g) * ld_k + 8 * m, x);
    st8(pending + (int64_t(n) * 3 + g) * kQsaD + 8 * m, x);
  }
}

// ---- decode: the new key of sequence b joins slot (n-1) % 4 of its block; slot 3 completes it.
// Run by one 16-lane group.
template <typename IO>
__device__ __forceinline__ void append_key(const QsaShape& sh, int b, int n, const QsaAppend& ap, int lane) {
  const int m = lane & 15;
  if (n < 1) return;
  const int j = (n - 1) & 3;
  const IO* k = static_cast<const IO*>(ap.k);
  IO* pending = static_cast<IO*>(ap.pending);
  float x[8];
  ld8(k + int64_t(b) * ap.ld_k + 8 * m, x);
  if (j < 3) {
    st8(pending + (int64_t(b) * 3 + j) * kQsaD + 8 * m, x);
    return;
  }
  const int64_t blk = n / 4 - 1;
  if (blk >= sh.cap) return;
  float w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = ap.norm_w[8 * m + i];
  float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jj = 0; jj < 3; ++jj) {  // token order, as in the prefill compression
    float p[8];
    ld8(pending + (int64_t(b) * 3 + jj) * kQsaD + 8 * m, p);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] += p[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] += x[e];
  const RopeLane rl = rope_lane(m, sh);
  finish_block(y, w, rl, 4 * blk, sh.eps, lane, static_cast<IO*>(ap.kbar) + (int64_t(b) * sh.cap + blk) * kQsaD + 8 * m);
}

// ---- per-row preparation: (sequence, position) and the rotated fp32 queries -------------------
// Prefill rows are tokens row0 + r of the packed batch (cu given); decode rows are sequences with
// position n_tok[r] - 1.
// Decode rows (cu == nullptr) also append their sequence's new key (group 0), before any score
// kernel reads the cache.
template <typename IO>
__global__ void __launch_bounds__(64) k_qsa_qprep(QsaShape sh, const IO* __restrict__ q, int64_t ld_q,
                                                  int64_t row0, const int32_t* __restrict__ cu, int n_seqs,
                                                  const int32_t* __restrict__ n_tok, QsaAppend ap,
                                                  float* __restrict__ qr, int2* __restrict__ info) {
  const int t = threadIdx.x, h = t >> 4, m = t & 15;
  if (!cu && ap.k && h == 0) append_key<IO>(sh, int(blockIdx.x), n_tok[blockIdx.x], ap, t);
  const int64_t r = blockIdx.x, row = row0 + r;
  int seq, pos;
  if (cu) {
    int lo = 0, hi = n_seqs;  // largest n with cu[n] <= row
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (int64_t(cu[mid]) <= row) lo = mid; else hi = mid;
    }
    seq = lo;
    pos = int(row - min(int64_t(cu[lo]), row));
  } else {
    seq = int(r);
    pos = n_tok[r] - 1;
  }
  float y[8];
  ld8(q + row * ld_q + h * kQsaD + 8 * m, y);
  const RopeLane rl = rope_lane(m, sh);
  rope8(y, rl, double(max(pos, 0)), t);
  if (std::is_same<IO, bf16>::value && cu) {
    // bf16 prefill: the MFMA score kernel's operands, rounded here once ([rows][4][128] bf16 in the
    // same buffer)
    *reinterpret_cast<short8*>(reinterpret_cast<uint16_t*>(qr) + r * (kQsaHeads * kQsaD) + h * kQsaD + 8 * m) =
        pack8(f32x4{y[0], y[1], y[2], y[3]}, f32x4{y[4], y[5], y[6], y[7]});
  } else {
    float* o = qr + r * (kQsaHeads * kQsaD) + h * kQsaD + 8 * m;
    *reinterpret_cast<float4*>(o) = make_float4(y[0], y[1], y[2], y[3]);
    *reinterpret_cast<float4*>(o + 4) = make_float4(y[4], y[5], y[6], y[7]);
  }
  if (t == 0) info[r] = make_int2(seq, pos);
}

__device__ __forceinline__ int64_t row_blocks(int pos, int64_t cap) {
  return pos < 0 ? 0 : min(int64_t(pos + 1) / 4, cap);
}

// Sum over the 4 heads of ReLU(dot) for one compressed key: p[h] are a lane's partial dots over its
// 8 dims. The heads are spread over the lanes while being reduced (lane bits 3, 2 pick the head), so
// the whole reduction takes 7 lane exchanges instead of 16. The exchanges stay inside the key's 16
// lanes (one DPP row), so they are DPP moves: lane ^ 8 is a rotation by 8; lane ^ 4 is a rotation
// by 4 (lanes with bit 2 set, reading lane - 4) or by 12 (reading lane + 4); lane ^ 2 and lane ^ 1
// are quad permutations; the last two sums add the four quads by rotations.
__device__ __forceinline__ float head_relu_sum(const float (&p)[4], int m) {
  const bool b3 = m & 8, b2 = m & 4;
  const float r0 = dpp_f32<0x128>(b3 ? p[0] : p[2]);  // lane ^ 8
  const float r1 = dpp_f32<0x128>(b3 ? p[1] : p[3]);
  const float k0 = (b3 ? p[2] : p[0]) + r0, k1 = (b3 ? p[3] : p[1]) + r1;  // heads 2 b3, 2 b3 + 1
  const float x = b2 ? k0 : k1;
  const float r4 = dpp_f32<0x124>(x), r12 = dpp_f32<0x12C>(x);
  float v = (b2 ? k1 : k0) + (b2 ? r4 : r12);  // head 2 b3 + b2, summed over 4 lanes
  v += dpp_f32<0x4E>(v);  // quad_perm [2, 3, 0, 1]: lane ^ 2
  v += dpp_f32<0xB1>(v);  // quad_perm [1, 0, 3, 2]: lane ^ 1
  v = fmaxf(v, 0.f);
  v += dpp_f32<0x124>(v);
  v += dpp_f32<0x128>(v);
  return v;
}

// ---- scores: grid (rows, block chunks of 1024); 16 groups of 16 lanes, one compressed key each --
template <typename IO>
__global__ void __launch_bounds__(256) k_qsa_score(QsaShape sh, const float* __restrict__ qr,
                                                   const int2* __restrict__ info, const IO* __restrict__ kbar,
                                                   float* __restrict__ scores, int64_t ld_s) {
  constexpr int N = vec16<IO>::N, V = 8 / N;
  const int t = threadIdx.x, g = t >> 4, m = t & 15;
  const int64_t r = blockIdx.x;
  const int2 in = info[r];
  const int64_t nb = row_blocks(in.y, sh.cap);
  const int64_t b0 = int64_t(blockIdx.y) * kScoreChunk;
  if (b0 >= nb) return;
  const int64_t end = min(b0 + kScoreChunk, nb);
  float qv[kQsaHeads][8];
#pragma unroll
  for (int h = 0; h < kQsaHeads; ++h) {
    const float* p = qr + r * (kQsaHeads * kQsaD) + h * kQsaD + 8 * m;
    const float4 a = *reinterpret_cast<const float4*>(p), c = *reinterpret_cast<const float4*>(p + 4);
    qv[h][0] = a.x; qv[h][1] = a.y; qv[h][2] = a.z; qv[h][3] = a.w;
    qv[h][4] = c.x; qv[h][5] = c.y; qv[h][6] = c.z; qv[h][7] = c.w;
  }
  // the cache is streamed once per call: non-temporal loads keep it from evicting the scores
  const IO* base = kbar + int64_t(in.x) * sh.cap * kQsaD + 8 * m;
  float* out = scores + r * ld_s;
  for (int64_t s = b0 + g; s < end; s += 16 * kScoreUnroll) {
    uint4 raw[kScoreUnroll][V];
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      const int64_t b = min(s + 16 * u, end - 1);  // clamped blocks are loaded, not stored
#pragma unroll
      for (int v = 0; v < V; ++v) raw[u][v] = ldnt16(base + b * kQsaD + v * N);
    }
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      float x[8];
#pragma unroll
      for (int v = 0; v < V; ++v) vec16<IO>::cvt(raw[u][v], x + v * N);
      float p[kQsaHeads];
#pragma unroll
      for (int h = 0; h < kQsaHeads; ++h) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) a = fmaf(qv[h][i], x[i], a);
        p[h] = a;
      }
      const float sc = head_relu_sum(p, m);
      if (m == 0 && s + 16 * u < end) out[s + 16 * u] = sc;
    }
  }
}

// ---- prefill scores on bf16 MFMA: one wave per 32 query rows (two 16-row tiles), 16 compressed
// keys per step -----------------------------------------------------------------------------------
// D_h = K Q_h^T for each head and tile (16x16x32 MFMA, fp32 accumulate), then sum_h ReLU(D_h). The
// keys are the A operand (the stored bf16 cache), shared by the two tiles; the rotated queries,
// which the query prep rounds to bf16 for this kernel, are the B operands, so lane (li, lq) ends a step with keys b0 + 4 lq .. + 3 of
// rows r0 + li and r0 + 16 + li and stores each as one 16-byte piece. A wave's rows can span
// sequences (packed batches): it runs once per sequence it touches. Every step issues the same
// memory instructions in every lane (so the waits for the prefetched keys are exact counts): the
// keys of step j + kMfmaRing are requested right after step j's MFMAs, and a lane stores its scores
// whether or not they are wanted: past the row's last block (inside the row's padding, which
// nothing reads) or, for a row of another sequence, past the last row, or a step past the slice (the
// loop runs whole rounds of the ring), into the spare row `rows` of the score buffer.
constexpr int kMfmaRing = 2;   // key steps in flight per wave (three: the same time, more spills)
constexpr int kMfmaTiles = 2;  // 16-row query tiles per wave
constexpr int kMfmaRows = 16 * kMfmaTiles * 4;  // query rows per workgroup

__global__ void __launch_bounds__(256, 2) k_qsa_score_mfma(QsaShape sh, const uint16_t* __restrict__ qr,
                                                        const int2* __restrict__ info, int64_t rows,
                                                        const uint16_t* __restrict__ kbar,
                                                        float* __restrict__ scores, int64_t ld_s) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, li = lane & 15, lq = lane >> 4;
  const int64_t r0 = (int64_t(blockIdx.x) * 4 + w) * (16 * kMfmaTiles);
  if (r0 >= rows) return;
  const int64_t rn = min(r0 + 16 * kMfmaTiles, rows);
  // this lane's output rows r0 + 16 tt + li
  int64_t row[kMfmaTiles];
  int oseq[kMfmaTiles], onb[kMfmaTiles];
#pragma unroll
  for (int tt = 0; tt < kMfmaTiles; ++tt) {
    row[tt] = min(r0 + 16 * tt + li, rn - 1);
    const int2 in = info[row[tt]];
    oseq[tt] = r0 + 16 * tt + li < rn ? in.x : -1;
    onb[tt] = int(row_blocks(in.y, sh.cap));
  }
  const int s_first = info[r0].x, s_last = info[rn - 1].x;
  const int c0 = blockIdx.y * kMfmaChunk;
  {  // most of the causal triangle's (rows, chunk) pairs are empty: leave before loading queries
    int most = 0;
#pragma unroll
    for (int tt = 0; tt < kMfmaTiles; ++tt) most = oseq[tt] >= 0 ? max(most, onb[tt]) : most;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) most = max(most, __shfl_xor(most, o, kWave));
    if (c0 >= most) return;
  }
  // B operand of tile tt, head h, k-step ks: row r0 + 16 tt + li, dims 32 ks + 8 lq .. + 7
  short8 a[kMfmaTiles][kQsaHeads][4];
#pragma unroll
  for (int tt = 0; tt < kMfmaTiles; ++tt)
#pragma unroll
    for (int h = 0; h < kQsaHeads; ++h)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        a[tt][h][ks] = ld_short8(qr + row[tt] * (kQsaHeads * kQsaD) + h * kQsaD + 32 * ks + 8 * lq);
      }
  float* const spare = scores + rows * ld_s + 4 * lq;

  for (int sq = s_first; sq <= s_last; ++sq) {
    int nbmax = 0;  // blocks of the wave's rows in this sequence (<= cap < 2^20)
#pragma unroll
    for (int tt = 0; tt < kMfmaTiles; ++tt) nbmax = oseq[tt] == sq ? max(nbmax, onb[tt]) : nbmax;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) nbmax = max(nbmax, __shfl_xor(nbmax, o, kWave));
    const int cend = __builtin_amdgcn_readfirstlane(min(nbmax, c0 + kMfmaChunk));  // this workgroup's slice
    if (c0 >= cend) continue;
    float* dst[kMfmaTiles];
#pragma unroll
    for (int tt = 0; tt < kMfmaTiles; ++tt)
      dst[tt] = oseq[tt] == sq ? scores + (r0 + 16 * tt + li) * ld_s + 4 * lq : spare;
    const uint16_t* kb = kbar + int64_t(sq) * sh.cap * kQsaD + 8 * lq;
    // A operands of the step at b0: key min(b0 + li, cend - 1), dims 32 ks + 8 lq .. + 7 (clamped
    // rows past the slice are loaded and their scores land in padding)
    auto load = [&](short8 (&kk)[4], int b0) {
      const uint16_t* p = kb + int64_t(min(b0 + li, cend - 1)) * kQsaD;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kk[ks] = ld_short8(p + 32 * ks);
    };
    auto step = [&](short8 (&kk)[4], int b0) {  // b0 past the slice: clamped keys, stored to the spare row
      f32x4 acc[kMfmaTiles][kQsaHeads];
#pragma unroll
      for (int tt = 0; tt < kMfmaTiles; ++tt)
#pragma unroll
        for (int h = 0; h < kQsaHeads; ++h) {
          acc[tt][h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) acc[tt][h] = mfma16x16x32(kk[ks], a[tt][h][ks], acc[tt][h]);
        }
      load(kk, b0 + 16 * kMfmaRing);
#pragma unroll
      for (int tt = 0; tt < kMfmaTiles; ++tt) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float t = 0.f;
#pragma unroll
          for (int h = 0; h < kQsaHeads; ++h) t += fmaxf(acc[tt][h][e], 0.f);
          v[e] = t;
        }
        *reinterpret_cast<f32x4*>(b0 < cend ? dst[tt] + b0 : spare) = v;
      }
    };
    short8 ring[kMfmaRing][4];
#pragma unroll
    for (int i = 0; i < kMfmaRing; ++i) {  // in ring order, as the loop consumes them
      load(ring[i], c0 + 16 * i);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int b0 = c0; b0 < cend; b0 += 16 * kMfmaRing) {
#pragma unroll
      for (int i = 0; i < kMfmaRing; ++i) step(ring[i], b0 + 16 * i);
    }
  }
}

// ---- exact top-k of up to 16384 keys held 16 per thread by 1024 threads ------------------------
// Keys are score bits with the sign cleared: scores are >= 0, so the unsigned order of the bits is
// the order of the scores. Thread t holds keys t * 16 .. t * 16 + 15 (index order = thread order,
// then slot order); a missing key (past the row) is kNoKey, which is negative as an int and so below
// every real key in signed compares and outside every bucket range. The k-th largest key is found
// digit by digit, each digit from a 2048-bin LDS histogram of the keys that match the digits found
// so far; then the keys above it and the first `need_eq` keys equal to it, in index order, are
// selected. The kernels issue few vector instructions per key: at 16 keys per thread they are bound
// by instruction issue, not by memory.
constexpr int kHistPad = 2048 + 2048 / 32;  // bin b at b + b / 32: the digit wave reads runs 33 words apart
constexpr int kGather = 256;                 // bucket sizes resolved by ranking instead of more digits
constexpr uint32_t kNoKey = 0xffffffffu;

__device__ __forceinline__ int hpad(int b) { return b + (b >> 5); }

template <int NT>
struct __attribute__((aligned(16))) SelLds {
  static constexpr int NW = NT / 64;
  uint32_t hist[3][kHistPad];    // one histogram per digit, all cleared up front
  uint32_t gkey[kGather];        // keys of the threshold bucket, when it is small
  uint32_t wmin[NW], wmax[NW], wpos[NW];
  uint32_t wcnt[NW];             // per wave: selected-above count << 16 | equal count
  uint32_t digit, above, ngather;
};

// Wave 0 finds the bin holding the need-th largest key in two wave scans: lane l first sums its run
// of c = nbins/64 bins (from the top bin down); the lane whose run crosses `need` is found, then the
// lanes take one bin each of that run (c <= 32) and a second scan finds the bin.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t n = __shfl_up(v, o, kWave);
    if (lane >= o) v += n;
  }
  return v;
}

template <typename LDS>
__device__ __forceinline__ void find_digit(const uint32_t* hist, int nbins, uint32_t need, LDS& L) {
  const int lane = threadIdx.x & 63, c = nbins >= 64 ? nbins / 64 : 1, top = nbins - 1 - lane * c;
  uint32_t sum = 0;
  for (int i = 0; i < c; ++i) sum += top - i >= 0 ? hist[hpad(top - i)] : 0u;
  const uint32_t incl = wave_incl_scan(sum, lane);
  const bool cross = incl - sum < need && need <= incl;
  const uint64_t who = __ballot(cross);
  const int src = int(__ffsll(static_cast<unsigned long long>(who))) - 1;  // exactly one lane crosses
  const uint32_t above_run = __shfl(incl - sum, src, kWave);
  const int top_run = nbins - 1 - src * c;
  const uint32_t h = (lane < c && top_run - lane >= 0) ? hist[hpad(top_run - lane)] : 0u;
  const uint32_t in2 = wave_incl_scan(h, lane) + above_run;
  if (lane < c && in2 - h < need && need <= in2) {
    L.digit = uint32_t(top_run - lane);
    L.above = in2 - h;
  }
}

// Threshold key T and how many keys equal to T to take (in index order), given more than k real
// keys. Zero keys (scores clipped to zero) are the smallest: when at most k keys are positive, all
// of those and the first k - n_pos zeros are taken. Otherwise the positive keys are bucketed over
// their own range [lo, lo + 2^bw), 11 bits per pass (bucketing by the top bits of the raw float
// pattern would put most keys of a wave into a few exponent bins and serialise the LDS atomics); a
// key is in the range when key - lo, as an unsigned number, is below 2^bw (zero and missing keys
// wrap far above it). After a pass, a bucket of at most kGather keys is resolved at once: its keys
// are gathered and wave 0 ranks them.
template <int NT, int S>
__device__ __forceinline__ void radix_threshold(const uint32_t (&key)[S], uint32_t k, SelLds<NT>& L,
                                                uint32_t* T_out, uint32_t* need_eq) {
  constexpr int NW = NT / 64;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  uint32_t mn = 0xffffffffu, np = 0;
  int mx = 0;
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const bool pos = int(key[j]) > 0;
    mn = min(mn, pos ? key[j] : 0xffffffffu);
    mx = max(mx, int(key[j]));
    np += pos;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = min(mn, uint32_t(__shfl_xor(mn, o, kWave)));
    mx = max(mx, __shfl_xor(mx, o, kWave));
    np += uint32_t(__shfl_xor(np, o, kWave));
  }
  if (lane == 0) {
    L.wmin[w] = mn;
    L.wmax[w] = uint32_t(mx);
    L.wpos[w] = np;
  }
  static_assert((3 * kHistPad) % 4 == 0, "histograms cleared in 16-byte pieces");
  for (int i = t; i < 3 * kHistPad / 4; i += NT) reinterpret_cast<uint4*>(&L.hist[0][0])[i] = make_uint4(0u, 0u, 0u, 0u);
  if (t == 0) L.ngather = 0;
  __syncthreads();
  uint32_t mxu = 0;
  mn = 0xffffffffu, np = 0;
#pragma unroll
  for (int u = 0; u < NW; ++u) {
    mn = min(mn, L.wmin[u]);
    mxu = max(mxu, L.wmax[u]);
    np += L.wpos[u];
  }
  if (np <= k) {
    *T_out = 0;
    *need_eq = k - np;
    return;
  }
  uint32_t lo = mn, need = k;
  int bw = 32 - __clz(mxu - mn);  // bits of the range: keys in [lo, lo + 2^bw), bw <= 31
  for (int pass = 0; pass < 3 && bw > 0; ++pass) {
    const int sh = max(bw - 11, 0), nbins = 1 << (bw - sh);
    const uint32_t range = 1u << bw;
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const uint32_t d = key[j] - lo;
      if (d < range) atomicAdd(&L.hist[pass][hpad(int(d >> sh))], 1u);
    }
    __syncthreads();
    if (t < kWave) find_digit(L.hist[pass], nbins, need, L);
    __syncthreads();
    const uint32_t dg = L.digit;
    const uint32_t cnt = L.hist[pass][hpad(int(dg))];
    need -= L.above;
    lo += dg << sh;
    bw = sh;
    if (bw > 0 && cnt <= kGather) {
      // the bucket [lo, lo + 2^bw) is small: gather its keys and rank them
      const uint32_t brange = 1u << bw;
#pragma unroll
      for (int j = 0; j < S; ++j)
        if (key[j] - lo < brange) L.gkey[atomicAdd(&L.ngather, 1u)] = key[j];
      __syncthreads();
      if (t < kWave) {
        const uint32_t n = L.ngather;
        for (uint32_t c = lane; c < n; c += kWave) {
          const uint32_t x = L.gkey[c];
          uint32_t gt = 0, eq = 0;
#pragma unroll 8
          for (uint32_t o = 0; o < n; ++o) {
            const uint32_t y = L.gkey[o];
            gt += y > x;
            eq += y == x;
          }
          if (gt < need && need <= gt + eq) {  // every lane that lands here holds the same key
            L.digit = x;
            L.above = gt;
          }
        }
      }
      __syncthreads();
      *T_out = L.digit;
      *need_eq = need - L.above;
      return;
    }
  }
  *T_out = lo;
  *need_eq = need;
}

// Selects (all real keys when n_valid <= k, else the top k) and calls emit(j, out_pos) for each
// selected key j of this thread, out_pos counting in index order (index = thread * S + j): one
// block-wide scan of each thread's counts (above | equal, packed) gives every thread its start.
// Returns the number selected.
// kSparse: emit needs only j (not key[j]), so the thread walks the set bits of its above / equal
// masks instead of every slot (a thread emits about k / NT keys; the wave loops as often as its
// busiest lane).
template <int NT, int S, bool kSparse = false, typename F>
__device__ __forceinline__ uint32_t select_topk(const uint32_t (&key)[S], uint32_t n_valid, uint32_t k,
                                                SelLds<NT>& L, F&& emit) {
  constexpr int NW = NT / 64;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const bool all = n_valid <= k;
  uint32_t T = 0, need_eq = 0;
  if (!all) radix_threshold<NT, S>(key, k, L, &T, &need_eq);
  // all: every real key counts as above (T = -1 as an int); else above means > T, equal means == T
  const int Ti = all ? -1 : int(T);
  const uint32_t Te = all ? kNoKey : T;
  uint32_t cnt = 0, mg = 0, me = 0;
  if constexpr (kSparse) {
#pragma unroll
    for (int j = 0; j < S; ++j) {
      mg |= uint32_t(int(key[j]) > Ti) << j;
      me |= uint32_t(key[j] == Te) << j;
    }
    cnt = (uint32_t(__popc(mg)) << 16) | uint32_t(__popc(me));
  } else {
#pragma unroll
    for (int j = 0; j < S; ++j) cnt += int(key[j]) > Ti ? 0x10000u : (key[j] == Te ? 1u : 0u);
  }
  const uint32_t incl = wave_incl_scan(cnt, lane);
  if (lane == 63) L.wcnt[w] = incl;
  __syncthreads();
  uint32_t pre = incl - cnt, tot = 0;
#pragma unroll
  for (int u = 0; u < NW; ++u) {
    const uint32_t x = L.wcnt[u];
    pre += u < w ? x : 0u;
    tot += x;
  }
  uint32_t gb = pre >> 16, eb = pre & 0xffffu;
  if constexpr (kSparse) {
    for (uint32_t m = mg | me; m != 0u; m &= m - 1u) {
      const int j = __ffs(m) - 1;
      const uint32_t below = (1u << j) - 1u;
      const uint32_t gbj = gb + uint32_t(__popc(mg & below)), ebj = eb + uint32_t(__popc(me & below));
      if ((mg >> j) & 1u) emit(j, gbj + min(ebj, need_eq));
      else if (ebj < need_eq) emit(j, gbj + ebj);
    }
  } else {
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const bool gt = int(key[j]) > Ti, eq = key[j] == Te;
      if (gt || (eq && eb < need_eq)) emit(j, gb + min(eb, need_eq));
      gb += gt;
      eb += eq;
    }
  }
  return (tot >> 16) + min(tot & 0xffffu, need_eq);
}

template <int NT>
__device__ __forceinline__ void finish_row(int32_t* sel_row, uint32_t count, uint32_t k, int pos, int32_t* n_sel,
                                           int32_t* tail) {
  for (uint32_t p = count + threadIdx.x; p < k; p += NT) sel_row[p] = -1;
  if (threadIdx.x == 0) {
    *n_sel = int32_t(count);
    *tail = pos < 0 ? 0 : 4 * ((pos + 1) / 4);
  }
}

// Segment pass: grid (rows, segments). A row with one segment is finished here; longer rows leave
// their segment's top-k (key, block) candidates for k_qsa_merge.
template <int NT>
__global__ void __launch_bounds__(NT, 8) k_qsa_select(QsaShape sh, const int2* __restrict__ info,
                                                            const float* __restrict__ scores, int64_t ld_s,
                                                            uint32_t* __restrict__ cand_key,
                                                            int32_t* __restrict__ cand_idx, int segmax,
                                                            int32_t* __restrict__ sel, int32_t* __restrict__ n_sel,
                                                            int32_t* __restrict__ tail) {
  __shared__ SelLds<NT> L;
  const int t = threadIdx.x;
  const int64_t r = blockIdx.x;
  const int sg = blockIdx.y;
  const int pos = info[r].y;
  const int64_t nb = row_blocks(pos, sh.cap);
  constexpr int SEG = NT * kSelPer;
  // smaller workgroups are launched only when every row fits one segment (cap <= SEG)
  const int nseg = SEG == kSelSeg ? int((nb + SEG - 1) / SEG) : int(nb > 0);
  if (sg >= max(nseg, 1)) return;
  const int64_t seg0 = int64_t(sg) * SEG;
  const uint32_t n = uint32_t(min(int64_t(SEG), nb - seg0 > 0 ? nb - seg0 : int64_t(0)));
  const float* row = scores + r * ld_s + seg0;
  const uint32_t k = uint32_t(sh.topk);
  // S keys per thread: the fewest slots that hold the segment, so short rows do less work per thread
  // (the select is bound by vector instruction issue, and most of it is per key)
  auto run = [&](auto s_tag) {
    constexpr int S = decltype(s_tag)::value;
    const uint32_t i0 = uint32_t(t) * S;  // this thread's first key
    uint32_t key[S];
#pragma unroll
    for (int q = 0; q < S / 4; ++q) {  // 16-byte pieces (the row stride is a multiple of 64 keys, so a
                                       // piece that starts before n stays inside the row)
      f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
      if (i0 + 4 * q < n) x = *reinterpret_cast<const f32x4*>(row + i0 + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        key[4 * q + e] = i0 + 4 * q + e < n ? (__float_as_uint(x[e]) & 0x7fffffffu) : kNoKey;
    }
    if (nseg <= 1) {
      int32_t* srow = sel + r * sh.topk;
      const uint32_t cnt = select_topk<NT, S, true>(key, n, k, L, [&](int j, uint32_t p) { srow[p] = int32_t(i0) + j; });
      finish_row<NT>(srow, cnt, k, pos, n_sel + r, tail + r);
    } else {
      const int64_t c0 = (r * segmax + sg) * int64_t(sh.topk);
      select_topk<NT, S>(key, n, k, L, [&](int j, uint32_t p) {
        cand_key[c0 + p] = key[j];
        cand_idx[c0 + p] = int32_t(seg0 + i0 + j);
      });
    }
  };
  if constexpr (NT == 1024) {  // decode rows (segments of 16384 scores): the short paths would spill
    run(std::integral_constant<int, kSelPer>{});
  } else {
    if (n <= 4u * NT)
      run(std::integral_constant<int, 4>{});
    else if (n <= 8u * NT)
      run(std::integral_constant<int, 8>{});
    else
      run(std::integral_constant<int, kSelPer>{});
  }
}

// Merge pass for rows of several segments: candidates of segment s sit at s * k .. s * k + c_s - 1,
// in block order, so list position order is block order.
template <int NT>
__global__ void __launch_bounds__(NT) k_qsa_merge(QsaShape sh, const int2* __restrict__ info,
                                                           const uint32_t* __restrict__ cand_key,
                                                           const int32_t* __restrict__ cand_idx, int segmax,
                                                           int32_t* __restrict__ sel, int32_t* __restrict__ n_sel,
                                                           int32_t* __restrict__ tail) {
  __shared__ SelLds<NT> L;
  const int t = threadIdx.x;
  const int64_t r = blockIdx.x;
  const int pos = info[r].y;
  const int64_t nb = row_blocks(pos, sh.cap);
  const int nseg = int((nb + kSelSeg - 1) / kSelSeg);
  if (nseg <= 1) return;
  const uint32_t k = uint32_t(sh.topk);
  const int64_t c0 = r * segmax * int64_t(sh.topk);
  uint32_t key[kSelPer], nv = 0;
  int32_t idx[kSelPer];
  const int64_t lim = int64_t(segmax) * k;  // this row's candidate slots; nothing past them is read
  if (k % 4 == 0) {  // 16-byte pieces of the candidate lists (c0 and lim are then multiples of 4)
#pragma unroll
    for (int q = 0; q < kSelPer / 4; ++q) {
      const int64_t p0 = int64_t(t) * kSelPer + 4 * q;
      uint4 kq = make_uint4(kNoKey, kNoKey, kNoKey, kNoKey);
      int4 iq = make_int4(0, 0, 0, 0);
      if (p0 < lim) {
        kq = *reinterpret_cast<const uint4*>(cand_key + c0 + p0);
        iq = *reinterpret_cast<const int4*>(cand_idx + c0 + p0);
      }
      key[4 * q] = kq.x; key[4 * q + 1] = kq.y; key[4 * q + 2] = kq.z; key[4 * q + 3] = kq.w;
      idx[4 * q] = iq.x; idx[4 * q + 1] = iq.y; idx[4 * q + 2] = iq.z; idx[4 * q + 3] = iq.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kSelPer; ++j) {
      const int64_t p = int64_t(t) * kSelPer + j;
      key[j] = p < lim ? cand_key[c0 + p] : kNoKey;
      idx[j] = p < lim ? cand_idx[c0 + p] : 0;
    }
  }
#pragma unroll
  for (int j = 0; j < kSelPer; ++j) {  // list position t * 16 + j: segment s, slot i; unfilled slots are no keys
    const uint32_t p = uint32_t(t * kSelPer + j), s = p / k, i = p - s * k;
    const int64_t cs = s < uint32_t(nseg) ? min(int64_t(k), min(int64_t(kSelSeg), nb - int64_t(s) * kSelSeg)) : 0;
    if (int64_t(i) >= cs) key[j] = kNoKey;
  }
  for (int s = 0; s < nseg; ++s) nv += uint32_t(min(int64_t(k), min(int64_t(kSelSeg), nb - int64_t(s) * kSelSeg)));
  int32_t* srow = sel + r * sh.topk;
  const uint32_t cnt = select_topk<NT, kSelPer>(key, nv, k, L, [&](int j, uint32_t p) { srow[p] = idx[j]; });
  finish_row<NT>(srow, cnt, k, pos, n_sel + r, tail + r);
}

// ---- launchers ----------------------------------------------------------------------------------
QsaWs plan_qsa_ws(const QsaShape& sh, int64_t rows, void* base, size_t* bytes) {
  QsaWs ws{};
  char* b = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t n) -> void* {
    void* r = b ? static_cast<void*>(b + off) : nullptr;
    off += (n + 255) & ~size_t(255);
    return r;
  };
  ws.segmax = int(std::max<int64_t>(1, (sh.cap + kSelSeg - 1) / kSelSeg));
  ws.ld_s = (sh.cap + 63) & ~int64_t(63);
  ws.qr = static_cast<float*>(take(sizeof(float) * size_t(rows) * kQsaHeads * kQsaD));
  ws.info = static_cast<int2*>(take(sizeof(int2) * size_t(rows)));
  // one spare row past the last: the MFMA score kernel's unwanted stores
  ws.scores = static_cast<float*>(take(sizeof(float) * size_t(rows + 1) * size_t(ws.ld_s)));
  const size_t nc = ws.segmax > 1 ? size_t(rows) * ws.segmax * size_t(sh.topk) : 0;
  ws.cand_key = static_cast<uint32_t*>(take(sizeof(uint32_t) * nc));
  ws.cand_idx = static_cast<int32_t*>(take(sizeof(int32_t) * nc));
  *bytes = off;
  return ws;
}

hipError_t launch_qsa_compress(const QsaShape& sh, int n_seqs, int64_t T, const int32_t* cu, const void* k,
                               int64_t ld_k, const float* norm_w, void* kbar, void* pending, hipStream_t s) {
  const int64_t nbmax = std::min<int64_t>(T / 4, sh.cap);
  const dim3 grid(unsigned(std::max<int64_t>(1, (nbmax + 63) / 64)), unsigned(n_seqs));
  if (sh.bf16)
    hipLaunchKernelGGL(k_qsa_compress<bf16>, grid, dim3(256), 0, s, sh, static_cast<const bf16*>(k), ld_k, cu, T,
                       norm_w, static_cast<bf16*>(kbar), static_cast<bf16*>(pending));
  else
    hipLaunchKernelGGL(k_qsa_compress<float>, grid, dim3(256), 0, s, sh, static_cast<const float*>(k), ld_k, cu, T,
                       norm_w, static_cast<float*>(kbar), static_cast<float*>(pending));
  return hipGetLastError();
}

hipError_t launch_qsa_rows(const QsaShape& sh, const QsaWs& ws, int64_t row0, int64_t rows, const int32_t* cu,
                           int n_seqs, const int32_t* n_tok, const QsaAppend& ap, const void* q, int64_t ld_q,
                           const void* kbar, int32_t* sel, int32_t* n_sel, int32_t* tail, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const dim3 rgrid(static_cast<unsigned>(rows));
  if (sh.bf16)
    hipLaunchKernelGGL(k_qsa_qprep<bf16>, rgrid, dim3(64), 0, s, sh, static_cast<const bf16*>(q), ld_q, row0, cu,
                       n_seqs, n_tok, ap, ws.qr, ws.info);
  else
    hipLaunchKernelGGL(k_qsa_qprep<float>, rgrid, dim3(64), 0, s, sh, static_cast<const float*>(q), ld_q, row0, cu,
                       n_seqs, n_tok, ap, ws.qr, ws.info);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 sgrid(unsigned(rows), unsigned(std::max<int64_t>(1, (sh.cap + kScoreChunk - 1) / kScoreChunk)));
  if (sh.cap > 0) {
    if (sh.bf16 && cu)  // prefill rows: many queries per sequence, a dense contraction
      hipLaunchKernelGGL(k_qsa_score_mfma,
                         dim3(static_cast<unsigned>((rows + kMfmaRows - 1) / kMfmaRows),
                              static_cast<unsigned>((sh.cap + kMfmaChunk - 1) / kMfmaChunk)),
                         dim3(256), 0, s, sh, reinterpret_cast<const uint16_t*>(ws.qr), ws.info, rows,
                         static_cast<const uint16_t*>(kbar), ws.scores, ws.ld_s);
    else if (sh.bf16)
      hipLaunchKernelGGL(k_qsa_score<bf16>, sgrid, dim3(256), 0, s, sh, ws.qr, ws.info,
                         static_cast<const bf16*>(kbar), ws.scores, ws.ld_s);
    else
      hipLaunchKernelGGL(k_qsa_score<float>, sgrid, dim3(256), 0, s, sh, ws.qr, ws.info,
                         static_cast<const float*>(kbar), ws.scores, ws.ld_s);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  int32_t* sel_r = sel + row0 * sh.topk;
  // one workgroup per row and segment; short rows (caches of <= 4096 or 8192 blocks) take smaller
  // workgroups, several of which share a CU
  const dim3 selgrid(static_cast<unsigned>(rows), static_cast<unsigned>(ws.segmax));
  if (sh.cap <= 256 * kSelPer)
    hipLaunchKernelGGL(k_qsa_select<256>, selgrid, dim3(256), 0, s, sh, ws.info, ws.scores, ws.ld_s, ws.cand_key,
                       ws.cand_idx, ws.segmax, sel_r, n_sel + row0, tail + row0);
  else if (sh.cap <= 512 * kSelPer)
    hipLaunchKernelGGL(k_qsa_select<512>, selgrid, dim3(512), 0, s, sh, ws.info, ws.scores, ws.ld_s, ws.cand_key,
                       ws.cand_idx, ws.segmax, sel_r, n_sel + row0, tail + row0);
  else
    hipLaunchKernelGGL(k_qsa_select<1024>, selgrid, dim3(1024), 0, s, sh, ws.info, ws.scores, ws.ld_s, ws.cand_key,
                       ws.cand_idx, ws.segmax, sel_r, n_sel + row0, tail + row0);
  e = hipGetLastError();
  if (e != hipSuccess || ws.segmax <= 1) return e;
  hipLaunchKernelGGL(k_qsa_merge<1024>, rgrid, dim3(1024), 0, s, sh, ws.info, ws.cand_key, ws.cand_idx, ws.segmax,
                     sel_r, n_sel + row0, tail + row0);
  return hipGetLastError();
}

}  // namespace gdn
