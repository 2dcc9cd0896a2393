// The layer's projections around the mixer: input projection (q | k | v, the gate logits and the
// decay / write gates from one fused input matrix) and the output projection.
//
// The paper reading "Qwen3.8-Flash-Next" (方法) sends the normalised residual stream through learned
// projections before the short conv, with a data-dependent decay gate and a write gate; the analysis
// notes "Qwen3.8-Flash-Next：架构、效率与技术谱系" (§07 optimizer table) describe the GDN input as one
// fused matrix of independent operators, 2-D input/output weights, and per-head alpha / beta
// vectors. The gate formula is not on the pages; the reading used here is
//     alpha = exp(-exp(A_h) softplus(a + delta_h)),   beta = sigmoid(b),
// with [a | b] = x W_ab and per-head vectors A, delta.
//
// Both projections are one bf16 MFMA GEMM kernel, out[t][n] = sum_k x[t][k] W[n][k] with fp32
// accumulation. The input projection runs it once over the stacked weight rows [W_qkv | W_z | W_ab]:
// column blocks of q | k | v and of the gate logits leave in bf16, and the 2 HV gate columns go
// through the gate formula in fp32 in the same epilogue (alpha is steep in a, so a must not be
// rounded to bf16 first). Weights are in the linear-layer layout [out features][in features],
// row-major, so both operands are K-contiguous rows.
//
// Kernel: a block computes an FT out features x TT tokens tile (256 x 256; 320 x 128 or 128 x 256 when
// those fill the chip's rounds better) with waves of FT / 2 features x a share of the tokens on 32x32x16
// bf16 MFMA: eight waves (two per SIMD, 128 x 64 each) for 256 x 256, so one wave's MFMAs run while the
// other waits at the LDS reads or the barrier; four (one per SIMD) for the other shapes (out features
// as the A operand, tokens as the B operand; each lane
// ends with runs of 4 consecutive output features of one token; the tile is staged in LDS and stored
// as 16-byte pieces of token rows). K advances in steps of 32 through a
// five-slot LDS ring filled by direct global->LDS loads three steps ahead. Blocks are numbered so that
// the 32 blocks an XCD runs at once form a 4 x 8 group of tiles that share their operand panels in
// that XCD's L2.
#include <atomic>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kKStep = 32;               // k per ring slot
constexpr int kRingG = 5;                // ring slots
constexpr int kAhead = kRingG - 2;       // k-steps loaded ahead of the one being multiplied
constexpr int kGroupM = 8, kGroupT = 4;  // tiles of a block group: 8 feature tiles x 4 token tiles
constexpr int kWaves256 = 8;             // waves of a 256 x 256 tile block
constexpr int kMaxGateHeads = 3072;      // value heads the epilogue's LDS holds gate vectors for

// Per tile shape: FT output features x TT tokens (each a multiple of 64) with WV waves, 2 along the
// features and WV / 2 along the tokens, each wave computing FT / 2 x TT / (WV / 2):
template <int FT, int TT, int WV> struct Geo {
  static constexpr int kPanelW = FT * kKStep * 2;                  // W panel bytes per slot
  static constexpr int kPanelX = TT * kKStep * 2;                  // x panel bytes per slot
  static constexpr int kSlot = kPanelW + kPanelX;
  static constexpr int kWLoads = FT / (16 * WV);                   // 1 KB W panel loads per wave and slot
  static constexpr int kXLoads = TT / (16 * WV);                   // 1 KB x panel loads per wave and slot
  static constexpr int kLoads = kWLoads + kXLoads;
  static constexpr int kMI = FT / 64;                              // 32-row feature tiles per wave
  static constexpr int kTW = TT / (WV / 2);                        // tokens per wave
  static constexpr int kNJ = kTW / 32;                             // 32-token tiles per wave
  static constexpr int kCLd = FT + 8;                              // bytes per token row of a wave's staged tile
  static constexpr int kFLd = FT / 2 + 4;                          // floats per token row of a staged fp32 gate tile
  static constexpr int kGateParams = WV * kTW * kCLd;              // exp(a_log), dt_bias in the epilogue
  static constexpr size_t kSmem = size_t(kRingG) * kSlot;
  static_assert(FT % (16 * WV) == 0 && TT % (16 * WV) == 0 && kTW % 32 == 0, "whole loads and tiles per wave");
  static_assert(kSmem <= 160 * 1024, "LDS budget");
  static_assert(size_t(kGateParams) + 8 * kMaxGateHeads <= kSmem, "gate vectors fit beside the staged tiles");
  static_assert(kTW * kCLd >= 32 * kFLd * 4, "a wave's staging area holds a 32-token fp32 gate tile");
};

// Rows of a panel are 64 bytes (four 16-byte pieces of k); piece p of row r sits at slot
// p ^ ((r >> 2) & 3), so the operand reads of 16 consecutive rows at one piece hit distinct banks.
__device__ __forceinline__ int pkey(int r) { return (r >> 2) & 3; }

struct GemmArgs {
  const uint16_t* x;        // [T][ld_x] bf16 activations
  int64_t ld_x, T;
  int K;                    // in features (a multiple of 32)
  const uint16_t* w[3];     // weight segments [rows][K]
  int64_t seg_end[3];       // cumulative row counts of the segments (output features)
  uint16_t* out[2];         // bf16 outputs of segments 0 and 1: [T][ld_out]
  int64_t ld_out[2];
  // segment 2, when gates != 0: the gate pre-activations [a | b] (2 hv columns)
  int gates, hv;
  const float *a_log, *dt_bias;
  float *alpha, *beta;      // [T][hv]
  int n_tiles_m, n_tiles_t;
};

// Source row of output feature n (clamped into the last segment's rows).
__device__ __forceinline__ const uint16_t* weight_row(const GemmArgs& a, int64_t n) {
  const int64_t N = a.seg_end[2];
  n = min(n, N - 1);
  if (n < a.seg_end[0]) return a.w[0] + n * a.K;
  if (n < a.seg_end[1]) return a.w[1] + (n - a.seg_end[0]) * a.K;
  return a.w[2] + (n - a.seg_end[1]) * a.K;
}

template <int FT, int TT, int WV>
__global__ void __launch_bounds__(64 * WV) k_gemm(GemmArgs a) {
  using G = Geo<FT, TT, WV>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // block -> tile: XCD x runs blocks b = 8 j + x; the 32 consecutive j of one XCD form one group
  const int b = int(blockIdx.x), x = b & 7, j = b >> 3;
  const int n_gm = (a.n_tiles_m + kGroupM - 1) / kGroupM;
  const int grp = (j / (kGroupM * kGroupT)) * 8 + x, in = j % (kGroupM * kGroupT);
  const int tmr = (grp % n_gm) * kGroupM + in % kGroupM, tt = (grp / n_gm) * kGroupT + in / kGroupM;
  if (tmr >= a.n_tiles_m || tt >= a.n_tiles_t) return;
  const int tm = a.n_tiles_m - 1 - tmr;  // the last feature tiles (the gate columns) go first
  const int64_t n0 = int64_t(tm) * FT, t0 = int64_t(tt) * TT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w & 1, wt = w >> 1;  // this wave's part: features (FT / 2) wm .., tokens kTW wt ..
  const uint32_t ring = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  const int nks = a.K / kKStep;

  // This wave's direct loads of one slot: W load i < kWLoads covers W panel rows 16 (kWLoads w + i) ..
  // + 15, x load i covers x panel rows 16 (kXLoads w + i - kWLoads) .. + 15; lane l takes row
  // 16 (.) + l / 4, slot l % 4.
  const uint16_t* src[G::kLoads];
  uint32_t dst[G::kLoads];
#pragma unroll
  for (int i = 0; i < G::kLoads; ++i) {
    const bool wl = i < G::kWLoads;
    const int blk = wl ? G::kWLoads * w + i : G::kXLoads * w + (i - G::kWLoads);
    const int r = 16 * blk + (lane >> 2), piece = (lane & 3) ^ pkey(r);
    src[i] = (wl ? weight_row(a, n0 + r) : a.x + min(t0 + r, a.T - 1) * a.ld_x) + 8 * piece;
    dst[i] = (wl ? 0 : G::kPanelW) + blk * 1024;
  }
  auto issue = [&](int ks, int slot) {
    const uint32_t sa = ring + uint32_t(slot * G::kSlot);
#pragma unroll
    for (int i = 0; i < G::kLoads; ++i) dma16(src[i] + int64_t(ks) * kKStep, sa + dst[i]);
  };
  auto barrier = []() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  // acc[i][jt]: 32 x 32 tile, element e: feature 8 (e / 4) + 4 hq + e % 4, token l32 (within tiles i, jt)
  const int l32 = lane & 31, hq = lane >> 5;
  f32x16 acc[G::kMI][G::kNJ];
#pragma unroll
  for (int i = 0; i < G::kMI; ++i)
#pragma unroll
    for (int jt = 0; jt < G::kNJ; ++jt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][jt][e] = 0.f;

  // waits until at most `later` k-steps issued after the next one are still in flight
  auto settle = [&](int later) {
    if (later >= 2) wait_vm<2 * G::kLoads>();
    else if (later == 1) wait_vm<G::kLoads>();
    else wait_vm<0>();
  };
  for (int k = 0; k < kAhead && k < nks; ++k) issue(k, k);
  settle(min(kAhead, nks) - 1);
  barrier();
  for (int ks = 0; ks < nks; ++ks) {
    if (ks + kAhead < nks) issue(ks + kAhead, (ks + kAhead) % kRingG);
    const unsigned char* sb = smem + size_t(ks % kRingG) * G::kSlot;
#pragma unroll
    for (int u = 0; u < 2; ++u) {  // two k-substeps of 16: pieces 2u + hq of the 64-byte rows
      short8 af[G::kMI], bf[G::kNJ];
#pragma unroll
      for (int i = 0; i < G::kMI; ++i) {
        const int r = (FT / 2) * wm + 32 * i + l32;
        af[i] = *reinterpret_cast<const short8*>(sb + r * 64 + (((2 * u + hq) ^ pkey(r)) << 4));
      }
#pragma unroll
      for (int jt = 0; jt < G::kNJ; ++jt) {
        const int r = G::kTW * wt + 32 * jt + l32;
        bf[jt] = *reinterpret_cast<const short8*>(sb + G::kPanelW + r * 64 + (((2 * u + hq) ^ pkey(r)) << 4));
      }
#pragma unroll
      for (int i = 0; i < G::kMI; ++i)
#pragma unroll
        for (int jt = 0; jt < G::kNJ; ++jt) acc[i][jt] = mfma32x32x16(af[i], bf[jt], acc[i][jt]);
    }
    // the next step has landed (later steps may stay in flight)
    settle(min(ks + kAhead, nks - 1) - (ks + 1));
    barrier();
  }

  // ---- epilogue. The bf16 outputs go through this wave's tile in LDS (the ring is free after the
  // last barrier) and leave as 16-byte pieces of token rows; the gate columns are finished from the
  // fp32 registers. ----
  unsigned char* const cs = smem + size_t(w) * G::kTW * G::kCLd;
#pragma unroll
  for (int i = 0; i < G::kMI; ++i)
#pragma unroll
    for (int jt = 0; jt < G::kNJ; ++jt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {  // features 32i + 8g + 4hq .. +3 of token 32jt + l32
        const f32x16& v = acc[i][jt];
        *reinterpret_cast<uint2*>(cs + (32 * jt + l32) * G::kCLd + (32 * i + 8 * g + 4 * hq) * 2) =
            make_uint2(pack_bf16x2(v[4 * g], v[4 * g + 1]), pack_bf16x2(v[4 * g + 2], v[4 * g + 3]));
      }
  const int64_t nw = n0 + (FT / 2) * wm;  // first feature of this wave's tile
  constexpr int kRowPieces = FT / 16;      // 16-byte pieces per staged token row (FT / 2 features)
#pragma unroll 4
  for (int k = 0; k < G::kTW * kRowPieces / 64; ++k) {
    const int pc = lane + 64 * k, tl = pc / kRowPieces, seg8 = pc % kRowPieces;
    const int64_t t = t0 + G::kTW * wt + tl, n = nw + 8 * seg8;
    if (t >= a.T || n >= a.seg_end[1]) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(cs + tl * G::kCLd + seg8 * 16);
    if (n < a.seg_end[0]) *reinterpret_cast<uint4*>(a.out[0] + t * a.ld_out[0] + n) = v;
    else *reinterpret_cast<uint4*>(a.out[1] + t * a.ld_out[1] + (n - a.seg_end[0])) = v;
  }
  if (!a.gates || nw + FT / 2 <= a.seg_end[1]) return;
  // Gate columns. exp(a_log) and dt_bias are staged in LDS by this wave (another wave of the block may
  // write the same values); then, per 32-token tile, the fp32 accumulators go to this wave's staging
  // area (its bf16 rows are all stored by now) and a compact loop applies the formula.
  float* const gp = reinterpret_cast<float*>(smem + G::kGateParams);
  for (int c = lane; c < a.hv; c += 64) {
    gp[c] = __expf(a.a_log[c]);
    gp[a.hv + c] = a.dt_bias[c];
  }
  float* const fs = reinterpret_cast<float*>(cs);  // [32 tokens][kFLd] fp32: every row holds the wave's FT / 2 columns
  const int c_lo = int(max<int64_t>(a.seg_end[1] - nw, 0)), c_hi = int(min<int64_t>(a.seg_end[2] - nw, FT / 2));
  const int nc = c_hi - c_lo;
#pragma unroll
  for (int jt = 0; jt < G::kNJ; ++jt) {
#pragma unroll
    for (int i = 0; i < G::kMI; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& v = acc[i][jt];
        *reinterpret_cast<float4*>(fs + l32 * G::kFLd + 32 * i + 8 * g + 4 * hq) =
            make_float4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
      }
    for (int e = lane; e < 32 * nc; e += 64) {
      const int tl = e / nc, c = c_lo + (e - tl * nc);
      const int64_t t = t0 + G::kTW * wt + 32 * jt + tl;
      if (t >= a.T) continue;
      const int col = int(nw + c - a.seg_end[1]);
      const float v = fs[tl * G::kFLd + c];
      if (col < a.hv) {
        const float uu = v + gp[a.hv + col];
        const float sp = fmaxf(uu, 0.f) + __logf(1.f + __expf(-fabsf(uu)));  // softplus without overflow
        a.alpha[t * a.hv + col] = __expf(-gp[col] * sp);
      } else {
        a.beta[t * a.hv + (col - a.hv)] = sigmoidf_(v);
      }
    }
  }
}

template <int FT, int TT, int WV = 4>
hipError_t launch_tiles(GemmArgs& a, hipStream_t s) {
  using G = Geo<FT, TT, WV>;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  // this instance's LDS limit is raised once per device (an idempotent call, so a race only repeats it)
  static std::atomic<uint64_t> raised{0};
  const uint64_t bit = uint64_t(1) << (dev & 63);
  if (!(raised.load() & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_gemm<FT, TT, WV>), hipFuncAttributeMaxDynamicSharedMemorySize,
                            int(G::kSmem));
    if (e != hipSuccess) return e;
    raised.fetch_or(bit);
  }
  a.n_tiles_m = int((a.seg_end[2] + FT - 1) / FT);
  a.n_tiles_t = int((a.T + TT - 1) / TT);
  const int n_gm = (a.n_tiles_m + kGroupM - 1) / kGroupM, n_gt = (a.n_tiles_t + kGroupT - 1) / kGroupT;
  const int64_t groups = int64_t(n_gm) * n_gt;
  const int64_t blocks = ((groups + 7) / 8) * 8 * kGroupM * kGroupT;  // every XCD walks whole groups
  hipLaunchKernelGGL((k_gemm<FT, TT, WV>), dim3(unsigned(blocks)), dim3(64 * WV), G::kSmem, s, a);
  return hipGetLastError();
}

// Tile shape by the number of tiles, one block per CU: 256 x 256 tiles, unless they fill less than one
// round of the chip's 256 CUs; then 320 x 128, or 128 x 256 when there are too few 256-wide tiles to
// occupy a quarter of the chip.
hipError_t launch_gemm(GemmArgs& a, hipStream_t s) {
  if (a.T == 0 || a.seg_end[2] == 0) return hipSuccess;
  auto tiles = [&](int ft, int tt) { return ((a.seg_end[2] + ft - 1) / ft) * ((a.T + tt - 1) / tt); };
  const int64_t t256 = tiles(256, 256);
  if (t256 < 64) return launch_tiles<128, 256>(a, s);
  // under one round of 256 x 256 tiles, 320 x 128 tiles (5/8 the work each) spread it over more CUs;
  // past that the larger tile's better ratio of MFMA work to operand traffic wins (measured: 427 against
  // 400 us for the input projection at T = 4096, 137 against 178 us for the output projection)
  if (t256 < 256 && tiles(320, 128) <= 256) return launch_tiles<320, 128>(a, s);
  return launch_tiles<256, 256, kWaves256>(a, s);
}

}  // namespace

hipError_t launch_in_proj(const Problem& p, int H, int64_t T, const void* x, int64_t ld_x, const void* w_qkv,
                          const void* w_z, const void* w_ab, const float* a_log, const float* dt_bias, void* qkv,
                          void* z, float* alpha, float* beta, hipStream_t s) {
  const int64_t C = p.C, vz = int64_t(p.hv) * p.dv;
  GemmArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.ld_x = ld_x;
  a.T = T;
  a.K = H;
  a.w[0] = static_cast<const uint16_t*>(w_qkv);
  a.w[1] = static_cast<const uint16_t*>(w_z);
  a.w[2] = static_cast<const uint16_t*>(w_ab);
  a.seg_end[0] = C;
  a.seg_end[1] = C + vz;
  a.seg_end[2] = C + vz + 2 * p.hv;
  a.out[0] = static_cast<uint16_t*>(qkv);
  a.out[1] = static_cast<uint16_t*>(z);
  a.ld_out[0] = C;
  a.ld_out[1] = vz;
  a.gates = 1;
  a.hv = p.hv;
  a.a_log = a_log;
  a.dt_bias = dt_bias;
  a.alpha = alpha;
  a.beta = beta;
  return launch_gemm(a, s);
}

hipError_t launch_out_proj(const Problem& p, int H, int64_t T, const void* o, const void* w_out, void* y,
                           hipStream_t s) {
  const int64_t vz = int64_t(p.hv) * p.dv;
  GemmArgs a{};
  a.x = static_cast<const uint16_t*>(o);
  a.ld_x = vz;
  a.T = T;
  a.K = int(vz);
  a.w[0] = a.w[1] = a.w[2] = static_cast<const uint16_t*>(w_out);
  a.seg_end[0] = a.seg_end[1] = a.seg_end[2] = H;
  a.out[0] = a.out[1] = static_cast<uint16_t*>(y);
  a.ld_out[0] = a.ld_out[1] = H;
  a.gates = 0;
  return launch_gemm(a, s);
}

}  // namespace gdn
