// Inter-chunk state propagation: the only sequential part of the chunked prefill.
//
// For each chunk of a sequence, from the chunk-start state S (fp32, kept in registers):
//     W  = U - Wk S                               (the chunk's effective writes beta_t e_t)
//     S <- exp(G_C) S + K^T diag(exp(G_C - G_i)) W  (state after the chunk)
// which is the update equations of the analysis notes "Qwen3.8-Flash-Next：架构、效率与技术谱系"
// (§03) applied to 64 tokens at once (U, Wk, G from the WY kernel). The chunk-start state and W are
// stored (bf16) for the output kernel, which then runs chunk-parallel.
//
// The d_v columns of S are independent in these products. One block serves a (sequence, value head,
// 32-column slice); each of its two compute waves owns one 16-column tile of S for all 128 rows,
// so both products of a chunk run on the wave's own registers:
//   * S is held in the row order pi (pi32 in gdn_device.h): the wave's accumulator tiles 2s and
//     2s + 1 are then, rounded to bf16, the B operand of rows 32s .. 32s + 31 -- W = U - Wk S needs
//     no exchange of S between waves;
//   * W is computed with its token rows in the order pi as well, so rounded W~ is directly the B
//     operand of K^T W~;
//   * the chunk-start state and W go to the output kernel as those same 16-byte operand pieces,
//     straight from registers.
// The only per-chunk synchronisation is the hand-over of the chunk's operands (A operands Wk and
// K^T, the wave's U, G), which two producer waves stream through an LDS ring; the compute waves
// read the next chunk's operands from the ring into registers while the current chunk's MFMAs
// run, and the barrier between chunks does not wait for those reads.
#include <atomic>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kSlices = 4;  // column slices per value head: one block each
constexpr int kTilesPerBlock = 128 / 16 / kSlices;  // 16-column tiles per block
constexpr int kComputeWaves = 2;
constexpr int kTilesPerWave = kTilesPerBlock / kComputeWaves;  // each A-operand read feeds this many MFMAs

struct StateArgs {
  const int32_t* seq_off;
  int n_units;  // sequences x QK heads
  int hk, hv, R;
  const float* G;
  const uint16_t *Wk, *U, *KT;
  uint16_t *ST, *WT;
  const float* state_in;
  float* state_out;
};

// ---- operand ring ------------------------------------------------------------------------------
// The chunk operands stream through a ring in LDS, filled by direct global->LDS loads (no VGPR
// destinations) that two producer waves issue kDepth-1 chunks ahead and wait for with explicit
// vmcnt counts (two chunks of loads exceed what one wave may have outstanding); the compute waves
// never stall on load issue. Every load moves 1 KB of consecutive
// global bytes (whole rows): such loads stream about twice as fast per CU as loads gathering
// 64-byte pieces of 16 rows. The 16-byte pieces of a row sit in LDS in an XOR order chosen so that
// the MFMA operand reads (rows pi(16t + i), i < 16, one piece) hit distinct banks.

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
// 16-byte global store of a register piece; non-temporal, since the pieces are read back only by
// the output kernel, while the ring's operands are reused from the caches by neighbouring blocks.
__device__ __forceinline__ void stg16(uint16_t* gptr, const short8& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<short8*>(gptr));
}

constexpr int kDepth = 4;  // ring slots
// Slot layout (bytes): Wk [64 rows][256 B], K^T [128 rows][128 B], U [compute waves][2 slabs]
// [1 KB], G [64] fp32.
constexpr int kULoads = 2 * kTilesPerBlock;
constexpr int kOffWk = 0, kOffKT = 16384, kOffU = 32768, kOffG = kOffU + 1024 * kULoads;
constexpr int kSlot = kOffG + 256;
constexpr int kLoadsPerChunk = 16 + 16 + kULoads + 1;  // Wk (4 rows each), K^T (8 rows each), U, G
constexpr size_t kStateSmem = size_t(kDepth) * kSlot;
// XOR keys: Wk row r (16 pieces) uses bits 0, 1, 3, 4 of r; K^T row r (8 pieces, two rows per 64
// banks) uses bits 1, 3, 4. Over the rows pi(16t + i), i < 16, both are one-to-one (per parity
// of r for K^T).
__device__ __forceinline__ int wk_key(int r) { return (r & 3) | (((r >> 3) & 3) << 2); }
__device__ __forceinline__ int kt_key(int r) { return ((r >> 1) & 1) | (((r >> 3) & 3) << 1); }

// Load i of chunk c into the ring slot at LDS address `slot`.
__device__ __forceinline__ void issue_load(const StateArgs& a, int64_t c, int h, int g, int sl, int lane,
                                           uint32_t slot, int i) {
  if (i < 16) {  // Wk rows 4i .. 4i+3
    const int r = 4 * i + (lane >> 4), piece = (lane & 15) ^ wk_key(r);
    dma16(a.Wk + (c * a.hv + h) * 8192 + r * 128 + piece * 8, slot + kOffWk + i * 1024);
  } else if (i < 32) {  // K^T rows 8k .. 8k+7
    const int k = i - 16, r = 8 * k + (lane >> 3), piece = (lane & 7) ^ kt_key(r);
    dma16(a.KT + (c * a.hk + g) * 8192 + r * 64 + piece * 8, slot + kOffKT + k * 1024);
  } else if (i < 32 + kULoads) {  // U: column tile kTilesPerBlock sl + (i - 32) / 2, token slab (i - 32) % 2
    const int k = i - 32;
    dma16(a.U + (c * a.hv + h) * 8192 + ((kTilesPerBlock * sl) * 2 + k) * 512 + lane * 8, slot + kOffU + k * 1024);
  } else {
    dma4(a.G + (c * a.hv + h) * 64 + lane, slot + kOffG);
  }
}

constexpr int kProducers = 2;  // waves issuing the ring loads; each has its own vmcnt budget
constexpr int kLoadsP0 = (kLoadsPerChunk + 1) / 2;  // loads [0, kLoadsP0) by producer 0, the rest by 1

__global__ void __launch_bounds__(64 * (kComputeWaves + kProducers)) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_state(StateArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // the R value heads of a QK head (both halves) read the same K^T tiles: keep them on one XCD
  int u, sub;
  xcd_item(int(blockIdx.x), a.R * kSlices, u, sub);
  if (u >= a.n_units) return;
  const int n = u / a.hk, g = u - n * a.hk;
  const int h = g * a.R + sub / kSlices, sl = sub % kSlices;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;  // compute waves first, then loaders
  const int li = lane & 15, lq = lane >> 4;
  const bool producer = (w >= kComputeWaves);
  const int pw = w - kComputeWaves;
  const int jc0 = kTilesPerBlock * sl + kTilesPerWave * w;  // this wave's first column tile
  const uint32_t ring = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  const int64_t c0 = a.seq_off[n], c1 = a.seq_off[n + 1];
  const int64_t clast = c1 > c0 ? c1 - 1 : c0;

  // S[v][m][r]: state row pi(16m + 4lq + r), column 16(jc0 + v) + li
  f32x4 S[kTilesPerWave][8];
  const size_t sbase = (size_t(n) * a.hv + h) * 128 * 128;
  if (!producer) {
#pragma unroll
    for (int v = 0; v < kTilesPerWave; ++v)
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S[v][m][r] = a.state_in ? a.state_in[sbase + size_t(pi32(16 * m + 4 * lq + r)) * 128 + 16 * (jc0 + v) + li] : 0.f;
    // settle these loads here, so no wait inside the loop has to cover them (the loop's own
    // stores would then be waited for too)
    wait_vm<0>();
  }
  // a producer issues its share of the loads of one chunk into one slot
  auto produce = [&](int64_t c, int slot) {
    const int64_t cc = min(c, clast);
    const uint32_t sa = ring + uint32_t(slot * kSlot);
    if (pw == 0) {
#pragma unroll
      for (int i = 0; i < kLoadsP0; ++i) issue_load(a, cc, h, g, sl, lane, sa, i);
    } else {
#pragma unroll
      for (int i = kLoadsP0; i < kLoadsPerChunk; ++i) issue_load(a, cc, h, g, sl, lane, sa, i);
    }
  };
  auto settle = [&]() {  // all but the last chunk issued have landed
    if (pw == 0) wait_vm<kLoadsP0>();
    else wait_vm<kLoadsPerChunk - kLoadsP0>();
  };
  // Block barrier without the memory fence of __syncthreads: LDS reads issued before it (the next
  // chunk's operands) stay in flight across it. The memory clobber keeps the compiler from moving
  // memory accesses across it; ring data is published by the producers' vmcnt waits before it.
  auto barrier = []() { asm volatile("s_barrier" ::: "memory"); };

  // A-operand rows (ring rows) of this lane: token pi(16t + li), state row pi(16m + li)
  int tok[4], srow[8];
#pragma unroll
  for (int t = 0; t < 4; ++t) tok[t] = pi32(16 * t + li);
#pragma unroll
  for (int m = 0; m < 8; ++m) srow[m] = pi32(16 * m + li);

  // Operands of one chunk, read from its ring slot into registers: Wk rows tok[t] and K^T rows
  // srow[m], columns 32s + 8lq .. +7 (piece 4s + lq) at their XOR slots; this wave's U pieces; G.
  struct Ops {
    short8 wk[4][4], kt[8][2];
    uint4 up[kTilesPerWave][2];
    float4 gt[4];
    float gc;
  };
  // LDS returns reads in issue order, so they are issued in the order the chunk step consumes
  // them (G, Wk, U, K^T): each wait then covers only what the next instruction needs.
  auto read_ops = [&](int slot, Ops& o) {
    const unsigned char* sb = smem + size_t(slot) * kSlot;
    const float* Gl = reinterpret_cast<const float*>(sb + kOffG);
#pragma unroll
    for (int k = 0; k < 4; ++k) o.gt[k] = *reinterpret_cast<const float4*>(Gl + 32 * (k >> 1) + 8 * lq + 4 * (k & 1));
    o.gc = Gl[63];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int r = tok[t];
        o.wk[t][s] = *reinterpret_cast<const short8*>(sb + kOffWk + r * 256 + (((4 * s + lq) ^ wk_key(r)) << 4));
      }
#pragma unroll
    for (int v = 0; v < kTilesPerWave; ++v)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        o.up[v][s] = *reinterpret_cast<const uint4*>(sb + kOffU + ((kTilesPerWave * w + v) * 2 + s) * 1024 + lane * 16);
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int r = srow[m];
        o.kt[m][s] = *reinterpret_cast<const short8*>(sb + kOffKT + r * 128 + (((4 * s + lq) ^ kt_key(r)) << 4));
      }
  };

  // Ring schedule (kDepth = 4 slots): the producers keep two chunks in flight and, before barrier
  // j, have chunk j + 2 landed; after barrier j - 1 the compute waves read chunk j + 1's operands
  // while they compute chunk j. The slot refilled after barrier j - 1 (chunk j + 3) held chunk j - 1,
  // whose operands were consumed before barrier j - 1.
  Ops op;
  if (c0 < c1) {
    if (producer) {
#pragma unroll
      for (int i = 0; i < 3; ++i) produce(c0 + i, i);
      settle();  // chunks c0 and c0 + 1 have landed
    }
    barrier();
    if (!producer) read_ops(0, op);
  }

  for (int64_t c = c0; c < c1; ++c) {
    const int64_t j = c - c0;
    if (producer) {
      produce(c + 3, int((j + 3) % kDepth));
      settle();  // chunk c + 2 has landed
      barrier();
      continue;
    }

    // chunk-start state in bf16: B operand of rows 32s .. +31 (rows 32s + 8lq .. +7 in this lane),
    // and the output kernel's piece (column tile jc0 + v, row slab s)
    short8 sbf[kTilesPerWave][4];
    uint16_t* stf = a.ST + (size_t(c) * a.hv + h) * 128 * 128;
#pragma unroll
    for (int v = 0; v < kTilesPerWave; ++v)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sbf[v][s] = pack8(S[v][2 * s], S[v][2 * s + 1]);
        stg16(stf + (((jc0 + v) * 4 + s) * 64 + lane) * 8, sbf[v][s]);
      }

    // W = U - Wk S, token rows in the order pi: W[t][r] is token pi(16t + 4lq + r) = 32(t/2) +
    // 8lq + 4(t%2) + r, whose U value is element 4(t%2) + r of this lane's U piece of slab t/2
    f32x4 W[kTilesPerWave][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x4 acc[kTilesPerWave];
#pragma unroll
      for (int v = 0; v < kTilesPerWave; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int v = 0; v < kTilesPerWave; ++v) acc[v] = mfma16x16x32(op.wk[t][s], sbf[v][s], acc[v]);
#pragma unroll
      for (int v = 0; v < kTilesPerWave; ++v) W[v][t] = acc[v];
    }
    short8 wbf[kTilesPerWave][2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float gt[8] = {op.gt[2 * s].x, op.gt[2 * s].y, op.gt[2 * s].z, op.gt[2 * s].w,
                           op.gt[2 * s + 1].x, op.gt[2 * s + 1].y, op.gt[2 * s + 1].z, op.gt[2 * s + 1].w};
      float dec[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) dec[e] = __expf(op.gc - gt[e]);
#pragma unroll
      for (int v = 0; v < kTilesPerWave; ++v) {
        const uint32_t uw[4] = {op.up[v][s].x, op.up[v][s].y, op.up[v][s].z, op.up[v][s].w};
        f32x4 wt[2], wd[2];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float uv = __uint_as_float(e & 1 ? uw[e >> 1] & 0xffff0000u : uw[e >> 1] << 16);
          const float wv = uv - W[v][2 * s + (e >> 2)][e & 3];
          wt[e >> 2][e & 3] = wv;
          wd[e >> 2][e & 3] = wv * dec[e];
        }
        wbf[v][s] = pack8(wd[0], wd[1]);   // W~ = diag(exp(G_C - G_i)) W: B operand of K^T W~
        // W, tokens 32s + 8lq .. +7: the output kernel's piece
        stg16(a.WT + (size_t(c) * a.hv + h) * 128 * 64 + (((jc0 + v) * 2 + s) * 64 + lane) * 8, pack8(wt[0], wt[1]));
      }
    }

    // S <- exp(G_C) S + K^T W~
    const float gC = __expf(op.gc);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      f32x4 acc[kTilesPerWave];
#pragma unroll
      for (int v = 0; v < kTilesPerWave; ++v) acc[v] = S[v][m] * gC;
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int v = 0; v < kTilesPerWave; ++v) acc[v] = mfma16x16x32(op.kt[m][s], wbf[v][s], acc[v]);
#pragma unroll
      for (int v = 0; v < kTilesPerWave; ++v) S[v][m] = acc[v];
    }
    // the next chunk's operands, over this one's MFMAs (unconditional, so that they share the
    // MFMAs' basic block; after the last chunk the slot's contents are read and not used)
    read_ops(int((j + 1) % kDepth), op);
    barrier();
  }
  if (producer) {
    wait_vm<0>();  // no load may still be writing this block's LDS when it exits
    return;
  }

  if (a.state_out) {
#pragma unroll
    for (int v = 0; v < kTilesPerWave; ++v)
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          a.state_out[sbase + size_t(pi32(16 * m + 4 * lq + r)) * 128 + 16 * (jc0 + v) + li] = S[v][m][r];
  }
}

hipError_t launch_state(const Problem& p, const Workspace& ws, const float* state_in, float* state_out,
                        hipStream_t s) {
  if (p.n_seqs == 0) return hipSuccess;
  const int R = p.hv / p.hk;
  const int64_t units = int64_t(p.n_seqs) * p.hk;
  StateArgs a{ws.seq_chunk_off, int(units), p.hk, p.hv, R, ws.G, ws.Wk, ws.U, ws.KT, ws.ST, ws.WT,
              state_in, state_out};
  // the kernel's LDS limit is raised once per device (an idempotent call, so a race only repeats it)
  static std::atomic<uint64_t> attr_set{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = uint64_t(1) << (dev & 63);
  if (!(attr_set.load() & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_state), hipFuncAttributeMaxDynamicSharedMemorySize,
                            int(kStateSmem));
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit);
  }
  hipLaunchKernelGGL(k_state, dim3(unsigned(xcd_blocks(units, R * kSlices))), dim3(64 * (kComputeWaves + kProducers)),
                     kStateSmem, s, a);
  return hipGetLastError();
}

}  // namespace gdn
