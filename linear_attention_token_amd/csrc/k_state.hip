// Inter-chunk state propagation: the only sequential part of the chunked prefill.
//
// For each chunk of a sequence, from the chunk-start state S (fp32, kept in registers):
//     W  = U - Wk S                               (the chunk's effective writes beta_t e_t)
//     S <- exp(G_C) S + K^T diag(exp(G_C - G_i)) W  (state after the chunk)
// which is the update equations of the analysis notes "Qwen3.8-Flash-Next：架构、效率与技术谱系"
// (§03) applied to 64 tokens at once (U, Wk, G from the WY kernel). The chunk-start state and W are
// stored (bf16) for the output kernel, which then runs chunk-parallel.
//
// The d_v columns of S are independent in these products, so a chain is split into 4 slices of
// 32 columns: one block of 4 compute waves per (sequence, value head, slice). Wave w owns state
// rows 32w..32w+31 (two 16-row MFMA tiles) and W rows 16w..16w+15 of the slice; S and W cross
// waves through LDS in bf16 as the B operand of the bf16 MFMAs, accumulation stays fp32. Each wave
// streams its own operands (A operands of Wk and K^T, its U tiles, G) through a private LDS ring
// (see below).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kSlice = 32;  // state columns per block
constexpr int kSlices = 128 / kSlice;

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

// ---- explicit memory operations -------------------------------------------------------------
// The chunk operands stream through a ring in LDS, filled by direct global->LDS loads (no VGPR
// destinations) that a fifth, producer wave issues kDepth-1 steps ahead and waits for with explicit
// vmcnt counts; the four compute waves never stall on load issue. Every load moves 1 KB of
// consecutive global bytes (whole rows): such loads stream about twice as fast per CU as loads
// gathering 64-byte pieces of 16 rows. The 16-byte pieces of a row are placed in LDS in an XOR
// order, so that the compute waves' MFMA operand reads (16 rows, the same columns) hit distinct
// banks. The compute waves write the chunk state and W with coalesced stores from LDS.

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
// The trailing s_nop covers the gfx9 hazard of a VALU overwriting the data VGPRs of a store wider
// than 8 bytes right after it (the compiler's hazard recognizer does not see inside inline asm).
__device__ __forceinline__ void st16(void* gptr, const void* lds_src) {
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(lds_src);
  asm volatile("global_store_dwordx4 %0, %1, off\n\ts_nop 1" ::"v"(gptr), "v"(v) : "memory");
}

constexpr int kDepth = 3;                       // ring slots: loads run kDepth - 1 steps ahead
constexpr int kNT = kSlice / 16;                // 16-column tiles per block
static_assert(kNT == 2, "one U tile pair per compute wave");
// Slot layout (bytes): Wk [64 rows][256 B], K^T [128 rows][128 B], U [4 waves][1 KB tile pair],
// G [64] fp32. Row r of Wk keeps its 16-byte piece q at slot q ^ (r % 16); row r of K^T keeps
// piece q at slot q ^ ((r / 2) % 8).
constexpr int kOffWk = 0, kOffKT = 16384, kOffU = 32768, kOffG = 36864;
constexpr int kSlot = kOffG + 256;
constexpr int kLoadsPerChunk = 16 + 16 + 4 + 1;  // Wk (4 rows each), K^T (8 rows each), U, G
constexpr int kStLd = 136;                      // bf16 row stride of S^T [cols][128 k]
constexpr int kWtLd = 72;                       // bf16 row stride of W~^T and W^T [cols][64 tokens]
constexpr size_t kStateSmem = size_t(kDepth) * kSlot + kSlice * kStLd * 2 + 2 * kSlice * kWtLd * 2;

// Load i of chunk c into the ring slot at LDS address `slot`.
__device__ __forceinline__ void issue_load(const StateArgs& a, int64_t c, int h, int g, int sl, int lane,
                                           uint32_t slot, int i) {
  if (i < 16) {  // Wk rows 4i .. 4i+3
    const int r = 4 * i + (lane >> 4), piece = (lane & 15) ^ (r & 15);
    dma16(a.Wk + (c * a.hv + h) * 8192 + r * 128 + piece * 8, slot + kOffWk + i * 1024);
  } else if (i < 32) {  // K^T rows 8k .. 8k+7
    const int k = i - 16, r = 8 * k + (lane >> 3), piece = (lane & 7) ^ ((r >> 1) & 7);
    dma16(a.KT + (c * a.hk + g) * 8192 + r * 64 + piece * 8, slot + kOffKT + k * 1024);
  } else if (i < 36) {  // U tile pair sl of accumulator row tile (wave) i - 32
    const int w = i - 32;
    dma16(a.U + (c * a.hv + h) * 8192 + (w * 4 + sl) * 512 + lane * 8, slot + kOffU + w * 1024);
  } else {
    dma4(a.G + (c * a.hv + h) * 64 + lane, slot + kOffG);
  }
}

__global__ void __launch_bounds__(320) k_state(StateArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // the R value heads of a QK head (all their slices) read the same K^T tiles: keep them on one XCD
  int u, sub;
  xcd_item(int(blockIdx.x), a.R * kSlices, u, sub);
  if (u >= a.n_units) return;
  const int n = u / a.hk, g = u - n * a.hk;
  const int h = g * a.R + sub / kSlices, sl = sub % kSlices;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;  // waves 0-3 compute, wave 4 loads
  const int li = lane & 15, lq = lane >> 4;
  const bool producer = (w == 4);
  uint16_t* STs = reinterpret_cast<uint16_t*>(smem + size_t(kDepth) * kSlot);
  uint16_t* WTs = STs + kSlice * kStLd;   // W~^T: B operand of K^T W~
  uint16_t* WUs = WTs + kSlice * kWtLd;    // W^T unscaled: staged for the coalesced store
  const uint32_t ring = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  const int64_t c0 = a.seq_off[n], c1 = a.seq_off[n + 1];
  const int64_t clast = c1 > c0 ? c1 - 1 : c0;

  // state rows 32w + 16m + 4lq + r, columns kSlice*sl + 16nt + li
  f32x4 S[2][kNT];
  const size_t sbase = (size_t(n) * a.hv + h) * 128 * 128;
  if (!producer) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S[m][nt][r] = a.state_in ? a.state_in[sbase + size_t(32 * w + 16 * m + 4 * lq + r) * 128 + kSlice * sl + 16 * nt + li] : 0.f;
    // settle these loads here, so no wait inside the loop has to cover them (the loop's own
    // stores would then be waited for too)
    wait_vm<0>();
  }
  // the producer issues loads [i0, i1) of one chunk into one slot
  auto produce = [&](int64_t c, int slot, int i0, int i1) {
    const int64_t cc = min(c, clast);
    const uint32_t sa = ring + uint32_t(slot * kSlot);
#pragma unroll
    for (int i = i0; i < i1; ++i) issue_load(a, cc, h, g, sl, lane, sa, i);
  };
  if (c0 < c1 && producer) {
#pragma unroll
    for (int i = 0; i < kDepth - 1; ++i) produce(c0 + i, i, 0, kLoadsPerChunk);
    wait_vm<(kDepth - 2) * kLoadsPerChunk>();  // chunk c0 has landed
  }

  for (int64_t c = c0; c < c1; ++c) {
    const int64_t j = c - c0;
    const int slot = int(j % kDepth);
    __syncthreads();  // B0: chunk c is in its ring slot
    if (producer) {
      // refill the slot read during step c - 1 (its reads finished before that step's B1), spread
      // over the step so no barrier waits for the producer
      const int fill = int((j + kDepth - 1) % kDepth);
      produce(c + kDepth - 1, fill, 0, 13);
      __syncthreads();  // B1
      produce(c + kDepth - 1, fill, 13, 26);
      __syncthreads();  // B2
      produce(c + kDepth - 1, fill, 26, kLoadsPerChunk);
      wait_vm<(kDepth - 2) * kLoadsPerChunk>();  // chunk c + 1 has landed
      continue;
    }

    const unsigned char* sb = smem + size_t(slot) * kSlot;
    // A operands: Wk rows 16w + li and K^T rows 32w + 16m + li, columns 32s + 8lq .. +7 (piece
    // 4s + lq), each at its XOR slot
    short8 wk[4], kt[2][2];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      wk[s] = *reinterpret_cast<const short8*>(sb + kOffWk + (16 * w + li) * 256 + (((4 * s + lq) ^ li) << 4));
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        kt[m][s] = *reinterpret_cast<const short8*>(sb + kOffKT + (32 * w + 16 * m + li) * 128 +
                                                    (((4 * s + lq) ^ (li >> 1)) << 4));
    uint2 uu[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
      uu[nt] = *reinterpret_cast<const uint2*>(sb + kOffU + w * 1024 + lane * 16 + nt * 8);
    const float* Gl = reinterpret_cast<const float*>(sb + kOffG);
    const float4 gr = *reinterpret_cast<const float4*>(Gl + 16 * w + 4 * lq);
    const float gc = Gl[63];

    // S (bf16) -> LDS as S^T
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const int col = 16 * nt + li, k0 = 32 * w + 16 * m + 4 * lq;
        *reinterpret_cast<uint2*>(&STs[col * kStLd + k0]) =
            make_uint2(pack_bf16x2(S[m][nt][0], S[m][nt][1]), pack_bf16x2(S[m][nt][2], S[m][nt][3]));
      }
    __syncthreads();  // B1
    // chunk-start state to the output kernel, in its MFMA operand pieces: piece (sl, nt, w) holds
    // columns 32sl + 16nt + (lane % 16), rows 32w + 8 (lane / 16) .. +7 -- 1 KB per store
    {
      uint16_t* stf = a.ST + (size_t(c) * a.hv + h) * 128 * 128;
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
        st16(stf + (((sl * kNT + nt) * 4 + w) * 64 + lane) * 8, &STs[(16 * nt + li) * kStLd + 32 * w + 8 * lq]);
    }

    // W = U - Wk S   (rows 16w + 4lq + r, columns 16nt + li)
    f32x4 Wt[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc = mfma16x16x32(wk[s], ld_short8(&STs[(16 * nt + li) * kStLd + 32 * s + 8 * lq]), acc);
      const uint2 u = uu[nt];
      Wt[nt][0] = __uint_as_float(u.x << 16) - acc[0];
      Wt[nt][1] = __uint_as_float(u.x & 0xffff0000u) - acc[1];
      Wt[nt][2] = __uint_as_float(u.y << 16) - acc[2];
      Wt[nt][3] = __uint_as_float(u.y & 0xffff0000u) - acc[3];
    }
    // W^T staged for the output kernel; W~ = diag(exp(G_C - G_i)) W to LDS as the B operand of K^T W~
    const float dec[4] = {__expf(gc - gr.x), __expf(gc - gr.y), __expf(gc - gr.z), __expf(gc - gr.w)};
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const int col = 16 * nt + li, t0 = 16 * w + 4 * lq;
      *reinterpret_cast<uint2*>(&WUs[col * kWtLd + t0]) =
          make_uint2(pack_bf16x2(Wt[nt][0], Wt[nt][1]), pack_bf16x2(Wt[nt][2], Wt[nt][3]));
      *reinterpret_cast<uint2*>(&WTs[col * kWtLd + t0]) =
          make_uint2(pack_bf16x2(Wt[nt][0] * dec[0], Wt[nt][1] * dec[1]),
                     pack_bf16x2(Wt[nt][2] * dec[2], Wt[nt][3] * dec[3]));
    }
    __syncthreads();  // B2
    // W^T to the output kernel, in its MFMA operand pieces: wave w stores piece (sl, nt, s) with
    // nt = w / 2, s = w % 2: columns 32sl + 16nt + (lane % 16), tokens 32s + 8 (lane / 16) .. +7
    {
      const int nt = w >> 1, s = w & 1;
      uint16_t* wtf = a.WT + (size_t(c) * a.hv + h) * 128 * 64;
      st16(wtf + (((sl * kNT + nt) * 2 + s) * 64 + lane) * 8, &WUs[(16 * nt + li) * kWtLd + 32 * s + 8 * lq]);
    }

    // S <- exp(G_C) S + K^T W~
    const float gC = __expf(gc);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        f32x4 acc = S[m][nt] * gC;
#pragma unroll
        for (int s = 0; s < 2; ++s)
          acc = mfma16x16x32(kt[m][s], ld_short8(&WTs[(16 * nt + li) * kWtLd + 32 * s + 8 * lq]), acc);
        S[m][nt] = acc;
      }
  }
  if (producer) {
    wait_vm<0>();  // no load may still be writing this block's LDS when it exits
    return;
  }

  if (a.state_out) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          a.state_out[sbase + size_t(32 * w + 16 * m + 4 * lq + r) * 128 + kSlice * sl + 16 * nt + li] = S[m][nt][r];
  }
}

hipError_t launch_state(const Problem& p, const Workspace& ws, const float* state_in, float* state_out,
                        hipStream_t s) {
  if (p.n_seqs == 0) return hipSuccess;
  const int R = p.hv / p.hk;
  const int64_t units = int64_t(p.n_seqs) * p.hk;
  StateArgs a{ws.seq_chunk_off, int(units), p.hk, p.hv, R, ws.G, ws.Wk, ws.U, ws.KT, ws.ST, ws.WT,
              state_in, state_out};
  static bool attr_set = false;  // same value on every device; idempotent, so a race is harmless
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_state),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, int(kStateSmem));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(k_state, dim3(unsigned(xcd_blocks(units, R * kSlices))), dim3(320),
                     kStateSmem, s, a);
  return hipGetLastError();
}

}  // namespace gdn
