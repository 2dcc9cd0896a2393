// Host-side declarations shared by the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

constexpr int kChunk = 64;      // tokens per chunk of the WY form
constexpr int kConvStrip = 8;   // tokens per thread of the conv kernel

// XCD-aware block numbering. The blocks of a launch are dealt round-robin over the chip's 8 XCDs
// (block b runs on XCD b % 8), each with its own L2. Work that reads the same tiles (the value heads
// of one QK head) forms a unit of `per_unit` blocks; numbering the blocks as xcd_item() decodes them
// puts all blocks of a unit on one XCD, back to back, so the first one's misses fill that XCD's L2
// for the others. Grids are 1-D with xcd_blocks() blocks; items past the last unit exit at once.
constexpr int kXcds = 8;
inline int64_t xcd_blocks(int64_t units, int per_unit) {
  return int64_t(kXcds) * per_unit * ((units + kXcds - 1) / kXcds);
}

// Problem description after validation; every launcher reads it.
struct Problem {
  int hk, hv, dk, dv;
  int n_seqs;
  int64_t T;
  int64_t C;          // conv channels: 2*hk*dk + hv*dv
  int64_t nc_max;     // bound on the number of 64-token chunks: T/64 + n_seqs
  uint32_t flags;
  float scale, l2_eps, norm_eps;
  int norm_stride;    // 0 or dv
  bool bf16;          // io dtype
};

// Device workspace regions. Offsets are computed by plan_workspace() and are 256-byte aligned.
struct Workspace {
  // both paths
  int32_t* seq_chunk_off = nullptr;  // [n_seqs + 1] first chunk of each sequence
  int4* chunk_tab = nullptr;         // [nc_max] (start token, length, sequence, 0)
  void* qhat = nullptr;              // [T][hk][dk]  work type
  void* khat = nullptr;              // [T][hk][dk]
  void* vhat = nullptr;              // [T][hv][dv]
  // chunked bf16 path only
  float* G = nullptr;                // fp32 [nc][hv][64]    in-chunk cumulative log decay
  uint16_t* Wk = nullptr;            // bf16 [nc][hv][64][128]  T diag(beta*gamma) K
  uint16_t* U = nullptr;             // bf16 [nc][hv][8 col tiles][2 token slabs][64 lanes][8]  T diag(beta) V
  uint16_t* KT = nullptr;            // bf16 [nc][hk][128][64]  K^T of each chunk
  uint16_t* ST = nullptr;            // bf16 [nc][hv][8 col tiles][4 row slabs][64 lanes][8] chunk-start state pieces
  uint16_t* WT = nullptr;            // bf16 [nc][hv][8 col tiles][2 token slabs][64 lanes][8] chunk write W pieces
  size_t bytes = 0;
};

// Records a message for gdn_last_error() on this thread and returns `st`.
gdn_status report(gdn_status st, const char* fmt, ...);

// gdn_prefill with every argument validated before any HIP call. With `scratch` set, the workspace is
// the device buffer scratch() returns (looked up after validation) and `workspace_bytes` its capacity;
// otherwise `workspace` as given.
using ScratchFn = gdn_status (*)(hipStream_t s, void** workspace);
gdn_status prefill_with(const gdn_cfg* cfg, int32_t n_seqs, int64_t total_tokens, const int32_t* cu_seqlens,
                        const int32_t* cu_seqlens_host, const void* q, const void* k, const void* v, int64_t ld_q,
                        int64_t ld_k, int64_t ld_v, const float* alpha, const float* beta, const void* gate,
                        const float* conv_w, const float* norm_w, const float* state_in, float* state_out,
                        const void* conv_in, void* conv_out, void* out, void* workspace, size_t workspace_bytes,
                        ScratchFn scratch, void* hip_stream);

// True when the chunked MFMA path serves this problem.
inline bool use_chunked(const Problem& p) { return p.bf16 && p.dk == 128 && p.dv == 128; }

// Carves `base` (may be null to only size it) into the regions the chosen path needs.
Workspace plan_workspace(const Problem& p, void* base);

// Conv-cache tail: conv_out[n][r] = the raw q/k/v input at position end - 3 + r of sequence n, or
// the matching conv_in row when the sequence is shorter than 3 (zeros without conv_in). Work item
// (n, channel group of 16 bytes); every thread reads its three rows before writing any, so
// conv_out may alias conv_in. Run by the standalone tail kernel or by extra output-kernel blocks.
struct ConvTailArgs {
  const int32_t* cu;
  int n_seqs;
  int64_t T, C, qk_ch;
  const void *q, *k, *v;
  int64_t ld_q, ld_k, ld_v;
  const void* conv_in;
  void* conv_out;
  int cblk;  // blocks of 256 channel groups per sequence
};
inline ConvTailArgs conv_tail_args(const Problem& p, const int32_t* cu, const void* q, const void* k,
                                   const void* v, int64_t ld_q, int64_t ld_k, int64_t ld_v,
                                   const void* conv_in, void* conv_out) {
  const int vec = p.bf16 ? 8 : 4;
  const int64_t groups = (p.C + vec - 1) / vec;
  return ConvTailArgs{cu, p.n_seqs, p.T, p.C, int64_t(p.hk) * p.dk, q, k, v, ld_q, ld_k, ld_v,
                      conv_in, conv_out, int((groups + 255) / 256)};
}

// ---- launchers (each returns hipGetLastError() after its launches) ----
hipError_t launch_conv(const Problem& p, const int32_t* cu, const void* q, const void* k, const void* v,
                       int64_t ld_q, int64_t ld_k, int64_t ld_v, const float* conv_w,
                       const void* conv_in, const Workspace& ws, bool work_bf16, hipStream_t s);
// (the conv launch also builds the chunk table when the chunked path runs)
hipError_t launch_conv_tail(const Problem& p, const int32_t* cu, const void* q, const void* k,
                            const void* v, int64_t ld_q, int64_t ld_k, int64_t ld_v,
                            const void* conv_in, void* conv_out, hipStream_t s);
hipError_t launch_sequential(const Problem& p, const int32_t* cu, const Workspace& ws,
                             const float* alpha, const float* beta, const void* gate,
                             const float* norm_w, const float* state_in, float* state_out, void* out,
                             hipStream_t s);
hipError_t launch_wy(const Problem& p, const Workspace& ws, const float* alpha, const float* beta,
                     hipStream_t s);
hipError_t launch_state(const Problem& p, const Workspace& ws, const float* state_in, float* state_out,
                        hipStream_t s);
// also writes the conv tail when tail.conv_out is set
hipError_t launch_output(const Problem& p, const Workspace& ws, const void* gate, const float* norm_w,
                         void* out, const ConvTailArgs& tail, hipStream_t s);
hipError_t launch_decode(const Problem& p, int batch, const void* q, const void* k, const void* v,
                         int64_t ld_q, int64_t ld_k, int64_t ld_v, const float* alpha, const float* beta,
                         const void* gate, const float* conv_w, const float* norm_w, void* conv_state,
                         float* state, void* out, hipStream_t s);

// Log of a speculative verify (multi-token decode), read back by the commit: per sequence b and
// draft token t, the normalised key of each QK head, the error e of each value head, alpha and
// beta, and (with the conv) the raw inputs. Regions are 256-byte aligned, in this order.
constexpr int kMaxDrafts = 8;   // draft tokens per verify
constexpr int kMaxMtpRatio = 4; // value heads per QK head on the verify path
struct MtpLog {
  float* kh = nullptr;   // fp32 [B][K][HK][d_k]
  float* e = nullptr;    // fp32 [B][K][HV][d_v]
  float* ab = nullptr;   // fp32 [B][K][HV][2]
  void* raw = nullptr;   // io   [B][K][C]
  size_t bytes = 0;
};
MtpLog plan_mtp_log(const Problem& p, int batch, int n_tok, void* base);
hipError_t launch_verify(const Problem& p, int batch, int n_tok, const void* q, const void* k, const void* v,
                         int64_t ld_q, int64_t ld_k, int64_t ld_v, const float* alpha, const float* beta,
                         const void* gate, const float* conv_w, const float* norm_w, const void* conv_state,
                         const float* state, void* out, const MtpLog& log, hipStream_t s);
hipError_t launch_commit(const Problem& p, int batch, int n_tok, const int32_t* n_accept, const MtpLog& log,
                         void* conv_state, float* state, hipStream_t s);

// Projections around the mixer (bf16), one MFMA GEMM kernel: the input projection over the stacked
// weights [W_qkv | W_z | W_ab] (q | k | v and gate logits in bf16, alpha and beta from the fp32 gate
// pre-activations), and the output projection.
hipError_t launch_in_proj(const Problem& p, int H, int64_t T, const void* x, int64_t ld_x, const void* w_qkv,
                          const void* w_z, const void* w_ab, const float* a_log, const float* dt_bias, void* qkv,
                          void* z, float* alpha, float* beta, hipStream_t s);
hipError_t launch_out_proj(const Problem& p, int H, int64_t T, const void* o, const void* w_out, void* y,
                           hipStream_t s);

}  // namespace gdn
