// Host-side declarations of the recurrence backward and the QSA indexer, shared by their kernel files
// and the C-ABI layer (kept apart from the mixer's own declarations).
#pragma once

#include "gdn_internal.h"
#include "qsa.h"

namespace gdn {

// The mixer's steps before the recurrence, backwards (conv + SiLU + L2), fp32, d = 128.
struct BwdMixArgs {
  const int32_t* cu;
  int n_seqs;
  int64_t T;
  int hk, hv;
  int64_t C;                    // 2 hk 128 + hv 128 conv channels
  float l2_eps;
  const float *q, *k, *v;       // raw inputs [T][HK][128], [T][HK][128], [T][HV][128]
  const float* conv_w;          // [C][4]
  const float* conv_in;         // [N][3][C] or null
  const float *dqa, *dka, *dva; // dL/d(normalised q, k; activated v): [T][HK][128], [T][HK][128], [T][HV][128]
  float* du;                    // workspace [T][C]: dL/d(conv output)
  float *dq, *dk, *dv;          // out: dL/d(raw inputs)
  float* dconv_w;               // out [C][4]
  float* dw_part;               // workspace [<= kConvWeightParts][C][4]: per-token-window-group parts of dconv_w
  float* dconv_in;              // out [N][3][C] or null
};
// Parts of the two weight derivatives that the backward sums in a fixed order: the norm gain's
// (kNormGateParts x 128 floats of workspace) and the conv weights' (up to kConvWeightParts x C x 4).
constexpr int kNormGateParts = 1024;
constexpr int kConvWeightParts = 256;
// dw_part: workspace of kNormGateParts x 128 floats
hipError_t launch_norm_gate_bwd(int64_t rows, const float* y, const float* z, const float* dout, const float* norm_w,
                                float eps, float* dy, float* dz, float* dnorm_w, float* dw_part, hipStream_t s);
hipError_t launch_mixer_input_bwd(const BwdMixArgs& m, hipStream_t s);

// ---- chunked backward of the recurrence (fp32, d = 128, 64-token chunks) ----
// Per-item arrays: item = chunk c x value head h (index c * hv + h), tiles zero-padded to 64 rows.
struct CBwdArgs {
  const int32_t* cu;
  int n_seqs;
  int64_t T;
  int hk, hv, R;
  float scale;
  int64_t nc_max;                 // chunk slots: T / 64 + n_seqs
  int32_t* seq_off;               // [n_seqs + 1] first chunk of each sequence
  int4* tab;                      // [nc_max] (start token, length, sequence, 0)
  const float *q, *k, *v;         // [T][HK][128], [T][HK][128], [T][HV][128] (normalised q, k; v)
  const float *alpha, *beta;      // [T][HV]
  const float *s0, *dy, *dsf;     // initial states (or null), dL/dy [T][HV][128], dL/dS_final (or null)
  float* y;                       // raw y [T][HV][128] written by the forward pass (or null)
  float *dv, *dalpha, *dbeta, *ds0;
  float *dqh, *dkh;               // [T][HV][128] per value head, before the group sums
  float *Qi, *Ki, *Vi, *dYi, *bV, *bgK, *U, *Wk, *W, *dW, *dKt, *X, *dWk, *dQ, *dK, *dbV, *dbgK;  // [I][64][128]
  float *Kt, *gQ;                 // [I][64][128]: diag(exp(G_C - G)) K, diag(exp(G)) Q
  float *KtT, *WkT;               // [I][128][64]: Kt^T, Wk^T
  float *S, *dS;                  // [I][128][128]: state at the chunk start; dL/d(state after the chunk)
  float *KK, *QK, *Am, *Pm, *Tm, *dP, *M1, *dT, *dA;  // [I][64][64]
  float *G, *bt;                  // [I][64]
  float* dgc;                     // [I][8][4] per-(slice, wave) parts of <S, dS'>
};
size_t cbwd_workspace_bytes(int n_seqs, int64_t T, int hv);
void cbwd_plan(CBwdArgs& a, void* base);  // sets nc_max and every workspace region
// forward: chunk table, gather, WY, forward chunk pass (writes y when a.y); backward: the rest, then
// dq, dk as sums over each QK head's value heads
hipError_t launch_cbwd(const CBwdArgs& a, bool forward, bool backward, float* dq, float* dk, hipStream_t s);

// ---- QSA compressed indexer ----
constexpr int kSelSeg = 16384;  // scores per select workgroup (1024 threads x 16)

struct QsaShape {
  int topk;
  int half;          // rope_dims / 2
  double theta[64];  // rotation angle per position of pair i: rope_base^(-i / half)
  float eps;         // RMSNorm eps
  bool bf16;         // io dtype
  int64_t cap;       // compressed-key cache capacity per sequence, in blocks
};

struct QsaWs {
  float* qr;          // [rows][4][128] rotated queries
  int2* info;         // [rows] (sequence, position)
  float* scores;      // [rows][ld_s]
  int64_t ld_s;
  uint32_t* cand_key; // [rows][segmax][topk] segment candidates (rows longer than one segment)
  int32_t* cand_idx;
  int segmax;
};

// Decode append: each row's new key k [rows][ld_k], the RMSNorm gain, and the caches it updates.
struct QsaAppend {
  const void* k;
  int64_t ld_k;
  const float* norm_w;
  void* pending;
  void* kbar;
};

QsaWs plan_qsa_ws(const QsaShape& sh, int64_t rows, void* base, size_t* bytes);
hipError_t launch_qsa_compress(const QsaShape& sh, int n_seqs, int64_t T, const int32_t* cu, const void* k,
                               int64_t ld_k, const float* norm_w, void* kbar, void* pending, hipStream_t s);
hipError_t launch_qsa_rows(const QsaShape& sh, const QsaWs& ws, int64_t row0, int64_t rows, const int32_t* cu,
                           int n_seqs, const int32_t* n_tok, const QsaAppend& ap, const void* q, int64_t ld_q,
                           const void* kbar, int32_t* sel, int32_t* n_sel, int32_t* tail, hipStream_t s);

}  // namespace gdn
