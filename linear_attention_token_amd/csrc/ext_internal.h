// Host-side declarations of the recurrence backward and the QSA indexer, shared by their kernel files
// and the C-ABI layer (kept apart from the mixer's own declarations).
#pragma once

#include "gdn_internal.h"
#include "qsa.h"

namespace gdn {

// ---- recurrence backward (fp32, d = 128) ----
// Each (sequence, value head) chain runs as 8 workgroups of 16 value columns.
constexpr int kBwdForward = 1, kBwdReverse = 2, kBwdWriteY = 4;  // BwdArgs::mode bits
struct BwdArgs {
  int mode;                      // forward pass (keep states), reverse pass, y output in the forward
  float* y;                      // [T][HV][128] raw recurrence output (kBwdWriteY)
  const int32_t* cu;
  int n_seqs;
  int64_t T;
  int hk, hv;
  float scale;
  const float *q, *k, *v;        // [T][HK][128], [T][HK][128], [T][HV][128]
  const float *alpha, *beta;     // [T][HV]
  const float* s0;               // [N][HV][128][128] or null (zeros)
  const float* dy;               // [T][HV][128]
  const float* dsf;              // [N][HV][128][128] or null (zeros)
  float *dqv, *dkv;              // workspace [T][HV][8 slices][128]: per-slice partials
  float *dalpha_part, *dbeta_part;  // workspace [T][HV][8]
  float* dv;                     // [T][HV][128] out
  float* ds0;                    // [N][HV][128][128] or null
  float* states;                 // workspace [T][HV][8 slices][2 rows][256 threads][4]: every state
  float* errs;                   // workspace [T][HV][128]
};
hipError_t launch_bwd(const BwdArgs& a, float* dq, float* dk, float* dalpha, float* dbeta, hipStream_t s);

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
  float* dw_part;               // workspace [ceil(T / 64)][C][4]: per-token-block parts of dconv_w
  float* dconv_in;              // out [N][3][C] or null
};
// dw_part: workspace of ceil(rows / 64) x 128 floats
hipError_t launch_norm_gate_bwd(int64_t rows, const float* y, const float* z, const float* dout, const float* norm_w,
                                float eps, float* dy, float* dz, float* dnorm_w, float* dw_part, hipStream_t s);
hipError_t launch_mixer_input_bwd(const BwdMixArgs& m, hipStream_t s);

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
