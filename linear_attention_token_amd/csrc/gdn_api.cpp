// C ABI of the GDN mixer: host-side validation, workspace layout and kernel dispatch.
// Every check runs before any HIP call, so a rejected call enqueues nothing and touches no output.
#include <stdarg.h>
#include <stdio.h>
#include <math.h>
#include <algorithm>
#include <string.h>

#include "ext_internal.h"

namespace gdn {

static thread_local char g_last_error[512] = "";
static thread_local void* const* g_stage_events = nullptr;

// Records the stage event `i` on `s` when stage timing is on.
static hipError_t mark(int i, hipStream_t s) {
  if (!g_stage_events) return hipSuccess;
  return hipEventRecord(static_cast<hipEvent_t>(g_stage_events[i]), s);
}

static gdn_status fail(gdn_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

gdn_status report(gdn_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static bool supported_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// Validates the configuration and fills the fields of Problem that depend on it alone.
static gdn_status check_cfg(const gdn_cfg* cfg, Problem& p) {
  if (!cfg) return fail(GDN_E_NULL, "cfg is NULL");
  if (cfg->io_dtype != GDN_BF16 && cfg->io_dtype != GDN_F32)
    return fail(GDN_E_DTYPE, "io_dtype %d is neither GDN_BF16 nor GDN_F32", cfg->io_dtype);
  if (cfg->n_qk_heads <= 0 || cfg->n_v_heads <= 0)
    return fail(GDN_E_SHAPE, "head counts must be positive (HK=%d, HV=%d)", cfg->n_qk_heads, cfg->n_v_heads);
  if (cfg->n_v_heads % cfg->n_qk_heads != 0)
    return fail(GDN_E_SHAPE, "HV=%d is not a multiple of HK=%d", cfg->n_v_heads, cfg->n_qk_heads);
  if (cfg->d_k <= 0 || cfg->d_v <= 0)
    return fail(GDN_E_SHAPE, "head dims must be positive (d_k=%d, d_v=%d)", cfg->d_k, cfg->d_v);
  if (!supported_dim(cfg->d_k) || !supported_dim(cfg->d_v))
    return fail(GDN_E_UNSUPPORTED, "head dims must be 16, 32, 64 or 128 (d_k=%d, d_v=%d)", cfg->d_k, cfg->d_v);
  if (cfg->conv_width != 4) return fail(GDN_E_UNSUPPORTED, "conv_width %d: only 4 is implemented", cfg->conv_width);
  if (cfg->flags & ~uint32_t(GDN_ALL)) return fail(GDN_E_VALUE, "unknown flag bits 0x%x", cfg->flags);
  if (!(cfg->l2_eps >= 0.f) || !(cfg->norm_eps >= 0.f))
    return fail(GDN_E_VALUE, "eps values must be >= 0 (l2_eps=%g, norm_eps=%g)", cfg->l2_eps, cfg->norm_eps);
  if (cfg->norm_head_stride != 0 && cfg->norm_head_stride != cfg->d_v)
    return fail(GDN_E_SHAPE, "norm_head_stride must be 0 or d_v (%d)", cfg->norm_head_stride);
  p.hk = cfg->n_qk_heads;
  p.hv = cfg->n_v_heads;
  p.dk = cfg->d_k;
  p.dv = cfg->d_v;
  p.C = 2 * int64_t(p.hk) * p.dk + int64_t(p.hv) * p.dv;
  p.flags = cfg->flags;
  p.scale = cfg->scale;
  p.l2_eps = cfg->l2_eps;
  p.norm_eps = cfg->norm_eps;
  p.norm_stride = cfg->norm_head_stride;
  p.bf16 = cfg->io_dtype == GDN_BF16;
  return GDN_OK;
}

Workspace plan_workspace(const Problem& p, void* base) {
  Workspace ws;
  char* b = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* r = b ? static_cast<void*>(b + off) : nullptr;
    off += align256(bytes);
    return r;
  };
  const bool chunked = use_chunked(p);
  const size_t wt = chunked ? 2 : 4;  // bytes of the normalised q/k/v work arrays
  ws.seq_chunk_off = static_cast<int32_t*>(take(sizeof(int32_t) * size_t(p.n_seqs + 1)));
  ws.chunk_tab = static_cast<int4*>(take(sizeof(int4) * size_t(chunked ? p.nc_max : 0)));
  ws.qhat = take(wt * size_t(p.T) * p.hk * p.dk);
  ws.khat = take(wt * size_t(p.T) * p.hk * p.dk);
  ws.vhat = take(wt * size_t(p.T) * p.hv * p.dv);
  if (chunked) {
    const size_t nc = size_t(p.nc_max);
    ws.G = static_cast<float*>(take(sizeof(float) * nc * p.hv * 64));
    ws.Wk = static_cast<uint16_t*>(take(2 * nc * p.hv * 64 * 128));
    ws.U = static_cast<uint16_t*>(take(2 * nc * p.hv * 64 * 128));
    ws.KT = static_cast<uint16_t*>(take(2 * nc * p.hk * 128 * 64));
    ws.ST = static_cast<uint16_t*>(take(2 * nc * p.hv * 128 * 128));
    ws.WT = static_cast<uint16_t*>(take(2 * nc * p.hv * 128 * 64));
  }
  ws.bytes = off;
  return ws;
}

static hipError_t run(hipError_t e, const char* what) {
  if (e != hipSuccess) fail(GDN_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return e;
}

// QSA indexer configuration and cache capacity -> QsaShape.
static gdn_status check_qsa(const qsa_cfg* cfg, int64_t cap, QsaShape& sh) {
  if (!cfg) return fail(GDN_E_NULL, "cfg is NULL");
  if (cfg->io_dtype != GDN_BF16 && cfg->io_dtype != GDN_F32)
    return fail(GDN_E_DTYPE, "io_dtype %d is neither GDN_BF16 nor GDN_F32", cfg->io_dtype);
  if (cfg->n_heads != 4 || cfg->d != 128 || cfg->block != 4)
    return fail(GDN_E_UNSUPPORTED, "only 4 heads of dim 128 and blocks of 4 are implemented (%d, %d, %d)",
                cfg->n_heads, cfg->d, cfg->block);
  if (cfg->topk < 1 || cfg->topk > 4096) return fail(GDN_E_UNSUPPORTED, "topk %d is outside 1..4096", cfg->topk);
  if (cfg->rope_dims < 0 || cfg->rope_dims > 128 || cfg->rope_dims % 16)
    return fail(GDN_E_UNSUPPORTED, "rope_dims %d must be a multiple of 16 in 0..128", cfg->rope_dims);
  if (!(cfg->rope_base > 0.f) || !(cfg->rope_base < 3.4e38f))
    return fail(GDN_E_VALUE, "rope_base %g must be positive and finite", cfg->rope_base);
  if (!(cfg->norm_eps >= 0.f)) return fail(GDN_E_VALUE, "norm_eps %g must be >= 0", cfg->norm_eps);
  if (cap < 0) return fail(GDN_E_SHAPE, "negative cap_blocks %lld", (long long)cap);
  const int64_t cap_max = int64_t(kSelSeg) * (kSelSeg / cfg->topk);
  if (cap > cap_max)
    return fail(GDN_E_UNSUPPORTED, "cap_blocks %lld exceeds %lld, the most a query can select from at topk %d",
                (long long)cap, (long long)cap_max, cfg->topk);
  sh.topk = cfg->topk;
  sh.half = cfg->rope_dims / 2;
  for (int i = 0; i < 64; ++i) sh.theta[i] = i < sh.half ? pow(double(cfg->rope_base), -double(i) / sh.half) : 0.0;
  sh.eps = cfg->norm_eps;
  sh.bf16 = cfg->io_dtype == GDN_BF16;
  sh.cap = cap;
  return GDN_OK;
}

}  // namespace gdn

using namespace gdn;

extern "C" {

void gdn_cfg_default(gdn_cfg* cfg) {
  if (!cfg) return;
  cfg->n_qk_heads = 16;
  cfg->n_v_heads = 48;
  cfg->d_k = 128;
  cfg->d_v = 128;
  cfg->conv_width = 4;
  cfg->io_dtype = GDN_BF16;
  cfg->flags = GDN_ALL;
  cfg->scale = 1.0f;
  cfg->l2_eps = 1e-6f;
  cfg->norm_eps = 1e-6f;
  cfg->norm_head_stride = 0;
}

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

gdn_status gdn_set_stage_events(void* const* events, int32_t n_events) {
  g_last_error[0] = 0;
  if (events && n_events != GDN_N_STAGES + 1)
    return fail(GDN_E_SHAPE, "need %d events, got %d", GDN_N_STAGES + 1, n_events);
  g_stage_events = events;
  return GDN_OK;
}

const char* gdn_last_error(void) { return g_last_error; }

const char* gdn_status_string(gdn_status st) {
  switch (st) {
    case GDN_OK: return "GDN_OK";
    case GDN_E_NULL: return "GDN_E_NULL: a required pointer is NULL";
    case GDN_E_SHAPE: return "GDN_E_SHAPE: inconsistent shapes or sequence lengths";
    case GDN_E_DTYPE: return "GDN_E_DTYPE: unknown io dtype";
    case GDN_E_ALIGN: return "GDN_E_ALIGN: pointer or stride not 16-byte aligned";
    case GDN_E_WORKSPACE: return "GDN_E_WORKSPACE: workspace missing or too small";
    case GDN_E_UNSUPPORTED: return "GDN_E_UNSUPPORTED: configuration not implemented";
    case GDN_E_HIP: return "GDN_E_HIP: HIP runtime error";
    case GDN_E_VALUE: return "GDN_E_VALUE: scalar parameter out of range";
  }
  return "unknown gdn_status";
}

// Every launch's grid, counted in work-items, must fit in 32 bits.
static bool launches_fit(const Problem& p) {
  const int64_t lim = (int64_t(1) << 32) - 1;
  const int vec = p.bf16 ? 8 : 4;
  const int64_t strips = (p.T + kConvStrip - 1) / kConvStrip;
  const int64_t cblk = ((p.C + vec - 1) / vec + 255) / 256;
  const int64_t conv = (int64_t(kXcds) * ((strips + kXcds - 1) / kXcds) * cblk + 1) * 256;
  const int64_t chunks = (xcd_blocks(p.nc_max * p.hk, p.hv / p.hk) + int64_t(p.n_seqs) * cblk) * 256;
  return conv <= lim && chunks <= lim;
}

gdn_status gdn_prefill_workspace(const gdn_cfg* cfg, int32_t n_seqs, int64_t total_tokens, size_t* bytes) {
  g_last_error[0] = 0;
  if (!bytes) return fail(GDN_E_NULL, "bytes is NULL");
  Problem p{};
  gdn_status st = check_cfg(cfg, p);
  if (st != GDN_OK) return st;
  if (n_seqs < 0 || total_tokens < 0) return fail(GDN_E_SHAPE, "negative n_seqs or total_tokens");
  if (n_seqs == 0 && total_tokens > 0) return fail(GDN_E_SHAPE, "tokens without sequences");
  if (total_tokens > (int64_t(1) << 31) - 1) return fail(GDN_E_UNSUPPORTED, "total_tokens >= 2^31");
  p.n_seqs = n_seqs;
  p.T = total_tokens;
  p.nc_max = total_tokens / kChunk + n_seqs;
  if (!launches_fit(p)) return fail(GDN_E_UNSUPPORTED, "too many tokens for one call; split the batch");
  *bytes = plan_workspace(p, nullptr).bytes;
  return GDN_OK;
}

}  // extern "C"

// gdn_prefill and gdn_prefill_static: every argument is validated first; with `scratch` set, the
// workspace comes from it (after validation, so a rejected call makes no HIP call at all) and
// `workspace_bytes` is the capacity it provides.
gdn_status gdn::prefill_with(const gdn_cfg* cfg, int32_t n_seqs, int64_t total_tokens,
                             const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                             const void* q, const void* k, const void* v,
                             int64_t ld_q, int64_t ld_k, int64_t ld_v,
                             const float* alpha, const float* beta, const void* gate,
                             const float* conv_w, const float* norm_w,
                             const float* state_in, float* state_out,
                             const void* conv_in, void* conv_out,
                             void* out, void* workspace, size_t workspace_bytes, ScratchFn scratch,
                             void* hip_stream) {
  g_last_error[0] = 0;
  Problem p{};
  gdn_status st = check_cfg(cfg, p);
  if (st != GDN_OK) return st;
  if (n_seqs < 0 || total_tokens < 0) return fail(GDN_E_SHAPE, "negative n_seqs (%d) or total_tokens (%lld)", n_seqs, (long long)total_tokens);
  if (n_seqs == 0 && total_tokens > 0) return fail(GDN_E_SHAPE, "tokens without sequences");
  if (total_tokens > (int64_t(1) << 31) - 1) return fail(GDN_E_UNSUPPORTED, "total_tokens >= 2^31");
  p.n_seqs = n_seqs;
  p.T = total_tokens;
  p.nc_max = total_tokens / kChunk + n_seqs;
  if (!launches_fit(p)) return fail(GDN_E_UNSUPPORTED, "too many tokens for one call; split the batch");
  const uint32_t f = p.flags;
  // required pointers
  if (n_seqs > 0 && !cu_seqlens) return fail(GDN_E_NULL, "cu_seqlens is NULL");
  if (total_tokens > 0) {
    if (!q || !k || !v) return fail(GDN_E_NULL, "q, k and v are required");
    if (!alpha || !beta) return fail(GDN_E_NULL, "alpha and beta are required");
    if (!out) return fail(GDN_E_NULL, "out is required");
    if ((f & GDN_GATE) && !gate) return fail(GDN_E_NULL, "gate is required with GDN_GATE");
    if ((f & GDN_NORM) && !norm_w) return fail(GDN_E_NULL, "norm_w is required with GDN_NORM");
  }
  if ((f & GDN_CONV) && !conv_w && (total_tokens > 0)) return fail(GDN_E_NULL, "conv_w is required with GDN_CONV");
  // strides and alignment
  const int64_t elem = p.bf16 ? 2 : 4;
  const int64_t qrow = int64_t(p.hk) * p.dk, vrow = int64_t(p.hv) * p.dv;
  if (ld_q < qrow || ld_k < qrow || ld_v < vrow)
    return fail(GDN_E_SHAPE, "row strides too small (ld_q=%lld, ld_k=%lld >= %lld; ld_v=%lld >= %lld)",
                (long long)ld_q, (long long)ld_k, (long long)qrow, (long long)ld_v, (long long)vrow);
  if ((ld_q * elem) % 16 || (ld_k * elem) % 16 || (ld_v * elem) % 16)
    return fail(GDN_E_ALIGN, "row strides must be multiples of 16 bytes");
  const void* ptrs[] = {q, k, v, gate, conv_w, norm_w, state_in, state_out, conv_in, conv_out, out};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(GDN_E_ALIGN, "a tensor pointer is not 16-byte aligned");
  if (!aligned4(alpha) || !aligned4(beta) || !aligned4(cu_seqlens))
    return fail(GDN_E_ALIGN, "alpha, beta and cu_seqlens must be 4-byte aligned");
  if (conv_in && conv_out && conv_in != conv_out) {
    // partial overlap is not allowed; exact aliasing is
    const char* a0 = static_cast<const char*>(conv_in);
    const char* b0 = static_cast<const char*>(conv_out);
    const size_t nb = size_t(n_seqs) * 3 * size_t(p.C) * size_t(elem);
    if (a0 < b0 + nb && b0 < a0 + nb) return fail(GDN_E_VALUE, "conv_in and conv_out overlap without being equal");
  }
  if (cu_seqlens_host) {
    if (cu_seqlens_host[0] != 0) return fail(GDN_E_SHAPE, "cu_seqlens[0] = %d, expected 0", cu_seqlens_host[0]);
    for (int i = 0; i < n_seqs; ++i)
      if (cu_seqlens_host[i + 1] < cu_seqlens_host[i]) return fail(GDN_E_SHAPE, "cu_seqlens decreases at %d", i);
    if (int64_t(cu_seqlens_host[n_seqs]) != total_tokens)
      return fail(GDN_E_SHAPE, "cu_seqlens[%d] = %d, expected total_tokens = %lld", n_seqs, cu_seqlens_host[n_seqs], (long long)total_tokens);
  }
  const Workspace need = plan_workspace(p, nullptr);
  if (scratch) {
    if (workspace_bytes < need.bytes)
      return fail(GDN_E_WORKSPACE, "this prefill needs %zu bytes of workspace; the static scratch holds %zu "
                  "(split the batch or call gdn_prefill with a workspace)", need.bytes, workspace_bytes);
  } else {
    if (!workspace && need.bytes > 0) return fail(GDN_E_WORKSPACE, "workspace is NULL (%zu bytes needed)", need.bytes);
    if (workspace_bytes < need.bytes) return fail(GDN_E_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need.bytes);
    if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u)) return fail(GDN_E_ALIGN, "workspace must be 256-byte aligned");
  }
  if (n_seqs == 0) return GDN_OK;

  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (scratch) {
    const gdn_status sst = scratch(s, &workspace);
    if (sst != GDN_OK) return sst;
  }
  const Workspace ws = plan_workspace(p, workspace);
  const bool chunked = use_chunked(p);
  const bool any = total_tokens > 0;
#define GDN_STEP(i, expr, what) \
  if (run(mark(i, s), "event record") != hipSuccess || (run((expr), what) != hipSuccess)) return GDN_E_HIP;
  GDN_STEP(0, hipSuccess, "")  // the chunk table is built inside the conv launch
  GDN_STEP(1, launch_conv(p, cu_seqlens, q, k, v, ld_q, ld_k, ld_v, conv_w, conv_in, ws, chunked, s), "conv")
  if (chunked) {
    // the output kernel's extra blocks write the conv tail (conv_in is no longer read by then)
    const ConvTailArgs tail = conv_tail_args(p, cu_seqlens, q, k, v, ld_q, ld_k, ld_v, conv_in, conv_out);
    GDN_STEP(2, any ? launch_wy(p, ws, alpha, beta, s) : hipSuccess, "wy")
    GDN_STEP(3, launch_state(p, ws, state_in, state_out, s), "state")
    GDN_STEP(4, any ? launch_output(p, ws, gate, norm_w, out, tail, s) : hipSuccess, "output")
    GDN_STEP(5, (conv_out && !any) ? launch_conv_tail(p, cu_seqlens, q, k, v, ld_q, ld_k, ld_v, conv_in, conv_out, s)
                                   : hipSuccess, "conv tail")
  } else {
    GDN_STEP(2, launch_sequential(p, cu_seqlens, ws, alpha, beta, gate, norm_w, state_in, state_out, out, s),
             "sequential")
    GDN_STEP(3, hipSuccess, "")
    GDN_STEP(4, hipSuccess, "")
    GDN_STEP(5, conv_out ? launch_conv_tail(p, cu_seqlens, q, k, v, ld_q, ld_k, ld_v, conv_in, conv_out, s)
                         : hipSuccess, "conv tail")
  }
  if (run(mark(GDN_N_STAGES, s), "event record") != hipSuccess) return GDN_E_HIP;
#undef GDN_STEP
  return GDN_OK;
}

extern "C" {

gdn_status gdn_prefill(const gdn_cfg* cfg, int32_t n_seqs, int64_t total_tokens,
                       const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                       const void* q, const void* k, const void* v,
                       int64_t ld_q, int64_t ld_k, int64_t ld_v,
                       const float* alpha, const float* beta, const void* gate,
                       const float* conv_w, const float* norm_w,
                       const float* state_in, float* state_out,
                       const void* conv_in, void* conv_out,
                       void* out, void* workspace, size_t workspace_bytes, void* hip_stream) {
  return prefill_with(cfg, n_seqs, total_tokens, cu_seqlens, cu_seqlens_host, q, k, v, ld_q, ld_k, ld_v, alpha,
                      beta, gate, conv_w, norm_w, state_in, state_out, conv_in, conv_out, out, workspace,
                      workspace_bytes, nullptr, hip_stream);
}

gdn_status gdn_decode_step(const gdn_cfg* cfg, int32_t batch,
                           const void* q, const void* k, const void* v,
                           int64_t ld_q, int64_t ld_k, int64_t ld_v,
                           const float* alpha, const float* beta, const void* gate,
                           const float* conv_w, const float* norm_w,
                           void* conv_state, float* state, void* out, void* hip_stream) {
  g_last_error[0] = 0;
  Problem p{};
  gdn_status st = check_cfg(cfg, p);
  if (st != GDN_OK) return st;
  if (batch < 0) return fail(GDN_E_SHAPE, "negative batch %d", batch);
  p.n_seqs = batch;
  p.T = batch;
  p.nc_max = 0;
  const uint32_t f = p.flags;
  if (batch > 0) {
    if (!q || !k || !v) return fail(GDN_E_NULL, "q, k and v are required");
    if (!alpha || !beta) return fail(GDN_E_NULL, "alpha and beta are required");
    if (!state) return fail(GDN_E_NULL, "state is required");
    if (!out) return fail(GDN_E_NULL, "out is required");
    if ((f & GDN_GATE) && !gate) return fail(GDN_E_NULL, "gate is required with GDN_GATE");
    if ((f & GDN_NORM) && !norm_w) return fail(GDN_E_NULL, "norm_w is required with GDN_NORM");
    if ((f & GDN_CONV) && (!conv_w || !conv_state)) return fail(GDN_E_NULL, "conv_w and conv_state are required with GDN_CONV");
  }
  const int64_t elem = p.bf16 ? 2 : 4;
  const int64_t qrow = int64_t(p.hk) * p.dk, vrow = int64_t(p.hv) * p.dv;
  if (ld_q < qrow || ld_k < qrow || ld_v < vrow) return fail(GDN_E_SHAPE, "row strides too small");
  if ((ld_q * elem) % 16 || (ld_k * elem) % 16 || (ld_v * elem) % 16)
    return fail(GDN_E_ALIGN, "row strides must be multiples of 16 bytes");
  const void* ptrs[] = {q, k, v, gate, conv_w, norm_w, conv_state, state, out};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(GDN_E_ALIGN, "a tensor pointer is not 16-byte aligned");
  if (!aligned4(alpha) || !aligned4(beta)) return fail(GDN_E_ALIGN, "alpha and beta must be 4-byte aligned");
  if (p.hv / p.hk > 64) return fail(GDN_E_UNSUPPORTED, "HV/HK = %d > 64", p.hv / p.hk);
  if (int64_t(batch) * p.hk * 768 > int64_t(UINT32_MAX))
    return fail(GDN_E_UNSUPPORTED, "batch x QK heads = %lld is too large for one launch", (long long)batch * p.hk);
  if (batch == 0) return GDN_OK;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (run(launch_decode(p, batch, q, k, v, ld_q, ld_k, ld_v, alpha, beta, gate, conv_w, norm_w, conv_state,
                        state, out, s), "decode") != hipSuccess)
    return GDN_E_HIP;
  return GDN_OK;
}

// Shape checks shared by the speculative-decoding entry points; fills p for B sequences of K drafts.
static gdn_status check_mtp(const gdn_cfg* cfg, int32_t batch, int32_t n_tok, Problem& p) {
  gdn_status st = check_cfg(cfg, p);
  if (st != GDN_OK) return st;
  if (batch < 0) return fail(GDN_E_SHAPE, "negative batch %d", batch);
  if (n_tok < 1) return fail(GDN_E_SHAPE, "n_tok = %d: a draft has at least one token", n_tok);
  if (n_tok > kMaxDrafts) return fail(GDN_E_UNSUPPORTED, "n_tok = %d > %d draft tokens", n_tok, kMaxDrafts);
  if (p.dk != 128 || p.dv != 128)
    return fail(GDN_E_UNSUPPORTED, "speculative decoding is implemented for d_k = d_v = 128 (got %d, %d)", p.dk, p.dv);
  if (p.hv / p.hk > kMaxMtpRatio)
    return fail(GDN_E_UNSUPPORTED, "speculative decoding needs HV/HK <= %d (got %d)", kMaxMtpRatio, p.hv / p.hk);
  if (int64_t(batch) * p.hk * 256 > int64_t(UINT32_MAX))
    return fail(GDN_E_UNSUPPORTED, "batch x QK heads = %lld is too large for one launch", (long long)batch * p.hk);
  p.n_seqs = batch;
  p.T = int64_t(batch) * n_tok;
  p.nc_max = 0;
  return GDN_OK;
}

gdn_status gdn_verify_log_bytes(const gdn_cfg* cfg, int32_t batch, int32_t n_tok, size_t* bytes) {
  g_last_error[0] = 0;
  if (!bytes) return fail(GDN_E_NULL, "bytes is NULL");
  Problem p{};
  const gdn_status st = check_mtp(cfg, batch, n_tok, p);
  if (st != GDN_OK) return st;
  *bytes = plan_mtp_log(p, batch, n_tok, nullptr).bytes;
  return GDN_OK;
}

gdn_status gdn_verify(const gdn_cfg* cfg, int32_t batch, int32_t n_tok,
                      const void* q, const void* k, const void* v,
                      int64_t ld_q, int64_t ld_k, int64_t ld_v,
                      const float* alpha, const float* beta, const void* gate,
                      const float* conv_w, const float* norm_w,
                      const void* conv_state, const float* state, void* out,
                      void* log, size_t log_bytes, void* hip_stream) {
  g_last_error[0] = 0;
  Problem p{};
  gdn_status st = check_mtp(cfg, batch, n_tok, p);
  if (st != GDN_OK) return st;
  const uint32_t f = p.flags;
  if (batch > 0) {
    if (!q || !k || !v) return fail(GDN_E_NULL, "q, k and v are required");
    if (!alpha || !beta) return fail(GDN_E_NULL, "alpha and beta are required");
    if (!state) return fail(GDN_E_NULL, "state is required");
    if (!out) return fail(GDN_E_NULL, "out is required");
    if (!log) return fail(GDN_E_NULL, "log is required");
    if ((f & GDN_GATE) && !gate) return fail(GDN_E_NULL, "gate is required with GDN_GATE");
    if ((f & GDN_NORM) && !norm_w) return fail(GDN_E_NULL, "norm_w is required with GDN_NORM");
    if ((f & GDN_CONV) && (!conv_w || !conv_state)) return fail(GDN_E_NULL, "conv_w and conv_state are required with GDN_CONV");
  }
  const int64_t elem = p.bf16 ? 2 : 4;
  const int64_t qrow = int64_t(p.hk) * p.dk, vrow = int64_t(p.hv) * p.dv;
  if (ld_q < qrow || ld_k < qrow || ld_v < vrow) return fail(GDN_E_SHAPE, "row strides too small");
  if ((ld_q * elem) % 16 || (ld_k * elem) % 16 || (ld_v * elem) % 16)
    return fail(GDN_E_ALIGN, "row strides must be multiples of 16 bytes");
  const void* ptrs[] = {q, k, v, gate, conv_w, norm_w, conv_state, state, out};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(GDN_E_ALIGN, "a tensor pointer is not 16-byte aligned");
  if (!aligned4(alpha) || !aligned4(beta)) return fail(GDN_E_ALIGN, "alpha and beta must be 4-byte aligned");
  if (log && (reinterpret_cast<uintptr_t>(log) & 255u)) return fail(GDN_E_ALIGN, "log must be 256-byte aligned");
  const MtpLog need = plan_mtp_log(p, batch, n_tok, nullptr);
  if (batch > 0 && log_bytes < need.bytes) return fail(GDN_E_WORKSPACE, "log has %zu bytes, %zu needed", log_bytes, need.bytes);
  if (batch == 0) return GDN_OK;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (run(launch_verify(p, batch, n_tok, q, k, v, ld_q, ld_k, ld_v, alpha, beta, gate, conv_w, norm_w, conv_state,
                        state, out, plan_mtp_log(p, batch, n_tok, log), s), "verify") != hipSuccess)
    return GDN_E_HIP;
  return GDN_OK;
}

gdn_status gdn_commit(const gdn_cfg* cfg, int32_t batch, int32_t n_tok, const int32_t* n_accept,
                      const void* log, size_t log_bytes, void* conv_state, float* state, void* hip_stream) {
  g_last_error[0] = 0;
  Problem p{};
  gdn_status st = check_mtp(cfg, batch, n_tok, p);
  if (st != GDN_OK) return st;
  if (batch > 0) {
    if (!n_accept) return fail(GDN_E_NULL, "n_accept is required");
    if (!log) return fail(GDN_E_NULL, "log is required");
    if (!state) return fail(GDN_E_NULL, "state is required");
    if ((p.flags & GDN_CONV) && !conv_state) return fail(GDN_E_NULL, "conv_state is required with GDN_CONV");
  }
  if ((state && !aligned16(state)) || (conv_state && !aligned16(conv_state)))
    return fail(GDN_E_ALIGN, "a tensor pointer is not 16-byte aligned");
  if (!aligned4(n_accept)) return fail(GDN_E_ALIGN, "n_accept must be 4-byte aligned");
  if (log && (reinterpret_cast<uintptr_t>(log) & 255u)) return fail(GDN_E_ALIGN, "log must be 256-byte aligned");
  const MtpLog need = plan_mtp_log(p, batch, n_tok, nullptr);
  if (batch > 0 && log_bytes < need.bytes) return fail(GDN_E_WORKSPACE, "log has %zu bytes, %zu needed", log_bytes, need.bytes);
  if (batch == 0) return GDN_OK;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  MtpLog L = plan_mtp_log(p, batch, n_tok, const_cast<void*>(log));
  if (run(launch_commit(p, batch, n_tok, n_accept, L, conv_state, state, s), "commit") != hipSuccess)
    return GDN_E_HIP;
  return GDN_OK;
}

gdn_status gdn_proj_workspace(size_t* bytes) {
  g_last_error[0] = 0;
  if (!bytes) return fail(GDN_E_NULL, "bytes is NULL");
  *bytes = 0;  // the projection kernels need no scratch
  return GDN_OK;
}

static gdn_status check_proj(const gdn_cfg* cfg, int32_t hidden, int64_t T, Problem& p) {
  gdn_status st = check_cfg(cfg, p);
  if (st != GDN_OK) return st;
  if (!p.bf16) return fail(GDN_E_UNSUPPORTED, "the projections are implemented for bf16 io");
  if (hidden <= 0 || hidden % 32) return fail(GDN_E_SHAPE, "hidden = %d must be a positive multiple of 32", hidden);
  if (T < 0 || T > int64_t(INT32_MAX) * 8) return fail(GDN_E_SHAPE, "T = %lld out of range", (long long)T);
  if (p.hv > 3072) return fail(GDN_E_UNSUPPORTED, "HV = %d > 3072 for the projection kernel", p.hv);
  return GDN_OK;
}

gdn_status gdn_in_proj(const gdn_cfg* cfg, int32_t hidden, int64_t T, const void* x, int64_t ld_x,
                       const void* w_qkv, const void* w_z, const void* w_ab, const float* a_log, const float* dt_bias,
                       void* qkv, void* z, float* alpha, float* beta, void* workspace, size_t workspace_bytes,
                       void* hip_stream) {
  g_last_error[0] = 0;
  Problem p{};
  gdn_status st = check_proj(cfg, hidden, T, p);
  if (st != GDN_OK) return st;
  if (T > 0) {
    if (!x || !w_qkv || !w_z || !w_ab || !a_log || !dt_bias) return fail(GDN_E_NULL, "x, the weights and the gate vectors are required");
    if (!qkv || !z || !alpha || !beta) return fail(GDN_E_NULL, "qkv, z, alpha and beta are required");
  }
  (void)workspace;
  (void)workspace_bytes;
  if (ld_x < hidden || ld_x % 8) return fail(GDN_E_SHAPE, "ld_x = %lld must be >= hidden and a multiple of 8", (long long)ld_x);
  const void* ptrs[] = {x, w_qkv, w_z, w_ab, qkv, z};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(GDN_E_ALIGN, "a tensor pointer is not 16-byte aligned");
  if (!aligned4(a_log) || !aligned4(dt_bias) || !aligned4(alpha) || !aligned4(beta))
    return fail(GDN_E_ALIGN, "a_log, dt_bias, alpha and beta must be 4-byte aligned");
  if (T == 0) return GDN_OK;
  if (run(launch_in_proj(p, hidden, T, x, ld_x, w_qkv, w_z, w_ab, a_log, dt_bias, qkv, z, alpha, beta,
                         static_cast<hipStream_t>(hip_stream)), "input projection") != hipSuccess)
    return GDN_E_HIP;
  return GDN_OK;
}

gdn_status gdn_out_proj(const gdn_cfg* cfg, int32_t hidden, int64_t T, const void* o, const void* w_out, void* y,
                        void* workspace, size_t workspace_bytes, void* hip_stream) {
  g_last_error[0] = 0;
  Problem p{};
  gdn_status st = check_proj(cfg, hidden, T, p);
  if (st != GDN_OK) return st;
  if (T > 0) {
    if (!o || !w_out || !y) return fail(GDN_E_NULL, "o, w_out and y are required");
  }
  (void)workspace;
  (void)workspace_bytes;
  const void* ptrs[] = {o, w_out, y};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(GDN_E_ALIGN, "a tensor pointer is not 16-byte aligned");
  if (T == 0) return GDN_OK;
  if (run(launch_out_proj(p, hidden, T, o, w_out, y, static_cast<hipStream_t>(hip_stream)), "output projection") !=
      hipSuccess)
    return GDN_E_HIP;
  return GDN_OK;
}

// Workspace of the recurrence backward: per (64-token chunk, value head) item the chunk's tiles, its WY
// factors and derivatives, the state at its start and the derivative of the state after it.
static size_t bwd_workspace_bytes(int32_t n_seqs, int64_t T, int hv) { return cbwd_workspace_bytes(n_seqs, T, hv); }

static gdn_status check_bwd(const gdn_cfg* cfg, int32_t n_seqs, int64_t T, Problem& p) {
  gdn_status st = check_cfg(cfg, p);
  if (st != GDN_OK) return st;
  if (cfg->io_dtype != GDN_F32) return fail(GDN_E_UNSUPPORTED, "the recurrence backward takes fp32 tensors");
  if (p.dk != 128 || p.dv != 128) return fail(GDN_E_UNSUPPORTED, "the recurrence backward needs d_k = d_v = 128");
  if (n_seqs < 0 || T < 0) return fail(GDN_E_SHAPE, "negative n_seqs or total_tokens");
  if (n_seqs == 0 && T != 0) return fail(GDN_E_SHAPE, "tokens without sequences");
  if (T >= (int64_t(1) << 31)) return fail(GDN_E_UNSUPPORTED, "total_tokens must stay below 2^31");
  // launch bounds: 8 blocks per (sequence, value head) chain, one block per (chunk, value head) item
  if (int64_t(n_seqs) * p.hv > (int64_t(1) << 27)) return fail(GDN_E_UNSUPPORTED, "too many (sequence, head) chains");
  if ((T / 64 + n_seqs) * int64_t(p.hv) >= (int64_t(1) << 31))
    return fail(GDN_E_UNSUPPORTED, "too many (64-token chunk, value head) items");
  return GDN_OK;
}

gdn_status gdn_recurrence_backward_workspace(const gdn_cfg* cfg, int32_t n_seqs, int64_t total_tokens, size_t* bytes) {
  g_last_error[0] = 0;
  Problem p{};
  gdn_status st = check_bwd(cfg, n_seqs, total_tokens, p);
  if (st != GDN_OK) return st;
  if (!bytes) return fail(GDN_E_NULL, "bytes is NULL");
  *bytes = bwd_workspace_bytes(n_seqs, total_tokens, p.hv);
  return GDN_OK;
}

gdn_status gdn_recurrence_backward(const gdn_cfg* cfg, int32_t n_seqs, int64_t total_tokens,
                                   const int32_t* cu_seqlens, const float* q, const float* k, const float* v,
                                   const float* alpha, const float* beta, const float* state_in, const float* dy,
                                   const float* dstate_out, float* dq, float* dk, float* dv, float* dalpha,
                                   float* dbeta, float* dstate_in, void* workspace, size_t workspace_bytes,
                                   void* hip_stream) {
  g_last_error[0] = 0;
  Problem p{};
  gdn_status st = check_bwd(cfg, n_seqs, total_tokens, p);
  if (st != GDN_OK) return st;
  if (n_seqs == 0) return GDN_OK;
  if (!cu_seqlens) return fail(GDN_E_NULL, "cu_seqlens is required");
  if (total_tokens > 0 && (!q || !k || !v || !alpha || !beta || !dy || !dq || !dk || !dv || !dalpha || !dbeta))
    return fail(GDN_E_NULL, "q, k, v, alpha, beta, dy and the gradient outputs are required");
  const void* ptrs[] = {q, k, v, state_in, dy, dstate_out, dq, dk, dv, dstate_in};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(GDN_E_ALIGN, "a tensor pointer is not 16-byte aligned");
  if (!aligned4(alpha) || !aligned4(beta) || !aligned4(dalpha) || !aligned4(dbeta) || !aligned4(cu_seqlens))
    return fail(GDN_E_ALIGN, "alpha, beta, dalpha, dbeta and cu_seqlens must be 4-byte aligned");
  const size_t need = bwd_workspace_bytes(n_seqs, total_tokens, p.hv);
  if (!workspace || workspace_bytes < need)
    return fail(GDN_E_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace ? workspace_bytes : 0, need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(GDN_E_ALIGN, "workspace must be 256-byte aligned");
  CBwdArgs a{};
  a.cu = cu_seqlens;
  a.n_seqs = n_seqs;
  a.T = total_tokens;
  a.hk = p.hk;
  a.hv = p.hv;
  a.R = p.hv / p.hk;
  a.scale = p.scale;
  a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.s0 = state_in; a.dy = dy; a.dsf = dstate_out;
  a.dv = dv; a.dalpha = dalpha; a.dbeta = dbeta; a.ds0 = dstate_in;
  cbwd_plan(a, workspace);
  if (run(launch_cbwd(a, true, true, dq, dk, static_cast<hipStream_t>(hip_stream)), "recurrence backward") != hipSuccess)
    return GDN_E_HIP;
  return GDN_OK;
}

// Workspace of the whole-mixer backward: the forward's normalised q/k/v, the recurrence backward's
// regions, y and dy, the recurrence-input derivatives and the conv-output derivatives.
static size_t mixer_bwd_workspace_bytes(const Problem& p, int64_t T) {
  const size_t th = size_t(T) * p.hv, tk = size_t(T) * p.hk;
  return align256(plan_workspace(p, nullptr).bytes) + bwd_workspace_bytes(p.n_seqs, T, p.hv) +
         2 * align256(sizeof(float) * th * 128) + 2 * align256(sizeof(float) * tk * 128) +
         align256(sizeof(float) * th * 128) + align256(sizeof(float) * size_t(T) * size_t(p.C)) +
         align256(sizeof(float) * kNormGateParts * 128) +
         align256(sizeof(float) * size_t(std::min<int64_t>((T + 15) / 16, kConvWeightParts)) * p.C * 4);
}

static gdn_status check_mixer_bwd(const gdn_cfg* cfg, int32_t n_seqs, int64_t T, Problem& p) {
  gdn_status st = check_bwd(cfg, n_seqs, T, p);
  if (st != GDN_OK) return st;
  if (cfg->flags != GDN_ALL) return fail(GDN_E_UNSUPPORTED, "gdn_backward needs every step on (flags = GDN_ALL)");
  if (cfg->norm_head_stride != 0) return fail(GDN_E_UNSUPPORTED, "gdn_backward needs one shared norm gain");
  p.n_seqs = n_seqs;
  p.T = T;
  p.nc_max = T / kChunk + n_seqs;
  return GDN_OK;
}

gdn_status gdn_backward_workspace(const gdn_cfg* cfg, int32_t n_seqs, int64_t total_tokens, size_t* bytes) {
  g_last_error[0] = 0;
  Problem p{};
  gdn_status st = check_mixer_bwd(cfg, n_seqs, total_tokens, p);
  if (st != GDN_OK) return st;
  if (!bytes) return fail(GDN_E_NULL, "bytes is NULL");
  *bytes = mixer_bwd_workspace_bytes(p, total_tokens);
  return GDN_OK;
}

gdn_status gdn_backward(const gdn_cfg* cfg, int32_t n_seqs, int64_t total_tokens, const int32_t* cu_seqlens,
                        const float* q, const float* k, const float* v, const float* alpha, const float* beta,
                        const float* gate, const float* conv_w, const float* norm_w, const float* state_in,
                        const float* conv_in, const float* dout, const float* dstate_out, float* dq, float* dk,
                        float* dv, float* dalpha, float* dbeta, float* dgate, float* dconv_w, float* dnorm_w,
                        float* dstate_in, float* dconv_in, void* workspace, size_t workspace_bytes,
                        void* hip_stream) {
  g_last_error[0] = 0;
  Problem p{};
  gdn_status st = check_mixer_bwd(cfg, n_seqs, total_tokens, p);
  if (st != GDN_OK) return st;
  if (n_seqs == 0) return GDN_OK;
  if (!cu_seqlens || !conv_w || !norm_w || !dconv_w || !dnorm_w)
    return fail(GDN_E_NULL, "cu_seqlens, conv_w, norm_w, dconv_w and dnorm_w are required");
  if (total_tokens > 0 && (!q || !k || !v || !alpha || !beta || !gate || !dout || !dq || !dk || !dv || !dalpha ||
                           !dbeta || !dgate))
    return fail(GDN_E_NULL, "the inputs, dout and the gradient outputs are required");
  const void* ptrs[] = {q, k, v, gate, conv_w, norm_w, state_in, conv_in, dout, dstate_out,
                        dq, dk, dv, dgate, dconv_w, dnorm_w, dstate_in, dconv_in};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(GDN_E_ALIGN, "a tensor pointer is not 16-byte aligned");
  if (!aligned4(alpha) || !aligned4(beta) || !aligned4(dalpha) || !aligned4(dbeta) || !aligned4(cu_seqlens))
    return fail(GDN_E_ALIGN, "alpha, beta, dalpha, dbeta and cu_seqlens must be 4-byte aligned");
  const size_t need = mixer_bwd_workspace_bytes(p, total_tokens);
  if (!workspace || workspace_bytes < need)
    return fail(GDN_E_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace ? workspace_bytes : 0, need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(GDN_E_ALIGN, "workspace must be 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  char* w = static_cast<char*>(workspace);
  const Workspace fws = plan_workspace(p, w);
  w += align256(fws.bytes);
  const size_t th = size_t(total_tokens) * p.hv, tk = size_t(total_tokens) * p.hk;
  CBwdArgs a{};
  a.cu = cu_seqlens;
  a.n_seqs = n_seqs;
  a.T = total_tokens;
  a.hk = p.hk;
  a.hv = p.hv;
  a.R = p.hv / p.hk;
  a.scale = p.scale;
  a.q = static_cast<const float*>(fws.qhat);
  a.k = static_cast<const float*>(fws.khat);
  a.v = static_cast<const float*>(fws.vhat);
  a.alpha = alpha; a.beta = beta; a.s0 = state_in; a.dsf = dstate_out; a.ds0 = dstate_in;
  a.dalpha = dalpha; a.dbeta = dbeta;
  cbwd_plan(a, w);
  w += align256(bwd_workspace_bytes(n_seqs, total_tokens, p.hv));
  float* y = reinterpret_cast<float*>(w);
  w += align256(sizeof(float) * th * 128);
  float* dy = reinterpret_cast<float*>(w);
  w += align256(sizeof(float) * th * 128);
  float* dqa = reinterpret_cast<float*>(w);
  w += align256(sizeof(float) * tk * 128);
  float* dka = reinterpret_cast<float*>(w);
  w += align256(sizeof(float) * tk * 128);
  float* dva = reinterpret_cast<float*>(w);
  w += align256(sizeof(float) * th * 128);
  float* du = reinterpret_cast<float*>(w);
  w += align256(sizeof(float) * size_t(total_tokens) * size_t(p.C));
  float* dw_part = reinterpret_cast<float*>(w);
  w += align256(sizeof(float) * kNormGateParts * 128);
  float* dcw_part = reinterpret_cast<float*>(w);
  a.y = y;
  a.dy = dy;
  a.dv = dva;
  const int64_t qrow = int64_t(p.hk) * 128, vrow = int64_t(p.hv) * 128;
  BwdMixArgs m{};
  m.cu = cu_seqlens;
  m.n_seqs = n_seqs;
  m.T = total_tokens;
  m.hk = p.hk;
  m.hv = p.hv;
  m.C = p.C;
  m.l2_eps = p.l2_eps;
  m.q = q; m.k = k; m.v = v; m.conv_w = conv_w; m.conv_in = conv_in;
  m.dqa = dqa; m.dka = dka; m.dva = dva; m.du = du;
  m.dq = dq; m.dk = dk; m.dv = dv; m.dconv_w = dconv_w; m.dconv_in = dconv_in; m.dw_part = dcw_part;
  if (run(launch_conv(p, cu_seqlens, q, k, v, qrow, qrow, vrow, conv_w, conv_in, fws, false, s), "backward conv") != hipSuccess ||
      run(launch_cbwd(a, true, false, dqa, dka, s), "backward forward pass") != hipSuccess ||
      run(launch_norm_gate_bwd(int64_t(th), y, gate, dout, norm_w, p.norm_eps, dy, dgate, dnorm_w, dw_part, s),
          "backward norm and gate") != hipSuccess ||
      run(launch_cbwd(a, false, true, dqa, dka, s), "backward recurrence") != hipSuccess ||
      run(launch_mixer_input_bwd(m, s), "backward conv, SiLU, L2") != hipSuccess)
    return GDN_E_HIP;
  return GDN_OK;
}

void qsa_cfg_default(qsa_cfg* cfg) {
  if (!cfg) return;
  cfg->n_heads = 4;
  cfg->d = 128;
  cfg->block = 4;
  cfg->topk = 512;
  cfg->rope_dims = 64;
  cfg->io_dtype = GDN_BF16;
  cfg->rope_base = 10000.f;
  cfg->norm_eps = 1e-6f;
}

gdn_status qsa_compress(const qsa_cfg* cfg, int32_t n_seqs, int64_t total_tokens, const int32_t* cu_seqlens,
                        const int32_t* cu_seqlens_host, const void* k, int64_t ld_k, const float* norm_w, void* kbar,
                        int64_t cap_blocks, void* pending, void* hip_stream) {
  g_last_error[0] = 0;
  QsaShape sh{};
  gdn_status st = check_qsa(cfg, cap_blocks, sh);
  if (st != GDN_OK) return st;
  if (n_seqs < 0 || total_tokens < 0) return fail(GDN_E_SHAPE, "negative n_seqs or total_tokens");
  if (n_seqs > 65535) return fail(GDN_E_UNSUPPORTED, "n_seqs %d > 65535", n_seqs);
  if (total_tokens >= (int64_t(1) << 31)) return fail(GDN_E_UNSUPPORTED, "total_tokens must stay below 2^31");
  if (n_seqs == 0 && total_tokens != 0) return fail(GDN_E_SHAPE, "tokens without sequences");
  if (n_seqs == 0) return GDN_OK;
  if (!cu_seqlens) return fail(GDN_E_NULL, "cu_seqlens is required");
  if (total_tokens > 0 && (!k || !norm_w || (!kbar && cap_blocks > 0)))
    return fail(GDN_E_NULL, "k, norm_w and kbar are required");
  const int64_t elem = sh.bf16 ? 2 : 4;
  if (ld_k < 128) return fail(GDN_E_SHAPE, "ld_k %lld < 128", (long long)ld_k);
  if ((ld_k * elem) % 16) return fail(GDN_E_ALIGN, "ld_k must be a multiple of 16 bytes");
  const void* ptrs[] = {k, norm_w, kbar, pending};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(GDN_E_ALIGN, "a tensor pointer is not 16-byte aligned");
  if (!aligned4(cu_seqlens)) return fail(GDN_E_ALIGN, "cu_seqlens must be 4-byte aligned");
  if (cu_seqlens_host) {
    if (cu_seqlens_host[0] != 0 || cu_seqlens_host[n_seqs] != total_tokens)
      return fail(GDN_E_SHAPE, "cu_seqlens must start at 0 and end at total_tokens");
    for (int i = 0; i < n_seqs; ++i) {
      const int64_t len = int64_t(cu_seqlens_host[i + 1]) - cu_seqlens_host[i];
      if (len < 0) return fail(GDN_E_SHAPE, "cu_seqlens decreases at %d", i);
      if (len / 4 > cap_blocks)
        return fail(GDN_E_SHAPE, "sequence %d has %lld blocks, cap_blocks is %lld", i, (long long)(len / 4),
                    (long long)cap_blocks);
    }
  }
  if (total_tokens == 0) return GDN_OK;
  if (run(launch_qsa_compress(sh, n_seqs, total_tokens, cu_seqlens, k, ld_k, norm_w, kbar, pending,
                              static_cast<hipStream_t>(hip_stream)), "qsa compress") != hipSuccess)
    return GDN_E_HIP;
  return GDN_OK;
}

gdn_status qsa_workspace(const qsa_cfg* cfg, int64_t rows, int64_t cap_blocks, size_t* bytes) {
  g_last_error[0] = 0;
  QsaShape sh{};
  gdn_status st = check_qsa(cfg, cap_blocks, sh);
  if (st != GDN_OK) return st;
  if (!bytes) return fail(GDN_E_NULL, "bytes is NULL");
  if (rows < 0) return fail(GDN_E_SHAPE, "negative rows");
  plan_qsa_ws(sh, rows, nullptr, bytes);
  return GDN_OK;
}

// Checks shared by qsa_select and qsa_decode.
static gdn_status check_qsa_rows(const QsaShape& sh, int64_t rows, const void* q, int64_t ld_q, const void* kbar,
                                 const int32_t* sel, const int32_t* n_sel, const int32_t* tail) {
  if (rows > 0 && (!q || !sel || !n_sel || !tail || (!kbar && sh.cap > 0)))
    return fail(GDN_E_NULL, "q, kbar, sel, n_sel and tail are required");
  const int64_t elem = sh.bf16 ? 2 : 4;
  if (ld_q < 512) return fail(GDN_E_SHAPE, "ld_q %lld < 4 * 128", (long long)ld_q);
  if ((ld_q * elem) % 16) return fail(GDN_E_ALIGN, "ld_q must be a multiple of 16 bytes");
  if ((q && !aligned16(q)) || (kbar && !aligned16(kbar)))
    return fail(GDN_E_ALIGN, "q and kbar must be 16-byte aligned");
  if (!aligned4(sel) || !aligned4(n_sel) || !aligned4(tail))
    return fail(GDN_E_ALIGN, "sel, n_sel and tail must be 4-byte aligned");
  return GDN_OK;
}

gdn_status qsa_select(const qsa_cfg* cfg, int32_t n_seqs, int64_t total_tokens, const int32_t* cu_seqlens,
                      const void* q, int64_t ld_q, const void* kbar, int64_t cap_blocks, int32_t* sel,
                      int32_t* n_sel, int32_t* tail, void* workspace, size_t workspace_bytes, void* hip_stream) {
  g_last_error[0] = 0;
  QsaShape sh{};
  gdn_status st = check_qsa(cfg, cap_blocks, sh);
  if (st != GDN_OK) return st;
  if (n_seqs < 0 || total_tokens < 0) return fail(GDN_E_SHAPE, "negative n_seqs or total_tokens");
  if (total_tokens >= (int64_t(1) << 31)) return fail(GDN_E_UNSUPPORTED, "total_tokens must stay below 2^31");
  if (n_seqs == 0 && total_tokens != 0) return fail(GDN_E_SHAPE, "tokens without sequences");
  if (total_tokens > 0 && !cu_seqlens) return fail(GDN_E_NULL, "cu_seqlens is required");
  if (cu_seqlens && !aligned4(cu_seqlens)) return fail(GDN_E_ALIGN, "cu_seqlens must be 4-byte aligned");
  st = check_qsa_rows(sh, total_tokens, q, ld_q, kbar, sel, n_sel, tail);
  if (st != GDN_OK) return st;
  if (total_tokens == 0) return GDN_OK;
  size_t one = 0;
  plan_qsa_ws(sh, 1, nullptr, &one);
  if (!workspace || workspace_bytes < one)
    return fail(GDN_E_WORKSPACE, "workspace has %zu bytes, at least %zu needed", workspace ? workspace_bytes : 0, one);
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(GDN_E_ALIGN, "workspace must be 256-byte aligned");
  int64_t lo = 1, hi = total_tokens;  // most rows whose workspace fits
  while (lo < hi) {
    const int64_t mid = hi - (hi - lo) / 2;
    size_t b = 0;
    plan_qsa_ws(sh, mid, nullptr, &b);
    if (b <= workspace_bytes) lo = mid; else hi = mid - 1;
  }
  size_t used = 0;
  const QsaWs ws = plan_qsa_ws(sh, lo, workspace, &used);
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  for (int64_t r0 = 0; r0 < total_tokens; r0 += lo)
    if (run(launch_qsa_rows(sh, ws, r0, std::min(lo, total_tokens - r0), cu_seqlens, n_seqs, nullptr, QsaAppend{},
                            q, ld_q, kbar, sel, n_sel, tail, s), "qsa select") != hipSuccess)
      return GDN_E_HIP;
  return GDN_OK;
}

gdn_status qsa_decode(const qsa_cfg* cfg, int32_t batch, const int32_t* n_tok, const void* q, int64_t ld_q,
                      const void* k, int64_t ld_k, const float* norm_w, void* pending, void* kbar,
                      int64_t cap_blocks, int32_t* sel, int32_t* n_sel, int32_t* tail, void* workspace,
                      size_t workspace_bytes, void* hip_stream) {
  g_last_error[0] = 0;
  QsaShape sh{};
  gdn_status st = check_qsa(cfg, cap_blocks, sh);
  if (st != GDN_OK) return st;
  if (batch < 0) return fail(GDN_E_SHAPE, "negative batch %d", batch);
  st = check_qsa_rows(sh, batch, q, ld_q, kbar, sel, n_sel, tail);
  if (st != GDN_OK) return st;
  if (batch > 0 && (!n_tok || !k || !norm_w || !pending)) return fail(GDN_E_NULL, "n_tok, k, norm_w and pending are required");
  const int64_t elem = sh.bf16 ? 2 : 4;
  if (ld_k < 128) return fail(GDN_E_SHAPE, "ld_k %lld < 128", (long long)ld_k);
  if ((ld_k * elem) % 16) return fail(GDN_E_ALIGN, "ld_k must be a multiple of 16 bytes");
  if ((k && !aligned16(k)) || (norm_w && !aligned16(norm_w)) || (pending && !aligned16(pending)))
    return fail(GDN_E_ALIGN, "k, norm_w and pending must be 16-byte aligned");
  if (!aligned4(n_tok)) return fail(GDN_E_ALIGN, "n_tok must be 4-byte aligned");
  if (batch == 0) return GDN_OK;
  size_t need = 0;
  plan_qsa_ws(sh, batch, nullptr, &need);
  if (!workspace || workspace_bytes < need)
    return fail(GDN_E_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace ? workspace_bytes : 0, need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(GDN_E_ALIGN, "workspace must be 256-byte aligned");
  const QsaWs ws = plan_qsa_ws(sh, batch, workspace, &need);
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const QsaAppend ap{k, ld_k, norm_w, pending, kbar};
  if (run(launch_qsa_rows(sh, ws, 0, batch, nullptr, batch, n_tok, ap, q, ld_q, kbar, sel, n_sel, tail, s),
          "qsa decode") != hipSuccess)
    return GDN_E_HIP;
  return GDN_OK;
}

}  // extern "C"
