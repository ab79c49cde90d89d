// capi.cpp - the extern "C" boundary declared in include/verify_attn.h.
//
// The pages' C-ABI shim takes device pointers and a stream, computes the grid itself,
// returns error codes ("The Glue That Connects", sections "What the Edit Actually Does" and
// "Assumptions Embedded in the Integration"; "The Glue That Makes Kernels Run", section "The
// Subject Message"), consumes the serving framework's native buffers directly and does no
// host-side preprocessing or synchronisation ("The Final Solder Joint", sections "Why the
// C-ABI Edit Matters" and "Assumptions and Design Decisions"). The pages' earlier version
// allocated its workspace with a raw device malloc on first use, which broke graph capture
// ("The Final Solder Joint", section "The Capture-Safety Constraint"); here the workspace is
// bound once at create and run() only enqueues kernels.
#include <algorithm>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <new>
#include <string>

#include "../../include/verify_attn.h"
#include "va_internal.h"


namespace {

thread_local std::string g_last_error;

hipEvent_t const kNoEvents[3] = {nullptr, nullptr, nullptr};

va_status fail(va_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

va_status ok() {
  g_last_error.clear();
  return VA_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device (the MFMA partial kernel runs one workgroup on each);
// 256, MI355X's count, when no device answers.
int32_t compute_units() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  return n;
}

// Bytes per partial-output dim: the MFMA kernel writes int16 codes with a scale per 128 dims,
// the fp32-input kernel fp32.
int part_elem_bytes(int32_t kernel) { return kernel == VA_KERNEL_MFMA ? 2 : 4; }

struct Derived {
  int32_t kernel, splits, rows_per_block, row_tiles, grid;
  int64_t part_rows;
  size_t bytes;
};

}  // namespace

struct verify_attn_ctx {
  verify_attn_config cfg;
  Derived d;          // kernel, split count, grid, workspace sizing
  void *ws_base;
  bool ws_owned;
  va::Workspace ws;
  hipEvent_t ev[3];  // profiling events (all NULL when off)
};

namespace {

// Checks a config and fills the derived launch parameters. Returns VA_OK or an error.
va_status derive(const verify_attn_config *c, Derived *d) {
  if (!c) return fail(VA_ERR_NULL, "config is NULL");
  if (c->num_heads < 1 || c->num_heads > 4096)
    return fail(VA_ERR_INVALID, "num_heads %d out of range [1, 4096]", c->num_heads);
  if (c->latent_dim != va::kLatent || c->rope_dim != va::kRope)
    return fail(VA_ERR_UNSUPPORTED, "latent_dim/rope_dim must be 512/64 (got %d/%d)",
                c->latent_dim, c->rope_dim);
  if (c->in_dtype != VA_BF16 && c->in_dtype != VA_FP32)
    return fail(VA_ERR_INVALID, "in_dtype %d unknown", c->in_dtype);
  if (c->out_dtype != VA_BF16 && c->out_dtype != VA_FP32)
    return fail(VA_ERR_INVALID, "out_dtype %d unknown", c->out_dtype);
  if (c->max_batch < 1 || c->max_q_per_req < 1 || c->max_q_tokens < 1)
    return fail(VA_ERR_INVALID, "max_batch, max_q_per_req and max_q_tokens must be >= 1");
  if (c->max_q_per_req > 65536 || c->max_q_tokens > (int64_t(1) << 26))
    return fail(VA_ERR_INVALID, "max_q_per_req or max_q_tokens too large");
  if (c->num_splits < 0 || c->num_splits > va::kMaxSplits)
    return fail(VA_ERR_INVALID, "num_splits %d out of range [0, %d]", c->num_splits,
                va::kMaxSplits);
  int32_t k = c->kernel;
  if (k == VA_KERNEL_AUTO) k = c->in_dtype == VA_BF16 ? VA_KERNEL_MFMA : VA_KERNEL_SIMPLE;
  if (k != VA_KERNEL_SIMPLE && k != VA_KERNEL_MFMA)
    return fail(VA_ERR_INVALID, "kernel %d unknown", c->kernel);
  if (k == VA_KERNEL_MFMA && c->in_dtype != VA_BF16)
    return fail(VA_ERR_UNSUPPORTED, "the MFMA kernel takes bf16 inputs only");

  const int64_t rows_cap = c->max_q_tokens * c->num_heads;
  int32_t s = c->num_splits;
  d->grid = 0;
  if (k == VA_KERNEL_SIMPLE) {
    d->rows_per_block = va::kSimpleHeadsPerBlock;
    d->row_tiles =
        int32_t(int64_t(c->max_q_per_req) * ceil_div(c->num_heads, va::kSimpleHeadsPerBlock));
    const int64_t blocks_per_split = int64_t(c->max_batch) * d->row_tiles;
    if (s == 0) {
      // enough workgroups to cover the compute units several times
      s = int32_t(ceil_div(2048, blocks_per_split));
      if (s < 1) s = 1;
      if (s > 64) s = 64;
    }
    if (blocks_per_split * s > 0x7fffffffLL)
      return fail(VA_ERR_INVALID, "launch grid too large");
    d->part_rows = int64_t(s) * rows_cap;
  } else {
    d->rows_per_block = va::kMfmaRowsPerBlock;
    d->row_tiles = int32_t(ceil_div(int64_t(c->max_q_per_req) * c->num_heads,
                                    va::kMfmaRowsPerBlock));
    // With s == 0 the work list is balanced on the device so that it holds at most `grid`
    // items (one per compute unit, a multiple of 8, at most kMaxSplits so that no row has more
    // splits than the combine takes) of kMfmaRowsPerBlock rows each when the requests have
    // fewer row tiles than that (else one item per row tile), which bounds the partial rows by
    // kMfmaRowsPerBlock * grid + rows_cap.
    static_assert(va::kMaxSplits % 8 == 0, "the grid is a multiple of 8");
    d->grid = int32_t(std::min<int64_t>(ceil_div(compute_units(), 8) * 8, va::kMaxSplits));
    d->part_rows = s == 0 ? int64_t(va::kMfmaRowsPerBlock) * d->grid + rows_cap
                          : int64_t(s) * rows_cap;
  }
  size_t off[7];
  d->bytes = va::workspace_layout(d->part_rows, rows_cap, part_elem_bytes(k), off);
  d->kernel = k;
  d->splits = s;
  return VA_OK;
}

// The workspace regions of a config with derived parameters `d`, laid over `base`.
va::Workspace bind_workspace(const verify_attn_config &cfg, const Derived &d, void *base) {
  size_t off[7];
  const int64_t rows_cap = cfg.max_q_tokens * cfg.num_heads;
  va::workspace_layout(d.part_rows, rows_cap, part_elem_bytes(d.kernel), off);
  char *b = static_cast<char *>(base);
  va::Workspace ws;
  ws.status = reinterpret_cast<uint32_t *>(b + off[0]);
  ws.zero_row = reinterpret_cast<const uint16_t *>(b + off[0] + va::kZeroRowOffset);
  ws.part_o = b + off[1];
  ws.part_scale = reinterpret_cast<float *>(b + off[2]);
  ws.part_i16 = part_elem_bytes(d.kernel) == 2;
  ws.part_lse = reinterpret_cast<float *>(b + off[3]);
  ws.part_max = reinterpret_cast<float *>(b + off[4]);
  ws.part_arg = reinterpret_cast<int32_t *>(b + off[5]);
  ws.row_info = reinterpret_cast<va::RowInfo *>(b + off[6]);
  ws.part_rows = d.part_rows;
  ws.rows_cap = rows_cap;
  ws.splits = d.splits;
  return ws;
}

// Host checks and the two launches of one verify step (both entry points). `ev` holds the
// optional profiling events (NULLs when off).
va_status launch_step(const verify_attn_config &cfg, const Derived &d, const va::Workspace &ws,
                      hipEvent_t const ev[3], const void *q, const void *kv_buffer,
                      int64_t num_slots, const int64_t *kv_indices, int64_t num_kv_indices,
                      const int32_t *kv_indptr, const int64_t *qo_indptr,
                      const uint8_t *custom_mask, int64_t mask_len, const int64_t *mask_indptr,
                      const int64_t *out_cache_loc, int32_t bs, int64_t num_tokens,
                      float sm_scale, void *out, float *out_lse, int32_t *out_argmax,
                      void *stream) {
  if (bs < 0 || bs > cfg.max_batch)
    return fail(VA_ERR_INVALID, "bs %d out of range [0, %d]", bs, cfg.max_batch);
  if (num_tokens < 0 || num_tokens > cfg.max_q_tokens)
    return fail(VA_ERR_INVALID, "num_tokens %lld out of range [0, %lld]",
                (long long)num_tokens, (long long)cfg.max_q_tokens);
  if (num_slots < 1) return fail(VA_ERR_INVALID, "num_slots must be >= 1");
  if (num_kv_indices < 0 || mask_len < 0)
    return fail(VA_ERR_INVALID, "num_kv_indices and mask_len must be >= 0");
  if (!(sm_scale > 0.f) || !isfinite(sm_scale))
    return fail(VA_ERR_INVALID, "sm_scale must be positive and finite");
  if (num_tokens == 0) return ok();
  if (!out) return fail(VA_ERR_NULL, "out is NULL");
  if (bs > 0) {
    if (!q || !kv_buffer || !kv_indptr || !qo_indptr || !mask_indptr)
      return fail(VA_ERR_NULL, "a required input pointer is NULL");
    if (num_kv_indices > 0 && !kv_indices) return fail(VA_ERR_NULL, "kv_indices is NULL");
    if (mask_len > 0 && !custom_mask) return fail(VA_ERR_NULL, "custom_mask is NULL");
  }
  va::RunArgs a;
  a.q = q;
  a.kv = kv_buffer;
  a.num_slots = num_slots;
  a.kv_indices = kv_indices;
  a.num_kv_indices = num_kv_indices;
  a.out_cache_loc = out_cache_loc;
  a.kv_indptr = kv_indptr;
  a.qo_indptr = qo_indptr;
  a.mask = custom_mask;
  a.mask_len = mask_len;
  a.mask_indptr = mask_indptr;
  a.bs = bs;
  a.num_tokens = num_tokens;
  a.H = cfg.num_heads;
  a.max_q_per_req = cfg.max_q_per_req;
  a.scale = sm_scale;
  a.out = out;
  a.out_lse = out_lse;
  a.out_argmax = out_argmax;
  a.out_bf16 = cfg.out_dtype == VA_BF16;
  a.want_argmax = out_argmax != nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (ev[0] && (e = hipEventRecord(ev[0], st)) != hipSuccess)
    return fail(VA_ERR_HIP, "hipEventRecord failed: %s", hipGetErrorString(e));
  if (bs > 0) {
    if (d.kernel == VA_KERNEL_SIMPLE)
      e = va::launch_simple_partial(a, ws, cfg.in_dtype == VA_FP32, st);
    else
      e = va::launch_mfma_partial(a, ws, d.rows_per_block, d.grid, st);
    if (e != hipSuccess)
      return fail(VA_ERR_HIP, "partial kernel launch failed: %s", hipGetErrorString(e));
  }
  if (ev[1] && (e = hipEventRecord(ev[1], st)) != hipSuccess)
    return fail(VA_ERR_HIP, "hipEventRecord failed: %s", hipGetErrorString(e));
  e = va::launch_combine(a, ws, st);
  if (e != hipSuccess)
    return fail(VA_ERR_HIP, "combine kernel launch failed: %s", hipGetErrorString(e));
  if (ev[2] && (e = hipEventRecord(ev[2], st)) != hipSuccess)
    return fail(VA_ERR_HIP, "hipEventRecord failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

size_t verify_attn_workspace_bytes(const verify_attn_config *cfg) {
  Derived d;
  if (derive(cfg, &d) != VA_OK) return 0;
  return d.bytes;
}

va_status verify_attn_create(const verify_attn_config *cfg, verify_attn_ctx **out) {
  if (!out) return fail(VA_ERR_NULL, "out is NULL");
  *out = nullptr;
  Derived d;
  va_status st = derive(cfg, &d);
  if (st != VA_OK) return st;
  const size_t bytes = d.bytes;
  void *base = cfg->workspace;
  bool owned = false;
  if (base) {
    if (cfg->workspace_bytes < bytes)
      return fail(VA_ERR_WORKSPACE, "workspace holds %zu bytes, %zu needed",
                  cfg->workspace_bytes, bytes);
    if (reinterpret_cast<uintptr_t>(base) & 255)
      return fail(VA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  } else {
    hipError_t e = hipMalloc(&base, bytes);
    if (e != hipSuccess)
      return fail(VA_ERR_HIP, "hipMalloc(%zu) failed: %s", bytes, hipGetErrorString(e));
    owned = true;
  }
  hipError_t e = hipMemset(base, 0, va::kHeaderBytes);  // status words and the zero row
  if (e != hipSuccess) {
    if (owned) (void)hipFree(base);
    return fail(VA_ERR_HIP, "hipMemset failed: %s", hipGetErrorString(e));
  }
  auto *x = new (std::nothrow) verify_attn_ctx();
  if (!x) {
    if (owned) (void)hipFree(base);
    return fail(VA_ERR_INVALID, "out of host memory");
  }
  x->cfg = *cfg;
  x->d = d;
  x->ws_base = base;
  x->ws_owned = owned;
  x->ev[0] = x->ev[1] = x->ev[2] = nullptr;
  x->ws = bind_workspace(x->cfg, d, base);
  *out = x;
  return ok();
}

va_status verify_attn_run(verify_attn_ctx *ctx, const void *q, const void *kv_buffer,
                          int64_t num_slots, const int64_t *kv_indices, int64_t num_kv_indices,
                          const int32_t *kv_indptr, const int64_t *qo_indptr,
                          const uint8_t *custom_mask, int64_t mask_len,
                          const int64_t *mask_indptr, const int64_t *out_cache_loc, int32_t bs,
                          int64_t num_tokens, float sm_scale, void *out, float *out_lse,
                          int32_t *out_argmax, void *stream) {
  if (!ctx) return fail(VA_ERR_NULL, "ctx is NULL");
  return launch_step(ctx->cfg, ctx->d, ctx->ws, ctx->ev, q, kv_buffer, num_slots, kv_indices,
                     num_kv_indices, kv_indptr, qo_indptr, custom_mask, mask_len, mask_indptr,
                     out_cache_loc, bs, num_tokens, sm_scale, out, out_lse, out_argmax, stream);
}

va_status verify_attn_run_static(const verify_attn_config *cfg, const void *q,
                                 const void *kv_buffer, int64_t num_slots,
                                 const int64_t *kv_indices, int64_t num_kv_indices,
                                 const int32_t *kv_indptr, const int64_t *qo_indptr,
                                 const uint8_t *custom_mask, int64_t mask_len,
                                 const int64_t *mask_indptr, const int64_t *out_cache_loc,
                                 int32_t bs, int64_t num_tokens, float sm_scale, void *out,
                                 float *out_lse, int32_t *out_argmax, void *stream) {
  Derived d;
  va_status st = derive(cfg, &d);
  if (st != VA_OK) return st;
  if (cfg->workspace)
    return fail(VA_ERR_INVALID, "verify_attn_run_static uses the library's static scratch; "
                                "cfg->workspace must be NULL");
  if (d.bytes > va::kStaticScratchBytes)
    return fail(VA_ERR_WORKSPACE,
                "the config needs %zu bytes of workspace, above the %zu-byte static scratch "
                "(lower max_q_tokens, num_heads or num_splits, or use verify_attn_create)",
                d.bytes, size_t(va::kStaticScratchBytes));
  if (num_tokens == 0 && bs >= 0 && bs <= cfg->max_batch)
    return launch_step(*cfg, d, va::Workspace{}, kNoEvents, q, kv_buffer, num_slots,
                       kv_indices, num_kv_indices, kv_indptr, qo_indptr, custom_mask, mask_len,
                       mask_indptr, out_cache_loc, bs, num_tokens, sm_scale, out, out_lse,
                       out_argmax, stream);
  void *base = nullptr;
  const hipError_t e = va::static_scratch(static_cast<hipStream_t>(stream), &base);
  if (e != hipSuccess)
    return fail(VA_ERR_HIP, "static scratch set-up failed: %s", hipGetErrorString(e));
  return launch_step(*cfg, d, bind_workspace(*cfg, d, base), kNoEvents, q, kv_buffer, num_slots,
                     kv_indices, num_kv_indices, kv_indptr, qo_indptr, custom_mask, mask_len,
                     mask_indptr, out_cache_loc, bs, num_tokens, sm_scale, out, out_lse,
                     out_argmax, stream);
}

va_status verify_attn_build_mask(verify_attn_ctx *ctx, const int64_t *parents,
                                 const int64_t *qo_indptr, const int32_t *kv_indptr,
                                 int32_t split_layout, int32_t bs, int64_t num_tokens,
                                 uint8_t *custom_mask, int64_t mask_len, int64_t *mask_indptr,
                                 int32_t write_mask_indptr, void *stream) {
  if (!ctx) return fail(VA_ERR_NULL, "ctx is NULL");
  if (bs < 0 || bs > ctx->cfg.max_batch)
    return fail(VA_ERR_INVALID, "bs %d out of range [0, %d]", bs, ctx->cfg.max_batch);
  if (num_tokens < 0 || num_tokens > ctx->cfg.max_q_tokens)
    return fail(VA_ERR_INVALID, "num_tokens %lld out of range [0, %lld]",
                (long long)num_tokens, (long long)ctx->cfg.max_q_tokens);
  if (ctx->cfg.max_q_per_req > va::kMaxTreeNodes)
    return fail(VA_ERR_UNSUPPORTED, "max_q_per_req above %d", va::kMaxTreeNodes);
  if (mask_len < 0) return fail(VA_ERR_INVALID, "mask_len must be >= 0");
  if (bs == 0) return ok();
  if (!qo_indptr || !kv_indptr || !mask_indptr || (num_tokens > 0 && (!parents || !custom_mask)))
    return fail(VA_ERR_NULL, "a required pointer is NULL");
  va::TreeArgs a;
  a.parents = parents;
  a.qo_indptr = qo_indptr;
  a.kv_indptr = kv_indptr;
  a.split_layout = split_layout != 0;
  a.bs = bs;
  a.num_tokens = num_tokens;
  a.max_q_per_req = ctx->cfg.max_q_per_req;
  a.mask = custom_mask;
  a.mask_len = mask_len;
  a.mask_indptr = mask_indptr;
  a.status = ctx->ws.status;
  const hipError_t e =
      va::launch_build_mask(a, write_mask_indptr != 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(VA_ERR_HIP, "mask build launch failed: %s", hipGetErrorString(e));
  return ok();
}

va_status verify_attn_accept(verify_attn_ctx *ctx, const int64_t *parents,
                             const int64_t *draft_tokens, const int64_t *target_tokens,
                             const int64_t *qo_indptr, int32_t bs, int64_t num_tokens,
                             int32_t *accept_len, int64_t *accept_path, int32_t max_path,
                             int64_t *next_token, void *stream) {
  if (!ctx) return fail(VA_ERR_NULL, "ctx is NULL");
  if (bs < 0 || bs > ctx->cfg.max_batch)
    return fail(VA_ERR_INVALID, "bs %d out of range [0, %d]", bs, ctx->cfg.max_batch);
  if (num_tokens < 0 || num_tokens > ctx->cfg.max_q_tokens)
    return fail(VA_ERR_INVALID, "num_tokens %lld out of range [0, %lld]",
                (long long)num_tokens, (long long)ctx->cfg.max_q_tokens);
  if (max_path < 1) return fail(VA_ERR_INVALID, "max_path must be >= 1");
  if (ctx->cfg.max_q_per_req > va::kMaxTreeNodes)
    return fail(VA_ERR_UNSUPPORTED, "max_q_per_req above %d", va::kMaxTreeNodes);
  if (bs == 0) return ok();
  if (!qo_indptr || !accept_len || !accept_path || !next_token ||
      (num_tokens > 0 && (!parents || !draft_tokens || !target_tokens)))
    return fail(VA_ERR_NULL, "a required pointer is NULL");
  va::AcceptArgs a;
  a.parents = parents;
  a.draft_tokens = draft_tokens;
  a.target_tokens = target_tokens;
  a.qo_indptr = qo_indptr;
  a.bs = bs;
  a.num_tokens = num_tokens;
  a.max_q_per_req = ctx->cfg.max_q_per_req;
  a.accept_len = accept_len;
  a.accept_path = accept_path;
  a.max_path = max_path;
  a.next_token = next_token;
  a.status = ctx->ws.status;
  const hipError_t e = va::launch_accept(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(VA_ERR_HIP, "accept launch failed: %s", hipGetErrorString(e));
  return ok();
}

va_status verify_attn_read_device_status(verify_attn_ctx *ctx, void *stream, uint32_t *flags) {
  if (!ctx || !flags) return fail(VA_ERR_NULL, "ctx or flags is NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  hipError_t e = hipStreamSynchronize(st);
  if (e == hipSuccess) e = hipMemcpy(&v, ctx->ws.status, sizeof v, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemset(ctx->ws.status, 0, sizeof v);
  if (e != hipSuccess) return fail(VA_ERR_HIP, "status read failed: %s", hipGetErrorString(e));
  *flags = v;
  return ok();
}

va_status verify_attn_set_profiling_events(verify_attn_ctx *ctx, void *before, void *between,
                                           void *after) {
  if (!ctx) return fail(VA_ERR_NULL, "ctx is NULL");
  const bool all = before && between && after;
  const bool two = before && between && !after;  // the next run's `before` ends this one
  const bool none = !before && !between && !after;
  if (!all && !two && !none)
    return fail(VA_ERR_INVALID, "pass three events, `before` and `between`, or none");
  ctx->ev[0] = static_cast<hipEvent_t>(before);
  ctx->ev[1] = static_cast<hipEvent_t>(between);
  ctx->ev[2] = static_cast<hipEvent_t>(after);
  return ok();
}

va_status verify_attn_get_info(const verify_attn_ctx *ctx, verify_attn_info *info) {
  if (!ctx || !info) return fail(VA_ERR_NULL, "ctx or info is NULL");
  info->kernel = ctx->d.kernel;
  info->num_splits = ctx->d.splits;
  info->rows_per_block = ctx->d.rows_per_block;
  info->row_tiles_per_req = ctx->d.row_tiles;
  info->workspace_bytes = ctx->d.bytes;
  info->partial_waves =
      ctx->d.kernel == VA_KERNEL_MFMA ? va::mfma_partial_waves(ctx->cfg.num_heads) : 4;
  return ok();
}

void verify_attn_destroy(verify_attn_ctx *ctx) {
  if (!ctx) return;
  if (ctx->ws_owned && ctx->ws_base) (void)hipFree(ctx->ws_base);
  delete ctx;
}

const char *verify_attn_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
