// Host side of the C ABI in include/tt.h: argument validation, launch
// planning and kernel launches.  Never allocates device memory.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <string>

#include <cmath>

#include "tt_internal.h"

namespace {

thread_local std::string g_err;

int fail(int status, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return status;
}

int ok() {
  g_err.clear();
  return TT_OK;
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

// Compute units of the current device; <= 0 when there is no usable device.
int device_cus(int *dev_out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return -1;
  }
  if (dev_out) *dev_out = dev;
  if (dev < kMaxDevices) {
    const int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return -1;
  }
  if (dev < kMaxDevices) g_cus[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Planning-only CU count: the device's when there is one, else MI355X's 256.
int planning_cus() {
  const int c = device_cus(nullptr);
  return c > 0 ? c : 256;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_desc(const tt_attn_desc *d) {
  if (!d) return fail(TT_ERR_NULL, "desc is NULL");
  if (d->dtype != TT_BF16 && d->dtype != TT_F32)
    return fail(TT_ERR_DTYPE, "dtype %d is neither TT_BF16 nor TT_F32", d->dtype);
  if (d->batch < 0 || d->batch > tt::kMaxBatch)
    return fail(TT_ERR_SHAPE, "batch %d outside [0, %d]", d->batch, tt::kMaxBatch);
  if (d->block < 1 || d->block > 64)
    return fail(TT_ERR_SHAPE, "block %d outside [1, 64]", d->block);
  if (d->heads_q < 1 || d->heads_kv < 1 || d->heads_q % d->heads_kv != 0)
    return fail(TT_ERR_SHAPE, "heads_q %d must be a positive multiple of heads_kv %d",
                d->heads_q, d->heads_kv);
  if (d->heads_q > 4096) return fail(TT_ERR_SHAPE, "heads_q %d > 4096", d->heads_q);
  if (d->page_size < 16 || d->page_size > 4096 || (d->page_size & (d->page_size - 1)) != 0)
    return fail(TT_ERR_SHAPE, "page_size %d is not a power of two in [16, 4096]", d->page_size);
  if (d->max_pages_per_seq < 1)
    return fail(TT_ERR_SHAPE, "max_pages_per_seq %d < 1", d->max_pages_per_seq);
  if (d->num_pages < 1) return fail(TT_ERR_SHAPE, "num_pages %d < 1", d->num_pages);
  if (d->max_ctx_len < 0 ||
      (long long)d->max_ctx_len > (long long)d->max_pages_per_seq * d->page_size)
    return fail(TT_ERR_SHAPE, "max_ctx_len %d outside [0, max_pages_per_seq * page_size]",
                d->max_ctx_len);
  if ((long long)d->max_ctx_len + 64 > (1ll << 30))
    return fail(TT_ERR_SHAPE, "max_ctx_len %d too large", d->max_ctx_len);
  if (!(isfinite(d->scale))) return fail(TT_ERR_SHAPE, "scale is not finite");
  if (d->dtype == TT_BF16) {
    if (d->head_dim != 64 && d->head_dim != 128)
      return fail(TT_ERR_UNSUPPORTED, "bf16 head_dim %d: only 64 and 128 are built", d->head_dim);
  } else if (d->head_dim < 1 || d->head_dim > 256) {
    return fail(TT_ERR_UNSUPPORTED, "f32 head_dim %d outside [1, 256]", d->head_dim);
  }
  return TT_OK;
}

}  // namespace

extern "C" {

const char *tt_status_str(int s) {
  switch (s) {
    case TT_OK: return "TT_OK";
    case TT_ERR_NULL: return "TT_ERR_NULL: a required pointer is NULL";
    case TT_ERR_SHAPE: return "TT_ERR_SHAPE: size out of range or inconsistent";
    case TT_ERR_DTYPE: return "TT_ERR_DTYPE: unknown element type";
    case TT_ERR_UNSUPPORTED: return "TT_ERR_UNSUPPORTED: not implemented in this build";
    case TT_ERR_WORKSPACE: return "TT_ERR_WORKSPACE: workspace missing or too small";
    case TT_ERR_NO_DEVICE: return "TT_ERR_NO_DEVICE: no usable HIP device";
    case TT_ERR_LAUNCH: return "TT_ERR_LAUNCH: kernel launch failed";
    default: return "unknown tt_status";
  }
}

const char *tt_last_error(void) { return g_err.c_str(); }

int tt_abi_version(void) { return TT_ABI_VERSION; }

int tt_block_attn_workspace_bytes(const tt_attn_desc *d, size_t *bytes) {
  if (!bytes) return fail(TT_ERR_NULL, "bytes is NULL");
  const int st = check_desc(d);
  if (st) return st;
  if (d->dtype == TT_F32 || d->batch == 0) {
    *bytes = 0;
    return ok();
  }
  const tt::AttnPlan plan = tt::plan_bf16_attn(*d, planning_cus());
  if (plan.tiles > tt::kMaxAttnTiles)
    return fail(TT_ERR_SHAPE, "%lld key tiles exceed what one launch indexes (%lld)", plan.tiles,
                tt::kMaxAttnTiles);
  *bytes = plan.ws_bytes;
  return ok();
}

static int block_attn(const tt_attn_desc *d, const void *q, const void *k_blk, const void *v_blk,
                      const void *k_pages, const void *v_pages, const int32_t *page_table,
                      const int32_t *ctx_lens, void *out, void *workspace, size_t workspace_bytes,
                      int causal, void *stream) {
  int st = check_desc(d);
  if (st) return st;
  if (d->batch == 0) return ok();
  if (!q || !k_blk || !v_blk || !ctx_lens || !out)
    return fail(TT_ERR_NULL, "q, k_blk, v_blk, ctx_lens and out are required");
  if (d->max_ctx_len > 0 && (!k_pages || !v_pages || !page_table))
    return fail(TT_ERR_NULL, "k_pages, v_pages and page_table are required when max_ctx_len > 0");
  const size_t vec = d->dtype == TT_BF16 ? 16 : 4;
  if (!aligned(q, vec) || !aligned(k_blk, vec) || !aligned(v_blk, vec) || !aligned(out, 8) ||
      (k_pages && !aligned(k_pages, vec)) || (v_pages && !aligned(v_pages, vec)) ||
      !aligned(page_table, 4) || !aligned(ctx_lens, 4))
    return fail(TT_ERR_UNSUPPORTED, "tensor pointers must be %zu-byte aligned (out: 8)", vec);
  int dev = -1;
  const int cus = device_cus(&dev);
  if (cus <= 0) return fail(TT_ERR_NO_DEVICE, "no HIP device");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (d->dtype == TT_BF16) {
    const tt::AttnPlan plan = tt::plan_bf16_attn(*d, cus);
    if (plan.tiles > tt::kMaxAttnTiles)
      return fail(TT_ERR_SHAPE, "%lld key tiles exceed what one launch indexes (%lld)", plan.tiles,
                  tt::kMaxAttnTiles);
    if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes))
      return fail(TT_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", plan.ws_bytes,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 16)) return fail(TT_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
    e = tt::launch_attn_bf16(plan, q, k_blk, v_blk, k_pages, v_pages, page_table, ctx_lens, out,
                             workspace, causal, s);
  } else {
    const float scale = d->scale > 0.f ? d->scale : 1.0f / sqrtf((float)d->head_dim);
    e = tt::launch_attn_f32(*d, scale, (const float *)q, (const float *)k_blk,
                            (const float *)v_blk, (const float *)k_pages, (const float *)v_pages,
                            page_table, ctx_lens, (float *)out, causal, s);
  }
  if (e != hipSuccess) return fail(TT_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int tt_block_attn(const tt_attn_desc *d, const void *q, const void *k_blk, const void *v_blk,
                  const void *k_pages, const void *v_pages, const int32_t *page_table,
                  const int32_t *ctx_lens, void *out, void *workspace, size_t workspace_bytes,
                  void *stream) {
  return block_attn(d, q, k_blk, v_blk, k_pages, v_pages, page_table, ctx_lens, out, workspace,
                    workspace_bytes, 0, stream);
}

int tt_chunk_attn(const tt_attn_desc *d, const void *q, const void *k_blk, const void *v_blk,
                  const void *k_pages, const void *v_pages, const int32_t *page_table,
                  const int32_t *ctx_lens, void *out, void *workspace, size_t workspace_bytes,
                  void *stream) {
  return block_attn(d, q, k_blk, v_blk, k_pages, v_pages, page_table, ctx_lens, out, workspace,
                    workspace_bytes, 1, stream);
}

int tt_kv_append(const tt_attn_desc *d, const void *k_blk, const void *v_blk, void *k_pages,
                 void *v_pages, const int32_t *page_table, int32_t *ctx_lens, void *stream) {
  int st = check_desc(d);
  if (st) return st;
  if (d->batch == 0) return ok();
  if (!k_blk || !v_blk || !k_pages || !v_pages || !page_table || !ctx_lens)
    return fail(TT_ERR_NULL, "every tensor argument of tt_kv_append is required");
  if (device_cus(nullptr) <= 0) return fail(TT_ERR_NO_DEVICE, "no HIP device");
  const hipError_t e = tt::launch_kv_append(*d, k_blk, v_blk, k_pages, v_pages, page_table,
                                            ctx_lens, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TT_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

static int check_unmask_shape(int32_t B, int32_t S, int32_t V) {
  if (B < 0 || B > (1 << 20)) return fail(TT_ERR_SHAPE, "batch %d outside [0, 2^20]", B);
  if (S < 1 || S > 64) return fail(TT_ERR_SHAPE, "block %d outside [1, 64]", S);
  if (V < 1) return fail(TT_ERR_SHAPE, "vocab %d < 1", V);
  if ((long long)B * S > 65535) return fail(TT_ERR_SHAPE, "batch * block %lld > 65535", (long long)B * S);
  return TT_OK;
}

int tt_unmask_workspace_bytes(int32_t B, int32_t S, int32_t V, size_t *bytes) {
  if (!bytes) return fail(TT_ERR_NULL, "bytes is NULL");
  const int st = check_unmask_shape(B, S, V);
  if (st) return st;
  *bytes = B == 0 ? 0 : tt::plan_unmask(B, S, V).ws_bytes;
  return ok();
}

// Checks of tt_unmask's arguments other than the workspace; *done is set
// when the call has nothing to do (B = 0).
static int check_unmask_args(const float *logits, uint8_t *mask, const int32_t *k_commit,
                             int32_t remaining_steps, int32_t B, int32_t S, int32_t V,
                             int32_t *ids_out, uint8_t *commit_out, float *conf_out,
                             uint32_t flags, bool *done) {
  *done = false;
  int st = check_unmask_shape(B, S, V);
  if (st) return st;
  if (flags & ~TT_UNMASK_UPDATE_MASK) return fail(TT_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
  if (!k_commit && remaining_steps < 1)
    return fail(TT_ERR_SHAPE, "remaining_steps %d < 1 with k_commit NULL", remaining_steps);
  if (B == 0) {
    *done = true;
    return TT_OK;
  }
  if (!logits || !mask || !ids_out || !commit_out)
    return fail(TT_ERR_NULL, "logits, mask, ids_out and commit_out are required");
  if (!aligned(logits, 4) || !aligned(ids_out, 4) || (k_commit && !aligned(k_commit, 4)) ||
      (conf_out && !aligned(conf_out, 4)))
    return fail(TT_ERR_UNSUPPORTED, "logits, ids_out, k_commit, conf_out must be 4-byte aligned");
  return TT_OK;
}

int tt_unmask(const float *logits, uint8_t *mask, const int32_t *k_commit, int32_t remaining_steps,
              int32_t B, int32_t S, int32_t V, int32_t *ids_out, uint8_t *commit_out,
              float *conf_out, uint32_t flags, void *workspace, size_t workspace_bytes,
              void *stream) {
  bool done = false;
  const int st = check_unmask_args(logits, mask, k_commit, remaining_steps, B, S, V, ids_out,
                                   commit_out, conf_out, flags, &done);
  if (st) return st;
  if (done) return ok();
  const tt::UnmaskPlan plan = tt::plan_unmask(B, S, V);
  if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes))
    return fail(TT_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", plan.ws_bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16)) return fail(TT_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  if (device_cus(nullptr) <= 0) return fail(TT_ERR_NO_DEVICE, "no HIP device");
  const hipError_t e = tt::launch_unmask(plan, logits, mask, k_commit, remaining_steps, ids_out,
                                         commit_out, conf_out, flags, workspace,
                                         (hipStream_t)stream);
  if (e != hipSuccess) return fail(TT_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

static_assert(TT_UNMASK_NOALLOC_MAX_BYTES == tt::kUnmaskStaticBytes,
              "the header states the static scratch size");

int tt_unmask_noalloc(const float *logits, uint8_t *mask, const int32_t *k_commit,
                      int32_t remaining_steps, int32_t B, int32_t S, int32_t V, int32_t *ids_out,
                      uint8_t *commit_out, float *conf_out, uint32_t flags, void *stream) {
  bool done = false;
  const int st = check_unmask_args(logits, mask, k_commit, remaining_steps, B, S, V, ids_out,
                                   commit_out, conf_out, flags, &done);
  if (st) return st;
  if (done) return ok();
  const tt::UnmaskPlan plan = tt::plan_unmask(B, S, V);
  if (plan.ws_bytes > tt::kUnmaskStaticBytes)
    return fail(TT_ERR_WORKSPACE,
                "tt_unmask_noalloc: batch %d x block %d x vocab %d needs %zu bytes of row partials, "
                "its static scratch holds %zu; use tt_unmask with a workspace",
                B, S, V, plan.ws_bytes, tt::kUnmaskStaticBytes);
  if (device_cus(nullptr) <= 0) return fail(TT_ERR_NO_DEVICE, "no HIP device");
  void *scratch = nullptr;
  hipError_t e = tt::unmask_static_scratch(&scratch);
  if (e != hipSuccess)
    return fail(TT_ERR_LAUNCH, "address of the static scratch: %s", hipGetErrorString(e));
  e = tt::launch_unmask(plan, logits, mask, k_commit, remaining_steps, ids_out, commit_out,
                        conf_out, flags, scratch, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TT_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int tt_unmask_threshold(const float *logits, uint8_t *mask, float gamma, int32_t B, int32_t S,
                        int32_t V, int32_t *ids_out, uint8_t *commit_out, float *conf_out,
                        int32_t *nsteps, uint32_t flags, void *workspace, size_t workspace_bytes,
                        void *stream) {
  int st = check_unmask_shape(B, S, V);
  if (st) return st;
  if (flags & ~TT_UNMASK_UPDATE_MASK) return fail(TT_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
  if (!std::isfinite(gamma)) return fail(TT_ERR_SHAPE, "gamma must be finite");
  if (B == 0) return ok();
  if (!logits || !mask || !ids_out || !commit_out)
    return fail(TT_ERR_NULL, "logits, mask, ids_out and commit_out are required");
  if (!aligned(logits, 4) || !aligned(ids_out, 4) || (nsteps && !aligned(nsteps, 4)) ||
      (conf_out && !aligned(conf_out, 4)))
    return fail(TT_ERR_UNSUPPORTED, "logits, ids_out, nsteps, conf_out must be 4-byte aligned");
  const tt::UnmaskPlan plan = tt::plan_unmask(B, S, V);
  if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes))
    return fail(TT_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", plan.ws_bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16)) return fail(TT_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  if (device_cus(nullptr) <= 0) return fail(TT_ERR_NO_DEVICE, "no HIP device");
  const hipError_t e = tt::launch_unmask_threshold(plan, logits, mask, gamma, ids_out, commit_out,
                                                   conf_out, nsteps, flags, workspace,
                                                   (hipStream_t)stream);
  if (e != hipSuccess) return fail(TT_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

// ---- LM head fused with the unmask ------------------------------------

static int check_lmhead_shape(int32_t B, int32_t S, int32_t V, int32_t H) {
  const int st = check_unmask_shape(B, S, V);
  if (st) return st;
  if (H < 32 || H > 65536 || H % 32 != 0)
    return fail(TT_ERR_SHAPE, "hidden size %d must be a multiple of 32 in [32, 65536]", H);
  // grids: one work-group per 256 x 256 logits tile, and one packing
  // work-group per (64-row group, 64-element stage), must each stay below 2^31
  const long long R = (long long)B * S;
  const long long row_tiles = (R + 255) / 256, vocab_tiles = ((long long)V + 255) / 256;
  const long long pack_groups = row_tiles * 4 * ((H + 63) / 64);
  if (row_tiles * vocab_tiles > INT32_MAX || pack_groups > INT32_MAX)
    return fail(TT_ERR_SHAPE, "batch*block %lld with vocab %d and hidden size %d is too large for one launch", R, V, H);
  return TT_OK;
}

static size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

// parts [R, chunks], then the hidden state in MFMA fragment order
static size_t lmhead_parts_bytes(int32_t B, int32_t S, int32_t V) {
  return round256((size_t)B * S * tt::lmhead_chunks(V) * sizeof(tt::UnmaskPart));
}
static size_t lmhead_ws_bytes(int32_t B, int32_t S, int32_t V, int32_t H) {
  return lmhead_parts_bytes(B, S, V) + round256(tt::lmhead_pack_bytes(B * S, H));
}

int tt_lmhead_unmask_workspace_bytes(int32_t B, int32_t S, int32_t V, int32_t H, size_t *bytes) {
  if (!bytes) return fail(TT_ERR_NULL, "bytes is NULL");
  const int st = check_lmhead_shape(B, S, V, H);
  if (st) return st;
  *bytes = B == 0 ? 0 : lmhead_ws_bytes(B, S, V, H);
  return ok();
}

// Validation and the fused head + tile reduction shared by the two commit
// forms; on success *parts points at the [B*S, lmhead_chunks(V)] partials in
// the workspace, which the commit kernels merge per row.
static int lmhead_rows(const void *hidden, const void *weight, int32_t B, int32_t S, int32_t V,
                       int32_t H, void *workspace, size_t workspace_bytes, hipStream_t s,
                       tt::UnmaskPart **parts) {
  if (!hidden || !weight) return fail(TT_ERR_NULL, "hidden and weight are required");
  if (!aligned(hidden, 16) || !aligned(weight, 16))
    return fail(TT_ERR_UNSUPPORTED, "hidden and weight must be 16-byte aligned");
  const size_t need = lmhead_ws_bytes(B, S, V, H);
  if (!workspace || workspace_bytes < need)
    return fail(TT_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16)) return fail(TT_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  if (device_cus(nullptr) <= 0) return fail(TT_ERR_NO_DEVICE, "no HIP device");
  const int R = B * S;
  *parts = (tt::UnmaskPart *)workspace;
  void *xpack = (unsigned char *)workspace + lmhead_parts_bytes(B, S, V);
  const hipError_t e = tt::launch_lmhead_parts(hidden, weight, R, H, V, *parts, xpack, s);
  if (e != hipSuccess) return fail(TT_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return TT_OK;
}

int tt_lmhead_unmask(const void *hidden, const void *weight, uint8_t *mask,
                     const int32_t *k_commit, int32_t remaining_steps, int32_t B, int32_t S,
                     int32_t V, int32_t H, int32_t *ids_out, uint8_t *commit_out, float *conf_out,
                     uint32_t flags, void *workspace, size_t workspace_bytes, void *stream) {
  int st = check_lmhead_shape(B, S, V, H);
  if (st) return st;
  if (flags & ~TT_UNMASK_UPDATE_MASK) return fail(TT_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
  if (!k_commit && remaining_steps < 1)
    return fail(TT_ERR_SHAPE, "remaining_steps %d < 1 with k_commit NULL", remaining_steps);
  if (B == 0) return ok();
  if (!mask || !ids_out || !commit_out)
    return fail(TT_ERR_NULL, "mask, ids_out and commit_out are required");
  if (!aligned(ids_out, 4) || (k_commit && !aligned(k_commit, 4)) || (conf_out && !aligned(conf_out, 4)))
    return fail(TT_ERR_UNSUPPORTED, "ids_out, k_commit, conf_out must be 4-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  tt::UnmaskPart *parts = nullptr;
  st = lmhead_rows(hidden, weight, B, S, V, H, workspace, workspace_bytes, s, &parts);
  if (st) return st;
  const hipError_t e = tt::launch_unmask_commit(parts, tt::lmhead_chunks(V), B, S, mask, k_commit,
                                                remaining_steps, ids_out, commit_out, conf_out, flags, s);
  if (e != hipSuccess) return fail(TT_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int tt_lmhead_unmask_threshold(const void *hidden, const void *weight, uint8_t *mask, float gamma,
                               int32_t B, int32_t S, int32_t V, int32_t H, int32_t *ids_out,
                               uint8_t *commit_out, float *conf_out, int32_t *nsteps,
                               uint32_t flags, void *workspace, size_t workspace_bytes,
                               void *stream) {
  int st = check_lmhead_shape(B, S, V, H);
  if (st) return st;
  if (flags & ~TT_UNMASK_UPDATE_MASK) return fail(TT_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
  if (!std::isfinite(gamma)) return fail(TT_ERR_SHAPE, "gamma must be finite");
  if (B == 0) return ok();
  if (!mask || !ids_out || !commit_out)
    return fail(TT_ERR_NULL, "mask, ids_out and commit_out are required");
  if (!aligned(ids_out, 4) || (nsteps && !aligned(nsteps, 4)) || (conf_out && !aligned(conf_out, 4)))
    return fail(TT_ERR_UNSUPPORTED, "ids_out, nsteps, conf_out must be 4-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  tt::UnmaskPart *parts = nullptr;
  st = lmhead_rows(hidden, weight, B, S, V, H, workspace, workspace_bytes, s, &parts);
  if (st) return st;
  const hipError_t e = tt::launch_unmask_threshold_commit(parts, tt::lmhead_chunks(V), B, S, mask, gamma,
                                                          ids_out, commit_out, conf_out, nsteps, flags, s);
  if (e != hipSuccess) return fail(TT_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
