// Internal declarations shared by the HIP sources of libtt.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "tt.h"

namespace tt {

// Raises a kernel's dynamic LDS limit to `bytes` on the current device, once
// per device: the attribute is per device, and `done` keeps one bit per
// device id below 64 (higher ids set it on every call).  Concurrent first
// calls may both set it, which is harmless.
inline hipError_t lds_limit_once(const void *kernel, int bytes, std::atomic<unsigned long long> &done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = dev >= 0 && dev < 64 ? 1ull << dev : 0ull;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Largest batch the attention planner keeps in LDS (per-sequence prefix sums).
constexpr int kMaxBatch = 2048;

// Shape and launch plan of one bf16 block-attention call.
struct AttnPlan {
  int B, S, Hq, Hkv, g, D;
  int page_size, max_pages, num_pages, max_ctx;
  int qchunks;       // ceil(S*g / 256) query-row chunks per (b, h_kv)
  int G;             // work-groups in the split launch
  float scale_log2;  // softmax scale * log2(e)
  size_t ws_bytes;   // workspace bytes
  long long tiles;   // upper bound on the flat tile count (the device indexes it in int)
};

// Largest flat tile count the device-side plan (int prefix sums and ranges)
// can index with headroom for the work-group range arithmetic.
constexpr long long kMaxAttnTiles = (1ll << 31) - (1ll << 20);

// Plans a bf16 call for a device with `cus` compute units.
AttnPlan plan_bf16_attn(const tt_attn_desc &d, int cus);

hipError_t launch_attn_bf16(const AttnPlan &p, const void *q, const void *k_blk,
                            const void *v_blk, const void *k_pages, const void *v_pages,
                            const int32_t *page_table, const int32_t *ctx_lens, void *out,
                            void *workspace, int causal, hipStream_t stream);

hipError_t launch_attn_f32(const tt_attn_desc &d, float scale, const float *q,
                           const float *k_blk, const float *v_blk, const float *k_pages,
                           const float *v_pages, const int32_t *page_table,
                           const int32_t *ctx_lens, float *out, int causal, hipStream_t stream);

hipError_t launch_kv_append(const tt_attn_desc &d, const void *k_blk, const void *v_blk,
                            void *k_pages, void *v_pages, const int32_t *page_table,
                            int32_t *ctx_lens, hipStream_t stream);

// Per (row, vocabulary chunk) partial of the unmask's row reduction:
// m = max, s = sum exp(l - m), idx = lowest index attaining m.  A chunk with
// no element has m = -inf, s = 0, idx = INT_MAX.
struct UnmaskPart {
  float m;
  float s;
  int idx;
  int pad;
};

struct UnmaskPlan {
  int B, S, V;
  int chunks;       // vocabulary chunks per row
  int chunk_len;    // elements per chunk (multiple of 4)
  size_t ws_bytes;
};

UnmaskPlan plan_unmask(int B, int S, int V);

// Size of the static row-partials array of tt_unmask_noalloc, and the
// current device's address of it (looked up on the first call on each
// device).  plan_unmask splits a row into ceil(512 / rows) chunks at most, so
// rows * chunks < max(rows, 1024) <= 65535 partials of 16 bytes: 1 MiB holds
// every shape the unmask accepts.
constexpr size_t kUnmaskStaticBytes = size_t(1) << 20;
hipError_t unmask_static_scratch(void **ptr);

hipError_t launch_unmask(const UnmaskPlan &p, const float *logits, uint8_t *mask,
                         const int32_t *k_commit, int remaining_steps, int32_t *ids,
                         uint8_t *commit, float *conf, uint32_t flags, void *workspace,
                         hipStream_t stream);

hipError_t launch_unmask_threshold(const UnmaskPlan &p, const float *logits, uint8_t *mask,
                                   float gamma, int32_t *ids, uint8_t *commit, float *conf,
                                   int32_t *nsteps, uint32_t flags, void *workspace,
                                   hipStream_t stream);

// The commit stage of tt_unmask / tt_unmask_threshold on row partials
// [B*S, chunks].
hipError_t launch_unmask_commit(const UnmaskPart *parts, int chunks, int B, int S, uint8_t *mask,
                                const int32_t *k_commit, int remaining_steps, int32_t *ids,
                                uint8_t *commit, float *conf, uint32_t flags, hipStream_t stream);
hipError_t launch_unmask_threshold_commit(const UnmaskPart *parts, int chunks, int B, int S,
                                          uint8_t *mask, float gamma, int32_t *ids,
                                          uint8_t *commit, float *conf, int32_t *nsteps,
                                          uint32_t flags, hipStream_t stream);

// LM head fused with the unmask's row reduction: hidden [R, H] and weight
// [V, H] in bf16 -> per (row, 256-entry vocabulary tile) partials [R, lmhead_chunks(V)].
// xpack: lmhead_pack_bytes(R, H) bytes of scratch (16-byte aligned) for the
// hidden state in MFMA fragment order.
int lmhead_chunks(int V);
size_t lmhead_pack_bytes(int R, int H);
hipError_t launch_lmhead_parts(const void *hidden, const void *weight, int R, int H, int V,
                               UnmaskPart *parts, void *xpack, hipStream_t stream);

}  // namespace tt
