// Block commit into the paged context cache ("The idea: freeze the reader,
// train the writer", paperfeed review: a resolved block is committed and the
// context tower's caches grow by it).  One work-group per sequence copies the
// block's S keys (token-major rows) and values (feature-major columns) to
// logical positions L_b .. L_b+S-1, then advances ctx_lens[b].  Pure data
// movement, bit-exact.
#include "tt_internal.h"

namespace tt {
namespace {

constexpr int kThreads = 256;

struct AppendParams {
  const void *k_blk, *v_blk;
  void *k_pages, *v_pages;
  const int32_t *page_table;
  int32_t *ctx_lens;
  int S, Hkv, D, page_size, max_pages, num_pages;
};

template <typename T>
__global__ __launch_bounds__(kThreads) void kv_append_kernel(AppendParams p) {
  __shared__ int ok;
  const int b = blockIdx.x;
  const int L = p.ctx_lens[b];
  const int32_t *pt = p.page_table + (size_t)b * p.max_pages;
  if (threadIdx.x == 0) {
    int good = L >= 0 && (long)L + p.S <= (long)p.max_pages * p.page_size;
    if (good) {
      for (int j = L / p.page_size; j <= (L + p.S - 1) / p.page_size; ++j)
        if (pt[j] < 0 || pt[j] >= p.num_pages) good = 0;
    }
    ok = good;
  }
  __syncthreads();
  if (!ok) return;
  const T *kb = (const T *)p.k_blk + (size_t)b * p.S * p.Hkv * p.D;
  const T *vb = (const T *)p.v_blk + (size_t)b * p.S * p.Hkv * p.D;
  T *kp = (T *)p.k_pages;
  T *vp = (T *)p.v_pages;
  const int n = p.S * p.Hkv * p.D;
  for (int e = threadIdx.x; e < n; e += kThreads) {
    const int t = e / (p.Hkv * p.D), h = (e / p.D) % p.Hkv, d = e % p.D;
    const int pos = L + t;
    const size_t pg = (size_t)pt[pos / p.page_size];
    const int off = pos % p.page_size;
    kp[((pg * p.Hkv + h) * p.page_size + off) * p.D + d] = kb[e];
    vp[((pg * p.Hkv + h) * p.D + d) * p.page_size + off] = vb[e];
  }
  __syncthreads();
  if (threadIdx.x == 0) p.ctx_lens[b] = L + p.S;
}

}  // namespace

hipError_t launch_kv_append(const tt_attn_desc &d, const void *k_blk, const void *v_blk,
                            void *k_pages, void *v_pages, const int32_t *page_table,
                            int32_t *ctx_lens, hipStream_t stream) {
  AppendParams p;
  p.k_blk = k_blk; p.v_blk = v_blk; p.k_pages = k_pages; p.v_pages = v_pages;
  p.page_table = page_table; p.ctx_lens = ctx_lens;
  p.S = d.block; p.Hkv = d.heads_kv; p.D = d.head_dim; p.page_size = d.page_size;
  p.max_pages = d.max_pages_per_seq; p.num_pages = d.num_pages;
  if (d.dtype == TT_BF16)
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, dim3(d.batch), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(kv_append_kernel<float>, dim3(d.batch), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace tt
