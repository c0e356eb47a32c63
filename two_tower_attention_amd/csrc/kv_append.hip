// Block commit into the paged context cache ("The idea: freeze the reader,
// train the writer", paperfeed review: a resolved block is committed and the
// context tower's caches grow by it).  Copies the block's S keys (token-major
// rows) and values (feature-major columns) of every (sequence, KV head) to
// logical positions L_b .. L_b+S-1, then advances ctx_lens[b].  Pure data
// movement, bit-exact.
//
// Grid (B, H_kv), one work-group per (sequence, KV head).  Every head reads
// L_b, so the length update runs afterwards in a second kernel (one thread
// per sequence) on the same stream.
#include "tt_internal.h"

namespace tt {
namespace {

constexpr int kThreads = 256;

struct AppendParams {
  const void *k_blk, *v_blk;
  void *k_pages, *v_pages;
  const int32_t *page_table;
  int32_t *ctx_lens;
  int B, S, Hkv, D, page_size, max_pages, num_pages;
  int vec;  // key rows may be copied in 16-byte chunks
};

// Whether every target slot of sequence b is backed by a valid page.
__device__ __forceinline__ bool target_ok(const AppendParams &p, int b, int L) {
  if (L < 0 || (long)L + p.S > (long)p.max_pages * p.page_size) return false;
  const int32_t *pt = p.page_table + (size_t)b * p.max_pages;
  for (int j = L / p.page_size; j <= (L + p.S - 1) / p.page_size; ++j)
    if (pt[j] < 0 || pt[j] >= p.num_pages) return false;
  return true;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void kv_append_kernel(AppendParams p) {
  const int b = blockIdx.x, h = blockIdx.y;
  const int L = p.ctx_lens[b];
  if (!target_ok(p, b, L)) return;
  const int32_t *pt = p.page_table + (size_t)b * p.max_pages;
  T *kp = (T *)p.k_pages;
  T *vp = (T *)p.v_pages;
  constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte chunk
  const int chunks = p.D / VEC;        // D is a multiple of VEC on the vector path
  if (p.vec && p.D % VEC == 0) {
    // keys: one 16-byte chunk per thread iteration
    for (int e = threadIdx.x; e < p.S * chunks; e += kThreads) {
      const int t = e / chunks, c = e % chunks;
      const int pos = L + t;
      const size_t pg = (size_t)pt[pos / p.page_size];
      const uint4 x = *(const uint4 *)((const T *)p.k_blk + (((size_t)b * p.S + t) * p.Hkv + h) * p.D + VEC * c);
      *(uint4 *)(kp + ((pg * p.Hkv + h) * p.page_size + pos % p.page_size) * p.D + VEC * c) = x;
    }
  } else {
    for (int e = threadIdx.x; e < p.S * p.D; e += kThreads) {
      const int t = e / p.D, d = e % p.D;
      const int pos = L + t;
      const size_t pg = (size_t)pt[pos / p.page_size];
      kp[((pg * p.Hkv + h) * p.page_size + pos % p.page_size) * p.D + d] =
          ((const T *)p.k_blk)[(((size_t)b * p.S + t) * p.Hkv + h) * p.D + d];
    }
  }
  // values: thread = (feature d, token t); consecutive threads write consecutive
  // slots of one feature row of the page
  for (int e = threadIdx.x; e < p.S * p.D; e += kThreads) {
    const int d = e / p.S, t = e % p.S;
    const int pos = L + t;
    const size_t pg = (size_t)pt[pos / p.page_size];
    vp[((pg * p.Hkv + h) * p.D + d) * p.page_size + pos % p.page_size] =
        ((const T *)p.v_blk)[(((size_t)b * p.S + t) * p.Hkv + h) * p.D + d];
  }
}

__global__ __launch_bounds__(kThreads) void advance_lens_kernel(AppendParams p) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= p.B) return;
  const int L = p.ctx_lens[b];
  if (target_ok(p, b, L)) p.ctx_lens[b] = L + p.S;
}

}  // namespace

hipError_t launch_kv_append(const tt_attn_desc &d, const void *k_blk, const void *v_blk,
                            void *k_pages, void *v_pages, const int32_t *page_table,
                            int32_t *ctx_lens, hipStream_t stream) {
  AppendParams p;
  p.k_blk = k_blk; p.v_blk = v_blk; p.k_pages = k_pages; p.v_pages = v_pages;
  p.page_table = page_table; p.ctx_lens = ctx_lens;
  p.B = d.batch; p.S = d.block; p.Hkv = d.heads_kv; p.D = d.head_dim; p.page_size = d.page_size;
  p.max_pages = d.max_pages_per_seq; p.num_pages = d.num_pages;
  p.vec = ((uintptr_t)k_blk % 16 == 0) && ((uintptr_t)k_pages % 16 == 0);
  const dim3 grid(d.batch, d.heads_kv);
  if (d.dtype == TT_BF16)
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(kv_append_kernel<float>, grid, dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(advance_lens_kernel, dim3((d.batch + kThreads - 1) / kThreads), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace tt
