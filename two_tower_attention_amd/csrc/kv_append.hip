// Block commit into the paged context cache ("The idea: freeze the reader,
// train the writer", paperfeed review: a resolved block is committed and the
// context tower's caches grow by it).  Copies the block's S keys (token-major
// rows) and values (feature-major columns) of every (sequence, KV head) to
// logical positions L_b .. L_b+S-1, then advances ctx_lens[b].  Pure data
// movement, bit-exact.
//
// One work-group per sequence covers all its KV heads, so it can advance
// ctx_lens[b] itself once every thread has read L_b (no second launch).
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

// LDS bytes of a pass: the values of `hp` heads, [S][hp][D]
constexpr int kStageBytes = 32 * 1024;
__host__ __device__ inline int heads_per_pass(int S, int Hkv, int D, int elem) {
  const int hp = kStageBytes / (S * D * elem);
  return hp < 1 ? 1 : hp > Hkv ? Hkv : hp;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void kv_append_kernel(AppendParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  T *sv = (T *)smem;  // values of the pass's heads [S][hp][D]
  const int b = blockIdx.x;
  const int L = p.ctx_lens[b];
  if (!target_ok(p, b, L)) return;  // uniform over the work-group
  const int32_t *__restrict__ pt = p.page_table + (size_t)b * p.max_pages;
  const T *__restrict__ kb = (const T *)p.k_blk + (size_t)b * p.S * p.Hkv * p.D;
  const T *__restrict__ vb = (const T *)p.v_blk + (size_t)b * p.S * p.Hkv * p.D;
  T *__restrict__ kp = (T *)p.k_pages;
  T *__restrict__ vp = (T *)p.v_pages;
  constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte chunk
  const bool vec = p.vec && p.D % VEC == 0;
  const int hp = heads_per_pass(p.S, p.Hkv, p.D, (int)sizeof(T));
  for (int h0 = 0; h0 < p.Hkv; h0 += hp) {
    const int nh = min(hp, p.Hkv - h0);
    const int row = nh * p.D;  // elements of one token's row in this pass
    if (vec) {
      // keys: token rows, 16-byte chunks straight to their page rows; values:
      // the same rows into LDS
      const int chunks = row / VEC;
      for (int e = threadIdx.x; e < p.S * chunks; e += kThreads) {
        const int t = e / chunks, c = e % chunks;
        const int hh = (VEC * c) / p.D, d = (VEC * c) % p.D;
        const size_t src = ((size_t)t * p.Hkv + h0) * p.D + VEC * c;
        const uint4 k = *(const uint4 *)(kb + src);
        const uint4 v = *(const uint4 *)(vb + src);
        const int pos = L + t;
        const size_t pg = (size_t)pt[pos / p.page_size];
        *(uint4 *)(kp + ((pg * p.Hkv + h0 + hh) * p.page_size + pos % p.page_size) * p.D + d) = k;
        *(uint4 *)(sv + t * row + VEC * c) = v;
      }
    } else {
      for (int e = threadIdx.x; e < p.S * row; e += kThreads) {
        const int t = e / row, j = e % row, hh = j / p.D, d = j % p.D;
        const size_t src = ((size_t)t * p.Hkv + h0) * p.D + j;
        const int pos = L + t;
        const size_t pg = (size_t)pt[pos / p.page_size];
        kp[((pg * p.Hkv + h0 + hh) * p.page_size + pos % p.page_size) * p.D + d] = kb[src];
        sv[t * row + j] = vb[src];
      }
    }
    __syncthreads();
    // values: thread = (head, feature, token), token fastest, so consecutive
    // threads write consecutive slots of one feature row of the page
    for (int e = threadIdx.x; e < p.S * row; e += kThreads) {
      const int j = e / p.S, t = e % p.S, hh = j / p.D, d = j % p.D;
      const int pos = L + t;
      const size_t pg = (size_t)pt[pos / p.page_size];
      vp[((pg * p.Hkv + h0 + hh) * p.D + d) * p.page_size + pos % p.page_size] = sv[t * row + j];
    }
    __syncthreads();  // sv is refilled by the next pass; every thread has read L_b
  }
  if (threadIdx.x == 0) p.ctx_lens[b] = L + p.S;  // only this work-group touches sequence b
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
  if (d.batch == 0) return hipSuccess;
  // the values of one pass's heads staged in LDS (at most 32 KiB: one head
  // is at most 64 * 128 * 4 bytes)
  const int elem = d.dtype == TT_BF16 ? 2 : 4;
  const size_t lds = (size_t)d.block * d.head_dim * elem *
                     heads_per_pass(d.block, d.heads_kv, d.head_dim, elem);
  if (d.dtype == TT_BF16)
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, dim3(d.batch), dim3(kThreads), lds, stream, p);
  else
    hipLaunchKernelGGL(kv_append_kernel<float>, dim3(d.batch), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace tt
