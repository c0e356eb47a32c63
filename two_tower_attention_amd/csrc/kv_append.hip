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
  int vec;   // block rows and key pages may be copied in 16-byte chunks
  int vvec;  // value pages are 16-byte aligned
};

// LDS bytes of a pass: the values of `hp` heads, [S][hp][D]
constexpr int kStageBytes = 32 * 1024;
__host__ __device__ inline int heads_per_pass(int S, int Hkv, int D, int elem) {
  const int hp = kStageBytes / (S * D * elem);
  return hp < 1 ? 1 : hp > Hkv ? Hkv : hp;
}
// Page ids of the block's target slots kept in LDS: S <= 64 tokens span at
// most 64/16 + 1 pages.
constexpr int kMaxTargetPages = 8;
// 16-byte chunks of the first pass's keys and values a thread loads before
// it knows L_b (the rest follow in the pass loop).
constexpr int kPre = 2;

template <typename T>
__global__ __launch_bounds__(kThreads) void kv_append_kernel(AppendParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  T *sv = (T *)smem;  // values of the pass's heads [S][hp][D]
  __shared__ int spg[kMaxTargetPages];
  __shared__ int bad;
  const int b = blockIdx.x;
  const T *__restrict__ kb = (const T *)p.k_blk + (size_t)b * p.S * p.Hkv * p.D;
  const T *__restrict__ vb = (const T *)p.v_blk + (size_t)b * p.S * p.Hkv * p.D;
  T *__restrict__ kp = (T *)p.k_pages;
  T *__restrict__ vp = (T *)p.v_pages;
  constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte chunk
  const bool vec = p.vec && p.D % VEC == 0;
  const int hp = heads_per_pass(p.S, p.Hkv, p.D, (int)sizeof(T));
  // The block's first chunks are loaded before L_b, so the two memory round
  // trips (the block's rows; L_b, then the page ids) overlap.
  uint4 pk[kPre], pvv[kPre];
  if (vec) {
    const int chunks = min(hp, p.Hkv) * p.D / VEC;
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
      const int e = threadIdx.x + i * kThreads;
      if (e < p.S * chunks) {
        const int t = e / chunks, c = e % chunks;
        const size_t src = (size_t)t * p.Hkv * p.D + VEC * c;
        pk[i] = *(const uint4 *)(kb + src);
        pvv[i] = *(const uint4 *)(vb + src);
      }
    }
  }
  const int L = p.ctx_lens[b];
  // Every target slot must be backed by a valid page: the page ids of the
  // slots' pages are read in parallel, checked, and kept in LDS.
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  const bool len_ok = L >= 0 && (long)L + p.S <= (long)p.max_pages * p.page_size;
  const int j0 = len_ok ? L / p.page_size : 0;
  const int npg = len_ok ? (L + p.S - 1) / p.page_size - j0 + 1 : 0;
  if ((int)threadIdx.x < npg) {
    const int pg = p.page_table[(size_t)b * p.max_pages + j0 + threadIdx.x];
    spg[threadIdx.x] = pg;
    if (pg < 0 || pg >= p.num_pages) bad = 1;
  }
  __syncthreads();
  if (!len_ok || bad) return;  // uniform over the work-group
  auto page_of = [&](int pos) { return (size_t)spg[pos / p.page_size - j0]; };
  for (int h0 = 0; h0 < p.Hkv; h0 += hp) {
    const int nh = min(hp, p.Hkv - h0);
    const int row = nh * p.D;  // elements of one token's row in this pass
    if (vec) {
      // keys: token rows, 16-byte chunks straight to their page rows; values:
      // the same rows into LDS
      const int chunks = row / VEC;
      auto load = [&](int e, uint4 &k, uint4 &v) {
        const int t = e / chunks, c = e % chunks;
        const size_t src = ((size_t)t * p.Hkv + h0) * p.D + VEC * c;
        k = *(const uint4 *)(kb + src);
        v = *(const uint4 *)(vb + src);
      };
      auto store = [&](int e, const uint4 &k, const uint4 &v) {
        const int t = e / chunks, c = e % chunks;
        const int hh = (VEC * c) / p.D, d = (VEC * c) % p.D;
        const int pos = L + t;
        *(uint4 *)(kp + ((page_of(pos) * p.Hkv + h0 + hh) * p.page_size + pos % p.page_size) * p.D + d) = k;
        *(uint4 *)(sv + t * row + VEC * c) = v;
      };
      // the first kPre chunks of a thread, unrolled so that the prefetched
      // registers are indexed by constants (a variable index would place
      // them in scratch memory)
#pragma unroll
      for (int i = 0; i < kPre; ++i) {
        const int e = threadIdx.x + i * kThreads;
        if (e < p.S * chunks) {
          uint4 k, v;
          if (h0 == 0) {
            k = pk[i];
            v = pvv[i];
          } else {
            load(e, k, v);
          }
          store(e, k, v);
        }
      }
      for (int e = threadIdx.x + kPre * kThreads; e < p.S * chunks; e += kThreads) {
        uint4 k, v;
        load(e, k, v);
        store(e, k, v);
      }
    } else {
      for (int e = threadIdx.x; e < p.S * row; e += kThreads) {
        const int t = e / row, j = e % row, hh = j / p.D, d = j % p.D;
        const size_t src = ((size_t)t * p.Hkv + h0) * p.D + j;
        const int pos = L + t;
        kp[((page_of(pos) * p.Hkv + h0 + hh) * p.page_size + pos % p.page_size) * p.D + d] = kb[src];
        sv[t * row + j] = vb[src];
      }
    }
    __syncthreads();
    // values: each feature row of a page takes the block's tokens as one run.
    // With L_b a multiple of VEC, runs of VEC tokens start 16-byte aligned and
    // never cross a page (pages hold a multiple of 16 tokens), so a thread
    // gathers VEC tokens of one feature row from LDS and stores them at once;
    // otherwise (and for a tail of fewer than VEC tokens) element by element,
    // consecutive threads writing consecutive slots of one feature row.
    const bool vs_ok = p.vvec && (L % VEC) == 0;
    const int runs = vs_ok ? p.S / VEC : 0;
    for (int e = threadIdx.x; e < runs * row; e += kThreads) {
      const int j = e / runs, r = e % runs, hh = j / p.D, d = j % p.D;
      const int t0 = VEC * r, pos = L + t0;
      T x[VEC];
#pragma unroll
      for (int k = 0; k < VEC; ++k) x[k] = sv[(t0 + k) * row + j];
      uint4 w;
      __builtin_memcpy(&w, x, sizeof w);
      *(uint4 *)(vp + ((page_of(pos) * p.Hkv + h0 + hh) * p.D + d) * p.page_size + pos % p.page_size) = w;
    }
    const int tdone = runs * VEC;  // tokens stored by the vector path
    const int tail = p.S - tdone;
    for (int e = threadIdx.x; e < tail * row; e += kThreads) {
      const int j = e / tail, t = tdone + e % tail, hh = j / p.D, d = j % p.D;
      const int pos = L + t;
      vp[((page_of(pos) * p.Hkv + h0 + hh) * p.D + d) * p.page_size + pos % p.page_size] = sv[t * row + j];
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
  p.vec = ((uintptr_t)k_blk % 16 == 0) && ((uintptr_t)v_blk % 16 == 0) &&
          ((uintptr_t)k_pages % 16 == 0);
  p.vvec = (uintptr_t)v_pages % 16 == 0;
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
