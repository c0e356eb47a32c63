// fp32 block attention for small problems ("The idea: freeze the reader,
// train the writer", paperfeed review): one wave per query row (b, t, h)
// walks the keys of [context (paged) ; block] in groups of 64 (one key per
// lane), with an fp32 online softmax and fp32 accumulation of O.  Not tuned:
// the bf16 MFMA kernel is the throughput path.
#include "tt_internal.h"

namespace tt {
namespace {

constexpr int kMaxD = 256;

struct F32Params {
  const float *q, *k_blk, *v_blk, *k_pages, *v_pages;
  const int32_t *page_table, *ctx_lens;
  float *out;
  int B, S, Hq, Hkv, g, D, page_size, max_pages, num_pages, max_ctx;
  int causal;  // chunk ingest: block position t sees block keys 0..t only
  float scale;
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__global__ __launch_bounds__(64) void attn_f32_kernel(F32Params p) {
  __shared__ float qs[kMaxD];
  __shared__ float ps[64];
  const int lane = threadIdx.x;
  const int row = blockIdx.x;
  const int b = row / (p.S * p.Hq), t = (row / p.Hq) % p.S, h = row % p.Hq;
  const int hk = h / p.g;
  const int L = min(max(p.ctx_lens[b], 0), p.max_ctx);
  const int N = L + (p.causal ? t + 1 : p.S);  // context, then the visible block keys
  const int32_t *pt = p.page_table + (size_t)b * p.max_pages;
  const float *qrow = p.q + (((size_t)b * p.S + t) * p.Hq + h) * p.D;
  for (int d = lane; d < p.D; d += 64) qs[d] = qrow[d];
  __syncthreads();

  float m = -INFINITY, l = 0.f;
  float o[kMaxD / 64] = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < N; j0 += 64) {
    const int j = j0 + lane;
    float s = -INFINITY;
    if (j < N) {
      const float *krow;
      if (j < L) {
        const int pg = min(max(pt[j / p.page_size], 0), p.num_pages - 1);
        krow = p.k_pages + (((size_t)pg * p.Hkv + hk) * p.page_size + j % p.page_size) * p.D;
      } else {
        krow = p.k_blk + (((size_t)b * p.S + (j - L)) * p.Hkv + hk) * p.D;
      }
      float acc = 0.f;
      for (int d = 0; d < p.D; ++d) acc = __builtin_fmaf(qs[d], krow[d], acc);
      s = acc * p.scale;
    }
    const float mn = fmaxf(m, wave_max(s));
    const float f = m == -INFINITY ? 0.f : expf(m - mn);
    l *= f;
#pragma unroll
    for (int k = 0; k < kMaxD / 64; ++k) o[k] *= f;
    m = mn;
    const float pj = j < N ? expf(s - m) : 0.f;
    l += pj;
    ps[lane] = pj;
    __syncthreads();
    const int nj = min(64, N - j0);
    for (int jj = 0; jj < nj; ++jj) {
      const int jg = j0 + jj;
      const float w = ps[jj];
      const float *vbase;
      size_t vstride;
      if (jg < L) {
        const int pg = min(max(pt[jg / p.page_size], 0), p.num_pages - 1);
        vbase = p.v_pages + ((size_t)pg * p.Hkv + hk) * p.D * p.page_size + jg % p.page_size;
        vstride = p.page_size;
      } else {
        vbase = p.v_blk + (((size_t)b * p.S + (jg - L)) * p.Hkv + hk) * p.D;
        vstride = 1;
      }
#pragma unroll
      for (int k = 0; k < kMaxD / 64; ++k) {
        const int d = lane + 64 * k;
        if (d < p.D) o[k] = __builtin_fmaf(w, vbase[(size_t)d * vstride], o[k]);
      }
    }
    __syncthreads();
  }
  const float inv = 1.f / wave_sum(l);
  float *orow = p.out + (((size_t)b * p.S + t) * p.Hq + h) * p.D;
#pragma unroll
  for (int k = 0; k < kMaxD / 64; ++k) {
    const int d = lane + 64 * k;
    if (d < p.D) orow[d] = o[k] * inv;
  }
}

}  // namespace

hipError_t launch_attn_f32(const tt_attn_desc &d, float scale, const float *q,
                           const float *k_blk, const float *v_blk, const float *k_pages,
                           const float *v_pages, const int32_t *page_table,
                           const int32_t *ctx_lens, float *out, int causal, hipStream_t stream) {
  F32Params p;
  p.causal = causal;
  p.q = q; p.k_blk = k_blk; p.v_blk = v_blk; p.k_pages = k_pages; p.v_pages = v_pages;
  p.page_table = page_table; p.ctx_lens = ctx_lens; p.out = out;
  p.B = d.batch; p.S = d.block; p.Hq = d.heads_q; p.Hkv = d.heads_kv;
  p.g = d.heads_q / d.heads_kv; p.D = d.head_dim; p.page_size = d.page_size;
  p.max_pages = d.max_pages_per_seq; p.num_pages = d.num_pages > 0 ? d.num_pages : 1;
  p.max_ctx = d.max_ctx_len; p.scale = scale;
  const long rows = (long)p.B * p.S * p.Hq;
  hipLaunchKernelGGL(attn_f32_kernel, dim3((unsigned)rows), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace tt
