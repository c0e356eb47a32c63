// Confidence unmask ("Training and sampling", paperfeed review; "Generating
// Text in Parallel Like Solving a Sudoku", kongchang explainer): for every
// row of logits the greedy id (lowest index among equal maxima) and its
// softmax probability 1/Z, Z = sum_v exp(l_v - max); then per sequence the
// k most confident masked slots are committed (equal confidence: lower slot),
// or, in the threshold form, every masked slot above gamma (the most
// confident one when none is).
//
// Kernel 1 (rowreduce) streams the fp32 logits once, HBM-bound: each work-
// group reduces one vocabulary chunk of one row to (max, lowest argmax,
// sum exp(l - max)) with an online rescale, 16-byte non-temporal loads, wave shuffles and
// LDS.  Kernel 2 (commit) gives one wave to a sequence: lane t merges the
// chunk partials of slot t, then ranks the masked slots by (conf desc, slot
// asc) and commits those ranked below k.
#include <limits.h>

#include <mutex>

#include "tt_internal.h"

namespace tt {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;       // 16-byte loads in flight per thread
constexpr int kTargetWGs = 512;  // work-groups the row split aims for
constexpr float kLog2e = 1.4426950408889634f;

typedef UnmaskPart Part;

// exp(x - m) for x <= m; m == -inf only when every x seen is -inf (-> 0).
__device__ __forceinline__ float ex(float x, float m) {
  return __builtin_amdgcn_exp2f((x - m) * kLog2e);
}

// 16-byte streaming load.  The logits are read once, so the load is marked
// non-temporal: on cold [512, 131072] fp32 logits this took a call from 54 to
// 48 us.
__device__ __forceinline__ float4 load4(const float *p) {
  const f32x4 v = __builtin_nontemporal_load((const f32x4 *)p);
  return make_float4(v[0], v[1], v[2], v[3]);
}

struct Acc {
  float m, s;
  int idx;
  __device__ void init() { m = -INFINITY; s = 0.f; idx = INT_MAX; }
  // Four consecutive elements starting at index i (in increasing order).
  __device__ __forceinline__ void add4(float x0, float x1, float x2, float x3, int i) {
    const float mx = fmaxf(fmaxf(x0, x1), fmaxf(x2, x3));
    if (mx > m) {
      idx = i + (x0 == mx ? 0 : x1 == mx ? 1 : x2 == mx ? 2 : 3);
      s = (m == -INFINITY) ? 0.f : s * ex(m, mx);
      m = mx;
    }
    const float mm = m == -INFINITY ? 0.f : m;
    s += ex(x0, mm) + ex(x1, mm) + ex(x2, mm) + ex(x3, mm);
  }
  __device__ __forceinline__ void add1(float x, int i) {
    if (x > m) {
      idx = i;
      s = (m == -INFINITY) ? 0.f : s * ex(m, x);
      m = x;
    }
    s += ex(x, m == -INFINITY ? 0.f : m);
  }
  // Merge another partial; on equal maxima keep the lower index.
  __device__ __forceinline__ void merge(float m2, float s2, int i2) {
    const float M = fmaxf(m, m2);
    const float a = (s == 0.f) ? 0.f : s * ex(m, M);
    const float b = (s2 == 0.f) ? 0.f : s2 * ex(m2, M);
    idx = (m2 > m) ? i2 : (m > m2) ? idx : min(idx, i2);
    m = M;
    s = a + b;
  }
};

// Merges the partials parts[first], parts[first + stride], ... below `end`
// into a, eight loads in flight at a time (the merge does not depend on the
// order: max, lowest index among equal maxima, rescaled sums).
__device__ __forceinline__ void merge_parts(Acc &a, const Part *parts, int first, int end,
                                            int stride) {
  constexpr int U = 8;
  for (int c0 = first; c0 < end; c0 += U * stride) {
    Part pt[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (c0 + u * stride < end) pt[u] = parts[c0 + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (c0 + u * stride < end) a.merge(pt[u].m, pt[u].s, pt[u].idx);
  }
}

__global__ __launch_bounds__(kThreads) void unmask_rowreduce_kernel(const float *logits, int V,
                                                                    int chunk_len, int chunks,
                                                                    int vec, Part *parts) {
  const int c = blockIdx.x, r = blockIdx.y;
  const float *row = logits + (size_t)r * V;
  const int begin = c * chunk_len;
  const int end = min(begin + chunk_len, V);
  const int tid = threadIdx.x;
  Acc a;
  a.init();
  if (vec) {  // V % 4 == 0 and 16-byte aligned rows; chunk_len % 4 == 0
    const int stride = 4 * kThreads;
    int i = begin + 4 * tid;
    for (; i + (kUnroll - 1) * stride < end; i += kUnroll * stride) {
      float4 x[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) x[u] = load4(row + i + u * stride);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) a.add4(x[u].x, x[u].y, x[u].z, x[u].w, i + u * stride);
    }
    for (; i < end; i += stride) {
      const float4 x = load4(row + i);
      a.add4(x.x, x.y, x.z, x.w, i);
    }
  } else {
    for (int i = begin + tid; i < end; i += kThreads) a.add1(row[i], i);
  }
  // wave reduction
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(a.m, o, 64);
    const float s2 = __shfl_xor(a.s, o, 64);
    const int i2 = __shfl_xor(a.idx, o, 64);
    a.merge(m2, s2, i2);
  }
  __shared__ float sm[kThreads / 64], ss[kThreads / 64];
  __shared__ int si[kThreads / 64];
  const int wave = tid >> 6;
  if ((tid & 63) == 0) { sm[wave] = a.m; ss[wave] = a.s; si[wave] = a.idx; }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kThreads / 64; ++w) a.merge(sm[w], ss[w], si[w]);
    Part pt;
    pt.m = a.m; pt.s = a.s; pt.idx = a.idx; pt.pad = 0;
    parts[(size_t)r * chunks + c] = pt;
  }
}

// Commit kernels: one work-group per sequence.  First the chunk partials of
// each row are merged into the row's confidence and id in LDS; then the first
// wave ranks the sequence's masked slots.  With few chunks per row (a
// one-wave work-group) lane t merges row t's chunks itself; with many (the
// fused LM head's 256-entry tiles) each wave takes rows wave, wave + waves,
// ..., its lane j chunks j, j + 64, ..., then a wave reduction.
constexpr int kCommitWaves = 16;
constexpr int kLanePerRowChunks = 8;  // at most this many chunks: lane per row

__device__ __forceinline__ void merge_rows(const Part *parts, int chunks, int S, const uint8_t *mask,
                                           float *cs, int *is, int *ms) {
  const int b = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int waves = blockDim.x >> 6;
  if (threadIdx.x < 64 && threadIdx.x >= S) {  // slots past the block take no part
    cs[threadIdx.x] = 0.f;
    is[threadIdx.x] = 0;
    ms[threadIdx.x] = 0;
  }
  if (waves == 1) {
    const int t = lane;
    if (t < S) {
      const size_t r = (size_t)b * S + t;
      Acc a;
      a.init();
      merge_parts(a, parts + r * chunks, 0, chunks, 1);
      cs[t] = 1.f / a.s;
      is[t] = a.idx == INT_MAX ? 0 : a.idx;
      ms[t] = mask[r] != 0;
    }
    __syncthreads();
    return;
  }
  for (int t = wave; t < S; t += waves) {
    const size_t r = (size_t)b * S + t;
    Acc a;
    a.init();
    merge_parts(a, parts + r * chunks, lane, chunks, 64);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float m2 = __shfl_xor(a.m, o, 64);
      const float s2 = __shfl_xor(a.s, o, 64);
      const int i2 = __shfl_xor(a.idx, o, 64);
      a.merge(m2, s2, i2);
    }
    if (lane == 0) {
      cs[t] = 1.f / a.s;
      is[t] = a.idx == INT_MAX ? 0 : a.idx;
      ms[t] = mask[r] != 0;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(64 * kCommitWaves) void unmask_commit_kernel(
    const Part *parts, int chunks, int S, uint8_t *mask, const int32_t *k_commit, int remaining,
    int32_t *ids, uint8_t *commit, float *conf, uint32_t flags) {
  __shared__ float cs[64];
  __shared__ int is[64], ms[64];
  merge_rows(parts, chunks, S, mask, cs, is, ms);
  if (threadIdx.x >= 64) return;
  const int b = blockIdx.x, t = threadIdx.x;
  const size_t r = (size_t)b * S + t;
  const float c = cs[t];
  const int mk = ms[t];
  int n = 0;
  for (int u = 0; u < S; ++u) n += ms[u];
  // ceil(n / remaining) in 64 bits: n + remaining - 1 overflows int for
  // remaining_steps near INT_MAX
  int kb = k_commit ? k_commit[b] : (int)(((long long)n + remaining - 1) / remaining);
  kb = min(max(kb, 0), n);
  if (t < S) {
    int rank = 0;
    for (int u = 0; u < S; ++u)
      rank += (ms[u] && (cs[u] > c || (cs[u] == c && u < t))) ? 1 : 0;
    const int com = (mk && rank < kb) ? 1 : 0;
    ids[r] = is[t];
    commit[r] = (uint8_t)com;
    if (conf) conf[r] = c;
    if ((flags & TT_UNMASK_UPDATE_MASK) && com) mask[r] = 0;
  }
}

// Threshold form: every masked slot with conf > gamma commits; if none does,
// the masked slot ranked first by (conf desc, slot asc) does.
__global__ __launch_bounds__(64 * kCommitWaves) void unmask_threshold_commit_kernel(
    const Part *parts, int chunks, int S, uint8_t *mask, float gamma, int32_t *ids,
    uint8_t *commit, float *conf, int32_t *nsteps, uint32_t flags) {
  __shared__ float cs[64];
  __shared__ int is[64], ms[64];
  merge_rows(parts, chunks, S, mask, cs, is, ms);
  if (threadIdx.x >= 64) return;
  const int b = blockIdx.x, t = threadIdx.x;
  const size_t r = (size_t)b * S + t;
  const float c = cs[t];
  const int mk = ms[t];
  int n = 0, n_above = 0;
  for (int u = 0; u < S; ++u) {
    n += ms[u];
    n_above += (ms[u] && cs[u] > gamma) ? 1 : 0;
  }
  if (t < S) {
    int com;
    if (n_above > 0) {
      com = (mk && c > gamma) ? 1 : 0;
    } else {
      int rank = 0;
      for (int u = 0; u < S; ++u)
        rank += (ms[u] && (cs[u] > c || (cs[u] == c && u < t))) ? 1 : 0;
      com = (mk && rank == 0) ? 1 : 0;
    }
    ids[r] = is[t];
    commit[r] = (uint8_t)com;
    if (conf) conf[r] = c;
    if ((flags & TT_UNMASK_UPDATE_MASK) && com) mask[r] = 0;
  }
  if (t == 0 && nsteps && n > 0) nsteps[b] += 1;
}

}  // namespace

// threads of a commit work-group: one wave when rows have few chunks, else a
// wave per row (up to kCommitWaves)
static int commit_threads(int chunks, int S) {
  return chunks <= kLanePerRowChunks ? 64 : 64 * (S < kCommitWaves ? S : kCommitWaves);
}

hipError_t launch_unmask_commit(const UnmaskPart *parts, int chunks, int B, int S, uint8_t *mask,
                                const int32_t *k_commit, int remaining_steps, int32_t *ids,
                                uint8_t *commit, float *conf, uint32_t flags, hipStream_t stream) {
  hipLaunchKernelGGL(unmask_commit_kernel, dim3(B), dim3(commit_threads(chunks, S)), 0, stream, parts,
                     chunks, S, mask, k_commit, remaining_steps, ids, commit, conf, flags);
  return hipGetLastError();
}

hipError_t launch_unmask_threshold_commit(const UnmaskPart *parts, int chunks, int B, int S,
                                          uint8_t *mask, float gamma, int32_t *ids,
                                          uint8_t *commit, float *conf, int32_t *nsteps,
                                          uint32_t flags, hipStream_t stream) {
  hipLaunchKernelGGL(unmask_threshold_commit_kernel, dim3(B), dim3(commit_threads(chunks, S)), 0,
                     stream, parts, chunks, S, mask, gamma, ids, commit, conf, nsteps, flags);
  return hipGetLastError();
}

UnmaskPlan plan_unmask(int B, int S, int V) {
  UnmaskPlan p{};
  p.B = B; p.S = S; p.V = V;
  const long rows = (long)B * S;
  const int per_wg = 4 * kThreads * kUnroll;  // elements one pass of a work-group covers
  const int max_chunks = (V + per_wg - 1) / per_wg;
  long want = rows > 0 ? (kTargetWGs + rows - 1) / rows : 1;  // aim for >= kTargetWGs work-groups
  if (want > max_chunks) want = max_chunks;
  if (want < 1) want = 1;
  int chunk_len = (int)((V + want - 1) / want);
  chunk_len = (chunk_len + 3) & ~3;
  p.chunk_len = chunk_len;
  p.chunks = (V + chunk_len - 1) / chunk_len;
  p.ws_bytes = (size_t)rows * p.chunks * sizeof(Part);
  return p;
}

static hipError_t launch_rowreduce(const UnmaskPlan &p, const float *logits, Part *parts,
                                   hipStream_t stream) {
  const int vec = (p.V % 4 == 0) && (((uintptr_t)logits & 15) == 0);
  hipLaunchKernelGGL(unmask_rowreduce_kernel, dim3(p.chunks, p.B * p.S), dim3(kThreads), 0,
                     stream, logits, p.V, p.chunk_len, p.chunks, vec, parts);
  return hipGetLastError();
}

hipError_t launch_unmask(const UnmaskPlan &p, const float *logits, uint8_t *mask,
                         const int32_t *k_commit, int remaining_steps, int32_t *ids,
                         uint8_t *commit, float *conf, uint32_t flags, void *workspace,
                         hipStream_t stream) {
  Part *parts = (Part *)workspace;
  hipError_t e = launch_rowreduce(p, logits, parts, stream);
  if (e != hipSuccess) return e;
  return launch_unmask_commit(parts, p.chunks, p.B, p.S, mask, k_commit, remaining_steps, ids,
                              commit, conf, flags, stream);
}

hipError_t launch_unmask_threshold(const UnmaskPlan &p, const float *logits, uint8_t *mask,
                                   float gamma, int32_t *ids, uint8_t *commit, float *conf,
                                   int32_t *nsteps, uint32_t flags, void *workspace,
                                   hipStream_t stream) {
  Part *parts = (Part *)workspace;
  hipError_t e = launch_rowreduce(p, logits, parts, stream);
  if (e != hipSuccess) return e;
  return launch_unmask_threshold_commit(parts, p.chunks, p.B, p.S, mask, gamma, ids, commit, conf,
                                        nsteps, flags, stream);
}

// Row partials of tt_unmask_noalloc: a static device array instead of a
// caller workspace, for callers that cannot allocate.  Each device holds its
// own copy until the process ends; in host code `scratch` names a host-side
// stand-in, so kernels get the device address that
// hipGetSymbolAddress reports, looked up once per device.
__device__ __align__(256) unsigned char scratch[kUnmaskStaticBytes];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kScratchDevices];
}  // namespace

hipError_t unmask_static_scratch(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace tt
