// bf16 block attention on gfx950 MFMA: split over a flat list of KV tiles
// ("stream-K" style) with an LSE combine across splits.
//
// Operation ("The idea: freeze the reader, train the writer", paperfeed
// review; "The 'Sky Bridges' Between Layers", kongchang explainer): the
// S*g query rows that share one KV head (S block slots x g heads of the GQA
// group) attend over [L_b context tokens read through the page table ; the
// S block tokens], softmax over all of them, no mask.
//
// Work decomposition.  A *unit* is (sequence b, KV head h, query chunk of up
// to 256 rows).  A unit's keys are cut into 64-token *tiles*: ceil(L_b/64)
// context tiles followed by one tile holding the S block tokens.  All tiles of
// all units form one flat list; work-group w of G takes the contiguous range
// [w*R, (w+1)*R), R = ceil(total/G).  Units wholly inside a range are finished
// in place; a unit cut by a range boundary leaves an unnormalised fp32 partial
// (O^T, running max, running sum) in one of the work-group's two workspace
// slots, and the combine kernel merges those partials.  Each block token is
// therefore seen exactly once, and no work-group holds more than two
// partials.  The plan is rebuilt on the device from ctx_lens, so the host
// never needs the lengths.
//
// Per work-group: 256 query rows, 32 * kQB of them per wave.
// Per tile: K (token-major) and V^T (feature-major, as stored in the pool) are
// staged through LDS; S^T = K . Q^T and O^T += V^T . P^T run on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation, Q stays in registers, and
// the online softmax works in the log2 domain with a lazily updated
// reference maximum (the accumulators are only rescaled when the running max
// grows by more than 2^8).
#include <float.h>

#include "tt_internal.h"

namespace tt {
namespace {

constexpr int kTile = 64;        // keys per tile
constexpr int kQRows = 256;      // query rows per unit
constexpr int kQB = 1;           // 32-row query blocks per wave
constexpr int kThreads = 64 * (kQRows / 32) / kQB;  // waves x 64 lanes
constexpr int kCombineThreads = kQRows;
constexpr int kMinTiles = 8;     // smallest range worth a work-group
constexpr float kLazy = 8.0f;    // rescale when max grows by > 2^kLazy

template <int D>
struct Geo {
  static constexpr int KS = D / 16;                     // MFMA k-steps over D
  static constexpr int DB = D / 32;                     // 32-row blocks of O^T
  static constexpr int KROW = D + 8;                    // LDS row pitch of K (elements)
  static constexpr int VROW = kTile + 8;                // LDS row pitch of V^T
  static constexpr int KCH = D / 8;                     // 16-byte chunks per key row
  static constexpr int KPT = kTile * KCH / kThreads;    // key chunks per thread
  static constexpr int VPT = D * (kTile / 8) / kThreads;  // value chunks per thread
  static constexpr int K_ELEMS = kTile * KROW;
  static constexpr int V_ELEMS = D * VROW;
  static constexpr size_t LDS_TILE_BYTES = (size_t)(K_ELEMS + V_ELEMS) * 2;
  static_assert(KPT >= 1 && VPT >= 1, "tile too small for the work-group");
};

struct Params {
  const __bf16 *q, *k_blk, *v_blk, *k_pages, *v_pages;
  const int32_t *page_table, *ctx_lens;
  __bf16 *out;
  float *ws_o;   // [2G][D][256] unnormalised O^T partials
  float *ws_ml;  // [2G][256][2]  (reference max in log2 units, sum)
  int B, S, Hq, Hkv, g, page_size, lps, max_pages, num_pages, max_ctx, qchunks, G;
  float sl2;
};

__device__ __forceinline__ int seq_len(const Params &p, int b) {
  const int L = p.ctx_lens[b];
  return min(max(L, 0), p.max_ctx);
}

__device__ __forceinline__ int seq_tiles(int L) { return (L + kTile - 1) / kTile + 1; }

// pre[b] = first flat tile of sequence b (all its units), pre[B] = total.
template <int NT>
__device__ void build_prefix(const Params &p, int *pre, int *scan) {
  const int tid = threadIdx.x;
  const int per = (p.B + NT - 1) / NT;
  const int upb = p.Hkv * p.qchunks;
  int local = 0;
  for (int i = 0; i < per; ++i) {
    const int b = tid * per + i;
    if (b < p.B) local += seq_tiles(seq_len(p, b)) * upb;
  }
  scan[tid] = local;
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {
    const int v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  int run = scan[tid] - local;
  for (int i = 0; i < per; ++i) {
    const int b = tid * per + i;
    if (b < p.B) {
      pre[b] = run;
      run += seq_tiles(seq_len(p, b)) * upb;
    }
  }
  if (tid == NT - 1) pre[p.B] = scan[tid];
  __syncthreads();
}

struct Unit {
  int b, h, qc, L, T, start, id;
};

// The unit that owns flat tile t.
__device__ Unit locate(const Params &p, const int *pre, int t) {
  int lo = 0, hi = p.B;  // pre[lo] <= t < pre[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= t) lo = mid; else hi = mid;
  }
  Unit u;
  u.b = lo;
  u.L = seq_len(p, lo);
  u.T = seq_tiles(u.L);
  const int ui = (t - pre[lo]) / u.T;
  u.h = ui / p.qchunks;
  u.qc = ui % p.qchunks;
  u.start = pre[lo] + ui * u.T;
  u.id = lo * p.Hkv * p.qchunks + ui;
  return u;
}

// Swap bits 2 and 3 of an MFMA row index.  Key row m of a 32-key block is
// stored at LDS row pi(m), so that the S^T accumulator registers 8c..8c+7 of
// lane half h hold keys 16c+8h .. 16c+8h+7 (contiguous), which is exactly the
// B-operand order P.V needs; no cross-lane shuffle of P is required.
__device__ __forceinline__ int pi_row(int m) {
  return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ __forceinline__ int clamp_page(int pg, int num_pages) {
  return min(max(pg, 0), num_pages - 1);
}

// Keep the first n (clamped to 0..8) bf16 lanes of an 8 x bf16 chunk, zero the rest.
__device__ __forceinline__ uint4 keep_first(uint4 v, int n) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 2 * i;
    const uint32_t m = e >= n ? 0u : (e + 1 >= n ? 0xFFFFu : 0xFFFFFFFFu);
    w[i] &= m;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ uint4 sel(bool c, uint4 a) {
  return c ? a : make_uint4(0, 0, 0, 0);
}

template <int D>
struct TileRegs {
  uint4 k[Geo<D>::KPT];
  uint4 v[Geo<D>::VPT];
};

// Global -> registers for context tile i of unit u (u.L >= 1 whenever a
// context tile exists).  Addresses past the context are clamped into it and the
// loaded values replaced by zeros, so the loads are branch-free.  `tile_page`
// is the physical page of the whole tile when page_size >= kTile (pages then
// never straddle a tile), else -1 and each chunk looks its page up.
template <int D>
__device__ __forceinline__ void load_ctx_tile(const Params &p, const Unit &u, int i,
                                              int tile_page, TileRegs<D> &r) {
  using G = Geo<D>;
  const int tid = threadIdx.x;
  const int tok0 = i * kTile;
  const int pmask = p.page_size - 1;
  const int32_t *pt = p.page_table + (size_t)u.b * p.max_pages;
#pragma unroll
  for (int kk = 0; kk < G::KPT; ++kk) {
    const int idx = tid + kThreads * kk;
    const int row = idx / G::KCH, c = idx % G::KCH;
    const int pos = tok0 + row;
    const bool valid = pos < u.L;
    const int posc = valid ? pos : u.L - 1;
    const int pg = tile_page >= 0 ? tile_page : clamp_page(pt[posc >> p.lps], p.num_pages);
    const uint4 x = *(const uint4 *)(p.k_pages +
                                     (((size_t)pg * p.Hkv + u.h) * p.page_size + (posc & pmask)) * D +
                                     8 * c);
    r.k[kk] = sel(valid, x);
  }
#pragma unroll
  for (int vv = 0; vv < G::VPT; ++vv) {
    const int idx = tid + kThreads * vv;
    const int d = idx >> 3, c = idx & 7;
    const int pos0 = tok0 + 8 * c;
    const int n = u.L - pos0;  // valid tokens in this 8-token chunk (may be <= 0 or >= 8)
    const int posc = n > 0 ? pos0 : ((u.L - 1) & ~7);
    const int pg = tile_page >= 0 ? tile_page : clamp_page(pt[posc >> p.lps], p.num_pages);
    const uint4 x = *(const uint4 *)(p.v_pages +
                                     (((size_t)pg * p.Hkv + u.h) * D + d) * p.page_size + (posc & pmask));
    r.v[vv] = keep_first(x, n);
  }
}

// Global -> registers for the block's own S keys/values (the unit's last tile).
template <int D>
__device__ __forceinline__ void load_blk_tile(const Params &p, const Unit &u, TileRegs<D> &r) {
  using G = Geo<D>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int kk = 0; kk < G::KPT; ++kk) {
    const int idx = tid + kThreads * kk;
    const int row = idx / G::KCH, c = idx % G::KCH;
    const int rc = min(row, p.S - 1);
    const uint4 x = *(const uint4 *)(p.k_blk + (((size_t)u.b * p.S + rc) * p.Hkv + u.h) * D + 8 * c);
    r.k[kk] = sel(row < p.S, x);
  }
  const uint16_t *vb = (const uint16_t *)p.v_blk;
#pragma unroll
  for (int vv = 0; vv < G::VPT; ++vv) {
    const int idx = tid + kThreads * vv;
    const int d = idx >> 3, c = idx & 7;
    uint32_t w[4];
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
      const int t0 = 8 * c + 2 * i2, t1 = t0 + 1;
      const uint32_t lo = vb[(((size_t)u.b * p.S + min(t0, p.S - 1)) * p.Hkv + u.h) * D + d];
      const uint32_t hi = vb[(((size_t)u.b * p.S + min(t1, p.S - 1)) * p.Hkv + u.h) * D + d];
      w[i2] = (t0 < p.S ? lo : 0u) | ((t1 < p.S ? hi : 0u) << 16);
    }
    r.v[vv] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Physical page of context tile i when one page covers the tile, else -1.
__device__ __forceinline__ int tile_page_of(const Params &p, const Unit &u, int i) {
  if (p.page_size < kTile || i >= u.T - 1) return -1;
  return clamp_page(p.page_table[(size_t)u.b * p.max_pages + ((i * kTile) >> p.lps)], p.num_pages);
}

template <int D>
__device__ __forceinline__ void load_tile(const Params &p, const Unit &u, int i, int tile_page,
                                          TileRegs<D> &r) {
  if (i < u.T - 1) load_ctx_tile<D>(p, u, i, tile_page, r);
  else load_blk_tile<D>(p, u, r);
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D> &r, __bf16 *Ks, __bf16 *Vs) {
  using G = Geo<D>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int kk = 0; kk < G::KPT; ++kk) {
    const int idx = tid + kThreads * kk;
    const int row = idx / G::KCH, c = idx % G::KCH;
    const int lrow = (row & ~31) | pi_row(row & 31);
    *(uint4 *)(Ks + lrow * G::KROW + 8 * c) = r.k[kk];
  }
#pragma unroll
  for (int vv = 0; vv < G::VPT; ++vv) {
    const int idx = tid + kThreads * vv;
    const int d = idx >> 3, c = idx & 7;
    *(uint4 *)(Vs + d * G::VROW + 8 * c) = r.v[vv];
  }
}

// Reductions over the lane pair (l, l ^ 32).  v_permlane32_swap exchanges the
// upper half of its first operand with the lower half of its second; feeding
// x as both operands leaves, at every lane, x[l % 32] in one output and
// x[l % 32 + 32] in the other, so a commutative op over the two outputs is the
// pair reduction, bit-identical in both halves.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
__device__ void run_unit(const Params &p, const Unit &u, int i0, int i1, bool complete,
                         int slot, __bf16 *Ks, __bf16 *Vs) {
  using G = Geo<D>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ln = lane & 31, hl = lane >> 5;
  const int M = p.S * p.g;
  constexpr int WROWS = 32 * kQB;  // query rows per wave

  // Q (B operand of S^T = K . Q^T): lane holds row ln of each 32-row block,
  // features 16*ks + 8*hl .. +7.
  bf16x8 qr[kQB][G::KS];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int qi = u.qc * kQRows + wave * WROWS + qb * 32 + ln;
    if (qi < M) {
      const int t = qi / p.g, j = qi % p.g;
      const __bf16 *src = p.q + (((size_t)u.b * p.S + t) * p.Hq + u.h * p.g + j) * D + 8 * hl;
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks) qr[qb][ks] = *(const bf16x8 *)(src + 16 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks) qr[qb][ks] = bf16x8{};
    }
  }

  f32x16 o[G::DB][kQB];
#pragma unroll
  for (int db = 0; db < G::DB; ++db)
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) o[db][qb] = f32x16{};
  float mref[kQB], lsum[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) { mref[qb] = -INFINITY; lsum[qb] = 0.f; }

  TileRegs<D> regs;
  load_tile<D>(p, u, i0, tile_page_of(p, u, i0), regs);
  store_tile<D>(regs, Ks, Vs);
  int next_page = tile_page_of(p, u, i0 + 1);
  __syncthreads();

  for (int i = i0; i < i1; ++i) {
    const bool more = i + 1 < i1;
    if (more) {
      load_tile<D>(p, u, i + 1, next_page, regs);
      next_page = tile_page_of(p, u, i + 2);
    }
    const int nvalid = (i < u.T - 1) ? min(kTile, u.L - i * kTile) : p.S;

    // ---- S^T[key][query] for two 32-key blocks
    f32x16 s[2][kQB];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) s[tb][qb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks) {
        const bf16x8 a = *(const bf16x8 *)(Ks + (32 * tb + ln) * G::KROW + 16 * ks + 8 * hl);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          s[tb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qr[qb][ks], s[tb][qb], 0, 0, 0);
      }
    }
    // key index of accumulator register r in lane half hl: 32*tb + 16*(r/8) + 8*hl + r%8
    if (nvalid < kTile) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * tb + 16 * (r >> 3) + 8 * hl + (r & 7);
          if (key >= nvalid) {
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) s[tb][qb][r] = -INFINITY;
          }
        }
    }

    // ---- online softmax (log2 domain), P rounded to bf16
    bf16x8 pk[2][kQB][2];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[tb][qb][r]);
      mx = pair_max(mx);
      const float mxs = mx * p.sl2;
      const bool need = mxs > mref[qb] + kLazy;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float f = need ? __builtin_amdgcn_exp2f(mref[qb] - mxs) : 1.f;
        if (need) mref[qb] = mxs;
        lsum[qb] *= f;
#pragma unroll
        for (int db = 0; db < G::DB; ++db) o[db][qb] *= f;
      }
      const float nm = -mref[qb];
      float acc = 0.f;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        f32x16 e;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[tb][qb][r], p.sl2, nm));
          acc += e[r];
        }
        f32x8 lo = {e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]};
        f32x8 hi = {e[8], e[9], e[10], e[11], e[12], e[13], e[14], e[15]};
        pk[tb][qb][0] = __builtin_convertvector(lo, bf16x8);
        pk[tb][qb][1] = __builtin_convertvector(hi, bf16x8);
      }
      lsum[qb] += acc;
    }

    // ---- O^T[d][query] += V^T . P^T
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int db = 0; db < G::DB; ++db) {
          const bf16x8 a =
              *(const bf16x8 *)(Vs + (32 * db + ln) * G::VROW + 32 * tb + 16 * cc + 8 * hl);
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb)
            o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[tb][qb][cc], o[db][qb], 0, 0, 0);
        }

    __syncthreads();
    if (more) store_tile<D>(regs, Ks, Vs);
    __syncthreads();
  }

  // ---- epilogue.  O^T accumulator register r of lane (hl, ln) in block db
  // holds feature 32*db + 8*(r/4) + 4*hl + r%4 of query row ln.
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const float ltot = pair_sum(lsum[qb]);
    const int qloc = wave * WROWS + qb * 32 + ln;
    const int qi = u.qc * kQRows + qloc;
    if (complete) {
      if (qi < M) {
        const float inv = 1.f / ltot;
        const int t = qi / p.g, j = qi % p.g;
        __bf16 *dst = p.out + (((size_t)u.b * p.S + t) * p.Hq + u.h * p.g + j) * D;
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            f32x4 v = {o[db][qb][4 * r4 + 0] * inv, o[db][qb][4 * r4 + 1] * inv,
                       o[db][qb][4 * r4 + 2] * inv, o[db][qb][4 * r4 + 3] * inv};
            *(bf16x4 *)(dst + 32 * db + 8 * r4 + 4 * hl) = __builtin_convertvector(v, bf16x4);
          }
      }
    } else {
      float *wo = p.ws_o + (size_t)slot * D * kQRows;
#pragma unroll
      for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int d = 32 * db + 8 * (r >> 2) + 4 * hl + (r & 3);
          wo[(size_t)d * kQRows + qloc] = o[db][qb][r];
        }
      if (hl == 0) {
        float *wm = p.ws_ml + ((size_t)slot * kQRows + qloc) * 2;
        wm[0] = mref[qb];
        wm[1] = ltot;
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void attn_split_kernel(Params p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int scan[kThreads];
  __bf16 *Ks = (__bf16 *)smem;
  __bf16 *Vs = Ks + Geo<D>::K_ELEMS;
  int *pre = (int *)(smem + Geo<D>::LDS_TILE_BYTES);
  build_prefix<kThreads>(p, pre, scan);
  const int total = pre[p.B];
  const int R = (total + p.G - 1) / p.G;
  const int t_begin = blockIdx.x * R;
  const int t_end = min(t_begin + R, total);
  bool first = true;
  for (int t = t_begin; t < t_end;) {
    const Unit u = locate(p, pre, t);
    const int i0 = t - u.start;
    const int i1 = min(t_end, u.start + u.T) - u.start;
    run_unit<D>(p, u, i0, i1, i0 == 0 && i1 == u.T, 2 * blockIdx.x + (first ? 0 : 1), Ks, Vs);
    first = false;
    t = u.start + i1;
  }
}

// One work-group per unit; merges the partials of units cut by a range
// boundary: O = sum_w 2^(m_w - M) O_w / sum_w 2^(m_w - M) l_w.
template <int D>
__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(Params p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int scan[kCombineThreads];
  int *pre = (int *)smem;
  build_prefix<kCombineThreads>(p, pre, scan);
  const int upb = p.Hkv * p.qchunks;
  const int uid = blockIdx.x;
  const int b = uid / upb, ui = uid % upb;
  const int h = ui / p.qchunks, qc = ui % p.qchunks;
  const int T = seq_tiles(seq_len(p, b));
  const int us = pre[b] + ui * T, ue = us + T;
  const int total = pre[p.B];
  const int R = (total + p.G - 1) / p.G;
  const int w_lo = us / R, w_hi = (ue - 1) / R;
  if (w_lo == w_hi) return;  // finished in place
  const int qloc = threadIdx.x;
  const int qi = qc * kQRows + qloc;
  if (qi >= p.S * p.g) return;

  float M = -INFINITY;
  for (int w = w_lo; w <= w_hi; ++w) {
    const int slot = 2 * w + (locate(p, pre, w * R).id == uid ? 0 : 1);
    M = fmaxf(M, p.ws_ml[((size_t)slot * kQRows + qloc) * 2]);
  }
  float lt = 0.f;
  for (int w = w_lo; w <= w_hi; ++w) {
    const int slot = 2 * w + (locate(p, pre, w * R).id == uid ? 0 : 1);
    const float *m = p.ws_ml + ((size_t)slot * kQRows + qloc) * 2;
    lt += __builtin_amdgcn_exp2f(m[0] - M) * m[1];
  }
  const float inv = 1.f / lt;
  const int t = qi / p.g, j = qi % p.g;
  __bf16 *dst = p.out + (((size_t)b * p.S + t) * p.Hq + h * p.g + j) * D;
  for (int dc = 0; dc < D / 8; ++dc) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int w = w_lo; w <= w_hi; ++w) {
      const int slot = 2 * w + (locate(p, pre, w * R).id == uid ? 0 : 1);
      const float wt = __builtin_amdgcn_exp2f(p.ws_ml[((size_t)slot * kQRows + qloc) * 2] - M) * inv;
      const float *src = p.ws_o + ((size_t)slot * D + 8 * dc) * kQRows + qloc;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += wt * src[(size_t)e * kQRows];
    }
    f32x8 v = {acc[0], acc[1], acc[2], acc[3], acc[4], acc[5], acc[6], acc[7]};
    *(bf16x8 *)(dst + 8 * dc) = __builtin_convertvector(v, bf16x8);
  }
}

template <int D>
hipError_t launch_d(const Params &prm, hipStream_t stream) {
  const size_t pre_bytes = (size_t)(prm.B + 1) * sizeof(int);
  hipLaunchKernelGGL(attn_split_kernel<D>, dim3(prm.G), dim3(kThreads),
                     Geo<D>::LDS_TILE_BYTES + pre_bytes, stream, prm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel<D>, dim3(prm.B * prm.Hkv * prm.qchunks), dim3(kCombineThreads),
                     pre_bytes, stream, prm);
  return hipGetLastError();
}

}  // namespace

AttnPlan plan_bf16_attn(const tt_attn_desc &d, int cus) {
  AttnPlan p{};
  p.B = d.batch; p.S = d.block; p.Hq = d.heads_q; p.Hkv = d.heads_kv;
  p.g = d.heads_q / d.heads_kv; p.D = d.head_dim;
  p.page_size = d.page_size; p.max_pages = d.max_pages_per_seq; p.num_pages = d.num_pages;
  p.max_ctx = d.max_ctx_len;
  p.qchunks = (p.S * p.g + kQRows - 1) / kQRows;
  const float scale = d.scale > 0.f ? d.scale : 1.0f / sqrtf((float)p.D);
  p.scale_log2 = scale * 1.4426950408889634f;
  const long tiles = (long)p.B * p.Hkv * p.qchunks * ((p.max_ctx + kTile - 1) / kTile + 1);
  long G = (tiles + kMinTiles - 1) / kMinTiles;
  if (G > cus) G = cus;
  if (G < 1) G = 1;
  p.G = (int)G;
  p.ws_bytes = (size_t)2 * G * ((size_t)p.D * kQRows + 2 * kQRows) * sizeof(float);
  return p;
}

hipError_t launch_attn_bf16(const AttnPlan &pl, const void *q, const void *k_blk,
                            const void *v_blk, const void *k_pages, const void *v_pages,
                            const int32_t *page_table, const int32_t *ctx_lens, void *out,
                            void *workspace, hipStream_t stream) {
  Params prm;
  prm.q = (const __bf16 *)q; prm.k_blk = (const __bf16 *)k_blk; prm.v_blk = (const __bf16 *)v_blk;
  prm.k_pages = (const __bf16 *)k_pages; prm.v_pages = (const __bf16 *)v_pages;
  prm.page_table = page_table; prm.ctx_lens = ctx_lens;
  prm.out = (__bf16 *)out;
  prm.ws_o = (float *)workspace;
  prm.ws_ml = prm.ws_o + (size_t)2 * pl.G * pl.D * kQRows;
  prm.B = pl.B; prm.S = pl.S; prm.Hq = pl.Hq; prm.Hkv = pl.Hkv; prm.g = pl.g;
  prm.page_size = pl.page_size; prm.lps = __builtin_ctz((unsigned)pl.page_size);
  prm.max_pages = pl.max_pages; prm.num_pages = pl.num_pages;
  prm.max_ctx = pl.max_ctx; prm.qchunks = pl.qchunks; prm.G = pl.G; prm.sl2 = pl.scale_log2;
  if (pl.max_ctx == 0) {  // no context is ever read; keep the pointers harmless
    prm.num_pages = 1;
  }
  return pl.D == 128 ? launch_d<128>(prm, stream) : launch_d<64>(prm, stream);
}

}  // namespace tt
