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
// to 256 rows).  The keys of a (b, h) pair are cut into 64-token *tiles*:
// ceil(L_b/64) context tiles, one tile holding the S block tokens, then
// kUnitPad virtual tiles that only stand for a unit's fixed cost.  The tiles
// of all (b, h) pairs form one flat list.  The G work-groups form G/Q teams
// of Q = (query chunks per pair) members; team k takes the range [k*R,
// (k+1)*R), R = ceil(total/(G/Q)), and member m computes query chunk m over
// it, so the Q chunks of a pair stream the same context tiles side by side.
// Ranges go to the work-groups so that each XCD holds a contiguous block of
// them: a team, and the teams that share a unit, then share an L2, and the
// context of a pair is fetched from HBM about once.  Units wholly inside a range are
// finished in place; a unit cut by a range boundary leaves a partial
// (O^T / l in bf16, running max and running sum l in fp32) in one of the
// work-group's two workspace slots, and the combine kernel merges those
// partials.  Each block token is therefore seen exactly once.  The plan is
// rebuilt on the device from ctx_lens, so the host never needs the lengths.
//
// Waves are split into a lead and a lag group sharing the SIMDs: the lag
// group runs one pipeline stage behind (P.V of the previous tile first), so
// the two waves on a SIMD are in different phases and one's softmax VALU
// work overlaps the other's MFMAs.
//
// Per work-group: 8 waves, 32 query rows each.  Context tiles stream from HBM
// straight into a ring of kStages LDS buffers with global_load_lds_dwordx4
// (no register staging); page ids of the range are cached in LDS first, so
// the tile loop issues no other vector-memory operation and the ring is
// synchronised with exact vmcnt waits.  Per tile: S^T = K . Q^T and
// O^T += V^T . P^T on v_mfma_f32_32x32x16_bf16 (fp32 accumulate), Q held in
// registers, online softmax in the log2 domain with a lazily updated
// reference maximum (accumulators are rescaled only when the running max
// grows by more than 2^8).
#include <float.h>

#include "tt_internal.h"

namespace tt {
namespace {

constexpr int kTile = 64;        // keys per tile
constexpr int kQRows = 256;      // query rows per unit
#ifndef TT_ATTN_STAGES
#define TT_ATTN_STAGES 4
#endif
constexpr int kThreads = 64 * (kQRows / 32);  // one wave per 32 query rows
constexpr int kStages = TT_ATTN_STAGES;  // LDS ring depth (tiles in flight + 1)
constexpr int kPageCache = 1024; // page ids cached per sub-range
constexpr int kMinTiles = 4;     // smallest range worth a work-group
// Each (sequence, KV head) tile run carries kUnitPad virtual tiles after its
// real ones: they stand for a unit's fixed cost (Q load, page-id cache,
// pipeline fill, block tile, epilogue) so that ranges which cut run
// boundaries get fewer real tiles.  A virtual tile holds no work.
#ifndef TT_ATTN_UNITPAD
#define TT_ATTN_UNITPAD 4
#endif
constexpr int kUnitPad = TT_ATTN_UNITPAD;
constexpr float kLazy = 8.0f;    // rescale when max grows by > 2^kLazy

template <int D>
struct Geo {
  static constexpr int KS = D / 16;                       // MFMA k-steps over D
  static constexpr int DB = D / 32;                       // 32-row blocks of O^T
  static constexpr int KCH = D / 8;                       // 16-byte chunks per key row
  static constexpr int KPT = kTile * KCH / kThreads;      // key chunks per thread
  static constexpr int VPT = D * (kTile / 8) / kThreads;  // value chunks per thread
  static constexpr int LPT = KPT + VPT;                   // direct loads per thread per tile
  static constexpr int K_BYTES = kTile * D * 2;           // key tile [64][D]
  static constexpr int V_BYTES = D * kTile * 2;           // value tile [D][64]
  static constexpr int STAGE_BYTES = K_BYTES + V_BYTES;
  static constexpr size_t RING_BYTES = (size_t)kStages * STAGE_BYTES;
  static_assert(KPT >= 1 && VPT >= 1, "tile too small for the work-group");
};

struct Params {
  const __bf16 *q, *k_blk, *v_blk, *k_pages, *v_pages;
  const int32_t *page_table, *ctx_lens;
  __bf16 *out;
  int *ws_pre;   // [B+1] flat-tile prefix, published for the combine
  __bf16 *ws_o; // [2G][D*256] partial O^T / l (bf16)
  float *ws_ml;  // [2G][256][2]  (reference max in log2 units, sum l)
  int B, S, Hq, Hkv, g, page_size, lps, max_pages, num_pages, max_ctx, qchunks, G;
  int causal;  // chunk ingest: block position t sees block keys 0..t only
  float sl2;
};

// real tiles of a (sequence, KV head) run: context tiles plus the block tile
__device__ __forceinline__ int real_tiles(int L) { return (L + kTile - 1) / kTile + 1; }
__device__ __forceinline__ int seq_tiles(int L) { return real_tiles(L) + kUnitPad; }

// pre[b] = first flat tile of sequence b (all its KV heads), pre[B] = total;
// lens[b] = clamped context length.  One wave scans 64 sequences per step.
__device__ void build_prefix(const Params &p, int *pre, int *lens) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int upb = p.Hkv;  // one tile run per (b, h); its query chunks share it
    int carry = 0;
    for (int base = 0; base < p.B; base += 64) {
      const int b = base + lane;
      const int L = b < p.B ? min(max(p.ctx_lens[b], 0), p.max_ctx) : 0;
      const int t = b < p.B ? seq_tiles(L) * upb : 0;
      int x = t;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      if (b < p.B) {
        pre[b] = carry + x - t;
        lens[b] = L;
      }
      carry += __shfl(x, 63, 64);
    }
    if (lane == 0) pre[p.B] = carry;
  }
  __syncthreads();
}

struct Unit {
  int b, h, qc, L, T, nreal, start, id;
};

// The unit of query chunk qc that owns flat tile t.
__device__ Unit locate(const Params &p, const int *pre, const int *lens, int t, int qc) {
  int lo = 0, hi = p.B;  // pre[lo] <= t < pre[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= t) lo = mid; else hi = mid;
  }
  Unit u;
  u.b = lo;
  u.L = lens[lo];
  u.T = seq_tiles(u.L);
  u.nreal = real_tiles(u.L);
  const int h = (t - pre[lo]) / u.T;
  u.h = h;
  u.qc = qc;
  u.start = pre[lo] + h * u.T;
  u.id = (lo * p.Hkv + h) * p.qchunks + qc;
  return u;
}

// Swap bits 2 and 3 of an MFMA row index.  Key row m of a 32-key block is
// stored at LDS row pi(m), so that the S^T accumulator registers 8c..8c+7 of
// lane half h hold keys 16c+8h .. 16c+8h+7 (contiguous), which is exactly the
// B-operand order P.V needs; no cross-lane shuffle of P is required.
__device__ __forceinline__ int pi_row(int m) {
  return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// LDS swizzles (16-byte slots).  Key tile: row r (D*2 bytes) keeps chunk c in
// slot c ^ (r mod KCH).  Value tile: row d (128 bytes) keeps token-chunk c in
// slot c ^ fv(d).  Each keeps the MFMA operand reads (32 consecutive rows,
// one chunk) free of bank conflicts.
template <int D>
__device__ __forceinline__ int k_off(int r, int c) {
  return r * (D * 2) + 16 * (c ^ (r & (Geo<D>::KCH - 1)));
}
__device__ __forceinline__ int v_off(int d, int c) {
  const int f = (d & 7) ^ ((d >> 3) & 1);
  return d * (kTile * 2) + 16 * (c ^ f);
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

typedef __attribute__((address_space(3))) void lds_void;

// Work-group barrier that orders LDS only.  __syncthreads() also fences
// global memory, which makes the compiler drain every outstanding vector
// load (vmcnt(0)) -- including the direct-to-LDS loads of tiles still in
// flight.  Tile arrival is awaited explicitly with wait_tiles() instead.
// The empty asm statements only stop the compiler from moving memory
// accesses across the barrier; lgkmcnt(0) completes this wave's LDS
// reads/writes before it signals arrival.
constexpr int lgkm0_imm() { return 15 | (7 << 4) | (0 << 8) | (3 << 14); }
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(lgkm0_imm());
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// vmcnt-only s_waitcnt immediate (gfx9 encoding; expcnt/lgkmcnt left at max).
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14); }

// Which waves issue the direct loads of a tile, at the start of their
// compute.  kIssuer 0: every wave its own share; 1: each lead wave w its
// share and that of its lag partner w + waves/2.  Issuing blocks a wave
// while the memory queue is full; with 1 the lag waves, which carry the
// longer compute, never block.  (Issuing later in the tile, or from the lag
// waves, measured slower.)
#ifndef TT_ATTN_ISSUER
#define TT_ATTN_ISSUER 1
#endif
constexpr int kIssuer = TT_ATTN_ISSUER;
#define TT_ATTN_ISSUE (kIssuer == 0 ? 1 : 2)
constexpr int kIssue = TT_ATTN_ISSUE;
constexpr int kWaves = kThreads / 64;
static_assert(kIssuer == 0 || kIssuer == 1, "issuer mode");

// Wait until at most `tiles_after` tiles' worth of this wave's direct loads
// are in flight.
template <int D>
__device__ __forceinline__ void wait_tiles(int tiles_after) {
  constexpr int L = Geo<D>::LPT * kIssue;
  if (tiles_after <= 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  else if (tiles_after == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(L));
  else if (tiles_after == 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * L));
  else __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * L));
  static_assert(3 * Geo<D>::LPT * kIssue < 64, "vmcnt range");
  static_assert(kStages <= 4, "wait_tiles covers up to 3 tiles in flight");
}

// Direct-load slots.  Each wave instruction fills 1 KiB of LDS contiguously
// (lane l -> bytes 16l..16l+15), and lane l fetches whichever key/value chunk
// the swizzled layout puts there.  An issuing wave iw owns NL = LPT-part *
// kIssue consecutive KiB of the key part and of the value part of a stage,
// so that its loads share one LDS base (M0) and differ only in the
// instruction's immediate offset, which applies to both addresses.
template <int D>
struct Share {
  static constexpr int NK = Geo<D>::KPT * kIssue;  // key loads per issuing wave
  static constexpr int NV = Geo<D>::VPT * kIssue;  // value loads per issuing wave
  static_assert(NK <= 4 && NV <= 4, "immediate offsets reach 4 KiB");
};
// Token t and chunk c fetched by this lane for key load n of issuing wave iw.
template <int D>
__device__ __forceinline__ void key_slot(int iw, int n, int &t, int &c) {
  using G = Geo<D>;
  const int slot = (iw * Share<D>::NK + n) * 64 + (threadIdx.x & 63);
  const int r = slot / G::KCH, s = slot % G::KCH;
  t = (r & ~31) | pi_row(r & 31);  // token within the tile
  c = s ^ (r & (G::KCH - 1));      // 16-byte feature chunk
}
// Feature row d and 8-token chunk c fetched for value load n.
template <int D>
__device__ __forceinline__ void value_slot(int iw, int n, int &d, int &c) {
  const int slot = (iw * Share<D>::NV + n) * 64 + (threadIdx.x & 63);
  d = slot >> 3;
  c = (slot & 7) ^ ((d & 7) ^ ((d >> 3) & 1));
}
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
// Index of this wave among the issuing waves (the lead waves come first).
__device__ __forceinline__ int issuer_id() { return wave_id(); }
// Positions past the context are clamped to a valid token: keys there are
// masked by score, values are zeroed in LDS before use.
__device__ __forceinline__ int key_pos(const Unit &u, int i, int t) {
  return min(i * kTile + t, u.L - 1);
}
__device__ __forceinline__ int value_pos(const Unit &u, int i, int c) {
  const int pos0 = i * kTile + 8 * c;
  return pos0 < u.L ? pos0 : ((u.L - 1) & ~7);
}

// Page ids behind this lane's direct loads of one tile, read from the LDS
// page-id cache one tile ahead of their use.  With pages of at least one
// tile (BIG), a tile lies inside one page: one id per tile, wave-uniform,
// and each lane's byte offsets from the tile's key / value start are the
// same for every tile (set once by lane_offsets).
template <int D, bool BIG>
struct TilePages {
  int k[Share<D>::NK], v[Share<D>::NV];
  __device__ __forceinline__ void lane_offsets(const Params &) {}
};
template <int D>
struct TilePages<D, true> {
  int pg;
  // value load n sits (n / 2) * 16 feature rows after load n % 2 (the slot
  // swizzle depends on n only through n % 2), so two offsets cover them
  unsigned ko[Share<D>::NK], vo[2];
  __device__ __forceinline__ void lane_offsets(const Params &p);
};

template <int D, bool BIG>
__device__ __forceinline__ void read_pages(const Params &p, const Unit &u, int i, const int *pcache,
                                           int pbase, TilePages<D, BIG> &pg) {
  if constexpr (BIG) {
    pg.pg = pcache[((i * kTile) >> p.lps) - pbase];
  } else {
    const int iw = issuer_id();
#pragma unroll
    for (int n = 0; n < Share<D>::NK; ++n) {
      int t, c;
      key_slot<D>(iw, n, t, c);
      pg.k[n] = pcache[(key_pos(u, i, t) >> p.lps) - pbase];
    }
#pragma unroll
    for (int n = 0; n < Share<D>::NV; ++n) {
      int d, c;
      value_slot<D>(iw, n, d, c);
      pg.v[n] = pcache[(value_pos(u, i, c) >> p.lps) - pbase];
    }
  }
}

template <int D>
__device__ __forceinline__ void TilePages<D, true>::lane_offsets(const Params &p) {
  const int iw = issuer_id();
#pragma unroll
  for (int n = 0; n < Share<D>::NK; ++n) {
    int t, c;
    key_slot<D>(iw, n, t, c);
    ko[n] = (unsigned)(t * D + 8 * c) * 2u;
  }
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    int d, c;
    value_slot<D>(iw, n, d, c);
    vo[n] = (unsigned)(d * p.page_size + 8 * c) * 2u;
  }
}

// Buffer descriptor over `bytes` bytes from `base` (raw, no stride; loads
// past `bytes` return zeros instead of touching memory).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

// One direct load through a buffer descriptor: bytes r + voff + soff ->
// LDS lds (+ 16 * lane).  The descriptor, soff and the LDS base are scalar
// per tile; the per-lane offset is fixed, so issuing takes no vector
// instructions.
__device__ __forceinline__ void dma_buf(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff,
                                        unsigned char *lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 16, voff, soff, 0, 0);
}

// One direct load: global `src` -> LDS lds + n KiB (+ 16 * lane).  The
// immediate offset n KiB is added by the hardware to both addresses.
__device__ __forceinline__ void dma(const __bf16 *src, unsigned char *lds, int n) {
  const unsigned char *g = (const unsigned char *)src;
  switch (n) {
    case 0: __builtin_amdgcn_global_load_lds((const void *)g, (lds_void *)lds, 16, 0, 0); break;
    case 1: __builtin_amdgcn_global_load_lds((const void *)(g - 1024), (lds_void *)lds, 16, 1024, 0); break;
    case 2: __builtin_amdgcn_global_load_lds((const void *)(g - 2048), (lds_void *)lds, 16, 2048, 0); break;
    default: __builtin_amdgcn_global_load_lds((const void *)(g - 3072), (lds_void *)lds, 16, 3072, 0); break;
  }
}

// Issue this wave's direct HBM->LDS loads of context tile i into `stage`.
// BIG: the tile's 64 tokens sit in one page, so the page base is scalar and
// each lane adds a fixed offset; positions past the context stay inside that
// page (masked keys, values zeroed in LDS).  Otherwise positions are clamped
// to the context and every lane looks up its own page.
template <int D, bool BIG>
__device__ __forceinline__ void issue_tile(const Params &p, const Unit &u, int i,
                                           unsigned char *stage, const TilePages<D, BIG> &pg) {
  using G = Geo<D>;
  const int iw = issuer_id();
  const int pmask = p.page_size - 1;
  unsigned char *kl = stage + iw * Share<D>::NK * 1024;
  unsigned char *vl = stage + G::K_BYTES + iw * Share<D>::NV * 1024;
  if constexpr (BIG) {
    const int page = __builtin_amdgcn_readfirstlane(pg.pg);
    const size_t block = ((size_t)page * p.Hkv + u.h) * p.page_size * D;  // (page, head) block
    const int off = (i * kTile) & pmask;                                   // tile start in the page
    // the key tile is contiguous; the value tile is D rows of kTile tokens,
    // page_size apart
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(p.k_pages + block + (size_t)off * D, G::K_BYTES);
    const __amdgpu_buffer_rsrc_t rv =
        buffer_rsrc(p.v_pages + block + off, ((D - 1) * p.page_size + kTile) * 2);
#pragma unroll
    for (int n = 0; n < Share<D>::NK; ++n) dma_buf(rk, pg.ko[n], 0u, kl + n * 1024);
#pragma unroll
    for (int n = 0; n < Share<D>::NV; ++n)
      dma_buf(rv, pg.vo[n & 1], (unsigned)((n >> 1) * 32 * p.page_size), vl + n * 1024);
  } else {
#pragma unroll
    for (int n = 0; n < Share<D>::NK; ++n) {
      int t, c;
      key_slot<D>(iw, n, t, c);
      const int pos = key_pos(u, i, t);
      dma(p.k_pages + (((size_t)pg.k[n] * p.Hkv + u.h) * p.page_size + (pos & pmask)) * D + 8 * c,
          kl, n);
    }
#pragma unroll
    for (int n = 0; n < Share<D>::NV; ++n) {
      int d, c;
      value_slot<D>(iw, n, d, c);
      const int pos = value_pos(u, i, c);
      dma(p.v_pages + (((size_t)pg.v[n] * p.Hkv + u.h) * D + d) * p.page_size + (pos & pmask), vl, n);
    }
  }
}

// The direct loads of one tile, issued at the start of an earlier tile's
// compute, followed by the page-id reads of the tile after it (awaited with
// the first operand batch).
template <int D, bool BIG>
struct TileLoads {
  const Params &p;
  const Unit &u;
  int i;                    // tile to load
  unsigned char *stage;     // its ring stage
  TilePages<D, BIG> &pg;    // its page ids; then those of tile i + 1
  const int *pcache;
  int pbase, c1;            // page-cache base, end of the sub-range
  __device__ __forceinline__ void issue() const {
    if (i >= c1) return;
    issue_tile<D, BIG>(p, u, i, stage, pg);
    if (i + 1 < c1) read_pages<D, BIG>(p, u, i + 1, pcache, pbase, pg);
  }
};

// No loads (block tile).
struct NoLoads {
  __device__ __forceinline__ void issue() const {}
};

// Zero the value columns of tokens >= nvalid in a landed tile.
template <int D>
__device__ __forceinline__ void zero_value_tail(unsigned char *stage, int nvalid) {
  unsigned char *vs = stage + Geo<D>::K_BYTES;
  for (int idx = threadIdx.x; idx < D * 8; idx += kThreads) {
    const int d = idx >> 3, c = idx & 7;
    const int n = nvalid - 8 * c;
    if (n < 8) {
      uint4 *ptr = (uint4 *)(vs + v_off(d, c));
      *ptr = keep_first(*ptr, n);
    }
  }
}

// The block's own S keys/values into `stage` (registers -> LDS, values
// transposed on the way); rows/columns >= S are zero.
template <int D>
__device__ __forceinline__ void stage_block_tile(const Params &p, const Unit &u,
                                                 unsigned char *stage) {
  using G = Geo<D>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int kk = 0; kk < G::KPT; ++kk) {
    const int idx = tid + kThreads * kk;
    const int t = idx / G::KCH, c = idx % G::KCH;
    const int tc = min(t, p.S - 1);
    uint4 x = *(const uint4 *)(p.k_blk + (((size_t)u.b * p.S + tc) * p.Hkv + u.h) * D + 8 * c);
    if (t >= p.S) x = make_uint4(0, 0, 0, 0);
    const int r = (t & ~31) | pi_row(t & 31);
    *(uint4 *)(stage + k_off<D>(r, c)) = x;
  }
  // values: token row t, features 8c..8c+7 loaded as one 16-byte chunk and
  // scattered into the feature-major tile (token t = column t).
#pragma unroll
  for (int kk = 0; kk < G::KPT; ++kk) {
    const int idx = tid + kThreads * kk;
    const int t = idx / G::KCH, c = idx % G::KCH;
    const int tc = min(t, p.S - 1);
    uint4 x = *(const uint4 *)(p.v_blk + (((size_t)u.b * p.S + tc) * p.Hkv + u.h) * D + 8 * c);
    if (t >= p.S) x = make_uint4(0, 0, 0, 0);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * c + e;
      const uint16_t val = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
      *(uint16_t *)(stage + G::K_BYTES + v_off(d, t >> 3) + 2 * (t & 7)) = val;
    }
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
struct Acc {
  f32x16 o[Geo<D>::DB];  // O^T, 32 features x 32 query rows per block
  float mref, lsum;      // reference max (log2 units), running sum
};

template <int D>
struct PTile {
  bf16x8 v[2][2];  // probabilities of a 64-key tile as P.V B-operands [32-key half][16-key chunk]
};

// Four MFMA A-operands read from LDS together.  A tile's score phase reads
// 2*KS key operands and its P.V phase 4*DB value operands, four per batch.
// Two batch buffers alternate: batch n+1 is read while batch n feeds the
// MFMAs.  Both phase lengths are even, so a phase's first batch always sits
// in buffer 0 and can be read during the previous phase.
struct Batch {
  bf16x8 v[4];
};

template <int D>
struct Phases {
  static constexpr int NQ = 2 * Geo<D>::KS / 4;  // score batches per tile
  static constexpr int NV = Geo<D>::DB;          // P.V batches per tile
  static_assert(NQ % 2 == 0 && NV % 2 == 0, "phases must hold an even number of batches");
};

// Completes this wave's outstanding LDS reads.  While direct-to-LDS loads
// are in flight the compiler treats LDS read completion as unordered and
// waits for all of them before a use; waiting here, before the next batch
// is issued, keeps exactly one batch in flight behind the MFMAs.
__device__ __forceinline__ void lds_wait() { __builtin_amdgcn_s_waitcnt(lgkm0_imm()); }

// Keeps the compiler from moving instructions across phase boundaries.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Score operand e of batch b, j = 4b + e: key half tb = j % 2, k-step
// ks = j / 2 (the two halves' accumulation chains interleave).
template <int D>
__device__ __forceinline__ void read_qk(const unsigned char *stage, int b, Batch &x) {
  const int lane = threadIdx.x & 63;
  const int ln = lane & 31, hl = lane >> 5;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = 4 * b + e, tb = j & 1, ks = j >> 1;
    x.v[e] = *(const bf16x8 *)(stage + k_off<D>(32 * tb + ln, 2 * ks + hl));
  }
}

// S^T (two 32-key halves) += K . Q^T for batch b
template <int D>
__device__ __forceinline__ void mfma_qk(const Batch &x, int b, const bf16x8 (&qr)[Geo<D>::KS],
                                        f32x16 (&s)[2]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = 4 * b + e, tb = j & 1, ks = j >> 1;
    s[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x.v[e], qr[ks], s[tb], 0, 0, 0);
  }
}

// P.V operand e of batch b, j = 4b + e = (2*tb + cc)*DB + db: feature block
// db, 16-key chunk cc of key half tb.
template <int D>
__device__ __forceinline__ void read_pv(const unsigned char *stage, int b, Batch &x) {
  constexpr int DB = Geo<D>::DB;
  const int lane = threadIdx.x & 63;
  const int ln = lane & 31, hl = lane >> 5;
  const unsigned char *Vs = stage + Geo<D>::K_BYTES;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = 4 * b + e, db = j % DB, tc = j / DB;
    x.v[e] = *(const bf16x8 *)(Vs + v_off(32 * db + ln, 2 * tc + hl));
  }
}

// O^T += V^T . P^T for batch b
template <int D>
__device__ __forceinline__ void mfma_pv(const Batch &x, int b, const PTile<D> &P, Acc<D> &A) {
  constexpr int DB = Geo<D>::DB;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = 4 * b + e, db = j % DB, tc = j / DB;
    A.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x.v[e], P.v[tc >> 1][tc & 1], A.o[db], 0, 0, 0);
  }
}

// Online softmax of a tile's scores (log2 domain): rescales the accumulators
// when the running max grows by more than 2^kLazy, returns P in bf16.
// Keys at or past klim (per lane: the lane's query row) are masked when
// `mask` (wave-uniform) is set.
template <int D>
__device__ __forceinline__ void softmax_tile(const Params &p, f32x16 (&s)[2], int klim, bool mask,
                                             Acc<D> &A, PTile<D> &P) {
  const int hl = (threadIdx.x & 63) >> 5;
  // key of register r of half tb in lane half hl: 32*tb + 16*(r/8) + 8*hl + r%8
  if (mask) {
    const int lim = klim - 8 * hl;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * tb + 16 * (r >> 3) + (r & 7) >= lim) s[tb][r] = -INFINITY;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[tb][r]);
  mx = pair_max(mx);
  const float mxs = mx * p.sl2;
  const bool need = mxs > A.mref + kLazy;
  if (__builtin_amdgcn_ballot_w64(need)) {
    const float f = need ? __builtin_amdgcn_exp2f(A.mref - mxs) : 1.f;
    if (need) A.mref = mxs;
    A.lsum *= f;
#pragma unroll
    for (int db = 0; db < Geo<D>::DB; ++db) A.o[db] *= f;
  }
  const float nm = -A.mref;
  float acc = 0.f;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    f32x16 e;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[tb][r], p.sl2, nm));
      acc += e[r];
    }
    const f32x8 lo = {e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]};
    const f32x8 hi = {e[8], e[9], e[10], e[11], e[12], e[13], e[14], e[15]};
    P.v[tb][0] = __builtin_convertvector(lo, bf16x8);
    P.v[tb][1] = __builtin_convertvector(hi, bf16x8);
  }
  A.lsum += acc;
}

// Score phase of a tile.  Expects its batch 0 in buf[0] (issued, not
// awaited).  With NEXT_V, issues P.V batch 0 of the same tile into buf[0]
// under the last score MFMAs.
template <int D, bool NEXT_V>
__device__ __forceinline__ void score_phase(const unsigned char *stage,
                                            const bf16x8 (&qr)[Geo<D>::KS], f32x16 (&s)[2],
                                            Batch (&buf)[2]) {
  constexpr int NQ = Phases<D>::NQ;
  s[0] = f32x16{};
  s[1] = f32x16{};
#pragma unroll
  for (int b = 0; b < NQ; ++b) {
    lds_wait();
    sched_fence();
    if (b + 1 < NQ) read_qk<D>(stage, b + 1, buf[(b + 1) & 1]);
    else if (NEXT_V) read_pv<D>(stage, 0, buf[0]);
    sched_fence();
    mfma_qk<D>(buf[b & 1], b, qr, s);
    sched_fence();
  }
}

// P.V phase of a tile whose probabilities are in P.  Expects its batch 0 in
// buf[0] (issued; complete already if READY).  With NEXT_K, issues score
// batch 0 of `kstage` into buf[0] under the last P.V MFMAs.
template <int D, bool READY, bool NEXT_K>
__device__ __forceinline__ void pv_phase(const unsigned char *stage, const unsigned char *kstage,
                                         const PTile<D> &P, Acc<D> &A, Batch (&buf)[2]) {
  constexpr int NV = Phases<D>::NV;
#pragma unroll
  for (int b = 0; b < NV; ++b) {
    if (b > 0 || !READY) lds_wait();
    sched_fence();
    if (b + 1 < NV) read_pv<D>(stage, b + 1, buf[(b + 1) & 1]);
    else if (NEXT_K) read_qk<D>(kstage, 0, buf[0]);
    sched_fence();
    mfma_pv<D>(buf[b & 1], b, P, A);
    sched_fence();
  }
}

// Lead role, whole tile: scores -> softmax -> P.V.  The first value batch is
// read under the last score MFMAs and lands during the softmax.
template <int D, typename Loads>
__device__ __forceinline__ void tile_lead(const Params &p, const unsigned char *stage, int klim,
                                          bool mask, const bf16x8 (&qr)[Geo<D>::KS], Acc<D> &A,
                                          PTile<D> &P, const Loads &ld) {
  Batch buf[2];
  f32x16 s[2];
  ld.issue();
  read_qk<D>(stage, 0, buf[0]);
  score_phase<D, true>(stage, qr, s, buf);
  softmax_tile<D>(p, s, klim, mask, A, P);
  sched_fence();
  pv_phase<D, false, false>(stage, nullptr, P, A, buf);
}

// Lag role: P.V of the previous tile (`prev`, probabilities in P, value
// batch 0 in buf[0], complete), then scores and softmax of this tile; the
// value batch 0 of this tile is read under the last score MFMAs, for the
// next call.  FIRST: no previous tile.
template <int D, bool FIRST, typename Loads>
__device__ __forceinline__ void tile_lag(const Params &p, const unsigned char *prev,
                                         const unsigned char *stage, int nvalid,
                                         const bf16x8 (&qr)[Geo<D>::KS], Acc<D> &A,
                                         PTile<D> &P, Batch (&buf)[2], const Loads &ld) {
  f32x16 s[2];
  ld.issue();
  if (FIRST) {
    read_qk<D>(stage, 0, buf[0]);
  } else {
    pv_phase<D, true, true>(prev, stage, P, A, buf);
  }
  score_phase<D, true>(stage, qr, s, buf);
  softmax_tile<D>(p, s, nvalid, nvalid < kTile, A, P);
}

// Start of context tile i of a sub-range [c0, c1): waits for the tile and
// zeroes the value tail of a partial tile.  Returns the tile's stage.
template <int D>
__device__ __forceinline__ unsigned char *begin_tile(const Unit &u, int i, int c0, int c1,
                                                     unsigned char *ring, int &nvalid) {
  constexpr int kAhead = kStages - 2;
  wait_tiles<D>(min(kAhead - 1, c1 - 1 - i));
  lds_barrier();   // tile i visible to all waves; tile i-2's stage free
  unsigned char *stage = ring + ((i - c0) % kStages) * Geo<D>::STAGE_BYTES;
  nvalid = min(kTile, u.L - i * kTile);
  if (nvalid < kTile) {
    zero_value_tail<D>(stage, nvalid);
    lds_barrier();
  }
  return stage;
}

// Context tiles [i0, ctx_end) of unit u through the LDS ring, in sub-ranges
// whose pages fit the page-id cache.  LAG selects the wave-group role.
// An idle wave (no valid query row) keeps the ring's barriers and issues its
// share of the loads but computes nothing.
template <int D, bool BIG, bool LAG>
__device__ __forceinline__ void context_tiles(const Params &p, const Unit &u, int i0, int ctx_end,
                                              unsigned char *ring, int *pcache,
                                              const bf16x8 (&qr)[Geo<D>::KS], Acc<D> &A,
                                              PTile<D> &P, bool idle) {
  using G = Geo<D>;
  constexpr int kAhead = kStages - 2;  // tiles prefetched beyond the current one
  // A sub-range of `sub` tiles starting at any in-page offset o (o < page_size)
  // spans floor((o + 64*sub - 1) / page_size) + 1 <= kPageCache pages when
  // 64*sub <= (kPageCache - 1) * page_size, so its page ids fit the cache.
  const int sub = max(1, ((kPageCache - 1) * p.page_size) / kTile);
  for (int c0 = i0; c0 < ctx_end; c0 += sub) {
    const int c1 = min(c0 + sub, ctx_end);
    const int pbase = (c0 * kTile) >> p.lps;
    const int plast = (min(c1 * kTile, u.L) - 1) >> p.lps;
    const int32_t *pt = p.page_table + (size_t)u.b * p.max_pages;
    for (int k = threadIdx.x; k <= plast - pbase; k += kThreads)
      pcache[k] = clamp_page(pt[pbase + k], p.num_pages);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();
    // the lag waves issue no loads when their lead partners carry them
    constexpr bool kIssues = kIssuer == 0 || !LAG;
    TilePages<D, BIG> pg;
    if (kIssues) {
      pg.lane_offsets(p);
#pragma unroll
      for (int j = 0; j < kAhead; ++j)
        if (c0 + j < c1) {
          read_pages<D, BIG>(p, u, c0 + j, pcache, pbase, pg);
          issue_tile<D, BIG>(p, u, c0 + j, ring + (j % kStages) * G::STAGE_BYTES, pg);
        }
      if (c0 + kAhead < c1) read_pages<D, BIG>(p, u, c0 + kAhead, pcache, pbase, pg);
    }
    // Per tile i, the loads of tile i + kAhead are issued during its compute.
    int nvalid;
    auto loads = [&](int i) {
      return TileLoads<D, BIG>{p, u, kIssues ? i + kAhead : c1,
                               ring + ((i - c0 + kAhead) % kStages) * G::STAGE_BYTES, pg, pcache,
                               pbase, c1};
    };
    if (idle) {
      for (int i = c0; i < c1; ++i) {
        begin_tile<D>(u, i, c0, c1, ring, nvalid);
        loads(i).issue();
      }
    } else if (!LAG) {
      for (int i = c0; i < c1; ++i) {
        const unsigned char *stage = begin_tile<D>(u, i, c0, c1, ring, nvalid);
        tile_lead<D>(p, stage, nvalid, nvalid < kTile, qr, A, P, loads(i));
      }
    } else {
      // the first tile has no predecessor; the last one's P.V drains after the loop
      Batch buf[2];
      const unsigned char *prev = begin_tile<D>(u, c0, c0, c1, ring, nvalid);
      tile_lag<D, true>(p, nullptr, prev, nvalid, qr, A, P, buf, loads(c0));
      for (int i = c0 + 1; i < c1; ++i) {
        const unsigned char *stage = begin_tile<D>(u, i, c0, c1, ring, nvalid);
        tile_lag<D, false>(p, prev, stage, nvalid, qr, A, P, buf, loads(i));
        prev = stage;
      }
      pv_phase<D, false, false>(prev, nullptr, P, A, buf);
    }
    lds_barrier();   // ring and page cache free for reuse
  }
}

// One unit's tiles [i0, i1) on this work-group.
//
// Context tiles stream through the LDS ring.  The waves are split into two
// groups that share the SIMDs (wave w and w + waves/2 sit on the same SIMD):
// the lead group runs scores -> softmax -> P.V on tile i, the lag group runs
// P.V of tile i-1 first and then scores -> softmax of tile i.  Within one
// barrier interval the two waves on a SIMD are then in different phases, so
// one wave's softmax (VALU) overlaps the other's MFMAs.  The lag group keeps
// its probabilities for one tile; a tile's stage therefore stays live for two
// iterations and only kStages - 2 tiles are prefetched.
template <int D, bool BIG>
__device__ void run_unit(const Params &p, const Unit &u, int i0, int i1, bool complete,
                         int slot, unsigned char *ring, int *pcache) {
  using G = Geo<D>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int ln = lane & 31, hl = lane >> 5;
  const int M = p.S * p.g;
  const bool lag = wave >= kWaves / 2;

  // Q (B operand of S^T = K . Q^T): lane holds query row 32*wave + ln,
  // features 16*ks + 8*hl .. +7.
  bf16x8 qr[G::KS];
  {
    const int qi = u.qc * kQRows + wave * 32 + ln;
    if (qi < M) {
      const int t = qi / p.g, j = qi % p.g;
      const __bf16 *src = p.q + (((size_t)u.b * p.S + t) * p.Hq + u.h * p.g + j) * D + 8 * hl;
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks) qr[ks] = *(const bf16x8 *)(src + 16 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks) qr[ks] = bf16x8{};
    }
  }
  Acc<D> A;
#pragma unroll
  for (int db = 0; db < G::DB; ++db) A.o[db] = f32x16{};
  A.mref = -INFINITY;
  A.lsum = 0.f;
  PTile<D> P;

  // ---- context tiles [i0, ctx_end): one loop instance per role, so that the
  // register allocation of each is independent (same barrier sequence)
  const int ctx_end = min(i1, u.nreal - 1);
  // a wave whose 32 query rows all lie past S*g (block sizes with S*g not a
  // multiple of 256) skips the compute
  const bool idle = u.qc * kQRows + wave * 32 >= M;
  if (lag) context_tiles<D, BIG, true>(p, u, i0, ctx_end, ring, pcache, qr, A, P, idle);
  else context_tiles<D, BIG, false>(p, u, i0, ctx_end, ring, pcache, qr, A, P, idle);
  // ---- the block's own S keys/values (the unit's last real tile)
  if (i0 < u.nreal && i1 >= u.nreal) {
    unsigned char *stage = ring;
    stage_block_tile<D>(p, u, stage);
    lds_barrier();
    // chunk ingest: the lane's query row (block position t) sees keys 0..t
    const int qt = (u.qc * kQRows + wave * 32 + ln) / p.g;
    const int klim = p.causal ? min(p.S, qt + 1) : p.S;
    if (!idle) tile_lead<D>(p, stage, klim, p.causal || p.S < kTile, qr, A, P, NoLoads{});
    lds_barrier();
  }

  // ---- epilogue.  O^T accumulator register r of lane (hl, ln) in block db
  // holds feature 32*db + 8*(r/4) + 4*hl + r%4 of query row ln.
  const float ltot = pair_sum(A.lsum);
  const float inv = 1.f / ltot;
  const int qloc = wave * 32 + ln;
  const int qi = u.qc * kQRows + qloc;
  if (complete) {
    if (qi < M) {
      const int t = qi / p.g, j = qi % p.g;
      __bf16 *dst = p.out + (((size_t)u.b * p.S + t) * p.Hq + u.h * p.g + j) * D;
#pragma unroll
      for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 v = {A.o[db][4 * r4 + 0] * inv, A.o[db][4 * r4 + 1] * inv,
                           A.o[db][4 * r4 + 2] * inv, A.o[db][4 * r4 + 3] * inv};
          *(bf16x4 *)(dst + 32 * db + 8 * r4 + 4 * hl) = __builtin_convertvector(v, bf16x4);
        }
    }
  } else if (!idle) {  // the combine reads no row of an idle wave
    // partial O^T / l in bf16, accumulator layout: 4 x bf16 (registers
    // 4*r4 .. 4*r4+3) of lane l at (((wave*DB + db)*4 + r4)*64 + l); features
    // 32*db + 8*r4 + 4*(l/32) + 0..3 of query row 32*wave + l%32.
    // Normalising keeps the values in V's range.
    bf16x4 *wo = (bf16x4 *)(p.ws_o + (size_t)slot * D * kQRows);
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 v = {A.o[db][4 * r4] * inv, A.o[db][4 * r4 + 1] * inv,
                         A.o[db][4 * r4 + 2] * inv, A.o[db][4 * r4 + 3] * inv};
        wo[((wave * G::DB + db) * 4 + r4) * 64 + lane] = __builtin_convertvector(v, bf16x4);
      }
    if (hl == 0) {
      float *wm = p.ws_ml + ((size_t)slot * kQRows + qloc) * 2;
      wm[0] = A.mref;
      wm[1] = ltot;
    }
  }
}

template <int D, bool BIG>
__global__ __launch_bounds__(kThreads, 1) void attn_split_kernel(Params p) {
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char *ring = smem;
  int *pcache = (int *)(smem + Geo<D>::RING_BYTES);
  int *pre = pcache + kPageCache;
  int *lens = pre + p.B + 1;
  build_prefix(p, pre, lens);
  if (blockIdx.x == 0)
    for (int k = threadIdx.x; k <= p.B; k += kThreads) p.ws_pre[k] = pre[k];
  const int total = pre[p.B];
  const int teams = p.G / p.qchunks;
  const int R = (total + teams - 1) / teams;
  // Index w of this work-group in range order.  Work-group ids are dealt to
  // the 8 XCDs round-robin, so XCD x = id % 8 takes a contiguous block of
  // indices: the members of a team, and the contributors of a unit, then
  // share its tiles and its Q through that XCD's L2.
  const int nx = p.G / 8, rx = p.G % 8, xcd = blockIdx.x % 8;
  const int w = xcd * nx + min(xcd, rx) + (int)blockIdx.x / 8;
  const int qc = w % p.qchunks;
  const int t_begin = (w / p.qchunks) * R;
  const int t_end = min(t_begin + R, total);
  bool first = true;
  for (int t = t_begin; t < t_end;) {
    const Unit u = locate(p, pre, lens, t, qc);
    const int i0 = t - u.start;
    const int i1 = min(t_end, u.start + u.T) - u.start;
    // slot 0 holds the partial of the range's first unit, slot 1 its last
    if (i0 < u.nreal)
      run_unit<D, BIG>(p, u, i0, i1, i0 == 0 && i1 >= u.nreal, 2 * w + (first ? 0 : 1), ring,
                  pcache);
    first = false;
    t = u.start + i1;
  }
}

// Merges the partials of units cut by a range boundary:
//   O = sum_w c_w (O_w / l_w) / sum_w c_w,  c_w = 2^(m_w - M) l_w,  M = max_w m_w.
// Work-group per (unit, 16-feature slice, 64-row chunk): lane = query row,
// and the contributors (the teams whose ranges meet the unit's real tiles,
// w_lo .. w_hi; of each, the member of the unit's query chunk) are dealt
// round-robin to the waves, each keeping an online (max, sum, O) over its
// share; the waves' states are then merged through LDS.  The member of team
// k for chunk qc is work-group index i = k * qchunks + qc; it left its partial
// in slot 2i, or 2i + 1 for team w_lo when its range began inside an earlier
// (b, h) pair.
constexpr int kCombineRows = 64;
constexpr int kCombineFeat = 16;
constexpr int kCombineWaves = 4;
constexpr int kCombineUnroll = 4;

template <int D>
__global__ __launch_bounds__(64 * kCombineWaves) void attn_combine_kernel(Params p) {
  const int upb = p.Hkv * p.qchunks;
  const int uid = blockIdx.x;
  const int b = uid / upb, ui = uid % upb;
  const int h = ui / p.qchunks, qc = ui % p.qchunks;
  const int pb = p.ws_pre[b];
  const int T = (p.ws_pre[b + 1] - pb) / p.Hkv;
  const int total = p.ws_pre[p.B];
  const int nreal = T - kUnitPad;
  const int us = pb + h * T;
  const int teams = p.G / p.qchunks;
  const int R = (total + teams - 1) / teams;
  // contributing teams; team k's member for query chunk qc is work-group
  // index k * qchunks + qc
  const int w_lo = us / R, w_hi = (us + nreal - 1) / R;
  if (w_lo == w_hi) return;  // finished in place by one work-group
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int qloc = blockIdx.z * kCombineRows + lane;
  const int qi = qc * kQRows + qloc;
  const bool row_ok = qi < p.S * p.g;
  const int lo_slot = 2 * (w_lo * p.qchunks + qc) + (w_lo * R != us ? 1 : 0);
  auto slot_of = [&](int w) { return w == w_lo ? lo_slot : 2 * (w * p.qchunks + qc); };

  // features f0 .. f0+15 of this row: 16-byte pieces at accumulator block
  // db = f0/32, register groups r4 = (f0%32)/8 + {0, 1}, lane halves hh = 0, 1
  const int f0 = kCombineFeat * blockIdx.y;
  const int db = f0 / 32, r40 = (f0 % 32) / 8;
  const int wv = qloc / 32, ln = qloc % 32;
  const size_t base = (((size_t)wv * (D / 32) + db) * 4 + r40) * 64 + ln;
  float acc[kCombineFeat];
#pragma unroll
  for (int e = 0; e < kCombineFeat; ++e) acc[e] = 0.f;
  float M = -INFINITY, lt = 0.f;
  constexpr int kStep = kCombineWaves * kCombineUnroll;
  for (int w0 = w_lo + wave * kCombineUnroll; row_ok && w0 <= w_hi; w0 += kStep) {
    f32x4 x[kCombineUnroll][4];
    float mw[kCombineUnroll], lw[kCombineUnroll];
#pragma unroll
    for (int k = 0; k < kCombineUnroll; ++k) {
      const int w = min(w0 + k, w_hi);
      const int slot = slot_of(w);
      const float *m = p.ws_ml + ((size_t)slot * kQRows + qloc) * 2;
      mw[k] = m[0];
      lw[k] = m[1];
      const bf16x4 *src = (const bf16x4 *)(p.ws_o + (size_t)slot * D * kQRows) + base;
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          x[k][2 * r + hh] = __builtin_convertvector(src[r * 64 + hh * 32], f32x4);
    }
#pragma unroll
    for (int k = 0; k < kCombineUnroll; ++k) {
      if (w0 + k > w_hi) break;
      if (mw[k] > M) {  // new running max: rescale what this wave holds
        const float f = __builtin_amdgcn_exp2f(M - mw[k]);
        lt *= f;
#pragma unroll
        for (int e = 0; e < kCombineFeat; ++e) acc[e] *= f;
        M = mw[k];
      }
      const float wt = __builtin_amdgcn_exp2f(mw[k] - M) * lw[k];   // partials hold O / l
      lt += wt;
      // x[k][2*r + hh][e] is feature f0 + 8*r + 4*hh + e
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[8 * r + 4 * hh + e] += wt * x[k][2 * r + hh][e];
    }
  }
  // merge the waves' (M, l, O) states
  __shared__ float st[kCombineWaves][kCombineFeat + 2][kCombineRows];
  st[wave][0][lane] = M;
  st[wave][1][lane] = lt;
#pragma unroll
  for (int e = 0; e < kCombineFeat; ++e) st[wave][2 + e][lane] = acc[e];
  __syncthreads();
  if (wave != 0 || !row_ok) return;
  float Mx = -INFINITY;
#pragma unroll
  for (int v = 0; v < kCombineWaves; ++v) Mx = fmaxf(Mx, st[v][0][lane]);
  float ltot = 0.f, o[kCombineFeat];
#pragma unroll
  for (int e = 0; e < kCombineFeat; ++e) o[e] = 0.f;
#pragma unroll
  for (int v = 0; v < kCombineWaves; ++v) {
    const float f = __builtin_amdgcn_exp2f(st[v][0][lane] - Mx);   // 0 for a wave without contributors
    ltot += f * st[v][1][lane];
#pragma unroll
    for (int e = 0; e < kCombineFeat; ++e) o[e] += f * st[v][2 + e][lane];
  }
  const float inv = 1.f / ltot;
  const int t = qi / p.g, j = qi % p.g;
  __bf16 *dst = p.out + (((size_t)b * p.S + t) * p.Hq + h * p.g + j) * D + f0;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    f32x8 v = {o[8 * c + 0] * inv, o[8 * c + 1] * inv, o[8 * c + 2] * inv, o[8 * c + 3] * inv,
               o[8 * c + 4] * inv, o[8 * c + 5] * inv, o[8 * c + 6] * inv, o[8 * c + 7] * inv};
    *(bf16x8 *)(dst + 8 * c) = __builtin_convertvector(v, bf16x8);
  }
}

template <int D, bool BIG>
hipError_t launch_split(const Params &prm, hipStream_t stream) {
  const size_t pre_bytes = (size_t)(2 * prm.B + 1) * sizeof(int);   // pre[] and lens[]
  const size_t split_lds = Geo<D>::RING_BYTES + kPageCache * sizeof(int) + pre_bytes;
  static std::atomic<unsigned long long> attr_done{0};  // per device
  const hipError_t e = lds_limit_once((const void *)attn_split_kernel<D, BIG>,
                                      (int)(Geo<D>::RING_BYTES + kPageCache * sizeof(int) +
                                            (2 * kMaxBatch + 1) * sizeof(int)),
                                      attr_done);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_split_kernel<D, BIG>), dim3(prm.G), dim3(kThreads), split_lds, stream, prm);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Params &prm, hipStream_t stream) {
  // pages of at least one tile: every tile lies inside one page
  hipError_t e = prm.page_size >= kTile ? launch_split<D, true>(prm, stream)
                                        : launch_split<D, false>(prm, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel<D>,
                     dim3(prm.B * prm.Hkv * prm.qchunks, D / kCombineFeat, kQRows / kCombineRows),
                     dim3(64 * kCombineWaves), 0, stream, prm);
  return hipGetLastError();
}

// bytes of the published prefix at the head of the workspace (256-aligned)
size_t ws_pre_bytes(int B) { return (((size_t)(B + 1) * sizeof(int)) + 255) & ~(size_t)255; }

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
  const long long tiles =
      (long long)p.B * p.Hkv * p.qchunks * ((p.max_ctx + kTile - 1) / kTile + 1 + kUnitPad);
  p.tiles = tiles;
  long long G = (tiles + kMinTiles - 1) / kMinTiles;
  if (G > cus) G = cus;
  if (G > 1024) G = 1024;  // the combine keeps one slot id per contributor in LDS
  // whole teams of qchunks work-groups (qchunks <= 1024: S <= 64 rows times
  // at most 4096 query heads over 256-row chunks)
  G = G / p.qchunks * p.qchunks;
  if (G < p.qchunks) G = p.qchunks;
  p.G = (int)G;
  p.ws_bytes = ws_pre_bytes(p.B) + (size_t)2 * G * ((size_t)p.D * kQRows * 2 + 2 * kQRows * sizeof(float));
  return p;
}

hipError_t launch_attn_bf16(const AttnPlan &pl, const void *q, const void *k_blk,
                            const void *v_blk, const void *k_pages, const void *v_pages,
                            const int32_t *page_table, const int32_t *ctx_lens, void *out,
                            void *workspace, int causal, hipStream_t stream) {
  Params prm;
  prm.causal = causal;
  prm.q = (const __bf16 *)q; prm.k_blk = (const __bf16 *)k_blk; prm.v_blk = (const __bf16 *)v_blk;
  prm.k_pages = (const __bf16 *)k_pages; prm.v_pages = (const __bf16 *)v_pages;
  prm.page_table = page_table; prm.ctx_lens = ctx_lens;
  prm.out = (__bf16 *)out;
  prm.ws_pre = (int *)workspace;
  prm.ws_o = (__bf16 *)((unsigned char *)workspace + ws_pre_bytes(pl.B));
  prm.ws_ml = (float *)(prm.ws_o + (size_t)2 * pl.G * pl.D * kQRows);
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
