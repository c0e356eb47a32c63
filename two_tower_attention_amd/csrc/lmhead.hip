// LM head fused with the confidence unmask's row reduction (gfx950).
//
// Operation ("Training and sampling", paperfeed review; "Generating Text in
// Parallel Like Solving a Sudoku", kongchang explainer): every masked
// position of the block is predicted through the model's output head, and
// the unmask rule reduces each row of logits to its greedy id and its
// confidence.  The head is a linear map, logits[r][v] = sum_h x[r][h] w[v][h]
// (x the final hidden state [R, H], w the head [V, H], bf16; fp32
// accumulation).  Here the logits never reach HBM: a work-group computes a
// 256 (vocabulary) x 256 (rows) tile of logits^T on MFMA and reduces it on
// the spot to, per row and 256-entry vocabulary chunk (one tile), the unmask's partial
// (max, lowest index of the max, sum exp(l - max)); the unmask's merge and
// commit kernels finish the rule.
//
// Work-group: a 256 (vocabulary) x 256 (hidden rows) tile of logits^T, 4
// waves, one per SIMD (so a wave may use all 512 registers of its lanes).
// Wave w owns hidden rows 64*w .. 64*w+63 against all 256 weight rows: 16
// MFMA accumulator blocks D[32 vocab][32 rows] (v_mfma_f32_32x32x16_bf16,
// A = weight rows, B = hidden rows).  A lane then holds one hidden row of
// every block, so the epilogue's row reductions are lane-local plus one
// lane-pair exchange.
//
// Operands.  The weight tile streams HBM -> LDS by direct loads through
// buffer descriptors into a ring of 4 stages of 64 reduction elements (128
// contiguous bytes of each of the 256 weight rows, 32 KiB); each 128-byte row
// keeps its 16-byte chunks XOR-swizzled by bits 1..3 of the row index
// (conflict-free operand reads).  A wave reads its 64 hidden rows only for
// itself, so they skip LDS and go from memory straight into the MFMA operand
// registers.  Loaded row-major, every such load would touch 32 rows (32
// cache lines) for 1 KiB; a first kernel therefore copies the hidden state
// once into fragment order (each 1 KiB MFMA operand contiguous), which costs
// one pass over R*H*2 bytes.
//
// Pipeline.  Stage s issues, after the MFMAs of each step t, two weight loads
// of stage s+3 and the hidden-row operands of step t of stage s+2, into the
// registers that step t just consumed.  Memory loads complete in issue order
// for the wait counter, so the wait for the hidden rows of step t, two stages
// later, also covers the weight stage loaded alongside them: every load has
// two stages to arrive, and the wait count is the same constant at every
// step.  Loads past the last stage read through empty descriptors (zero, no
// memory traffic), which keeps the counts uniform.
#include <limits.h>

#include <type_traits>

#include "tt_internal.h"

namespace tt {
namespace {

constexpr int kVT = 256;                          // vocabulary rows per work-group tile
constexpr int kRT = 256;                          // hidden rows per work-group tile
constexpr int kWR = 64;                           // hidden rows per wave
constexpr int kChunk = kVT;                       // vocabulary entries per partial (one tile)
constexpr int kKS = 64;                           // reduction elements per stage
constexpr int kSlots = 4;                         // weight ring stages
constexpr int kThreads = 256;                     // 4 waves
constexpr int kSteps = kKS / 16;                  // MFMA reduction steps per stage
constexpr int kRowBytes = kKS * 2;                // 128 bytes of a weight row per stage
constexpr int kRowsPerLoad = 1024 / kRowBytes;    // 8 rows per 1 KiB direct load
constexpr int kStageBytes = kVT * kRowBytes;      // 32 KiB
constexpr int kLoads = kStageBytes / 1024 / 4;    // weight loads per wave per stage
constexpr int kXLoads = (kWR / 32) * kSteps;      // hidden-row loads per wave per stage
constexpr int kFrag = 1024;                       // one MFMA operand of a wave: 64 lanes x 16 B
static_assert(kLoads == 2 * kSteps, "two weight loads per reduction step");
static_assert(kRT == 4 * kWR, "4 waves cover the row tile");

// Physical 16-byte slot of logical chunk c in weight row r: rows r and r + 2
// share banks (128-byte rows), so the XOR runs over bits 1..3 of r and 16
// consecutive rows cover all 64 banks.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

struct LmParams {
  const __bf16 *xp, *w;  // xp: hidden rows in fragment order
  UnmaskPart *parts;     // [R, NC]
  int R, H, V, NC;
};

// Fragment order of the hidden state: for row tile rt, wave w, stage s,
// step t and row block rb, one 1 KiB fragment whose lane l = 32*hl + ln holds
// x[256*rt + 64*w + 32*rb + ln][64*s + 16*t + 8*hl .. +7], zero past R and
// past H.  Fragment index ((((rt*4 + w)*nst + s)*kSteps + t)*2 + rb).
// One work-group per (64-row group f = rt*4 + w, stage s): it reads the
// group's 64 rows x 128 bytes with whole-row loads, transposes them through
// LDS and writes the stage's 8 fragments (8 KiB) contiguously.
__global__ __launch_bounds__(256) void lmhead_pack_kernel(const __bf16 *__restrict__ x,
                                                          bf16x8 *__restrict__ xp, int R, int H,
                                                          int nst) {
  __shared__ bf16x8 tile[kWR][kKS / 8 + 1];  // [row][16-byte chunk], padded against bank conflicts
  const int s = blockIdx.x % nst;
  const long long f = blockIdx.x / nst;
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = tid / 4, c = 2 * (tid % 4) + u;
    const long long gr = f * kWR + row;
    const int k = s * kKS + 8 * c;
    bf16x8 v = {};
    if (gr < R && k < H) v = *(const bf16x8 *)(x + gr * H + k);
    tile[row][c] = v;
  }
  __syncthreads();
  bf16x8 *dst = xp + ((size_t)f * nst + s) * (kSteps * 2 * 64);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = tid + 256 * u;       // 16-byte unit of the stage: fragment e / 64, lane e % 64
    const int frag = e >> 6, lane = e & 63;
    const int t = frag >> 1, rb = frag & 1;
    dst[e] = tile[32 * rb + (lane & 31)][2 * t + (lane >> 5)];
  }
}

// lgkmcnt(0) only (gfx9 encoding): completes this wave's LDS reads.
__device__ __forceinline__ void lds_wait() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}
// Work-group barrier ordering LDS only (no global fence, which would drain
// the direct loads still in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  lds_wait();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct WOps {
  bf16x8 v[8];  // weight blocks 0..7 of one reduction step
};
struct XOps {
  bf16x8 v[kSteps][2];  // this wave's two hidden-row blocks, per step
};

__global__ __launch_bounds__(kThreads, 1) void lmhead_kernel(LmParams p) {
  extern __shared__ __align__(16) unsigned char ring[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 31, hl = lane >> 5;

  // Tile order.  Work-groups are dealt to the 8 XCDs round-robin (id % 8),
  // and each XCD has its own L2.  The row tiles of one vocabulary tile read
  // the same weight rows, so they go to ids 8 apart: same XCD, dispatched
  // together, and the weight tile leaves HBM once.  (Vocabulary tiles past the
  // last multiple of 8 use plain order.)
  const int nrt = (p.R + kRT - 1) / kRT;
  const int nvt = (p.V + kVT - 1) / kVT;
  const int full = (nvt / 8) * 8 * nrt;
  int rt, vt;
  if ((int)blockIdx.x < full) {
    const int q = blockIdx.x / (8 * nrt), rem = blockIdx.x % (8 * nrt);
    rt = rem / 8;
    vt = 8 * q + rem % 8;
  } else {
    const int j = blockIdx.x - full;
    rt = j % nrt;
    vt = (nvt / 8) * 8 + j / nrt;
  }
  const int r0 = rt * kRT, v0 = vt * kVT;
  const int w_rows = min(kVT, p.V - v0);
  const __bf16 *wb = p.w + (size_t)v0 * p.H;
  const int nst = (p.H + kKS - 1) / kKS;

  // Weight loads: load n = 8*wave + j of a stage fills tile rows 8n .. 8n+7
  // (1 KiB); lane l holds row 8n + l/8, physical chunk l%8, i.e. logical
  // chunk (l%8) ^ ((8n + l/8) >> 1 & 7), which depends on n only through
  // j % 2.  One descriptor per wave and stage starts at the wave's first row
  // (64*wave) and ends at the tile's last vocabulary row, and the per-lane
  // offset carries the row, so rows past the vocabulary read as zero.
  const int lrow = lane >> 3;
  const int wrow0 = kLoads * kRowsPerLoad * wave;
  unsigned voffw[2];
  voffw[0] = (unsigned)((lrow * p.H + 8 * ((lane & 7) ^ ((lrow >> 1) & 7))) * 2);
  voffw[1] = (unsigned)((lrow * p.H + 8 * ((lane & 7) ^ (((8 + lrow) >> 1) & 7))) * 2);
  auto wrsrc = [&](int s) {
    const int k0 = s * kKS;
    const int bytes = k0 < p.H ? max(0, ((w_rows - wrow0) * p.H - k0) * 2) : 0;
    return buffer_rsrc(wb + (size_t)wrow0 * p.H + min(k0, p.H), bytes);
  };
  auto wload = [&](const __amdgpu_buffer_rsrc_t &r, int s, int j) {
    const int n = kLoads * wave + j;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(ring + (s % kSlots) * kStageBytes + n * 1024), 16,
                                             voffw[j & 1] + (unsigned)(j * kRowsPerLoad * p.H * 2), 0, 0, 0);
  };
  // Hidden rows: this wave's fragments, stage after stage (8 KiB each); the
  // descriptor ends after the last stage, so later stages read as zero.
  const __amdgpu_buffer_rsrc_t xr =
      buffer_rsrc(p.xp + (size_t)(rt * 4 + wave) * nst * (kXLoads * kFrag / 2), nst * kXLoads * kFrag);
  auto xload = [&](int s, int t, int rb, XOps &x) {
    x.v[t][rb] = __builtin_bit_cast(
        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(xr, (unsigned)(16 * lane + ((s * kSteps + t) * 2 + rb) * kFrag),
                                                      0, 0));
  };

  // operand read offsets of this lane in a stage, step t: row ln of a 32-row
  // block, logical chunk 2*t + hl (block b adds 4 KiB, an immediate)
  unsigned loff[kSteps];
#pragma unroll
  for (int t = 0; t < kSteps; ++t) loff[t] = (unsigned)(ln * kRowBytes + 16 * swz(ln, 2 * t + hl));
  auto wread1 = [&](int s, int t, int b, WOps &o) {
    o.v[b] = *(const bf16x8 *)(ring + (s % kSlots) * kStageBytes + loff[t] + b * 32 * kRowBytes);
  };
  auto wread = [&](int s, int t, WOps &o) {
#pragma unroll
    for (int b = 0; b < 8; ++b) wread1(s, t, b, o);
  };

  f32x16 acc[8][2];
#pragma unroll
  for (int vb = 0; vb < 8; ++vb)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) acc[vb][rb] = f32x16{};

  // Prologue: the loads that stages -3, -2 and -1 would have issued, in the
  // same order: W(0); then per step t, W(1) loads 2t, 2t+1 and X(0) step t;
  // the same for W(2) and X(1).
  XOps xa, xb;
  WOps wa, wb2;
  {
    const __amdgpu_buffer_rsrc_t r = wrsrc(0);
#pragma unroll
    for (int j = 0; j < kLoads; ++j) wload(r, 0, j);
  }
#pragma unroll
  for (int s = 1; s <= 2; ++s) {
    const __amdgpu_buffer_rsrc_t r = wrsrc(s);
#pragma unroll
    for (int t = 0; t < kSteps; ++t) {
      wload(r, s, 2 * t);
      xload(s - 1, t, 0, s == 1 ? xa : xb);
      wload(r, s, 2 * t + 1);
      xload(s - 1, t, 1, s == 1 ? xa : xb);
    }
  }
  vm_wait<2 * (kLoads + kXLoads)>();  // W(0)
  lds_barrier();
  wread(0, 0, wa);

  // Per step: 16 MFMAs (row block 0 first), the next step's 8 weight operand
  // reads one after each of the first 8 MFMAs, and one memory load after
  // every 4 MFMAs, alternating weight and hidden-row (a load waits for room
  // in the memory queue, and the wave is the only one on its SIMD, so loads
  // go where matrix work is queued, never in bursts).  The hidden-row load
  // of row block rb follows the last MFMA that reads it.  At step t of stage
  // s the loads after X(s) step t are the rest of stage s-2 (steps t+1..3),
  // all of stage s-1 and steps 0..t-1 of stage s: always 28.
  constexpr int kPerStep = kLoads / kSteps + kXLoads / kSteps;
  constexpr int kWaitX = kPerStep * (2 * kSteps - 1);
  static_assert(kWaitX < 64, "vmcnt range");
  auto stage = [&](int s, XOps &xc) {
    const __amdgpu_buffer_rsrc_t rn = wrsrc(s + 3);
#pragma unroll
    for (int t = 0; t < kSteps; ++t) {
      WOps &cur = (t & 1) ? wb2 : wa;
      WOps &nxt = (t & 1) ? wa : wb2;
      lds_wait();
      vm_wait<kWaitX>();  // X(s) step t; at t = 3 also W(s+1), loaded before it
      if (t == kSteps - 1) {
        // W(s+1) visible after the barrier, and every wave has finished
        // reading W(s-1), whose slot W(s+3) takes
        lds_barrier();
      }
      // the next step's operands: this stage's, or the next stage's first
      // (after the last stage an unused read)
      const int rs = t + 1 < kSteps ? s : s + 1, rstep = (t + 1) % kSteps;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const int rb = m >> 3, vb = m & 7;
        acc[vb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.v[vb], xc.v[t][rb], acc[vb][rb], 0, 0, 0);
        if (m < 8) wread1(rs, rstep, m, nxt);
        if ((m & 7) == 3) wload(rn, s + 3, 2 * t + rb);
        if ((m & 7) == 7) xload(s + 2, t, rb, xc);  // into the registers just consumed
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // two stages per iteration: xa holds the hidden rows of even stages, xb of
  // odd ones; the next weight operands always sit in wa (kSteps is even).
  // An odd stage count gets one more stage, whose operands read as zero.
  for (int s = 0; s < nst; s += 2) {
    stage(s, xa);
    stage(s + 1, xb);
  }
  // the loads past the last stage complete before the work-group's LDS is
  // released
  vm_wait<0>();

  // Epilogue.  Accumulator register q of lane (hl, ln) in block (vb, rb)
  // holds the logit of vocabulary entry 32*vb + 8*(q/4) + 4*hl + q%4 of the
  // tile and hidden row 64*wave + 32*rb + ln of the tile.  Per row: max and
  // lowest index over the lane's 128 entries, then over the lane pair
  // (l, l ^ 32), then sum exp(l - max) the same way; one partial per row and
  // vocabulary tile.  Entries past the vocabulary (a ragged last tile) count
  // as -inf.
  constexpr float kLog2e = 1.4426950408889634f;
  const int lim = p.V - v0;
  auto reduce = [&](int rb, auto ragged) {
    constexpr bool kRagged = decltype(ragged)::value;
    auto val = [&](int vb, int q) {
      const float l = acc[vb][rb][q];
      return !kRagged || 32 * vb + 8 * (q >> 2) + 4 * hl + (q & 3) < lim ? l : -INFINITY;
    };
    float m = -INFINITY;
    int idx = INT_MAX;
#pragma unroll
    for (int vb = 0; vb < 8; ++vb)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float l = val(vb, q);
        if (l > m) {  // entries visited in increasing order: keeps the lowest
          m = l;
          idx = v0 + 32 * vb + 8 * (q >> 2) + 4 * hl + (q & 3);
        }
      }
    auto mi = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    auto ii = __builtin_amdgcn_permlane32_swap((unsigned)idx, (unsigned)idx, false, false);
    const float ma = __uint_as_float(mi[0]), mb = __uint_as_float(mi[1]);
    const int ia = (int)ii[0], ib = (int)ii[1];
    const float M = fmaxf(ma, mb);
    const int I = min(ma == M ? ia : INT_MAX, mb == M ? ib : INT_MAX);
    float sum = 0.f;
#pragma unroll
    for (int vb = 0; vb < 8; ++vb)
#pragma unroll
      for (int q = 0; q < 16; ++q) sum += __builtin_amdgcn_exp2f((val(vb, q) - M) * kLog2e);
    auto si = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum), __float_as_uint(sum), false, false);
    const float S = __uint_as_float(si[0]) + __uint_as_float(si[1]);
    const int row = r0 + kWR * wave + 32 * rb + ln;
    if (hl == 0 && row < p.R) {
      UnmaskPart pt;
      pt.m = M;
      pt.s = S;
      pt.idx = I;
      pt.pad = 0;
      p.parts[(size_t)row * p.NC + vt] = pt;
    }
  };
  if (lim >= kVT) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) reduce(rb, std::false_type{});
  } else {  // the ragged last tile: entries past the vocabulary count as -inf
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) reduce(rb, std::true_type{});
  }
}

}  // namespace

int lmhead_chunks(int V) { return (V + kChunk - 1) / kChunk; }

size_t lmhead_pack_bytes(int R, int H) {
  const size_t nrt = (size_t)(R + kRT - 1) / kRT, nst = (size_t)(H + kKS - 1) / kKS;
  return nrt * 4 * nst * kXLoads * kFrag;
}

hipError_t launch_lmhead_parts(const void *hidden, const void *weight, int R, int H, int V,
                               UnmaskPart *parts, void *xpack, hipStream_t stream) {
  static std::atomic<unsigned long long> attr_done{0};  // per device
  const hipError_t e = lds_limit_once((const void *)lmhead_kernel, kSlots * kStageBytes, attr_done);
  if (e != hipSuccess) return e;
  const int nst = (H + kKS - 1) / kKS;
  const long long groups = (long long)((R + kRT - 1) / kRT) * 4 * nst;  // (64-row group, stage) pairs
  hipLaunchKernelGGL(lmhead_pack_kernel, dim3((unsigned)groups), dim3(256), 0, stream,
                     (const __bf16 *)hidden, (bf16x8 *)xpack, R, H, nst);
  LmParams prm;
  prm.xp = (const __bf16 *)xpack;
  prm.w = (const __bf16 *)weight;
  prm.parts = parts;
  prm.R = R;
  prm.H = H;
  prm.V = V;
  prm.NC = lmhead_chunks(V);
  const long long tiles = (long long)((V + kVT - 1) / kVT) * ((R + kRT - 1) / kRT);
  hipLaunchKernelGGL(lmhead_kernel, dim3((unsigned)tiles), dim3(kThreads), kSlots * kStageBytes,
                     stream, prm);
  return hipGetLastError();
}

}  // namespace tt
