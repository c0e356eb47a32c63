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
// the spot to, per row and 128-entry vocabulary chunk, the unmask's partial
// (max, lowest index of the max, sum exp(l - max)); the unmask's merge and
// commit kernels finish the rule.
//
// Work-group: 4 waves, one per SIMD (all 512 VGPRs of a lane are the wave's),
// as a 2 x 2 grid of 128 x 128 wave tiles: wave (vw, rw) owns vocabulary rows
// 128*vw.. and hidden rows 128*rw.. of the tile, 16 MFMA accumulator blocks
// D[32 vocab][32 rows] (v_mfma_f32_32x32x16_bf16, A = weight rows, B =
// hidden rows).  A lane then holds one hidden row of each block, so the
// epilogue's row reductions are lane-local plus one lane-pair exchange.
//
// Operands stream HBM -> LDS by direct loads through buffer descriptors into
// a ring of kSlots stages; a stage is kKS reduction elements of the tile's
// 256 weight rows and 256 hidden rows.  Small stages in many slots keep the
// loads issued well ahead of their use (the ring's lead time is (kSlots - 2)
// stages).  Inside a stage each row keeps its 16-byte chunks XOR-swizzled by
// the row's position in its 256-byte group, which keeps the operand reads
// (32 consecutive rows, one chunk) free of bank conflicts; each direct load
// fills 1 KiB of rows, and a lane fetches whichever chunk the swizzle puts at
// its slot.  One per-lane offset serves every load: load n of a tile adds its
// first row as a scalar offset.
#include <limits.h>

#include "tt_internal.h"

namespace tt {
namespace {

constexpr int kVT = 256;                        // vocabulary rows per work-group tile
constexpr int kRT = 256;                        // hidden rows per work-group tile
constexpr int kChunk = 128;                     // vocabulary entries per partial
#ifndef TT_LM_KS
#define TT_LM_KS 32
#endif
#ifndef TT_LM_SLOTS
#define TT_LM_SLOTS 4
#endif
constexpr int kKS = TT_LM_KS;                   // reduction elements per stage
constexpr int kSlots = TT_LM_SLOTS;             // ring stages
constexpr int kThreads = 256;                   // 4 waves
constexpr int kNCh = kKS / 8;                   // 16-byte chunks per row per stage
constexpr int kSteps = kKS / 16;                // MFMA reduction steps per stage
constexpr int kRowBytes = kKS * 2;              // bytes of one row per stage
constexpr int kRowsPerLoad = 1024 / kRowBytes;  // rows one 1 KiB direct load fills
constexpr int kSwz = 16 / kNCh;                 // rows per 256 bytes: the swizzle's row period
constexpr int kTileBytes = kVT * kRowBytes;     // one operand's part of a stage
constexpr int kStageBytes = 2 * kTileBytes;     // weight part, then hidden part
constexpr int kLoads = kTileBytes / 1024 / 4;   // 1 KiB loads per wave per operand per stage
static_assert(kVT == kRT, "both operand parts of a stage have the same shape");
static_assert(kKS == 16 || kKS == 32, "stage depth");
static_assert(kLoads * 4 * 1024 == kTileBytes, "the waves share a stage's loads evenly");
static_assert(kSlots >= 3 && (kSlots - 3) * 2 * kLoads < 64, "ring depth");
static_assert(kSlots * kStageBytes <= 160 * 1024, "ring fits the LDS");

// Physical 16-byte slot of logical chunk c in row r: XOR with the row's
// position in its 256-byte group, so 16 consecutive rows cover all banks.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r / kSwz) % kNCh); }

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

struct LmParams {
  const __bf16 *x, *w;
  UnmaskPart *parts;  // [R, NC]
  int R, H, V, NC;
};

// Operands of one 16-element reduction step: 4 weight blocks, 4 hidden blocks.
struct Ops {
  bf16x8 w[4], x[4];
};

// Reads the wave's operands of one reduction step of a stage.  Row r of a
// part keeps logical chunk c at r * kRowBytes + 16 * swz(r, c); the wave's
// rows are 32*b + ln of its 128-row half, so the swizzle depends on ln only
// and the block offset goes into the instruction's immediate.
__device__ __forceinline__ void read_ops(const unsigned char *stage, unsigned lane_off, int vw,
                                         int rw, Ops &o) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    o.w[b] = *(const bf16x8 *)(stage + (128 * vw + 32 * b) * kRowBytes + lane_off);
    o.x[b] = *(const bf16x8 *)(stage + kTileBytes + (128 * rw + 32 * b) * kRowBytes + lane_off);
  }
}

// The four MFMAs of weight block vb (128 cycles of matrix-core work).
__device__ __forceinline__ void mfma_row(const Ops &o, int vb, f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
    acc[vb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.w[vb], o.x[rb], acc[vb][rb], 0, 0, 0);
}

// lgkmcnt(0) only (gfx9 encoding): completes this wave's LDS reads.
__device__ __forceinline__ void lds_wait() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}
// vmcnt(n) only.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}
// Wait until at most `stages` stages of this wave's direct loads are in flight.
template <int PER, int MAX>
__device__ __forceinline__ void wait_stages(int stages) {
  if constexpr (MAX > 0) {
    if (stages >= MAX) {
      vm_wait<PER * MAX>();
      return;
    }
    wait_stages<PER, MAX - 1>(stages);
  } else {
    vm_wait<0>();
  }
}
// Work-group barrier ordering LDS only (no global fence, which would drain
// the direct loads still in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  lds_wait();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(kThreads, 1) void lmhead_kernel(LmParams p) {
  extern __shared__ __align__(16) unsigned char ring[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 31, hl = lane >> 5;
  const int vw = wave >> 1, rw = wave & 1;
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
  const int w_rows = min(kVT, p.V - v0), x_rows = min(kRT, p.R - r0);
  const __bf16 *wb = p.w + (size_t)v0 * p.H;
  const __bf16 *xb = p.x + (size_t)r0 * p.H;
  const int nst = p.H / kKS;

  // Direct loads: lane l of a load fills bytes 16l.. of 1 KiB = tile rows
  // kRowsPerLoad*n + l/kNCh (n = the load), physical chunk l%kNCh, i.e. the
  // logical chunk that swz() puts there; rows past the operand's end read as
  // zero (descriptor range).  Load n adds n*kRowsPerLoad rows as a scalar
  // offset, which leaves the swizzle unchanged (kRowsPerLoad is a multiple of
  // its row period times kNCh).
  static_assert(kRowsPerLoad % (kSwz * kNCh) == 0, "load boundaries keep the swizzle");
  const int lrow = lane / kNCh;
  const unsigned voff = (unsigned)((lrow * p.H + 8 * swz(lrow, lane % kNCh)) * 2);
  // Load j (0 .. 2*kLoads-1) of this wave for stage s: weight part first.
  // Issued one at a time between MFMA groups: the wave is the only one on
  // its SIMD, and a load that waits for room in the memory queue holds up
  // its instruction stream, so each load sits behind 128 cycles of queued
  // matrix-core work instead of in a burst.
  auto issue_one = [&](int s, int j) {
    unsigned char *st = ring + (s % kSlots) * kStageBytes;
    const int k0 = s * kKS;
    const bool wpart = j < kLoads;
    const int n = kLoads * wave + (wpart ? j : j - kLoads);
    const __amdgpu_buffer_rsrc_t r =
        wpart ? buffer_rsrc(wb + k0, (w_rows * p.H - k0) * 2) : buffer_rsrc(xb + k0, (x_rows * p.H - k0) * 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(st + (wpart ? 0 : kTileBytes) + n * 1024), 16,
                                             voff, (unsigned)(n * kRowsPerLoad * p.H * 2), 0, 0);
  };
  auto issue = [&](int s) {
    if (s >= nst) return;
#pragma unroll
    for (int j = 0; j < 2 * kLoads; ++j) issue_one(s, j);
  };
  constexpr int kPer = 2 * kLoads;  // direct loads per wave per stage

  // operand read offsets of this lane for reduction step t of a stage:
  // row ln of a 32-row block, logical chunk 2*t + hl
  unsigned loff[kSteps];
#pragma unroll
  for (int t = 0; t < kSteps; ++t) loff[t] = (unsigned)(ln * kRowBytes + 16 * swz(ln, 2 * t + hl));

  f32x16 acc[4][4];
#pragma unroll
  for (int vb = 0; vb < 4; ++vb)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) acc[vb][rb] = f32x16{};

  // Prologue: stages 0 .. kSlots-2 in flight, stage 0 landed and visible.
  // In iteration s, stage s + 1 is awaited (it was issued kSlots - 3
  // iterations earlier), so the operands of its first step can be read
  // under the last MFMAs of stage s; stage s + kSlots - 1 then takes the
  // slot of stage s - 1, which every wave has finished reading.
  for (int s = 0; s < kSlots - 1; ++s) issue(s);
  wait_stages<kPer, kSlots - 2>(min(kSlots - 2, nst - 1));
  lds_barrier();
  Ops buf[2];
  read_ops(ring, loff[0], vw, rw, buf[0]);

  // One stage: operands of its first step are in `cur`; the next stage's
  // first operands end up in `cur` (two steps per stage) or `nxt` (one).
  static_assert(2 * kLoads == 4 * kSteps, "one load per MFMA group");
  auto stage = [&](int s, Ops &cur, Ops &nxt) {
    if (s + 1 < nst) {
      wait_stages<kPer, kSlots - 3>(min(kSlots - 3, nst - 2 - s));
      lds_barrier();
    }
    const int sn = s + kSlots - 1;  // stage loaded into the slot of stage s - 1
    const bool load = sn < nst;
    const unsigned char *st = ring + (s % kSlots) * kStageBytes;
    const unsigned char *st1 = ring + ((s + 1) % kSlots) * kStageBytes;
#pragma unroll
    for (int t = 0; t < kSteps; ++t) {
      const Ops &o = t == 0 ? cur : nxt;
      lds_wait();
      __builtin_amdgcn_sched_barrier(0);
      if (t + 1 < kSteps) read_ops(st, loff[t + 1], vw, rw, nxt);
      else if (s + 1 < nst) read_ops(st1, loff[0], vw, rw, kSteps == 2 ? cur : nxt);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int vb = 0; vb < 4; ++vb) {
        mfma_row(o, vb, acc);
        __builtin_amdgcn_sched_barrier(0);
        if (load) issue_one(sn, 4 * t + vb);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  for (int s = 0; s < nst; ++s) {
    stage(s, buf[0], buf[1]);
    if (kSteps == 1) buf[0] = buf[1];  // register moves, under the MFMAs
  }

  // Epilogue.  Accumulator register q of lane (hl, ln) in block (vb, rb)
  // holds the logit of vocabulary entry 32*vb + 8*(q/4) + 4*hl + q%4 of the
  // wave's half and hidden row 32*rb + ln of its half.  Per row: max and
  // lowest index over the lane's 64 entries, then over the lane pair
  // (l, l ^ 32), then sum exp(l - max) the same way.
  const int vbase = v0 + 128 * vw;
  if (vbase >= p.V) return;  // this wave's half lies past the vocabulary
  const int chunk = vbase / kChunk;
  constexpr float kLog2e = 1.4426950408889634f;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    float m = -INFINITY;
    int idx = INT_MAX;
#pragma unroll
    for (int vb = 0; vb < 4; ++vb)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int v = vbase + 32 * vb + 8 * (q >> 2) + 4 * hl + (q & 3);
        const float l = acc[vb][rb][q];
        if (v < p.V && l > m) {  // entries visited in increasing v: keeps the lowest
          m = l;
          idx = v;
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
    for (int vb = 0; vb < 4; ++vb)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int v = vbase + 32 * vb + 8 * (q >> 2) + 4 * hl + (q & 3);
        const float e = __builtin_amdgcn_exp2f((acc[vb][rb][q] - M) * kLog2e);
        sum += v < p.V ? e : 0.f;
      }
    auto si = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum), __float_as_uint(sum), false, false);
    const float S = __uint_as_float(si[0]) + __uint_as_float(si[1]);
    const int row = r0 + 128 * rw + 32 * rb + ln;
    if (hl == 0 && row < p.R) {
      UnmaskPart pt;
      pt.m = M;
      pt.s = S;
      pt.idx = I;
      pt.pad = 0;
      p.parts[(size_t)row * p.NC + chunk] = pt;
    }
  }
}

}  // namespace

int lmhead_chunks(int V) { return (V + kChunk - 1) / kChunk; }

hipError_t launch_lmhead_parts(const void *hidden, const void *weight, int R, int H, int V,
                               UnmaskPart *parts, hipStream_t stream) {
  static bool attr_done = false;  // benign race: every caller sets the same value
  if (!attr_done) {
    const hipError_t e = hipFuncSetAttribute((const void *)lmhead_kernel,
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             kSlots * kStageBytes);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  LmParams prm;
  prm.x = (const __bf16 *)hidden;
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
