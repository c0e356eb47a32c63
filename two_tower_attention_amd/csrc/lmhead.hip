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
// a ring of kSlots stages; a stage is 32 reduction elements (64 bytes) of the
// tile's 256 weight rows and 256 hidden rows.  Inside a stage each 64-byte
// row keeps its four 16-byte chunks XOR-swizzled by bits 2..3 of the row
// index, which keeps the operand reads (32 consecutive rows, one chunk)
// free of bank conflicts; each direct load fills 1 KiB = 16 rows, and a lane
// fetches whichever chunk the swizzle puts at its slot.  One per-lane offset
// serves every load: load n of a tile adds n * 16 rows as a scalar offset.
#include <limits.h>

#include "tt_internal.h"

namespace tt {
namespace {

constexpr int kVT = 256;                        // vocabulary rows per work-group tile
constexpr int kRT = 256;                        // hidden rows per work-group tile
constexpr int kChunk = 128;                     // vocabulary entries per partial
constexpr int kKS = 32;                         // reduction elements per stage
constexpr int kSlots = 4;                       // ring stages (kSlots - 1 in flight)
constexpr int kThreads = 256;                   // 4 waves
constexpr int kRowBytes = kKS * 2;              // 64 bytes of one row per stage
constexpr int kTileBytes = kVT * kRowBytes;     // 16 KiB: one operand's part of a stage
constexpr int kStageBytes = 2 * kTileBytes;     // weight part, then hidden part
constexpr int kLoads = kTileBytes / 1024 / 4;   // 4 KiB-loads per wave per operand per stage
static_assert(kVT == kRT, "both operand parts of a stage have the same shape");
static_assert(kLoads * 4 * 1024 == kTileBytes, "the waves share a stage's loads evenly");

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

// Reads the wave's operands of reduction step ks (0, 1) of a stage.  Row r
// of a part, logical chunk c sits at r * 64 + 16 * (c ^ ((r >> 2) & 3)); the
// wave's rows are 32*b + ln of its 128-row half, so the XOR term depends on
// ln only and the block offset goes into the instruction's immediate.
__device__ __forceinline__ void read_ops(const unsigned char *stage, unsigned lane_off, int vw,
                                         int rw, Ops &o) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    o.w[b] = *(const bf16x8 *)(stage + (128 * vw + 32 * b) * kRowBytes + lane_off);
    o.x[b] = *(const bf16x8 *)(stage + kTileBytes + (128 * rw + 32 * b) * kRowBytes + lane_off);
  }
}

__device__ __forceinline__ void mfma_ops(const Ops &o, f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int vb = 0; vb < 4; ++vb)
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
  const int nrt = (p.R + kRT - 1) / kRT;
  const int rt = blockIdx.x % nrt, vt = blockIdx.x / nrt;  // the row tiles of a vocabulary tile run together
  const int r0 = rt * kRT, v0 = vt * kVT;
  const int w_rows = min(kVT, p.V - v0), x_rows = min(kRT, p.R - r0);
  const __bf16 *wb = p.w + (size_t)v0 * p.H;
  const __bf16 *xb = p.x + (size_t)r0 * p.H;
  const int nst = p.H / kKS;

  // Direct loads: lane l of a load fills bytes 16l.. of 1 KiB = tile rows
  // 16n + l/4 (n = the load), physical chunk l%4, i.e. logical chunk
  // (l%4) ^ ((l/16)%4); rows past the operand's end read as zero (descriptor
  // range).
  const unsigned voff = (unsigned)(((lane >> 2) * p.H + 8 * ((lane & 3) ^ ((lane >> 4) & 3))) * 2);
  auto issue = [&](int s) {
    if (s >= nst) return;
    unsigned char *st = ring + (s % kSlots) * kStageBytes;
    const int k0 = s * kKS;
    const __amdgpu_buffer_rsrc_t rw_ = buffer_rsrc(wb + k0, (w_rows * p.H - k0) * 2);
    const __amdgpu_buffer_rsrc_t rx_ = buffer_rsrc(xb + k0, (x_rows * p.H - k0) * 2);
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int n = kLoads * wave + j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw_, (lds_void *)(st + n * 1024), 16, voff,
                                               (unsigned)(n * 32 * p.H), 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int n = kLoads * wave + j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx_, (lds_void *)(st + kTileBytes + n * 1024), 16,
                                               voff, (unsigned)(n * 32 * p.H), 0, 0);
    }
  };
  constexpr int kPer = 2 * kLoads;  // direct loads per wave per stage

  const int xo = (ln >> 2) & 3;
  const unsigned off0 = (unsigned)(ln * kRowBytes + 16 * ((0 + hl) ^ xo));  // step 0: chunks 0, 1
  const unsigned off1 = (unsigned)(ln * kRowBytes + 16 * ((2 + hl) ^ xo));  // step 1: chunks 2, 3

  f32x16 acc[4][4];
#pragma unroll
  for (int vb = 0; vb < 4; ++vb)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) acc[vb][rb] = f32x16{};

  // prologue: stages 0 .. kSlots-2 in flight, stage 0 landed and visible
  for (int s = 0; s < kSlots - 1; ++s) issue(s);
  if (nst >= 3) vm_wait<2 * kPer>();
  else if (nst == 2) vm_wait<kPer>();
  else vm_wait<0>();
  lds_barrier();
  Ops buf[2];
  read_ops(ring, off0, vw, rw, buf[0]);

  for (int s = 0; s < nst; ++s) {
    // Stage s + 1 landed and visible to all waves; every wave is past stage
    // s - 1, whose slot takes stage s + kSlots - 1.
    if (s + 1 < nst) {
      if (s + 2 < nst) vm_wait<kPer>();
      else vm_wait<0>();
      lds_barrier();
    }
    issue(s + kSlots - 1);
    const unsigned char *st = ring + (s % kSlots) * kStageBytes;
    lds_wait();
    __builtin_amdgcn_sched_barrier(0);
    read_ops(st, off1, vw, rw, buf[1]);
    __builtin_amdgcn_sched_barrier(0);
    mfma_ops(buf[0], acc);
    __builtin_amdgcn_sched_barrier(0);
    lds_wait();
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 < nst) read_ops(ring + ((s + 1) % kSlots) * kStageBytes, off0, vw, rw, buf[0]);
    __builtin_amdgcn_sched_barrier(0);
    mfma_ops(buf[1], acc);
    __builtin_amdgcn_sched_barrier(0);
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
