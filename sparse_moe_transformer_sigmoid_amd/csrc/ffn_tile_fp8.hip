// Grouped expert FFN with fp8 e4m3 weights (128 x 128 blocks) and dynamically
// quantised activations, tiled schedule for many rows per expert.
// ("Kimi K2 . Down projection", config.json quantization_config: fmt e4m3,
// weight_block_size [128, 128], activation_scheme dynamic.)
//
// Data movement as in the bf16 tile kernel -- both operands go global -> LDS
// by DMA (global_load_lds_dwordx4), 128-byte unpadded LDS rows with the slot
// swizzle chunk ^ ((row >> 1) & 7), XCD-chunked order of the work items --
// but with separate LDS rings for the weight rows (six stages, each half of
// a step's rows) and the grouped rows (three stages), the DMA issued from
// inline asm and waited for with counted s_waitcnt.  A 128-byte row is 128
// fp8 K-elements: exactly one quantisation block per K step, so each step is
// two v_mfma_scale_f32_32x32x64_f8f6f4 (unit e8m0 scales) per 32x32 output
// tile into a fresh partial, added to the fp32 accumulator scaled by
// weight-block scale x row scale:
//   acc += (sum_k q_w q_a) * s_w[block][kb] * s_a[row][kb].
// The block is 256 weight rows x 128 grouped rows in 8 waves of 64 x 64.
// gate_up writes the SwiGLU output already quantised for the down projection
// (e4m3 codes + one scale per row and 128 channels); down writes bf16.
#include "kernels.h"

namespace moe {

namespace {

constexpr int kBM = 128;                      // grouped rows per work item
constexpr int kBW = 256;                      // weight rows per slab
constexpr int kRowB = 128;                    // bytes per LDS row = K elements per step
constexpr int kWStage = (kBW / 2) * kRowB;    // 16 KB: one half of a step's weight rows
constexpr int kXData = kBM * kRowB;           // 16 KB: a step's grouped rows
constexpr int kXStage = kXData + 8 * 64 * 4;  // + their row scales: 64 slots per wave
constexpr int kMaxKB = 64;                     // K blocks (K <= 8192) of the weight-scale table
constexpr int kXcd = 8;

// Global -> LDS DMA issued from inline asm, so that the compiler neither
// tracks it nor places its own (full) waits for it: every wait on these
// loads is an explicit s_waitcnt vmcnt(n) below.  The instruction has no
// register result (lane i writes 16 or 4 bytes at LDS address m0 + 16 i or
// m0 + 4 i); its address operands are read at issue.  SADDR form: a
// wave-uniform 64-bit base in SGPRs plus a 32-bit lane byte offset.
template <bool NT = false>
__device__ __forceinline__ void dma16(uint64_t base, uint32_t voff, uint32_t lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds);
  if (NT)
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(m0v), "v"(voff), "s"(base) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0v), "v"(voff), "s"(base) : "memory", "m0");
}
__device__ __forceinline__ void dma4(uint64_t base, uint32_t voff, uint32_t lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(m0v), "v"(voff), "s"(base) : "memory", "m0");
}
// a wave-uniform pointer as a 64-bit SGPR base (each half through uint32_t:
// readfirstlane returns int, which would sign-extend the low word)
__device__ __forceinline__ uint64_t sbase(const void* p) {
  const uint64_t b = reinterpret_cast<uint64_t>(p);
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32)));
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b)));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
// LDS byte address of a __shared__ object (an address-space cast)
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)(p)));
}

__device__ __forceinline__ f32x16 mma_fp8_32(const uint4& a0, const uint4& a1, const uint4& b0,
                                             const uint4& b1, const f32x16& c) {
  i32x8 av, bv;
  av[0] = a0.x; av[1] = a0.y; av[2] = a0.z; av[3] = a0.w;
  av[4] = a1.x; av[5] = a1.y; av[6] = a1.z; av[7] = a1.w;
  bv[0] = b0.x; bv[1] = b0.y; bv[2] = b0.z; bv[3] = b0.w;
  bv[4] = b1.x; bv[5] = b1.y; bv[6] = b1.z; bv[7] = b1.w;
  // formats 0 = fp8 e4m3 for A and B; scale 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, 127, 0, 127);
}

}  // namespace

// MODE 0: gate_up (K = H; slab = 128 features = 128 gate + 128 up rows)
// MODE 1: down    (K = F or Fs; slab = 256 output rows)
// A K step (one 128-wide quantisation block) is taken in two halves, each
// over one half of the slab's weight rows (gate_up: the gate rows, then the
// up rows; down: output rows o0 + [0, 128), then o0 + 128 + [0, 128)) and
// all 128 grouped rows.  The weight halves stream through a ring of six
// 16 KB stages (the DMA of half h + 5 is issued during half h, so five
// halves -- 80 KB of weights -- are in flight per block), the grouped rows
// through a ring of three 16 KB stages (+ their row scales; the DMA of step
// s + 2 during step s).  8 waves, two per SIMD: wave (wm, wn) owns weight
// rows 32*wm + [0, 32) of each half (gate_up: gate then up rows of features
// o0 + 32*wm + [0, 32)) and grouped rows 64*wn + [0, 64); while one wave of
// a SIMD applies the scales of its partial products (VALU), the other's
// MFMAs run.  WNT: the weight DMA carries the nontemporal hint.  The LDS
// rings and table are the kernel's (one allocation for both copies of this
// body that the kernel inlines).
template <int MODE, bool WNT>
__device__ __forceinline__ void tile_fp8_body(const FfnArgs& a, int slab, const Tile& tl, uint8_t* ws0,
                                              uint8_t* ws1, uint8_t* ws2, uint8_t* ws3, uint8_t* ws4,
                                              uint8_t* ws5, uint8_t* xs0, uint8_t* xs1, uint8_t* xs2,
                                              float* wscale) {
  const bool sh = tl.group == a.E;
  const int Fg = sh ? a.Fs : a.F;
  const int64_t TK = static_cast<int64_t>(a.T) * a.k;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;        // 32 weight rows (per half) x 64 grouped rows
  const int r32 = lane & 31, kh = lane >> 5;
  const int drow = lane >> 3;
  const int dch[2] = {(lane & 7) ^ ((drow >> 1) & 7), (lane & 7) ^ ((4 + (drow >> 1)) & 7)};

  // ---- weights: this wave's DMA fills rows 16*wave + [0, 16) of each half
  // (2 instructions of 8 rows); the compute side reads rows 32*wm + [0, 32) ----
  int K, o0;
  const uint8_t* wdma[2];            // wave-uniform: the first of the wave's 16 DMA rows, per half
  const float* wsc[2];               // weight-block scale rows of the two halves
  int64_t KB;
  if (MODE == 0) {
    K = a.H;
    KB = K / 128;
    o0 = slab * (kBW / 2);
    if (o0 >= Fg) return;
    const int64_t wofs = sh ? 0 : static_cast<int64_t>(tl.group) * a.F * a.H;
    const uint8_t* wg = static_cast<const uint8_t*>(sh ? a.sh_gate : a.w_gate) + wofs;
    const uint8_t* wu = static_cast<const uint8_t*>(sh ? a.sh_up : a.w_up) + wofs;
    wdma[0] = wg + static_cast<int64_t>(o0 + 16 * wave) * K;
    wdma[1] = wu + static_cast<int64_t>(o0 + 16 * wave) * K;
    const int64_t sofs = (sh ? 0 : static_cast<int64_t>(tl.group) * (a.F / 128) * KB) + (o0 / 128) * KB;
    wsc[0] = (sh ? a.sh_s_gate : a.s_gate) + sofs;
    wsc[1] = (sh ? a.sh_s_up : a.s_up) + sofs;
  } else {
    K = Fg;
    KB = K / 128;
    o0 = slab * kBW;
    const int64_t wofs = sh ? 0 : static_cast<int64_t>(tl.group) * a.H * a.F;
    const uint8_t* wd = static_cast<const uint8_t*>(sh ? a.sh_down : a.w_down) + wofs;
    wdma[0] = wd + static_cast<int64_t>(o0 + 16 * wave) * K;
    wdma[1] = wd + static_cast<int64_t>(o0 + kBW / 2 + 16 * wave) * K;
    const int64_t sofs = (sh ? 0 : static_cast<int64_t>(tl.group) * (a.H / 128) * KB) + (o0 / 128) * KB;
    wsc[0] = (sh ? a.sh_s_down : a.s_down) + sofs;
    wsc[1] = wsc[0] + KB;
  }
  // (two scalars, not an array: a select between array elements became a
  // dynamically indexed array, which the compiler placed in LDS)
  const uint64_t wbase0 = sbase(wdma[0]), wbase1 = sbase(wdma[1]);
  // lane offset of weight DMA instruction g (rows 8 g + drow of the wave's 16)
  uint32_t woff[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) woff[g] = static_cast<uint32_t>((8 * g + drow) * K + dch[g] * 16);
  // ---- grouped rows: this wave's DMA fills rows 16*wave + [0, 16) of a
  // grouped-row stage; lane offsets from the (wave-uniform) start of the code
  // rows: token * H (gathered routed rows), else the row index * row length
  // (under 2^32 bytes: tile_fp8_shapes_ok) ----
  const uint8_t* xrow0;   // wave-uniform
  if (MODE == 0)
    xrow0 = sh ? static_cast<const uint8_t*>(a.xs) : static_cast<const uint8_t*>(a.xr);
  else
    xrow0 = sh ? static_cast<const uint8_t*>(a.hq_sh) : static_cast<const uint8_t*>(a.hq);
  const uint64_t xbase = sbase(xrow0);
  uint32_t xoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int tr = 16 * wave + 8 * i + drow;
    const int64_t p = tl.row0 + min(tr, tl.rows - 1);
    int64_t r, ld;
    if (MODE == 0) {
      r = sh ? p - TK : (a.xr_rows ? a.xr_rows[p] : p);
      ld = a.H;
    } else {
      r = sh ? p - TK : p;
      ld = sh ? a.Fs : a.F;
    }
    xoff[i] = static_cast<uint32_t>(r * ld + dch[i] * 16);
  }
  // ---- weight-block scales of the two halves, all K blocks, into LDS once
  // (read there at every half step) ----
  for (int i = tid; i < KB; i += 512) {
    wscale[i] = wsc[0][i];
    wscale[kMaxKB + i] = wsc[1][i];
  }
  // ---- row scales: lane l of this wave copies the scale of grouped row
  // 16*wave + l % 16 for each step into the stage's 64 slots of the wave
  // (kXData + 256 * wave + 4 * l; the compute side reads l < 16) ----
  // gate_up reads them K-block-major ([K block][grouped row], gathered by
  // the same launch: a step's 16 rows are 64 contiguous bytes); down reads
  // h's row-major scales ([row][K block])
  uint64_t rbase;   // wave-uniform start of the scale rows
  uint32_t roff;    // this lane's row, in bytes
  uint32_t rstep;   // bytes from one K block to the next
  {
    const int tr = 16 * wave + (lane & 15);
    const int64_t p = tl.row0 + min(tr, tl.rows - 1);
    if (MODE == 0) {
      rbase = sbase(a.xrs_t);
      roff = static_cast<uint32_t>(p * 4);
      rstep = static_cast<uint32_t>((TK + a.T) * 4);
    } else {
      rbase = sbase(sh ? a.h_sh_scales : a.h_scales);
      roff = static_cast<uint32_t>((sh ? p - TK : p) * KB * 4);
      rstep = 4;
    }
  }
  const int steps = static_cast<int>(KB), halves = 2 * steps;
  // the DMA of weight half hh (step hh / 2, half hh % 2; clamped to the last
  // one, whose data then lands in a stage nobody reads again): 2 issues
  auto dma_w = [&](int hh, uint8_t* st) {
    hh = min(hh, halves - 1);
    const uint32_t ko = static_cast<uint32_t>(hh >> 1) * kRowB;
    const uint32_t l = lds_addr(st) + 16 * wave * kRowB;
    const uint64_t b = (hh & 1) ? wbase1 : wbase0;
    dma16<WNT>(b, woff[0] + ko, l);
    dma16<WNT>(b, woff[1] + ko, l + 8 * kRowB);
  };
  // the DMA of the grouped rows of step s (clamped likewise): 2 row issues,
  // then the 16 row scales
  auto dma_x = [&](int s, uint8_t* st) {
    s = min(s, steps - 1);
    const uint32_t ko = static_cast<uint32_t>(s) * kRowB;
    const uint32_t l = lds_addr(st);
    dma16(xbase, xoff[0] + ko, l + (16 * wave) * kRowB);
    dma16(xbase, xoff[1] + ko, l + (16 * wave + 8) * kRowB);
    dma4(rbase, roff + rstep * static_cast<uint32_t>(s), l + kXData + 256 * wave);
  };

  f32x16 acc[2][2];   // [half][grouped-row tile]
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][n][i] = 0.f;

  const int sw = (r32 >> 1) & 7;
  const int arow = (32 * wm + r32) * kRowB;
  const int brow = (64 * wn + r32) * kRowB;
  // grouped row r = 64 wn + 32 n + r32 has its scale at kXData + 256 (r / 16) + 4 (r % 16)
  const int srow = kXData + 256 * (4 * wn + (r32 >> 4)) + 4 * (r32 & 15);
  // fragments of one 32-row tile: MFMA i (0, 1) takes chunks kh*4 + 2i, +1
  auto frag = [&](const uint8_t* st, int row, uint4 (&f)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) f[c] = *reinterpret_cast<const uint4*>(st + row + (((kh * 4 + c) ^ sw) * 16));
  };
  // The partial products of the previous half step and their scales: folded
  // into that half's accumulators during the next half step, while its MFMAs
  // run (the fold does not wait on them).  Each accumulator still takes its
  // K blocks in order.  Before the first half step: zeros (a fold of 0 x 0).
  f32x16 pp[2];
  float psc[2] = {0.f, 0.f};
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int i = 0; i < 16; ++i) pp[n][i] = 0.f;
  // One half step: weight half h of step s from stage w against the grouped
  // rows' fragments bf (read from the step's stage in the first half, kept
  // in registers for the second): two 32x32 tiles' partial products, then
  // the previous half step's partials folded into its accumulators (of half
  // 1 - h) while these MFMAs run; issue() runs the half step's DMA between
  // them.  Then the counted wait: at most `keep` of this wave's DMA issues
  // may still be outstanding (those of the last four half steps that the
  // next half step does not read), and this wave's LDS reads are done
  // (lgkmcnt); then the barrier.
  auto half = [&](const uint8_t* w, auto hc, int s, const uint4 (&bf)[2][4], const float (&rs)[2], auto issue,
                  auto keep) {
    constexpr int h = decltype(hc)::value;
    const float ws = wscale[h * kMaxKB + s];
    uint4 af[4];
    frag(w, arow, af);
    f32x16 p[2];
    auto part = [&](int n) {
      f32x16 z;
#pragma unroll
      for (int i = 0; i < 16; ++i) z[i] = 0.f;
      z = mma_fp8_32(af[0], af[1], bf[n][0], bf[n][1], z);
      p[n] = mma_fp8_32(af[2], af[3], bf[n][2], bf[n][3], z);
    };
    part(0);
    part(1);
    issue();
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[1 - h][n][i] = fmaf(pp[n][i], psc[n], acc[1 - h][n][i]);
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      pp[n] = p[n];
      psc[n] = ws * rs[n];
    }
    // (fenced against the scheduler: nothing moves across the wait)
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (decltype(keep)::value == 14)
      asm volatile("s_waitcnt vmcnt(14) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(11) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // One step s on grouped-row stage x and weight stages w0 (half 0), w1
  // (half 1): the first half issues the grouped rows of step s + 2 (into xn,
  // the stage of step s - 1) and weight half 2s + 5 (into wp, the stage of
  // half 2s - 1); the second issues weight half 2s + 6 (into w0).  Waits:
  // after the first half the next one needs weight half 2s + 1 (issued
  // during half 2s - 4: 14 issues since); after the second, the next step
  // needs weight half 2s + 2 and the grouped rows of step s + 1 (issued
  // during half 2s - 2 before its 2 weight issues: 11 issues since).
  auto step = [&](uint8_t* x, uint8_t* xn, uint8_t* w0, uint8_t* w1, uint8_t* wp, int s) {
    uint4 bf[2][4];
    frag(x, brow, bf[0]);
    frag(x, brow + 32 * kRowB, bf[1]);
    const float rs[2] = {*reinterpret_cast<const float*>(x + srow),
                         *reinterpret_cast<const float*>(x + srow + 512)};
    half(w0, std::integral_constant<int, 0>(), s, bf, rs, [&] { dma_x(s + 2, xn); dma_w(2 * s + 5, wp); },
         std::integral_constant<int, 14>());
    half(w1, std::integral_constant<int, 1>(), s, bf, rs, [&] { dma_w(2 * s + 6, w0); },
         std::integral_constant<int, 11>());
  };

  // as if issued by half steps -5 .. -1: weight halves 0..4 and the grouped
  // rows of steps 0 and 1 (same order, so the same counted wait: the first
  // step needs weight half 0 and grouped rows 0, 11 issues before the end)
  dma_w(0, ws0);
  dma_x(0, xs0);
  dma_w(1, ws1);
  dma_w(2, ws2);
  dma_x(1, xs1);
  dma_w(3, ws3);
  dma_w(4, ws4);
  // (lgkmcnt: the weight-scale table written above is visible after the barrier)
  asm volatile("s_waitcnt vmcnt(11) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // steps in threes (grouped-row stages 0, 1, 2; weight stages 0..5)
  int s = 0;
  for (; s + 2 < steps; s += 3) {
    step(xs0, xs2, ws0, ws1, ws5, s);
    step(xs1, xs0, ws2, ws3, ws1, s + 1);
    step(xs2, xs1, ws4, ws5, ws3, s + 2);
  }
  if (s < steps) step(xs0, xs2, ws0, ws1, ws5, s);
  if (s + 1 < steps) step(xs1, xs0, ws2, ws3, ws1, s + 1);
  // the last half step's partials (half 1)
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[1][n][i] = fmaf(pp[n][i], psc[n], acc[1][n][i]);
  // no DMA may still be writing LDS when the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: lane holds weight rows 8*(i/4) + 4*kh + (i%4) of each
  // 32-row tile, for grouped row 64*wn + 32*n + r32 ----
  if (MODE == 0) {
    // h = SiLU(gate) * up, quantised here for the down projection: the slab's
    // 128 features are one 128-channel group ("Kimi K2 . Down projection",
    // activation_scheme dynamic), held by the four waves wm of a row half
    // wn, 16 values per lane.  s = amax / 448 (1 for an all-zero group),
    // codes e4m3(h / s) with the division in fp32 -- the same arithmetic as
    // the activation-quant kernel.  The row maxima meet in LDS, in the
    // weight-scale table: no DMA ever targets it (a stage may still receive a
    // refill that another wave issued in the last step, which only that
    // wave's own vmcnt(0) above waits for), and the last half step's barrier
    // came after every wave's reads of the table (lgkmcnt(0)).
    float hv[2][16], rmax[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        hv[n][i] = silu(acc[0][n][i]) * acc[1][n][i];
        m = fmaxf(m, fabsf(hv[n][i]));
      }
      rmax[n] = fmaxf(m, __shfl_xor(m, 32, 64));
    }
    float* gmax = wscale;   // [4 wm][128 rows]
    if (kh == 0) {
#pragma unroll
      for (int n = 0; n < 2; ++n) gmax[128 * wm + 64 * wn + 32 * n + r32] = rmax[n];
    }
    __syncthreads();
    const int64_t gidx = o0 / 128;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int tr = 64 * wn + 32 * n + r32;
      if (tr >= tl.rows) continue;
      const float amax = fmaxf(fmaxf(gmax[tr], gmax[128 + tr]), fmaxf(gmax[256 + tr], gmax[384 + tr]));
      const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
      const int64_t p = tl.row0 + tr;
      uint8_t* dst = sh ? static_cast<uint8_t*>(a.hq_sh) + (p - TK) * a.Fs : static_cast<uint8_t*>(a.hq) + p * a.F;
      dst += o0 + 32 * wm + 4 * kh;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint32_t c = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) c |= static_cast<uint32_t>(f32_to_e4m3(hv[n][4 * g + e] / sc)) << (8 * e);
        *reinterpret_cast<uint32_t*>(dst + 8 * g) = c;
      }
      if (wm == 0 && kh == 0) {
        float* sdst = sh ? a.h_sh_scales + (p - TK) * (a.Fs / 128) : a.h_scales + p * (a.F / 128);
        sdst[gidx] = sc;
      }
    }
    return;
  }
  // down: y in bf16 (half m holds output rows o0 + 128 m + 32 wm + .)
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int tr = 64 * wn + 32 * n + r32;
    if (tr >= tl.rows) continue;
    const int64_t p = tl.row0 + tr;
    uint16_t* dst = sh ? static_cast<uint16_t*>(a.y_sh) + (p - TK) * a.H
                       : static_cast<uint16_t*>(a.y) + p * a.H;
    dst += o0 + 32 * wm + 4 * kh;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 v2;
        v2.x = static_cast<uint32_t>(f32_to_bf16(acc[m][n][4 * g + 0])) |
               (static_cast<uint32_t>(f32_to_bf16(acc[m][n][4 * g + 1])) << 16);
        v2.y = static_cast<uint32_t>(f32_to_bf16(acc[m][n][4 * g + 2])) |
               (static_cast<uint32_t>(f32_to_bf16(acc[m][n][4 * g + 3])) << 16);
        *reinterpret_cast<uint2*>(dst + (kBW / 2) * m + 8 * g) = v2;
      }
  }
}

// WNT: the weight DMA of routed tiles carries the nontemporal hint (each
// routed weight slab is expected to be read by one tile only); never that
// of the shared expert, whose slabs every token tile reads.  The block
// branches once, on its tile, between two inlined copies of the pipeline (a
// branch per DMA issue made the kernel spill).
template <int MODE, bool WNT>
__global__ __launch_bounds__(512) void ffn_tile_fp8(FfnArgs a, int slabs) {
  // the rings as separate objects (compile-time LDS addresses)
  __shared__ __attribute__((aligned(16))) uint8_t ws0[kWStage], ws1[kWStage], ws2[kWStage], ws3[kWStage],
      ws4[kWStage], ws5[kWStage];
  __shared__ __attribute__((aligned(16))) uint8_t xs0[kXStage], xs1[kXStage], xs2[kXStage];
  __shared__ float wscale[4 * kBM];   // [half][K block] (kMaxKB each); the epilogue's row maxima
  static_assert(2 * kMaxKB <= 4 * kBM, "weight-scale table fits");
  const int ntile = *a.tile_count;
  const int total = slabs * ntile;
  const int per = (total + kXcd - 1) / kXcd;
  const int j = blockIdx.x / kXcd;
  const int v = (blockIdx.x % kXcd) * per + j;
  if (j >= per || v >= total) return;
  // tile-major: the slabs of one tile side by side on an XCD, so its
  // grouped rows are fetched once per XCD.  Measured on the K2 fp8 layer:
  // down 1-2 % faster than slab-major (T = 512..8192); gate_up on the
  // current kernel 1.2 % faster at T = 2048 and 4096 (FETCH_SIZE -16 % at
  // T = 4096), unchanged at 512 and 1024.
  const int tix = v / slabs;
  const int slab = v - tix * slabs;
  const Tile tl = a.tiles[tix];
  // (without the hint one copy serves every tile)
  if (WNT && tl.group != a.E)
    tile_fp8_body<MODE, WNT>(a, slab, tl, ws0, ws1, ws2, ws3, ws4, ws5, xs0, xs1, xs2, wscale);
  else
    tile_fp8_body<MODE, false>(a, slab, tl, ws0, ws1, ws2, ws3, ws4, ws5, xs0, xs1, xs2, wscale);
}

// The row scales of the grouped rows of the tiled fp8 gate_up in
// K-block-major order: st[kb][p] = the scale of grouped row p's activation
// row in K block kb (routed rows p < T k through the row -> token map, shared
// row T k + t = token t).  A thread per grouped row, so the writes of one K
// block are contiguous across the block; routed rows past offsets[E] (unused
// capacity) are skipped.
__global__ __launch_bounds__(256) void gather_scales_t(FfnArgs a) {
  const int64_t TK = static_cast<int64_t>(a.T) * a.k, R = TK + a.T;
  const int64_t p = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (p >= R) return;
  const int KB = a.H / 128;
  const float* src;
  if (p < TK) {
    if (p >= a.offsets[a.E]) return;
    src = a.xr_scales + static_cast<int64_t>(a.xr_rows ? a.xr_rows[p] : p) * KB;
  } else {
    if (a.Fs == 0) return;
    src = a.xs_scales + (p - TK) * KB;
  }
  for (int kb = 0; kb < KB; ++kb) a.xrs_t[kb * R + p] = src[kb];
}

int tile_fp8_rows() { return kBM; }

// slabs must divide the weight dimensions, and every K fits the LDS table of
// weight-block scales
bool tile_fp8_shapes_ok(int64_t T, int k, int H, int F, int Fs) {
  // DMA lane offsets are 32-bit: x codes (T rows of H), h codes (T k routed
  // rows of F, T shared rows of Fs), row scales (per 128 channels)
  const int64_t lim = 0xffffffffLL;
  return F % (kBW / 2) == 0 && Fs % (kBW / 2) == 0 && H % kBW == 0 && H <= 128 * kMaxKB &&
         F <= 128 * kMaxKB && Fs <= 128 * kMaxKB && T * H <= lim && T * k * F <= lim && T * Fs <= lim &&
         (T * k + T) * (H / 128) * 4 <= lim && T * k * (F / 128) * 4 <= lim;
}

template <int MODE>
static hipError_t launch_tile_fp8(const FfnArgs& a, int slabs, hipStream_t st) {
  // a multiple of 8: block b serves item (b % 8) * per + b / 8 with
  // per = ceil(items / 8), which needs 8 * per blocks to reach every item
  const int64_t blocks = (static_cast<int64_t>(slabs) * a.tile_bound + kXcd - 1) / kXcd * kXcd;
  // the hint on gate_up only: on down (tile-major, 56 slabs per token tile)
  // it cost more than it gained (K2 fp8 T=2048: layer 3.67 -> 3.75 ms with
  // it on both, gate_up alone 2.23 -> 2.20)
  if (a.w_once && MODE == 0)
    hipLaunchKernelGGL((ffn_tile_fp8<MODE, true>), dim3(static_cast<unsigned>(blocks)), dim3(512), 0, st, a,
                       slabs);
  else
    hipLaunchKernelGGL((ffn_tile_fp8<MODE, false>), dim3(static_cast<unsigned>(blocks)), dim3(512), 0, st, a,
                       slabs);
  return hipGetLastError();
}

// gate_up writes h already quantised (e4m3 codes + per-128 scales); its row
// scales are gathered into K-block-major order first
hipError_t launch_gate_up_tile_fp8(const FfnArgs& a, hipStream_t st) {
  if (a.xrs_t == nullptr || a.offsets == nullptr) return hipErrorInvalidValue;
  const int64_t R = static_cast<int64_t>(a.T) * a.k + a.T;
  hipLaunchKernelGGL(gather_scales_t, dim3(static_cast<unsigned>((R + 255) / 256)), dim3(256), 0, st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_tile_fp8<0>(a, std::max(a.F, a.Fs) / (kBW / 2), st);
}

hipError_t launch_down_tile_fp8(const FfnArgs& a, hipStream_t st) {
  return launch_tile_fp8<1>(a, a.H / kBW, st);
}

}  // namespace moe
