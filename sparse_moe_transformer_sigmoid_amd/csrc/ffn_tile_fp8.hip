// Grouped expert FFN with fp8 e4m3 weights (128 x 128 blocks) and dynamically
// quantised activations, tiled schedule for many rows per expert.
// ("Kimi K2 . Down projection", config.json quantization_config: fmt e4m3,
// weight_block_size [128, 128], activation_scheme dynamic.)
//
// Data movement as in the bf16 tile kernel -- both operands go global -> LDS
// by DMA (global_load_lds_dwordx4), 128-byte unpadded LDS rows with the slot
// swizzle chunk ^ ((row >> 1) & 7), XCD-chunked order of the work items --
// but with three LDS stages, the DMA issued from inline asm and waited for
// with counted s_waitcnt (the next step's DMA issues and the next row-tile's
// LDS reads interleaved with the MFMAs).  A 128-byte row is 128 fp8
// K-elements: exactly one quantisation block per K step, so each step is two
// v_mfma_scale_f32_32x32x64_f8f6f4 (unit e8m0 scales) per 32x32 output tile
// into a fresh partial, added to the fp32 accumulator scaled by weight-block
// scale x row scale:
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
constexpr int kData = (kBW + kBM) * kRowB;    // 48 KB of operands per stage
constexpr int kStage = kData + 8 * 64 * 4;     // + grouped-row scales: 64 slots per wave
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
// 8 waves, two per SIMD: wave (wm, wn) owns LDS weight rows 64*wm + [0, 64)
// (gate_up: 32 gate then 32 up rows of features o0 + 32*wm + [0, 32)) and
// grouped rows 64*wn + [0, 64); while one wave of a SIMD applies the scales
// of its partial products (VALU), the other's MFMAs run.
// WNT: the weight DMA carries the nontemporal hint (each weight slab is
// expected to be read by one tile only)
template <int MODE, bool WNT>
__global__ __launch_bounds__(512) void ffn_tile_fp8(FfnArgs a, int slabs) {
  // three stages as separate objects
  __shared__ __attribute__((aligned(16))) uint8_t st0[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st1[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st2[kStage];
  __shared__ float wscale[4][2][kMaxKB];        // [wm][gate/up or down][K block]
  const int ntile = *a.tile_count;
  const int total = slabs * ntile;
  const int per = (total + kXcd - 1) / kXcd;
  const int j = blockIdx.x / kXcd;
  const int v = (blockIdx.x % kXcd) * per + j;
  if (j >= per || v >= total) return;
  // gate_up: slab-major (the tiles of one weight slab side by side on an
  // XCD); down: tile-major (the slabs of one tile side by side, so its h rows
  // are fetched once per XCD).  Measured on the K2 fp8 layer, T = 512..8192:
  // tile-major down 1-2 % faster, tile-major gate_up 4 % slower.
  int slab, tix;
  if (MODE == 1) {
    tix = v / slabs;
    slab = v - tix * slabs;
  } else {
    slab = v / ntile;
    tix = v - slab * ntile;
  }
  const Tile tl = a.tiles[tix];
  const bool sh = tl.group == a.E;
  const int Fg = sh ? a.Fs : a.F;
  const int64_t TK = static_cast<int64_t>(a.T) * a.k;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;        // 64 weight rows x 64 grouped rows
  const int r32 = lane & 31, kh = lane >> 5;
  const int drow = lane >> 3;
  const int dch[2] = {(lane & 7) ^ ((drow >> 1) & 7), (lane & 7) ^ ((4 + (drow >> 1)) & 7)};

  // ---- weights: this wave's DMA fills LDS rows 32*wave + [0, 32) (4
  // instructions of 8 rows); the compute side reads rows 64*wm + [0, 64) ----
  int K, o0;
  const uint8_t* wdma;               // wave-uniform: the first of the wave's 32 DMA rows
  const float* wsc[2];               // scale rows of the wave's two 32-row tiles
  int64_t KB;
  if (MODE == 0) {
    K = a.H;
    KB = K / 128;
    o0 = slab * (kBW / 2);
    if (o0 >= Fg) return;
    const int64_t wofs = sh ? 0 : static_cast<int64_t>(tl.group) * a.F * a.H;
    const uint8_t* wg = static_cast<const uint8_t*>(sh ? a.sh_gate : a.w_gate) + wofs;
    const uint8_t* wu = static_cast<const uint8_t*>(sh ? a.sh_up : a.w_up) + wofs;
    // LDS rows 64 q + [0, 32) = gate features o0 + 32 q + ., + [32, 64) = up
    const int q = wave >> 1, half = wave & 1;
    wdma = (half ? wu : wg) + static_cast<int64_t>(o0 + 32 * q) * K;
    const int64_t sofs = (sh ? 0 : static_cast<int64_t>(tl.group) * (a.F / 128) * KB) + ((o0 + 32 * wm) / 128) * KB;
    wsc[0] = (sh ? a.sh_s_gate : a.s_gate) + sofs;
    wsc[1] = (sh ? a.sh_s_up : a.s_up) + sofs;
  } else {
    K = Fg;
    KB = K / 128;
    o0 = slab * kBW;
    const int64_t wofs = sh ? 0 : static_cast<int64_t>(tl.group) * a.H * a.F;
    const uint8_t* wd = static_cast<const uint8_t*>(sh ? a.sh_down : a.w_down) + wofs;
    wdma = wd + static_cast<int64_t>(o0 + 32 * wave) * K;
    const int64_t sofs = (sh ? 0 : static_cast<int64_t>(tl.group) * (a.H / 128) * KB) + ((o0 + 64 * wm) / 128) * KB;
    wsc[0] = wsc[1] = (sh ? a.sh_s_down : a.s_down) + sofs;
  }
  const uint64_t wbase = sbase(wdma);
  // lane offset of weight DMA instruction g (rows 8 g + drow of the wave's 32)
  uint32_t woff[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) woff[g] = static_cast<uint32_t>((8 * g + drow) * K + dch[g & 1] * 16);
  // ---- grouped rows: this wave's DMA fills LDS rows kBW + 16*wave + [0, 16);
  // lane offsets from the (wave-uniform) start of the code rows: token * H
  // (gathered routed rows), else the row index * row length (under 2^32
  // bytes: tile_fp8_shapes_ok) ----
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
    xoff[i] = static_cast<uint32_t>(r * ld + dch[i & 1] * 16);
  }
  // ---- weight-block scales of the four 64-row groups, all K blocks, into
  // LDS once (read there at every step) ----
  if (wn == 0)
    for (int i = lane; i < 2 * KB; i += 64) wscale[wm][i / KB][i % KB] = wsc[i / KB][i % KB];
  // ---- row scales: lane l of this wave copies the scale of grouped row
  // 16*wave + l % 16 for each step into the stage's 64 slots of the wave
  // (kData + 256 * wave + 4 * l; the compute side reads l < 16) ----
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
  // the 7 DMA issues of step s into stage st: 4 x 8 weight rows, 2 x 8
  // grouped rows, then the 16 row scales
  auto dma = [&](int g, int s, const uint8_t* st) {
    const uint32_t ko = static_cast<uint32_t>(s) * kRowB;
    const uint32_t l = lds_addr(st);
    if (g < 4) {
      dma16<WNT>(wbase, woff[g] + ko, l + (32 * wave + 8 * g) * kRowB);
    } else if (g < 6) {
      dma16(xbase, xoff[g - 4] + ko, l + (kBW + 16 * wave + 8 * (g - 4)) * kRowB);
    } else {
      dma4(rbase, roff + rstep * static_cast<uint32_t>(s), l + kData + 256 * wave);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][n][i] = 0.f;

  const int steps = static_cast<int>(KB);
  const int sw = (r32 >> 1) & 7;
  const int arow = (64 * wm + r32) * kRowB;
  const int brow = (kBW + 64 * wn + r32) * kRowB;
  // grouped row r = 64 wn + 32 n + r32 has its scale at kData + 256 (r / 16) + 4 (r % 16)
  const int srow = kData + 256 * (4 * wn + (r32 >> 4)) + 4 * (r32 & 15);
  // fragments of one 32-row tile: MFMA i (0, 1) takes chunks kh*4 + 2i, +1
  auto frag = [&](const uint8_t* st, int row, uint4 (&f)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) f[c] = *reinterpret_cast<const uint4*>(st + row + (((kh * 4 + c) ^ sw) * 16));
  };
  // One K step s (one 128-wide quantisation block) on stage rd while the DMA
  // of step sd (= s + 2, clamped) fills stage wr: the four 32x32 tiles t =
  // (m, n), the partial product of tile t+1 computed before tile t's is
  // scaled into the accumulator (MFMA and VALU work overlap).
  auto step = [&](const uint8_t* rd, const uint8_t* wr, int s, int sd) {
    const float ws[2] = {wscale[wm][0][s], wscale[wm][1][s]};
    const float rs[2] = {*reinterpret_cast<const float*>(rd + srow),
                         *reinterpret_cast<const float*>(rd + srow + 512)};
    uint4 af[2][4], bf[2][4];
    frag(rd, arow, af[0]);
    frag(rd, arow + 32 * kRowB, af[1]);
    frag(rd, brow, bf[0]);
    frag(rd, brow + 32 * kRowB, bf[1]);
    f32x16 p[2];
    auto part = [&](int t) {
      const int m = t >> 1, n = t & 1;
      f32x16 z;
#pragma unroll
      for (int i = 0; i < 16; ++i) z[i] = 0.f;
      z = mma_fp8_32(af[m][0], af[m][1], bf[n][0], bf[n][1], z);
      p[t & 1] = mma_fp8_32(af[m][2], af[m][3], bf[n][2], bf[n][3], z);
    };
    auto fold = [&](int t) {
      const int m = t >> 1, n = t & 1;
      // gate_up: m = 0 gate rows, 1 up rows; down: one block
      const float sc = ws[m] * rs[n];
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][n][i] = fmaf(p[t & 1][i], sc, acc[m][n][i]);
    };
    part(0);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < 3) part(t + 1);
      dma(2 * t, sd, wr);
      if (t < 3) dma(2 * t + 1, sd, wr);
      fold(t);
    }
    // this wave's DMA of step s + 1 has landed once at most the 7 issued
    // during this step are outstanding; this wave's LDS reads are done
    // (lgkmcnt); then the barrier.  (__syncthreads would also wait for the
    // DMA of step s + 2.)
    // (fenced against the scheduler: nothing moves across the wait; K2 fp8
    // T=4096 4.38 -> 4.34 ms, T=1024 3.25 -> 3.21)
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(7) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

#pragma unroll
  for (int g = 0; g < 7; ++g) dma(g, 0, st0);
#pragma unroll
  for (int g = 0; g < 7; ++g) dma(g, min(1, steps - 1), st1);
  // (lgkmcnt: the weight-scale table written above is visible after the barrier)
  asm volatile("s_waitcnt vmcnt(7) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // steps in threes (stages 0, 1, 2); a DMA index past the end re-loads the
  // last step's (in-bounds) data into a stage nobody reads again
  const int last = steps - 1;
  int s = 0;
  for (; s + 2 < steps; s += 3) {
    step(st0, st2, s, min(s + 2, last));
    step(st1, st0, s + 1, min(s + 3, last));
    step(st2, st1, s + 2, min(s + 4, last));
  }
  if (s < steps) step(st0, st2, s, min(s + 2, last));
  if (s + 1 < steps) step(st1, st0, s + 1, min(s + 3, last));
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
    // wave's own vmcnt(0) above waits for), and the last step's barrier came
    // after every wave's reads of the table (lgkmcnt(0)).
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
    static_assert(sizeof(wscale) >= 4 * kBM * sizeof(float), "row maxima fit the scale table");
    float* gmax = &wscale[0][0][0];   // [4 wm][128 rows]
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
  // down: y in bf16
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int tr = 64 * wn + 32 * n + r32;
    if (tr >= tl.rows) continue;
    const int64_t p = tl.row0 + tr;
    uint16_t* dst = sh ? static_cast<uint16_t*>(a.y_sh) + (p - TK) * a.H
                       : static_cast<uint16_t*>(a.y) + p * a.H;
    dst += o0 + 64 * wm + 4 * kh;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 v2;
        v2.x = static_cast<uint32_t>(f32_to_bf16(acc[m][n][4 * g + 0])) |
               (static_cast<uint32_t>(f32_to_bf16(acc[m][n][4 * g + 1])) << 16);
        v2.y = static_cast<uint32_t>(f32_to_bf16(acc[m][n][4 * g + 2])) |
               (static_cast<uint32_t>(f32_to_bf16(acc[m][n][4 * g + 3])) << 16);
        *reinterpret_cast<uint2*>(dst + 32 * m + 8 * g) = v2;
      }
  }
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
