// Grouped expert FFN with fp8 e4m3 weights (128 x 128 blocks) and dynamically
// quantised activations, tiled schedule for many rows per expert.
// ("Kimi K2 . Down projection", config.json quantization_config: fmt e4m3,
// weight_block_size [128, 128], activation_scheme dynamic.)
//
// Same data movement as the bf16 tile kernel: both operands go global -> LDS
// by DMA (global_load_lds_dwordx4), 128-byte unpadded LDS rows with the slot
// swizzle chunk ^ ((row >> 1) & 7), two stages held in separate __shared__
// objects, the next step's DMA issues and the next row-tile's LDS reads
// interleaved with the MFMAs, XCD-chunked (slab, tile) order.  A 128-byte
// row is 128 fp8 K-elements: exactly one quantisation block per K step, so
// each step is two v_mfma_scale_f32_32x32x64_f8f6f4 (unit e8m0 scales) per
// 32x32 output tile into a fresh partial, added to the fp32 accumulator
// scaled by weight-block scale x row scale:
//   acc += (sum_k q_w q_a) * s_w[block][kb] * s_a[row][kb].
// The partials need registers next to the accumulators, so the block is 256
// weight rows x 128 grouped rows, 4 waves of 128 x 64.
// gate_up writes the SwiGLU output in fp32 (re-quantised per row and 128
// channels before the down projection); down writes bf16.
#include "kernels.h"

namespace moe {

namespace {

constexpr int kBM = 128;                      // grouped rows per work item
constexpr int kBW = 256;                      // weight rows per slab
constexpr int kRowB = 128;                    // bytes per LDS row = K elements per step
constexpr int kStage = (kBW + kBM) * kRowB;   // 48 KB
constexpr int kXcd = 8;

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(1))) void* glb_ptr;

__device__ __forceinline__ void dma16(const void* g, uint8_t* l) {
  __builtin_amdgcn_global_load_lds((glb_ptr)(g), (lds_ptr)(l), 16, 0, 0);
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
template <int MODE>
__global__ __launch_bounds__(256) void ffn_tile_fp8(FfnArgs a, int slabs) {
  // two stages as separate objects (no alias between a DMA into one and the
  // LDS reads of the other, as in the bf16 tile kernel)
  __shared__ __attribute__((aligned(16))) uint8_t st0[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st1[kStage];
  const int ntile = *a.tile_count;
  const int total = slabs * ntile;
  const int per = (total + kXcd - 1) / kXcd;
  const int j = blockIdx.x / kXcd;
  const int v = (blockIdx.x % kXcd) * per + j;
  if (j >= per || v >= total) return;
  const int slab = v / ntile;
  const Tile tl = a.tiles[v - slab * ntile];
  const bool sh = tl.group == a.E;
  const int Fg = sh ? a.Fs : a.F;
  const int64_t TK = static_cast<int64_t>(a.T) * a.k;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;        // 128 weight rows x 64 grouped rows
  const int r32 = lane & 31, kh = lane >> 5;
  const int drow = lane >> 3;
  const int dch[2] = {(lane & 7) ^ ((drow >> 1) & 7), (lane & 7) ^ ((4 + (drow >> 1)) & 7)};

  // ---- weight rows: LDS rows 128*wm + [0, 128); this wave's DMA covers
  // LDS rows 64*wave + [0, 64) (8 instructions of 8 rows) ----
  int K, o0;
  const uint8_t* wdma;               // first weight row of this wave's DMA share
  const float* wsc[2];               // scale rows of the wave's two 64-row halves (compute side)
  int64_t KB;
  if (MODE == 0) {
    K = a.H;
    KB = K / 128;
    o0 = slab * (kBW / 2);
    if (o0 >= Fg) return;
    const int64_t wofs = sh ? 0 : static_cast<int64_t>(tl.group) * a.F * a.H;
    const uint8_t* wg = static_cast<const uint8_t*>(sh ? a.sh_gate : a.w_gate) + wofs;
    const uint8_t* wu = static_cast<const uint8_t*>(sh ? a.sh_up : a.w_up) + wofs;
    // LDS rows 128 q + [0, 64) = gate features o0 + 64 q + ., + [64, 128) = up
    const int q = wave >> 1, half = wave & 1;
    wdma = (half ? wu : wg) + static_cast<int64_t>(o0 + 64 * q + drow) * K;
    const int64_t sofs = (sh ? 0 : static_cast<int64_t>(tl.group) * (a.F / 128) * KB) +
                         static_cast<int64_t>((o0 + 64 * wm) / 128) * KB;
    wsc[0] = (sh ? a.sh_s_gate : a.s_gate) + sofs;
    wsc[1] = (sh ? a.sh_s_up : a.s_up) + sofs;
  } else {
    K = Fg;
    KB = K / 128;
    o0 = slab * kBW;
    const int64_t wofs = sh ? 0 : static_cast<int64_t>(tl.group) * a.H * a.F;
    const uint8_t* wd = static_cast<const uint8_t*>(sh ? a.sh_down : a.w_down) + wofs;
    wdma = wd + static_cast<int64_t>(o0 + 64 * wave + drow) * K;
    const int64_t sofs = (sh ? 0 : static_cast<int64_t>(tl.group) * (a.H / 128) * KB) +
                         static_cast<int64_t>((o0 + 128 * wm) / 128) * KB;
    wsc[0] = wsc[1] = (sh ? a.sh_s_down : a.s_down) + sofs;
  }
  const int64_t rstride8 = static_cast<int64_t>(8) * K;
  // ---- grouped rows: this wave's DMA covers LDS rows kBW + 32*wave + [0, 32) ----
  const uint8_t* xb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tr = 32 * wave + 8 * i + drow;
    const int64_t p = tl.row0 + min(tr, tl.rows - 1);
    const uint8_t* base;
    if (MODE == 0) {
      if (sh) base = static_cast<const uint8_t*>(a.xs) + (p - TK) * a.H;
      else base = static_cast<const uint8_t*>(a.xr) + (a.xr_rows ? a.xr_rows[p] : p) * a.H;
    } else {
      base = sh ? static_cast<const uint8_t*>(a.hq_sh) + (p - TK) * a.Fs
                : static_cast<const uint8_t*>(a.hq) + p * a.F;
    }
    xb[i] = base + dch[i & 1] * 16;
  }
  // ---- row scales of this lane's two grouped rows (compute side) ----
  const float* rsc[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int tr = 64 * wn + 32 * n + r32;
    const int64_t p = tl.row0 + min(tr, tl.rows - 1);
    if (MODE == 0) {
      if (sh) rsc[n] = a.xs_scales + (p - TK) * KB;
      else rsc[n] = a.xr_scales + (a.xr_rows ? a.xr_rows[p] : p) * KB;
    } else {
      rsc[n] = sh ? a.h_sh_scales + (p - TK) * KB : a.h_scales + p * KB;
    }
  }

  // DMA instruction g (0..11) of step s into stage st: 0-7 weight rows, 8-11 grouped rows
  auto dma = [&](int g, int s, uint8_t* st) {
    const int64_t ko = static_cast<int64_t>(s) * kRowB;
    if (g < 8) dma16(wdma + g * rstride8 + ko + dch[g & 1] * 16, st + (64 * wave + 8 * g) * kRowB);
    else dma16(xb[g - 8] + ko, st + (kBW + 32 * wave + 8 * (g - 8)) * kRowB);
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][n][i] = 0.f;

  const int steps = static_cast<int>(KB);
  const int sw = (r32 >> 1) & 7;
  const int arow = (128 * wm + r32) * kRowB;
  const int brow = (kBW + 64 * wn + r32) * kRowB;
  // fragments of one 32-row tile: MFMA i (0, 1) takes chunks kh*4 + 2i, +1
  auto frag = [&](const uint8_t* st, int row, uint4 (&f)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) f[c] = *reinterpret_cast<const uint4*>(st + row + (((kh * 4 + c) ^ sw) * 16));
  };
  // scales of the step being computed (loaded one step ahead)
  float ws[2], rs[2];
  auto scales = [&](int s, float (&w)[2], float (&r)[2]) {
    w[0] = wsc[0][s];
    w[1] = wsc[1][s];
    r[0] = rsc[0][s];
    r[1] = rsc[1][s];
  };
  // one K step (one 128-wide quantisation block): the weight row-tiles m = 0..3
  // in turn, the next one's fragments read while the current one computes,
  // three of the next step's 12 DMA issues per row-tile
  auto step = [&](const uint8_t* rd, uint8_t* wr, int sn) {
    float nws[2], nrs[2];
    scales(sn, nws, nrs);
    uint4 bf[2][4], af[2][4];
    frag(rd, brow, bf[0]);
    frag(rd, brow + 32 * kRowB, bf[1]);
    frag(rd, arow, af[0]);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int c = m & 1;
      if (m < 3) frag(rd, arow + 32 * (m + 1) * kRowB, af[c ^ 1]);
#pragma unroll
      for (int g = 0; g < 3; ++g) dma(3 * m + g, sn, wr);
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        f32x16 p;
#pragma unroll
        for (int i = 0; i < 16; ++i) p[i] = 0.f;
        p = mma_fp8_32(af[c][0], af[c][1], bf[n][0], bf[n][1], p);
        p = mma_fp8_32(af[c][2], af[c][3], bf[n][2], bf[n][3], p);
        // gate_up: m = 0, 1 are gate rows, 2, 3 up rows; down: one block
        const float sc = (m < 2 ? ws[0] : ws[1]) * rs[n];
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[m][n][i] = fmaf(p[i], sc, acc[m][n][i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    ws[0] = nws[0];
    ws[1] = nws[1];
    rs[0] = nrs[0];
    rs[1] = nrs[1];
  };

  scales(0, ws, rs);
#pragma unroll
  for (int g = 0; g < 12; ++g) dma(g, 0, st0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // steps in pairs (stage 0 then 1); a step past the end re-loads the last
  // step's (in-bounds) data into the stage nobody reads again
  int s = 0;
  for (; s + 1 < steps; s += 2) {
    step(st0, st1, s + 1);
    step(st1, st0, min(s + 2, steps - 1));
  }
  if (s < steps) step(st0, st1, s);

  // ---- epilogue: lane holds weight rows 8*(i/4) + 4*kh + (i%4) of each
  // 32-row sub-tile, for grouped row 64*wn + 32*n + r32 ----
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int tr = 64 * wn + 32 * n + r32;
    if (tr >= tl.rows) continue;
    const int64_t p = tl.row0 + tr;
    if (MODE == 0) {
      float* dst = sh ? static_cast<float*>(a.h_sh) + (p - TK) * a.Fs : static_cast<float*>(a.h) + p * a.F;
      dst += o0 + 64 * wm + 4 * kh;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float4 h;
          h.x = silu(acc[m][n][4 * g + 0]) * acc[m + 2][n][4 * g + 0];
          h.y = silu(acc[m][n][4 * g + 1]) * acc[m + 2][n][4 * g + 1];
          h.z = silu(acc[m][n][4 * g + 2]) * acc[m + 2][n][4 * g + 2];
          h.w = silu(acc[m][n][4 * g + 3]) * acc[m + 2][n][4 * g + 3];
          *reinterpret_cast<float4*>(dst + 32 * m + 8 * g) = h;
        }
    } else {
      uint16_t* dst = sh ? static_cast<uint16_t*>(a.y_sh) + (p - TK) * a.H
                         : static_cast<uint16_t*>(a.y) + p * a.H;
      dst += o0 + 128 * wm + 4 * kh;
#pragma unroll
      for (int m = 0; m < 4; ++m)
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
}

int tile_fp8_rows() { return kBM; }

bool tile_fp8_shapes_ok(int H, int F, int Fs) {
  return F % (kBW / 2) == 0 && Fs % (kBW / 2) == 0 && H % kBW == 0;
}

template <int MODE>
static hipError_t launch_tile_fp8(const FfnArgs& a, int slabs, hipStream_t st) {
  const int64_t blocks = static_cast<int64_t>(slabs) * a.tile_bound;
  hipLaunchKernelGGL((ffn_tile_fp8<MODE>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, a,
                     slabs);
  return hipGetLastError();
}

hipError_t launch_gate_up_tile_fp8(const FfnArgs& a, hipStream_t st) {
  hipError_t e = launch_tile_fp8<0>(a, std::max(a.F, a.Fs) / (kBW / 2), st);
  if (e != hipSuccess) return e;
  e = launch_act_quant_f32(static_cast<const float*>(a.h), static_cast<int64_t>(a.T) * a.k, a.F,
                           static_cast<uint8_t*>(a.hq), a.h_scales, st);
  if (e != hipSuccess || a.Fs == 0) return e;
  return launch_act_quant_f32(static_cast<const float*>(a.h_sh), a.T, a.Fs, static_cast<uint8_t*>(a.hq_sh),
                              a.h_sh_scales, st);
}

hipError_t launch_down_tile_fp8(const FfnArgs& a, hipStream_t st) {
  return launch_tile_fp8<1>(a, a.H / kBW, st);
}

}  // namespace moe
