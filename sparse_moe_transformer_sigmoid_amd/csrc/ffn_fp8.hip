// Grouped expert FFN with fp8 e4m3 weights in 128x128 blocks and dynamically
// quantised activations ("Kimi K2 . Down projection", config.json
// quantization_config: fmt e4m3, weight_block_size [128, 128],
// activation_scheme dynamic).
//
// Same transposed weight-streaming layout as the bf16 kernels (weights on the
// MFMA M side), with two differences:
//  * one v_mfma_scale_f32_16x16x128_f8f6f4 (unit e8m0 scales) covers exactly
//    one 128-wide K block, so each partial product is rescaled once by the
//    weight block scale times the token's activation scale before it joins
//    the fp32 accumulator: acc += (sum_k qw qa) * s_w * s_a;
//  * a work item covers up to 16 * NT grouped rows (NT = 1, 2, 4 sub-tiles of
//    16, chosen from the rows per expert) so that an expert with tens of rows
//    streams its weights once per item; all NT sub-tiles are computed (rows
//    past the tile repeat its last row and are not stored), which keeps the
//    loop free of divergent control flow.
// Each wave's loads for its next K step (operands and scales) are issued
// before the current step's MFMAs, so a load's latency overlaps a step of
// compute instead of stalling every step.  As in the bf16 stream, weights
// are loaded in whole 128-byte lines with the nontemporal hint (gate_up: not
// the shared expert's) and pass through a per-wave LDS scratch into the
// MFMA layout.
// The SwiGLU output is written in fp32; one activation-quant launch turns the
// routed and shared rows into e4m3 codes + per-128 scales for the down
// projection.
#include "kernels.h"

namespace moe {

namespace {

constexpr int kWK = 4;   // waves splitting K

__device__ __forceinline__ f32x4 mma_fp8(const uint4 (&a)[2], const uint4 (&b)[2]) {
  i32x8 av, bv;
  av[0] = a[0].x; av[1] = a[0].y; av[2] = a[0].z; av[3] = a[0].w;
  av[4] = a[1].x; av[5] = a[1].y; av[6] = a[1].z; av[7] = a[1].w;
  bv[0] = b[0].x; bv[1] = b[0].y; bv[2] = b[0].z; bv[3] = b[0].w;
  bv[4] = b[1].x; bv[5] = b[1].y; bv[6] = b[1].z; bv[7] = b[1].w;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  // formats: 0 = fp8 e4m3 for A and B; scales 127 = 2^0 (no e8m0 scaling)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, zero, 0, 0, 0, 127, 0, 127);
}

// One wave's operands of one K step (one 128-wide quantisation block) and
// their scales.
//  a: NA weight row-tiles of 16 rows x 128 bytes as loaded: load g covers
//     rows 8 g + [0, 8) in whole 128-byte lines (lane L: row L / 8, 16-byte
//     chunk L % 8), with the nontemporal hint;
//  b: NT token sub-tiles in the MFMA layout: lane (r = L % 16, q = L / 16)
//     holds chunks q and q + 4 of row r (the MFMA's K order, permuted the same
//     way for the weights when they are read back from LDS).
template <int NA, int NT>
struct Frag8 {
  uint4 a[NA][2];
  uint4 b[NT][2];
  float ws[NA];
  float bs[NT];
};

// NTW: the weight loads carry the nontemporal hint (a routed tile's; not
// the shared expert's, whose slabs every token tile reads)
template <int NA, int NT, bool NTW>
__device__ __forceinline__ void load_frag8(Frag8<NA, NT>& f, const uint8_t* const (&pa)[NA],
                                           const float* const (&wsc)[NA],
                                           const uint8_t* const (&pb)[NT],
                                           const float* const (&bsc)[NT], int64_t ld8, int s) {
  const int koff = s * 128;
#pragma unroll
  for (int m = 0; m < NA; ++m) {
    const uint4* w0 = reinterpret_cast<const uint4*>(pa[m] + koff);
    const uint4* w1 = reinterpret_cast<const uint4*>(pa[m] + ld8 + koff);
    f.a[m][0] = NTW ? load_nt(w0) : *w0;
    f.a[m][1] = NTW ? load_nt(w1) : *w1;
    f.ws[m] = wsc[m][s];
  }
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const uint4* p = reinterpret_cast<const uint4*>(pb[n] + koff);
    f.b[n][0] = p[0];
    f.b[n][1] = p[4];
    f.bs[n] = bsc[n][s];
  }
}

// Per-wave LDS scratch from the loaded weight layout to the MFMA layout: row
// rho (0..15) of tile m holds its 8 chunks, chunk c at slot c ^ ((rho >> 1)
// & 7), which keeps the 8-row writes and the 16-row reads of one chunk free
// of bank conflicts (rows 128 B apart pair up by parity).
template <int NA, int NT>
__device__ __forceinline__ void mma_frag8(const Frag8<NA, NT>& f, uint4 (*scr)[16][8], f32x4 (&acc)[NA][NT]) {
  const int lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
#pragma unroll
  for (int m = 0; m < NA; ++m)
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int rho = (lane >> 3) + 8 * g;
      scr[m][rho][(lane & 7) ^ ((rho >> 1) & 7)] = f.a[m][g];
    }
  // the reads take chunks other lanes of this wave wrote (LDS executes one
  // wave's accesses in order)
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
  uint4 w[NA][2];
#pragma unroll
  for (int m = 0; m < NA; ++m) {
    w[m][0] = scr[m][r][q ^ ((r >> 1) & 7)];
    w[m][1] = scr[m][r][(q + 4) ^ ((r >> 1) & 7)];
  }
  // the next step's writes overwrite what these reads take
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int m = 0; m < NA; ++m) {
      const f32x4 c = mma_fp8(w[m], f.b[n]);
      const float sc = f.ws[m] * f.bs[n];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[m][n][i] = fmaf(c[i], sc, acc[m][n][i]);
    }
}

// One wave's K loop for NA weight row-tiles of 16 rows and NT token
// sub-tiles (steps wave, wave + kWK, ..., the next step's loads in flight
// during the current step's MFMAs); then the kWK partial sums are added in
// LDS in wave order (wave 0 keeps them).  pa[m]: this lane's load position
// in tile m (row L / 8, byte 16 (L % 8)); ld8: 8 rows in bytes; pb[n]: token
// row r + 16 q.
// The K loop's LDS (per-wave layout scratch, partial-sum exchange): one
// allocation per shape, shared by both copies of the loop a kernel inlines.
template <int NA, int NT>
struct StreamLds8 {
  uint4 scr[kWK][NA][16][8];
  f32x4 red[kWK - 1][NA][NT][64];
};
template <int NA, int NT>
__device__ __forceinline__ StreamLds8<NA, NT>& stream_lds8() {
  __shared__ StreamLds8<NA, NT> l;
  return l;
}

template <int NA, int NT, bool NTW>
__device__ __forceinline__ void stream_k_fp8(const uint8_t* const (&pa)[NA],
                                             const float* const (&wsc)[NA],
                                             const uint8_t* const (&pb)[NT],
                                             const float* const (&bsc)[NT], int64_t ld8, int steps,
                                             f32x4 (&acc)[NA][NT]) {
  auto& scr = stream_lds8<NA, NT>().scr;
  auto& red = stream_lds8<NA, NT>().red;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int m = 0; m < NA; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  int s = wave;
  Frag8<NA, NT> cur, nxt;
  if (s < steps) load_frag8<NA, NT, NTW>(cur, pa, wsc, pb, bsc, ld8, s);
#pragma unroll 1
  while (s < steps) {
    const int sn = s + kWK;
    if (sn < steps) load_frag8<NA, NT, NTW>(nxt, pa, wsc, pb, bsc, ld8, sn);
    mma_frag8(cur, scr[wave], acc);
    cur = nxt;
    s = sn;
  }
  if (wave > 0)
#pragma unroll
    for (int m = 0; m < NA; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n) red[wave - 1][m][n][lane] = acc[m][n];
  __syncthreads();
  if (wave == 0)
#pragma unroll
    for (int w = 0; w < kWK - 1; ++w)
#pragma unroll
      for (int m = 0; m < NA; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[m][n] += red[w][m][n][lane];
}

}  // namespace

// gate_up: block = 16 * NF intermediate features (16 NF gate + 16 NF up
// weight rows) of one work item (<= 16 * NT grouped rows); h written in fp32.
template <int NT, int NF = 1>
__global__ __launch_bounds__(256) void gate_up_stream_fp8(FfnArgs a) {
  const int ti = blockIdx.y;
  if (ti >= *a.tile_count) return;
  const Tile tl = a.tiles[ti];
  const bool sh = tl.group == a.E;
  const int Fg = sh ? a.Fs : a.F;
  const int f0 = blockIdx.x * 16 * NF;
  if (f0 >= Fg) return;
  const int lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
  const int64_t H = a.H, KB = a.H / 128, TK = static_cast<int64_t>(a.T) * a.k;
  const uint8_t* wg = static_cast<const uint8_t*>(sh ? a.sh_gate : a.w_gate);
  const uint8_t* wu = static_cast<const uint8_t*>(sh ? a.sh_up : a.w_up);
  const float* sg = sh ? a.sh_s_gate : a.s_gate;
  const float* su = sh ? a.sh_s_up : a.s_up;
  const int64_t wofs = sh ? 0 : static_cast<int64_t>(tl.group) * a.F * H;
  const int64_t lrow = f0 + (lane >> 3), lch = 16 * (lane & 7);     // load position
  const uint8_t* pa[2 * NF];
  const float* wsc[2 * NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    // the weight-block scale row of features f0 + 16 j (128-row blocks)
    const int64_t sofs = (sh ? 0 : static_cast<int64_t>(tl.group) * (a.F / 128) * KB) + ((f0 + 16 * j) / 128) * KB;
    pa[j] = wg + wofs + (lrow + 16 * j) * H + lch;
    pa[NF + j] = wu + wofs + (lrow + 16 * j) * H + lch;
    wsc[j] = sg + sofs;
    wsc[NF + j] = su + sofs;
  }
  const uint8_t* pb[NT];
  const float* bsc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int64_t p = tl.row0 + min(n * 16 + r, tl.rows - 1);
    int64_t row;
    const uint8_t* base;
    const float* sbase;
    if (sh) {
      row = p - TK;
      base = static_cast<const uint8_t*>(a.xs);
      sbase = a.xs_scales;
    } else {
      row = a.xr_rows ? a.xr_rows[p] : p;
      base = static_cast<const uint8_t*>(a.xr);
      sbase = a.xr_scales;
    }
    pb[n] = base + row * H + q * 16;
    bsc[n] = sbase + row * KB;
  }
  f32x4 acc[2 * NF][NT];
  // (one branch per block between two copies of the K loop)
  if (sh)
    stream_k_fp8<2 * NF, NT, false>(pa, wsc, pb, bsc, 8 * H, static_cast<int>(KB), acc);
  else
    stream_k_fp8<2 * NF, NT, true>(pa, wsc, pb, bsc, 8 * H, static_cast<int>(KB), acc);
  if ((threadIdx.x >> 6) != 0) return;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    if (n * 16 + r >= tl.rows) continue;
    const int64_t pr = tl.row0 + n * 16 + r;
    float* dst = sh ? static_cast<float*>(a.h_sh) + (pr - TK) * a.Fs : static_cast<float*>(a.h) + pr * a.F;
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      float4 v;
      v.x = silu(acc[j][n][0]) * acc[NF + j][n][0];
      v.y = silu(acc[j][n][1]) * acc[NF + j][n][1];
      v.z = silu(acc[j][n][2]) * acc[NF + j][n][2];
      v.w = silu(acc[j][n][3]) * acc[NF + j][n][3];
      *reinterpret_cast<float4*>(dst + f0 + 16 * j + 4 * q) = v;
    }
  }
}

// down: block = 32 hidden outputs of one work item; input = quantised h
template <int NT>
__global__ __launch_bounds__(256) void down_stream_fp8(FfnArgs a) {
  const int ti = blockIdx.y;
  if (ti >= *a.tile_count) return;
  const Tile tl = a.tiles[ti];
  const bool sh = tl.group == a.E;
  const int Fg = sh ? a.Fs : a.F;
  const int h0 = blockIdx.x * 32;
  const int lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
  const int64_t KB = Fg / 128, TK = static_cast<int64_t>(a.T) * a.k;
  const uint8_t* wd = static_cast<const uint8_t*>(sh ? a.sh_down : a.w_down);
  const float* sd = sh ? a.sh_s_down : a.s_down;
  const int64_t wofs = sh ? 0 : static_cast<int64_t>(tl.group) * a.H * a.F;
  const int64_t sofs = (sh ? 0 : static_cast<int64_t>(tl.group) * (a.H / 128) * KB) + (h0 / 128) * KB;
  const int lch = 16 * (lane & 7);                                   // load position
  const uint8_t* pa[2] = {wd + wofs + static_cast<int64_t>(h0 + (lane >> 3)) * Fg + lch,
                          wd + wofs + static_cast<int64_t>(h0 + 16 + (lane >> 3)) * Fg + lch};
  const float* wsc[2] = {sd + sofs, sd + sofs};
  const uint8_t* pb[NT];
  const float* bsc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int64_t p = tl.row0 + min(n * 16 + r, tl.rows - 1);
    if (sh) {
      pb[n] = static_cast<const uint8_t*>(a.hq_sh) + (p - TK) * a.Fs + q * 16;
      bsc[n] = a.h_sh_scales + (p - TK) * KB;
    } else {
      pb[n] = static_cast<const uint8_t*>(a.hq) + p * a.F + q * 16;
      bsc[n] = a.h_scales + p * KB;
    }
  }
  f32x4 acc[2][NT];
  // (one copy of the K loop, every weight load with the hint: a second copy
  // for the shared tiles cost this kernel registers and occupancy, K2 fp8
  // T=128 down 0.687 -> 0.702 ms)
  stream_k_fp8<2, NT, true>(pa, wsc, pb, bsc, 8 * static_cast<int64_t>(Fg), static_cast<int>(KB), acc);
  if ((threadIdx.x >> 6) != 0) return;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    if (n * 16 + r >= tl.rows) continue;
    const int64_t pr = tl.row0 + n * 16 + r;
    uint16_t* dst = sh ? static_cast<uint16_t*>(a.y_sh) + (pr - TK) * a.H : static_cast<uint16_t*>(a.y) + pr * a.H;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      uint2 v;
      v.x = static_cast<uint32_t>(f32_to_bf16(acc[m][n][0])) | (static_cast<uint32_t>(f32_to_bf16(acc[m][n][1])) << 16);
      v.y = static_cast<uint32_t>(f32_to_bf16(acc[m][n][2])) | (static_cast<uint32_t>(f32_to_bf16(acc[m][n][3])) << 16);
      *reinterpret_cast<uint2*>(dst + h0 + 16 * m + 4 * q) = v;
    }
  }
}

hipError_t launch_gate_up_fp8(const FfnArgs& a, hipStream_t st) {
  // 32 features per block when that grid keeps >= 3000 blocks, as for bf16
  const dim3 grid(std::max(a.F, a.Fs) / 16, static_cast<unsigned>(a.tile_bound));
  const bool nf2 = static_cast<int64_t>(grid.x / 2) * a.tile_bound >= 3000;
  const dim3 grid2(grid.x / 2, grid.y);
  switch (a.bm) {
    case 16:
      if (nf2) hipLaunchKernelGGL((gate_up_stream_fp8<1, 2>), grid2, dim3(256), 0, st, a);
      else hipLaunchKernelGGL((gate_up_stream_fp8<1, 1>), grid, dim3(256), 0, st, a);
      break;
    case 32:
      if (nf2) hipLaunchKernelGGL((gate_up_stream_fp8<2, 2>), grid2, dim3(256), 0, st, a);
      else hipLaunchKernelGGL((gate_up_stream_fp8<2, 1>), grid, dim3(256), 0, st, a);
      break;
    case 64:
      if (nf2) hipLaunchKernelGGL((gate_up_stream_fp8<4, 2>), grid2, dim3(256), 0, st, a);
      else hipLaunchKernelGGL((gate_up_stream_fp8<4, 1>), grid, dim3(256), 0, st, a);
      break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // SwiGLU output (routed and shared rows, one launch) -> e4m3 codes +
  // per-128 scales for the down projection
  return launch_act_quant_f32(static_cast<const float*>(a.h), static_cast<int64_t>(a.T) * a.k, a.F,
                              static_cast<uint8_t*>(a.hq), a.h_scales, static_cast<const float*>(a.h_sh),
                              a.Fs > 0 ? a.T : 0, a.Fs > 0 ? a.Fs : 128, static_cast<uint8_t*>(a.hq_sh),
                              a.h_sh_scales, st);
}

hipError_t launch_down_fp8(const FfnArgs& a, hipStream_t st) {
  dim3 grid(a.H / 32, static_cast<unsigned>(a.tile_bound));
  switch (a.bm) {
    case 16: hipLaunchKernelGGL(down_stream_fp8<1>, grid, dim3(256), 0, st, a); break;
    case 32: hipLaunchKernelGGL(down_stream_fp8<2>, grid, dim3(256), 0, st, a); break;
    case 64: hipLaunchKernelGGL(down_stream_fp8<4>, grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
