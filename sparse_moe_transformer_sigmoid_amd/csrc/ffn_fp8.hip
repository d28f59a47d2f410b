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
//  * a work item covers up to 64 grouped rows (4 sub-tiles of 16) so that an
//    expert with tens of rows streams its weights once per 64 rows; all four
//    sub-tiles are computed (rows past the tile repeat its last row and are
//    not stored), which keeps the loop free of divergent control flow.
// The SwiGLU output is written in fp32; the activation-quant kernel turns it
// into e4m3 codes + per-128 scales for the down projection.
#include "kernels.h"

namespace moe {

namespace {

constexpr int kWK = 4;   // waves splitting K
constexpr int kNT = 4;   // 16-row sub-tiles per work item

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

__device__ __forceinline__ void load32(uint4 (&d)[2], const uint8_t* p) {
  const uint4* s = reinterpret_cast<const uint4*>(p);
  d[0] = s[0];
  d[1] = s[1];
}

// One wave's K loop for NA weight row-tiles of 16 rows and up to kNT token
// sub-tiles; then the kWK partial sums are added in LDS (wave 0 keeps them).
template <int NA>
__device__ __forceinline__ void stream_k_fp8(const uint8_t* const (&pa)[NA],
                                             const float* const (&wsc)[NA],
                                             const uint8_t* const (&pb)[kNT],
                                             const float* const (&bsc)[kNT], int steps,
                                             f32x4 (&acc)[NA][kNT]) {
  __shared__ f32x4 red[kWK - 1][NA][kNT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int m = 0; m < NA; ++m)
#pragma unroll
    for (int n = 0; n < kNT; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int s = wave; s < steps; s += kWK) {
    const int koff = s * 128;
    uint4 a[NA][2], b[kNT][2];
    float ws[NA], bs[kNT];
#pragma unroll
    for (int m = 0; m < NA; ++m) {
      load32(a[m], pa[m] + koff);
      ws[m] = wsc[m][s];
    }
    // sub-tiles past the tile's rows point at its last valid row, so every
    // load is in bounds
#pragma unroll
    for (int n = 0; n < kNT; ++n) {
      load32(b[n], pb[n] + koff);
      bs[n] = bsc[n][s];
    }
#pragma unroll
    for (int n = 0; n < kNT; ++n)
#pragma unroll
      for (int m = 0; m < NA; ++m) {
          const f32x4 c = mma_fp8(a[m], b[n]);
          const float sc = ws[m] * bs[n];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[m][n][i] = fmaf(c[i], sc, acc[m][n][i]);
      }
  }
  if (wave > 0)
#pragma unroll
    for (int m = 0; m < NA; ++m)
#pragma unroll
      for (int n = 0; n < kNT; ++n) red[wave - 1][m][n][lane] = acc[m][n];
  __syncthreads();
  if (wave == 0)
#pragma unroll
    for (int w = 0; w < kWK - 1; ++w)
#pragma unroll
      for (int m = 0; m < NA; ++m)
#pragma unroll
        for (int n = 0; n < kNT; ++n) acc[m][n] += red[w][m][n][lane];
}

}  // namespace

// gate_up: block = 16 intermediate features (16 gate + 16 up weight rows) of
// one work item (<= 64 grouped rows); h written in fp32.
__global__ __launch_bounds__(256) void gate_up_stream_fp8(FfnArgs a) {
  const int ti = blockIdx.y;
  if (ti >= *a.tile_count) return;
  const Tile tl = a.tiles[ti];
  const bool sh = tl.group == a.E;
  const int Fg = sh ? a.Fs : a.F;
  const int f0 = blockIdx.x * 16;
  if (f0 >= Fg) return;
  const int lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
  const int64_t H = a.H, KB = a.H / 128, TK = static_cast<int64_t>(a.T) * a.k;
  const uint8_t* wg = static_cast<const uint8_t*>(sh ? a.sh_gate : a.w_gate);
  const uint8_t* wu = static_cast<const uint8_t*>(sh ? a.sh_up : a.w_up);
  const float* sg = sh ? a.sh_s_gate : a.s_gate;
  const float* su = sh ? a.sh_s_up : a.s_up;
  const int64_t wofs = sh ? 0 : static_cast<int64_t>(tl.group) * a.F * H;
  const int64_t sofs = (sh ? 0 : static_cast<int64_t>(tl.group) * (a.F / 128) * KB) + (f0 / 128) * KB;
  const uint8_t* pa[2] = {wg + wofs + (f0 + r) * H + q * 32, wu + wofs + (f0 + r) * H + q * 32};
  const float* wsc[2] = {sg + sofs, su + sofs};
  const uint8_t* pb[kNT];
  const float* bsc[kNT];
#pragma unroll
  for (int n = 0; n < kNT; ++n) {
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
    pb[n] = base + row * H + q * 32;
    bsc[n] = sbase + row * KB;
  }
  f32x4 acc[2][kNT];
  stream_k_fp8<2>(pa, wsc, pb, bsc, static_cast<int>(KB), acc);
  if ((threadIdx.x >> 6) != 0) return;
#pragma unroll
  for (int n = 0; n < kNT; ++n) {
    if (n * 16 + r >= tl.rows) continue;
    const int64_t pr = tl.row0 + n * 16 + r;
    float* dst = sh ? static_cast<float*>(a.h_sh) + (pr - TK) * a.Fs : static_cast<float*>(a.h) + pr * a.F;
    float4 v;
    v.x = silu(acc[0][n][0]) * acc[1][n][0];
    v.y = silu(acc[0][n][1]) * acc[1][n][1];
    v.z = silu(acc[0][n][2]) * acc[1][n][2];
    v.w = silu(acc[0][n][3]) * acc[1][n][3];
    *reinterpret_cast<float4*>(dst + f0 + 4 * q) = v;
  }
}

// down: block = 32 hidden outputs of one work item; input = quantised h
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
  const uint8_t* pa[2] = {wd + wofs + static_cast<int64_t>(h0 + r) * Fg + q * 32,
                          wd + wofs + static_cast<int64_t>(h0 + 16 + r) * Fg + q * 32};
  const float* wsc[2] = {sd + sofs, sd + sofs};
  const uint8_t* pb[kNT];
  const float* bsc[kNT];
#pragma unroll
  for (int n = 0; n < kNT; ++n) {
    const int64_t p = tl.row0 + min(n * 16 + r, tl.rows - 1);
    if (sh) {
      pb[n] = static_cast<const uint8_t*>(a.hq_sh) + (p - TK) * a.Fs + q * 32;
      bsc[n] = a.h_sh_scales + (p - TK) * KB;
    } else {
      pb[n] = static_cast<const uint8_t*>(a.hq) + p * a.F + q * 32;
      bsc[n] = a.h_scales + p * KB;
    }
  }
  f32x4 acc[2][kNT];
  stream_k_fp8<2>(pa, wsc, pb, bsc, static_cast<int>(KB), acc);
  if ((threadIdx.x >> 6) != 0) return;
#pragma unroll
  for (int n = 0; n < kNT; ++n) {
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

int fp8_tile_rows() { return 16 * kNT; }

hipError_t launch_gate_up_fp8(const FfnArgs& a, hipStream_t st) {
  dim3 grid(std::max(a.F, a.Fs) / 16, static_cast<unsigned>(a.tile_bound));
  hipLaunchKernelGGL(gate_up_stream_fp8, grid, dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // SwiGLU output -> e4m3 codes + per-128 scales for the down projection
  e = launch_act_quant_f32(static_cast<const float*>(a.h), static_cast<int64_t>(a.T) * a.k, a.F,
                           static_cast<uint8_t*>(a.hq), a.h_scales, st);
  if (e != hipSuccess || a.Fs == 0) return e;
  return launch_act_quant_f32(static_cast<const float*>(a.h_sh), a.T, a.Fs,
                              static_cast<uint8_t*>(a.hq_sh), a.h_sh_scales, st);
}

hipError_t launch_down_fp8(const FfnArgs& a, hipStream_t st) {
  dim3 grid(a.H / 32, static_cast<unsigned>(a.tile_bound));
  hipLaunchKernelGGL(down_stream_fp8, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
