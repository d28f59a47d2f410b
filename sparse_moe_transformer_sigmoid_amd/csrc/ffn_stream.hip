// Grouped expert FFN, weight-streaming schedule (few rows per expert, the
// memory-bound decode regime: "MoE GEMMs remain memory-bound" -- "Behind
// Kimi-K2's Config", section 2.1, Decode bullet).
//
// Expert form ("Kimi K2 . Down projection"): y = W_down (silu(W_gate a) *
// (W_up a)), weights [out][in].
//
// Layout of the work: the output is computed transposed, Y^T = W A^T, so the
// long weight dimension is the MFMA M side and up to 16 grouped rows (tokens)
// form N.  A block is 4 waves that split the K loop of one 16-row (gate_up:
// 16 gate + 16 up rows) or 64-row (down; 32-row for 64-row work items)
// weight slab, K steps of 128 (64 for 64-row items) dealt round-robin to
// the waves.  The weights are loaded in whole 128-byte lines per instruction
// (with the nontemporal hint, except the shared expert's, whose slabs every
// token tile reads) and pass through a per-wave LDS scratch into the
// MFMA layout (16x16x32 bf16; the K order inside a step permuted the same way
// for both operands); each weight byte is read exactly once per tile of 16
// rows.  The four partial sums
// meet in LDS in a fixed order (deterministic).  Grid: x = weight slab, y =
// work-list tile; tiles past the device-side count exit at once.
#include "kernels.h"

namespace moe {

namespace {

constexpr int kWK = 4;  // waves splitting K

// K elements per wave step: 128 for up to 32 rows, 64 for 64-row items, so
// that the double-buffered operands stay in registers
template <int NT>
constexpr int step_k() { return NT <= 2 ? 128 : 64; }

// One wave's operands for one K step.
//  a: NA weight row-tiles of 16 rows as loaded -- each load instruction
//     covers 8 rows x 128 contiguous bytes (lane L: row L / 8 (+ 8 for the
//     second row group), 16-byte chunk L % 8 of a 128-byte line), the
//     nontemporal form: full lines per instruction stream from HBM at
//     ~7.1 TB/s against ~5.9 for 64 bytes of each of 16 rows per instruction
//     (16 GB reads shaped like these slabs, on MI355X).  Load j of a tile is
//     row group j % 2, line j / 2.
//  b: NT token sub-tiles of 16 rows in the MFMA layout: lane (r = L % 16,
//     q = L / 16) holds elements 32 i + 8 q + [0, 8) of row r for MFMA i.
template <int NA, int NT, int KS>
struct Frag {
  uint4 a[NA][KS / 32];
  uint4 b[NT][KS / 32];
};

// NTW: the weight loads carry the nontemporal hint (weights read once: a
// routed tile's; not the shared expert's, whose slabs every token tile reads)
template <int NA, int NT, int KS, bool NTW>
__device__ __forceinline__ void load_frag(Frag<NA, NT, KS>& f, const uint16_t* const (&pa)[NA],
                                          const uint16_t* const (&pb)[NT], int64_t ld8, int koff) {
#pragma unroll
  for (int m = 0; m < NA; ++m)
#pragma unroll
    for (int j = 0; j < KS / 32; ++j) {
      const uint4* w = reinterpret_cast<const uint4*>(pa[m] + (j & 1) * ld8 + koff + (j >> 1) * 64);
      f.a[m][j] = NTW ? load_nt(w) : *w;
    }
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const uint4* s = reinterpret_cast<const uint4*>(pb[n] + koff);
#pragma unroll
    for (int i = 0; i < KS / 32; ++i) f.b[n][i] = s[4 * i];
  }
}

// Per-wave LDS scratch that turns the loaded weight layout into the MFMA
// layout: row rho (0..15) of tile m holds KS / 8 16-byte chunks, chunk c at
// slot c ^ swz(rho).  The swizzle keeps both the 8-row x 8-chunk writes and
// the 16-row reads of one chunk free of bank conflicts (16 lanes of 16 bytes
// per LDS cycle): rows 256 B apart (KS = 128) differ in their slot, rows
// 128 B apart (KS = 64) pair up by parity.
template <int KS>
__device__ __forceinline__ int swz(int rho) {
  return KS == 128 ? (rho ^ ((rho & 1) << 3)) : ((rho >> 1) & 7);
}

template <int NA, int NT, int KS>
__device__ __forceinline__ void mma_frag(const Frag<NA, NT, KS>& f, uint4 (*scr)[16][KS / 8],
                                         f32x4 (&acc)[NA][NT]) {
  const int lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
  // loaded layout -> LDS
#pragma unroll
  for (int m = 0; m < NA; ++m)
#pragma unroll
    for (int j = 0; j < KS / 32; ++j) {
      const int rho = (lane >> 3) + 8 * (j & 1), c = 8 * (j >> 1) + (lane & 7);
      scr[m][rho][c ^ swz<KS>(rho)] = f.a[m][j];
    }
  // the reads below take chunks other lanes of this wave wrote: keep them
  // after the writes (LDS executes one wave's accesses in order)
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
#pragma unroll
  for (int i = 0; i < KS / 32; ++i) {
    uint4 a[NA];
#pragma unroll
    for (int m = 0; m < NA; ++m) a[m] = scr[m][r][(4 * i + q) ^ swz<KS>(r)];
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int m = 0; m < NA; ++m)
        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[m]),
                                                            __builtin_bit_cast(bf16x8, f.b[n][i]),
                                                            acc[m][n], 0, 0, 0);
  }
  // the next step's writes overwrite what these reads take
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// K loop of one wave over steps wave, wave+kWK, ... (double-buffered loads),
// then the kWK partial sums are added in LDS in wave order; wave 0 returns
// the total.  pa[m]: this lane's load position in weight tile m (row L / 8,
// byte 16 (L % 8)); ld8: 8 rows, in elements; pb[n]: token row r + 8 q.
// Both operands use the same K order, so the MFMA sums run over the full step.
// The K loop's LDS (per-wave layout scratch, partial-sum exchange): one
// allocation per shape, shared by both copies of the loop a kernel inlines.
template <int NA, int NT, int KS>
struct StreamLds {
  uint4 scr[kWK][NA][16][KS / 8];
  f32x4 red[kWK - 1][NA][NT][64];
};
template <int NA, int NT, int KS>
__device__ __forceinline__ StreamLds<NA, NT, KS>& stream_lds() {
  __shared__ StreamLds<NA, NT, KS> l;
  return l;
}

template <int NA, int NT, int KS, bool NTW>
__device__ __forceinline__ void stream_k(const uint16_t* const (&pa)[NA],
                                         const uint16_t* const (&pb)[NT], int64_t ld8, int steps,
                                         f32x4 (&acc)[NA][NT]) {
  static_assert(KS == 128 || KS == 64, "K step of one or two 128-byte lines per row");
  auto& scr = stream_lds<NA, NT, KS>().scr;
  auto& red = stream_lds<NA, NT, KS>().red;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int m = 0; m < NA; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  int s = wave;
  Frag<NA, NT, KS> cur, nxt;
  if (s < steps) load_frag<NA, NT, KS, NTW>(cur, pa, pb, ld8, s * KS);
#pragma unroll 1
  while (s < steps) {
    const int sn = s + kWK;
    if (sn < steps) load_frag<NA, NT, KS, NTW>(nxt, pa, pb, ld8, sn * KS);
    mma_frag(cur, scr[wave], acc);
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
#pragma unroll 1
    for (int w = 0; w < kWK - 1; ++w)
#pragma unroll
      for (int m = 0; m < NA; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[m][n] += red[w][m][n][lane];
}

__device__ __forceinline__ void store_bf16x4(uint16_t* dst, float a, float b, float c, float d) {
  uint2 v;
  v.x = static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
  v.y = static_cast<uint32_t>(f32_to_bf16(c)) | (static_cast<uint32_t>(f32_to_bf16(d)) << 16);
  *reinterpret_cast<uint2*>(dst) = v;
}

}  // namespace

// gate_up: block = 16 * NF intermediate features (16 NF gate + 16 NF up
// weight rows) of one work item of up to 16*NT grouped rows.  Sub-tiles past
// the item's rows read its last row again (in bounds, not stored), which
// keeps the K loop free of divergent control flow.
template <int NT, int NF = 1>
__global__ __launch_bounds__(256) void gate_up_stream_bf16(FfnArgs a) {
  constexpr int KS = step_k<NT>();
  const int ti = blockIdx.y;
  if (ti >= *a.tile_count) return;
  const Tile tl = a.tiles[ti];
  const bool sh = tl.group == a.E;
  const int Fg = sh ? a.Fs : a.F;
  const int f0 = blockIdx.x * 16 * NF;
  if (f0 >= Fg) return;
  const int lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
  const int64_t H = a.H, TK = static_cast<int64_t>(a.T) * a.k;
  const uint16_t* wg = static_cast<const uint16_t*>(sh ? a.sh_gate : a.w_gate);
  const uint16_t* wu = static_cast<const uint16_t*>(sh ? a.sh_up : a.w_up);
  const int64_t wofs = sh ? 0 : static_cast<int64_t>(tl.group) * a.F * H;
  const int64_t lrow = f0 + (lane >> 3), lch = 8 * (lane & 7);
  const uint16_t* pa[2 * NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    pa[j] = wg + wofs + (lrow + 16 * j) * H + lch;
    pa[NF + j] = wu + wofs + (lrow + 16 * j) * H + lch;
  }
  const uint16_t* pb[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int64_t p = tl.row0 + min(16 * n + r, tl.rows - 1);
    const uint16_t* b = sh ? static_cast<const uint16_t*>(a.xs) + (p - TK) * H
                           : static_cast<const uint16_t*>(a.xr) + (a.xr_rows ? a.xr_rows[p] : p) * H;
    pb[n] = b + q * 8;
  }
  f32x4 acc[2 * NF][NT];
  // (one branch per block between two copies of the K loop)
  if (sh)
    stream_k<2 * NF, NT, KS, false>(pa, pb, 8 * H, a.H / KS, acc);
  else
    stream_k<2 * NF, NT, KS, true>(pa, pb, 8 * H, a.H / KS, acc);
  if ((threadIdx.x >> 6) != 0) return;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    if (16 * n + r >= tl.rows) continue;
    const int64_t pr = tl.row0 + 16 * n + r;
    uint16_t* dst = sh ? static_cast<uint16_t*>(a.h_sh) + (pr - TK) * a.Fs
                       : static_cast<uint16_t*>(a.h) + pr * a.F;
#pragma unroll
    for (int j = 0; j < NF; ++j)
      store_bf16x4(dst + f0 + 16 * j + 4 * q, silu(acc[j][n][0]) * acc[NF + j][n][0],
                   silu(acc[j][n][1]) * acc[NF + j][n][1], silu(acc[j][n][2]) * acc[NF + j][n][2],
                   silu(acc[j][n][3]) * acc[NF + j][n][3]);
  }
}

// down: block = 16 * NA hidden outputs of one work item
template <int NT, int NA>
__global__ __launch_bounds__(256) void down_stream_bf16(FfnArgs a) {
  constexpr int KS = step_k<NT>();
  const int ti = blockIdx.y;
  if (ti >= *a.tile_count) return;
  const Tile tl = a.tiles[ti];
  const bool sh = tl.group == a.E;
  const int Fg = sh ? a.Fs : a.F;
  const int h0 = blockIdx.x * 16 * NA;
  const int lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
  const int64_t TK = static_cast<int64_t>(a.T) * a.k;
  const uint16_t* wd = static_cast<const uint16_t*>(sh ? a.sh_down : a.w_down);
  const int64_t wofs = sh ? 0 : static_cast<int64_t>(tl.group) * a.H * a.F;
  const uint16_t* pa[NA];
#pragma unroll
  for (int m = 0; m < NA; ++m)
    pa[m] = wd + wofs + static_cast<int64_t>(h0 + 16 * m + (lane >> 3)) * Fg + 8 * (lane & 7);
  const uint16_t* pb[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int64_t p = tl.row0 + min(16 * n + r, tl.rows - 1);
    pb[n] = (sh ? static_cast<const uint16_t*>(a.h_sh) + (p - TK) * a.Fs
                : static_cast<const uint16_t*>(a.h) + p * a.F) + q * 8;
  }
  f32x4 acc[NA][NT];
  if (sh)
    stream_k<NA, NT, KS, false>(pa, pb, 8 * static_cast<int64_t>(Fg), Fg / KS, acc);
  else
    stream_k<NA, NT, KS, true>(pa, pb, 8 * static_cast<int64_t>(Fg), Fg / KS, acc);
  if ((threadIdx.x >> 6) != 0) return;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    if (16 * n + r >= tl.rows) continue;
    const int64_t pr = tl.row0 + 16 * n + r;
    uint16_t* dst = sh ? static_cast<uint16_t*>(a.y_sh) + (pr - TK) * a.H
                       : static_cast<uint16_t*>(a.y) + pr * a.H;
#pragma unroll
    for (int m = 0; m < NA; ++m)
      store_bf16x4(dst + h0 + 16 * m + 4 * q, acc[m][n][0], acc[m][n][1], acc[m][n][2], acc[m][n][3]);
  }
}

// ---------------------------------------------------------------------------
// fp32 path: plain FMA, one thread per output element, the input row staged
// in LDS.  Grid: x = 256 outputs, y = grouped row.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int find_group(const int32_t* offsets, int E, int64_t p) {
  int lo = 0, hi = E;  // offsets[lo] <= p < offsets[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= p) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(256) void gate_up_simple_f32(FfnArgs a) {
  extern __shared__ float row[];
  const int64_t p = blockIdx.y;
  const int64_t TK = static_cast<int64_t>(a.T) * a.k;
  const bool sh = p >= TK;
  const int H = a.H, Fg = sh ? a.Fs : a.F;
  const float* src = sh ? static_cast<const float*>(a.xs) + (p - TK) * H
                        : static_cast<const float*>(a.xr) + (a.xr_rows ? a.xr_rows[p] : p) * H;
  for (int i = threadIdx.x; i < H; i += blockDim.x) row[i] = src[i];
  __syncthreads();
  const int f = blockIdx.x * blockDim.x + threadIdx.x;
  if (f >= Fg) return;
  const int e = sh ? 0 : find_group(a.offsets, a.E, p);
  const float* wg = sh ? static_cast<const float*>(a.sh_gate)
                       : static_cast<const float*>(a.w_gate) + static_cast<int64_t>(e) * a.F * H;
  const float* wu = sh ? static_cast<const float*>(a.sh_up)
                       : static_cast<const float*>(a.w_up) + static_cast<int64_t>(e) * a.F * H;
  wg += static_cast<int64_t>(f) * H;
  wu += static_cast<int64_t>(f) * H;
  float g = 0.f, u = 0.f;
  for (int i = 0; i < H; ++i) {
    g = fmaf(row[i], wg[i], g);
    u = fmaf(row[i], wu[i], u);
  }
  float* dst = sh ? static_cast<float*>(a.h_sh) + (p - TK) * a.Fs : static_cast<float*>(a.h) + p * a.F;
  dst[f] = g / (1.0f + expf(-g)) * u;
}

__global__ __launch_bounds__(256) void down_simple_f32(FfnArgs a) {
  extern __shared__ float row[];
  const int64_t p = blockIdx.y;
  const int64_t TK = static_cast<int64_t>(a.T) * a.k;
  const bool sh = p >= TK;
  const int H = a.H, Fg = sh ? a.Fs : a.F;
  const float* src = sh ? static_cast<const float*>(a.h_sh) + (p - TK) * a.Fs
                        : static_cast<const float*>(a.h) + p * a.F;
  for (int i = threadIdx.x; i < Fg; i += blockDim.x) row[i] = src[i];
  __syncthreads();
  const int o = blockIdx.x * blockDim.x + threadIdx.x;
  if (o >= H) return;
  const int e = sh ? 0 : find_group(a.offsets, a.E, p);
  const float* wd = sh ? static_cast<const float*>(a.sh_down)
                       : static_cast<const float*>(a.w_down) + static_cast<int64_t>(e) * H * a.F;
  wd += static_cast<int64_t>(o) * Fg;
  float y = 0.f;
  for (int i = 0; i < Fg; ++i) y = fmaf(row[i], wd[i], y);
  float* dst = sh ? static_cast<float*>(a.y_sh) + (p - TK) * H : static_cast<float*>(a.y) + p * H;
  dst[o] = y;
}

// sub-tiles of 16 rows per work item: bm = 16 * NT.  32 features per block
// (NF = 2) when that grid still has >= 3000 blocks, else 16.  Measured whole
// layer, NF 2 against 1: K2 T=128 2.85 against 2.87 ms (gate_up), T=256
// 3.20 against 3.25, T=300 5.18 against 5.28 ms, T=384 5.33 against 5.48,
// Moonlight T=256 0.303 against 0.332, T=512 0.390 against 0.435; but K2
// T=1 0.095 against 0.090 ms (gate_up) and T=2 0.166 against 0.158, where
// the grid is a few hundred blocks.
hipError_t launch_gate_up_stream(const FfnArgs& a, hipStream_t st) {
  const dim3 grid(std::max(a.F, a.Fs) / 16, static_cast<unsigned>(a.tile_bound));
  const bool nf2 = static_cast<int64_t>(grid.x / 2) * a.tile_bound >= 3000;
  const dim3 grid2(grid.x / 2, grid.y);
  switch (a.bm) {
    case 16:
      if (nf2) hipLaunchKernelGGL((gate_up_stream_bf16<1, 2>), grid2, dim3(256), 0, st, a);
      else hipLaunchKernelGGL((gate_up_stream_bf16<1, 1>), grid, dim3(256), 0, st, a);
      break;
    case 32:
      if (nf2) hipLaunchKernelGGL((gate_up_stream_bf16<2, 2>), grid2, dim3(256), 0, st, a);
      else hipLaunchKernelGGL((gate_up_stream_bf16<2, 1>), grid, dim3(256), 0, st, a);
      break;
    case 64:
      if (nf2) hipLaunchKernelGGL((gate_up_stream_bf16<4, 2>), grid2, dim3(256), 0, st, a);
      else hipLaunchKernelGGL((gate_up_stream_bf16<4, 1>), grid, dim3(256), 0, st, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// 32 outputs per block
hipError_t launch_down_stream(const FfnArgs& a, hipStream_t st) {
  const unsigned tiles = static_cast<unsigned>(a.tile_bound);
  // 64 output rows per block up to 32-row items (K = F is short: 16 steps
  // of 128, so a larger slab keeps more bytes in flight per wave; measured
  // K2 decode down 1.65 -> 1.60 ms at T=128), 32 rows for 64-row items
  switch (a.bm) {
    case 16: hipLaunchKernelGGL((down_stream_bf16<1, 4>), dim3(a.H / 64, tiles), dim3(256), 0, st, a); break;
    case 32: hipLaunchKernelGGL((down_stream_bf16<2, 4>), dim3(a.H / 64, tiles), dim3(256), 0, st, a); break;
    case 64: hipLaunchKernelGGL((down_stream_bf16<4, 2>), dim3(a.H / 32, tiles), dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_simple_f32(const FfnArgs& a, bool gate_up, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(a.T) * a.k + (a.Fs > 0 ? a.T : 0);
  if (gate_up) {
    dim3 grid((std::max(a.F, a.Fs) + 255) / 256, static_cast<unsigned>(rows));
    hipLaunchKernelGGL(gate_up_simple_f32, grid, dim3(256), a.H * sizeof(float), st, a);
  } else {
    dim3 grid((a.H + 255) / 256, static_cast<unsigned>(rows));
    hipLaunchKernelGGL(down_simple_f32, grid, dim3(256), std::max(a.F, a.Fs) * sizeof(float), st, a);
  }
  return hipGetLastError();
}

}  // namespace moe

namespace moe {

// Rows per work-list tile and the kernel family of one call, from the
// expected rows per expert r = T*k / E (the row capacity for one rank's
// share).  The thresholds are whole-layer measurements on MI355X over
// Kimi-K2 decode (T = 1..2048), the DeepSeek-V3 and Moonlight shapes,
// expert-parallel rank shares and the dense layer (figures beside each rule
// below):
//  * bf16 from r = 7 on (32 for a single expert): the LDS-tiled MFMA
//    kernels (128 rows x 512 weight rows per block); when that grid is small
//    (few, fat experts) the K loop is split over up to 8 (gate_up) or 16
//    (down) blocks;
//  * below, or when the shapes do not fit the tiles: the weight-streaming
//    kernels with work items of 16 rows below 6 rows per expert, 32 below 12
//    and 64 beyond (128-row items run at half occupancy and were slower in
//    every case);
//  * fp8: the fp8 tiled kernel from r = 12 on, else its streaming kernel
//    with the same 16 / 32 / 64-row work items.
FfnPlan ffn_plan(const FfnArgs& a, int weight_dtype, int act_dtype) {
  if (act_dtype == MOE_F32) return {16, FfnPlan::kSimple};
  const int64_t rows = static_cast<int64_t>(a.T) * a.k;
  const double per_expert = static_cast<double>(rows) / a.E;
  const int stream_bm = per_expert < 6.0 ? 16 : (per_expert < 12.0 ? 32 : 64);
  // bf16 tiled from 7 rows per expert (K2 T=384, 8 rows: 5.08 ms tiled
  // against 5.37 streamed; T=448 5.12 against 5.45; DeepSeek-V3 T=256 3.55
  // against 3.68).  fp8 streams its 32-row items up to 12 rows per expert
  // (T=512: 2.85 ms against 3.05 tiled) but not 64-row ones (T=640: 4.00
  // against 3.12).
  if (weight_dtype == MOE_FP8_E4M3) {
    if (per_expert >= 12.0 && tile_fp8_shapes_ok(a.T, a.k, a.H, a.F, a.Fs)) {
      FfnPlan p{tile_fp8_rows(), FfnPlan::kTiled};
      p.w_once = per_expert <= 64.0;   // as for bf16 below (gate_up only: K2 fp8 T=512 layer 3.15 -> 3.10 ms)
      return p;
    }
    return {stream_bm, FfnPlan::kStream};
  }
  // one expert (a dense layer) gives the tiled grid few items: streaming
  // wins below 32 rows (dense T=16: 0.218 ms streamed, 0.238 tiled; T=32
  // ties; T=64 0.294 against 0.252)
  const double tiled_min = a.E == 1 ? 32.0 : 7.0;
  if (per_expert >= tiled_min && tile_shapes_ok(a.T, a.H, a.F, a.Fs)) {
    // few work items (few, fat experts: one expert-parallel rank, the dense
    // layer) split the K loop so that the grid still fills the chip
    FfnPlan p{tile_rows(), FfnPlan::kTiled};
    // expected work items with the rows spread evenly over the experts
    const int64_t per_e = (rows + a.E - 1) / a.E;
    const int64_t items = a.E * ((per_e + 127) / 128) + (a.Fs > 0 ? (a.T + 127) / 128 : 0);
    p.ks_gu = tile_ksplit(items * (std::max(a.F, a.Fs) / 256), a.H, a.H, 8, 256, true);
    p.ks_dn = tile_ksplit(items * (a.H / 512), a.F, a.Fs > 0 ? a.Fs : a.F, 16, 128, false);
    // up to 64 expected rows per expert every expert fits one 128-row tile,
    // so each weight slab is read once: the nontemporal weight DMA (K2 T=512
    // 5.77 -> 5.48 ms, T=1024 6.17 -> 5.97, T=2048 6.51 -> 6.35).  With more
    // rows the slabs are re-read through L2 by an expert's tiles, and the
    // hint cost the T=8192 prefill 8 %.
    // One expert (a dense layer): its row count is exact, T * k.
    p.w_once = per_expert <= 64.0 || (a.E == 1 && rows <= 128 && a.T <= 128);
    return p;
  }
  return {stream_bm, FfnPlan::kStream};
}

hipError_t launch_gate_up(const FfnArgs& a, int act_dtype, int weight_dtype, hipStream_t st) {
  if (act_dtype == MOE_F32) return launch_simple_f32(a, true, st);
  if (weight_dtype == MOE_BF16)
    return a.kind == FfnPlan::kTiled ? launch_gate_up_tile(a, st) : launch_gate_up_stream(a, st);
  if (weight_dtype == MOE_FP8_E4M3)
    return a.kind == FfnPlan::kTiled ? launch_gate_up_tile_fp8(a, st) : launch_gate_up_fp8(a, st);
  return hipErrorNotSupported;
}

hipError_t launch_down(const FfnArgs& a, int act_dtype, int weight_dtype, hipStream_t st) {
  if (act_dtype == MOE_F32) return launch_simple_f32(a, false, st);
  if (weight_dtype == MOE_BF16)
    return a.kind == FfnPlan::kTiled ? launch_down_tile(a, st) : launch_down_stream(a, st);
  if (weight_dtype == MOE_FP8_E4M3)
    return a.kind == FfnPlan::kTiled ? launch_down_tile_fp8(a, st) : launch_down_fp8(a, st);
  return hipErrorNotSupported;
}

}  // namespace moe
