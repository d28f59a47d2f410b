// Grouped expert FFN, tiled schedule for many rows per expert (the
// compute-bound prefill regime: "prefill is compute-bound" -- "Behind
// Kimi-K2's Config", section 2.1, Prefill bullet).
//
// Expert form ("Kimi K2 . Down projection"): y = W_down (silu(W_gate a) *
// (W_up a)), weights [out][in].
//
// Work item = up to 128 grouped rows of one expert (a tile of the work list)
// x one slab of weight rows.  Still computed transposed (C[weight row][row]),
// with 32x32x16 bf16 MFMA:
//  * the 128 grouped rows (gathered on the fly through the row -> token map)
//    are staged through LDS once per K step of 64 and shared by all waves;
//  * each wave streams its own 64 weight rows straight from global memory
//    into registers (nobody else needs them), double-buffered one step ahead;
//  * gate_up: a wave owns 32 features = 32 gate + 32 up rows, so SiLU * up is
//    applied on matching accumulators in the epilogue; down: a wave owns 64
//    output rows.
// LDS rows are padded to 144 bytes so the 16-byte fragment reads of 8
// consecutive lanes hit distinct banks.  The slab count per expert is a
// multiple of 8, so every tile of one weight slab runs on the same XCD (L2).
#include "kernels.h"

namespace moe {

namespace {

constexpr int kBM = 128;          // grouped rows per work item
constexpr int kBK = 64;           // K elements per step
constexpr int kLds = kBK + 8;     // LDS row stride in bf16 elements (144 B)

__device__ __forceinline__ f32x16 mma32(const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

}  // namespace

// MODE 0: gate_up (K = H, 4 waves = 128 features per block)
// MODE 1: down    (K = F or Fs, 2 waves = 128 output rows per block)
template <int MODE, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void ffn_tile_bf16(FfnArgs a) {
  constexpr int NT = 64 * WAVES;                 // threads
  constexpr int CHUNKS = kBM * kBK * 2 / 16;     // 16-byte chunks of one row tile
  constexpr int CPT = CHUNKS / NT;               // chunks per thread
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][kBM * kLds];

  const int ti = blockIdx.y;
  if (ti >= *a.tile_count) return;
  const Tile tl = a.tiles[ti];
  const bool sh = tl.group == a.E;
  const int Fg = sh ? a.Fs : a.F;
  const int64_t TK = static_cast<int64_t>(a.T) * a.k;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r32 = lane & 31, kh = lane >> 5;

  // ---- weight rows of this wave (A operand, 2 sub-tiles of 32 rows) ----
  int K, o0;
  const uint16_t* pw[2];
  if (MODE == 0) {
    K = a.H;
    o0 = blockIdx.x * (32 * WAVES);
    if (o0 >= Fg) return;
    const int64_t wofs = sh ? 0 : static_cast<int64_t>(tl.group) * a.F * a.H;
    const uint16_t* wg = static_cast<const uint16_t*>(sh ? a.sh_gate : a.w_gate) + wofs;
    const uint16_t* wu = static_cast<const uint16_t*>(sh ? a.sh_up : a.w_up) + wofs;
    const int64_t row = o0 + 32 * wave + r32;
    pw[0] = wg + row * K + kh * 32;
    pw[1] = wu + row * K + kh * 32;
  } else {
    K = Fg;
    o0 = blockIdx.x * (64 * WAVES);
    const int64_t wofs = sh ? 0 : static_cast<int64_t>(tl.group) * a.H * a.F;
    const uint16_t* wd = static_cast<const uint16_t*>(sh ? a.sh_down : a.w_down) + wofs;
    const int64_t row = o0 + 64 * wave + r32;
    pw[0] = wd + row * K + kh * 32;
    pw[1] = wd + (row + 32) * K + kh * 32;
  }

  // ---- grouped-row tile (B operand) staging: source pointers per chunk ----
  const uint16_t* src[CPT];
  int ldo[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int idx = tid + c * NT;
    const int tr = idx >> 3, cc = idx & 7;     // row of the tile, 16-byte column
    const int64_t p = tl.row0 + min(tr, tl.rows - 1);
    const uint16_t* base;
    if (MODE == 0) {
      if (sh) base = static_cast<const uint16_t*>(a.xs) + (p - TK) * a.H;
      else base = static_cast<const uint16_t*>(a.xr) + (a.xr_rows ? a.xr_rows[p] : p) * a.H;
    } else {
      base = sh ? static_cast<const uint16_t*>(a.h_sh) + (p - TK) * a.Fs
                : static_cast<const uint16_t*>(a.h) + p * a.F;
    }
    src[c] = base + cc * 8;
    ldo[c] = tr * kLds + cc * 8;
  }

  f32x16 acc[2][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][n][i] = 0.f;

  const int steps = K / kBK;
  uint4 stage[CPT];
  uint4 wcur[2][4], wnxt[2][4];
#pragma unroll
  for (int c = 0; c < CPT; ++c) stage[c] = *reinterpret_cast<const uint4*>(src[c]);
#pragma unroll
  for (int c = 0; c < CPT; ++c) *reinterpret_cast<uint4*>(&lds[0][ldo[c]]) = stage[c];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) wcur[m][i] = reinterpret_cast<const uint4*>(pw[m])[i];
  __syncthreads();

  // Straight-line loop body: the prefetch of the last step re-reads that step
  // (in bounds) and its LDS write lands in the buffer nobody reads any more.
  for (int s = 0; s < steps; ++s) {
    const int buf = s & 1;
    {
      const int ko = min(s + 1, steps - 1) * kBK;
#pragma unroll
      for (int c = 0; c < CPT; ++c) stage[c] = *reinterpret_cast<const uint4*>(src[c] + ko);
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) wnxt[m][i] = reinterpret_cast<const uint4*>(pw[m] + ko)[i];
    }
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const uint4* bp = reinterpret_cast<const uint4*>(&lds[buf][(32 * n + r32) * kLds + kh * 32]);
      uint4 b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) b[i] = bp[i];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < 2; ++m) acc[m][n] = mma32(wcur[m][i], b[i], acc[m][n]);
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) *reinterpret_cast<uint4*>(&lds[buf ^ 1][ldo[c]]) = stage[c];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) wcur[m][i] = wnxt[m][i];
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 8*(i/4) + 4*kh + (i%4) of each 32-row
  // weight sub-tile, for grouped row 32*n + r32 ----
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int tr = 32 * n + r32;
    if (tr >= tl.rows) continue;
    const int64_t p = tl.row0 + tr;
    if (MODE == 0) {
      uint16_t* dst = sh ? static_cast<uint16_t*>(a.h_sh) + (p - TK) * a.Fs
                         : static_cast<uint16_t*>(a.h) + p * a.F;
      dst += o0 + 32 * wave + 4 * kh;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 v;
        const float h0 = silu(acc[0][n][4 * g + 0]) * acc[1][n][4 * g + 0];
        const float h1 = silu(acc[0][n][4 * g + 1]) * acc[1][n][4 * g + 1];
        const float h2 = silu(acc[0][n][4 * g + 2]) * acc[1][n][4 * g + 2];
        const float h3 = silu(acc[0][n][4 * g + 3]) * acc[1][n][4 * g + 3];
        v.x = static_cast<uint32_t>(f32_to_bf16(h0)) | (static_cast<uint32_t>(f32_to_bf16(h1)) << 16);
        v.y = static_cast<uint32_t>(f32_to_bf16(h2)) | (static_cast<uint32_t>(f32_to_bf16(h3)) << 16);
        *reinterpret_cast<uint2*>(dst + 8 * g) = v;
      }
    } else {
      uint16_t* dst = sh ? static_cast<uint16_t*>(a.y_sh) + (p - TK) * a.H
                         : static_cast<uint16_t*>(a.y) + p * a.H;
      dst += o0 + 64 * wave + 4 * kh;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint2 v;
          v.x = static_cast<uint32_t>(f32_to_bf16(acc[m][n][4 * g + 0])) |
                (static_cast<uint32_t>(f32_to_bf16(acc[m][n][4 * g + 1])) << 16);
          v.y = static_cast<uint32_t>(f32_to_bf16(acc[m][n][4 * g + 2])) |
                (static_cast<uint32_t>(f32_to_bf16(acc[m][n][4 * g + 3])) << 16);
          *reinterpret_cast<uint2*>(dst + 32 * m + 8 * g) = v;
        }
    }
  }
}

int tile_rows() { return kBM; }

hipError_t launch_gate_up_tile(const FfnArgs& a, hipStream_t st) {
  dim3 grid(std::max(a.F, a.Fs) / 128, static_cast<unsigned>(a.tile_bound));
  hipLaunchKernelGGL((ffn_tile_bf16<0, 4>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_down_tile(const FfnArgs& a, hipStream_t st) {
  dim3 grid(a.H / 128, static_cast<unsigned>(a.tile_bound));
  hipLaunchKernelGGL((ffn_tile_bf16<1, 2>), grid, dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
