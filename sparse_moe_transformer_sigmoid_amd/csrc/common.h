// Device helpers shared by the HIP kernels of libmoe (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

// 16-byte load with the nontemporal hint (global_load_dwordx4 ... nt), for
// weight bytes read once, in instructions that each cover whole 128-byte
// lines (with partly covered lines the hint costs re-fetches).
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

constexpr int kWave = 64;

// ---- bf16 <-> fp32 -------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// round to nearest even; NaN stays NaN
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// element access for the two activation dtypes
template <typename T> struct Act;
template <> struct Act<float> {
  static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Act<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// ---- e4m3fn (OCP fp8: 1-4-3, bias 7, max 448, no inf) ---------------------
// Round to nearest, ties to even, saturating at +-448.  |v| below 2^-6 uses
// the subnormal spacing 2^-9; the code of a normal value is
// ((e + 6) << 3) + m with m = rint(|v| * 2^(3-e)) in [8, 16], which carries a
// mantissa overflow into the exponent field by itself.
__device__ __forceinline__ uint8_t f32_to_e4m3(float v) {
  uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = fabsf(v);
  uint32_t code;
  if (!(a < 448.0f)) {
    code = 0x7eu;  // saturate (also NaN -> 448: inputs are finite by construction)
  } else if (a < 0.015625f) {
    code = static_cast<uint32_t>(rintf(a * 512.0f));  // 0..8; 8 is the smallest normal
  } else {
    int e = static_cast<int>((__float_as_uint(a) >> 23) & 0xffu) - 127;  // -6..8
    float m = rintf(a * __uint_as_float(static_cast<uint32_t>(127 + 3 - e) << 23));
    code = static_cast<uint32_t>((e + 6) << 3) + static_cast<uint32_t>(m);
  }
  return static_cast<uint8_t>(code | sign);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Dynamic activation quantisation of one 128-channel group held by a wave as
// two values per lane: s = amax / 448 (1 for an all-zero group), codes
// e4m3(v / s), the division in fp32.  Returns the lane's two codes.
__device__ __forceinline__ uint16_t quant_pair(float v0, float v1, float& s) {
  const float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
  s = amax > 0.f ? amax / 448.0f : 1.0f;
  return static_cast<uint16_t>(f32_to_e4m3(v0 / s)) | (static_cast<uint16_t>(f32_to_e4m3(v1 / s)) << 8);
}

// ---- dynamic fp8 activation quantisation ------------------------------------
// ("Kimi K2 . Down projection", config.json quantization_config: fmt e4m3,
// activation_scheme dynamic.)  Per row and 128-channel group: s = amax / 448
// (1 for an all-zero group), codes e4m3(v / s) with the division in fp32.
// Rows come in up to two sets (groups [0, n0) of the first, then those of the
// second); 16 lanes hold one group (8 values each), a wave GPW groups (4 per
// load), every load issued before the arithmetic.
template <typename In>
struct QuantSeg {
  const In* src;
  int64_t R;
  int C;
  uint8_t* codes;
  float* scales;
};

// 8 consecutive values of a row (16 bytes of bf16, 32 of fp32)
__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(static_cast<uint16_t>(w[i] & 0xffffu));
    v[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(w[i] >> 16));
  }
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// the groups of block `blk` (4 waves of GPW groups) of a 256-thread launch
template <typename In, int GPW>
__device__ __forceinline__ void quant_groups(const QuantSeg<In>& s0, const QuantSeg<In>& s1, int64_t blk) {
  const int lane = threadIdx.x & 63, sub = lane & 15;
  const int64_t n0 = s0.R * (s0.C / 128);
  const int64_t total = n0 + s1.R * (s1.C / 128);
  const int64_t g0 = (blk * 4 + (threadIdx.x >> 6)) * GPW + (lane >> 4);
  // group gi: its set, its index inside the set and its first value
  auto locate = [&](int64_t gi, const QuantSeg<In>*& sg, int64_t& off, int64_t& gs) {
    sg = gi < n0 ? &s0 : &s1;
    gs = gi < n0 ? gi : gi - n0;
    const int groups = sg->C / 128;
    const int64_t row = gs / groups;
    off = row * sg->C + (gs - row * groups) * 128 + 8 * sub;
  };
  float v[GPW / 4][8];
#pragma unroll
  for (int i = 0; i < GPW / 4; ++i) {
    const int64_t gi = g0 + 4 * i;
    if (gi < total) {
      const QuantSeg<In>* sg;
      int64_t off, gs;
      locate(gi, sg, off, gs);
      load8(sg->src + off, v[i]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] = 0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < GPW / 4; ++i) {
    const int64_t gi = g0 + 4 * i;
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[i][e]));
    // the group's 16 lanes (xor offsets below 16 stay inside them)
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    if (gi >= total) continue;   // (after the shuffles, which every lane joins)
    const float sc = m > 0.f ? m / 448.0f : 1.0f;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo |= static_cast<uint32_t>(f32_to_e4m3(v[i][e] / sc)) << (8 * e);
      hi |= static_cast<uint32_t>(f32_to_e4m3(v[i][4 + e] / sc)) << (8 * e);
    }
    const QuantSeg<In>* sg;
    int64_t off, gs;
    locate(gi, sg, off, gs);
    *reinterpret_cast<uint2*>(sg->codes + off) = make_uint2(lo, hi);
    if (sub == 0) sg->scales[gs] = sc;
  }
}

// ---- grouped-GEMM work list ----------------------------------------------
// One entry per (group, tile of up to BM grouped rows).  Groups 0..E-1 are the
// routed experts (rows [offsets[e], offsets[e+1]) of the grouped order), group
// E is the shared expert (rows T*k + t for token t).
struct Tile {
  int32_t group;
  int32_t row0;   // first grouped row of the tile
  int32_t rows;   // 1..BM
  int32_t pad;
};

}  // namespace moe
