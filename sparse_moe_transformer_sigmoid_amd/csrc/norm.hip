// Pre-MoE RMSNorm ("Kimi K2 Base" architecture table: RMSNorm; raw config
// fields: rms_norm_eps 1e-06): u = x / sqrt(mean(x^2) + eps) * g, computed in
// fp64 and rounded once (to nearest even) to the activation dtype, the input
// the router and the experts then see.  With fp8 expert weights the same pass
// also quantises u per 128 channels for the expert GEMMs (the arithmetic of
// the standalone activation-quant kernel, on the rounded u).
//
// One block of 4 waves per row; a wave owns 128-channel groups wave, wave+4,
// ..., two values per lane.  The sum of squares of the (exactly squared)
// inputs is accumulated in fp64 per lane, then added across lanes and waves
// in a fixed order, so a row's result does not depend on the launch.
#include "kernels.h"

namespace moe {

namespace {

__device__ __forceinline__ double wave_sum_f64(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// nearest bf16 (ties to even) of an fp64 value: the 45 low mantissa bits are
// rounded away directly (no intermediate fp32 rounding); magnitudes below
// 2^-126 become a signed zero
__device__ __forceinline__ uint16_t f64_to_bf16(double v) {
  const uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
  const uint16_t sign = static_cast<uint16_t>((b >> 48) & 0x8000u);
  const uint64_t mag = b & 0x7fffffffffffffffull;
  if (mag < (static_cast<uint64_t>(1023 - 126) << 52)) return sign;
  const uint64_t low = mag & ((1ull << 45) - 1);
  uint64_t kept = mag >> 45;  // 11-bit exponent | 7-bit mantissa
  if (low > (1ull << 44) || (low == (1ull << 44) && (kept & 1u))) ++kept;
  const uint64_t e = (kept >> 7) - 1023 + 127;
  return static_cast<uint16_t>(sign | static_cast<uint16_t>((e << 7) | (kept & 0x7fu)));
}

__device__ __forceinline__ void load2(const uint16_t* p, float& a, float& b) {
  const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
  a = bf16_to_f32(static_cast<uint16_t>(v & 0xffffu));
  b = bf16_to_f32(static_cast<uint16_t>(v >> 16));
}
__device__ __forceinline__ void load2(const float* p, float& a, float& b) {
  const float2 v = *reinterpret_cast<const float2*>(p);
  a = v.x;
  b = v.y;
}
// round two fp64 values to the storage type, store them, return them as fp32
__device__ __forceinline__ void store2(uint16_t* p, double a, double b, float& ra, float& rb) {
  const uint16_t ha = f64_to_bf16(a), hb = f64_to_bf16(b);
  *reinterpret_cast<uint32_t*>(p) = static_cast<uint32_t>(ha) | (static_cast<uint32_t>(hb) << 16);
  ra = bf16_to_f32(ha);
  rb = bf16_to_f32(hb);
}
__device__ __forceinline__ void store2(float* p, double a, double b, float& ra, float& rb) {
  ra = static_cast<float>(a);
  rb = static_cast<float>(b);
  *reinterpret_cast<float2*>(p) = make_float2(ra, rb);
}

}  // namespace

template <typename T, bool QUANT>
__global__ __launch_bounds__(256) void rmsnorm_rows(const T* __restrict__ x, const T* __restrict__ g,
                                                    double eps, int H, T* __restrict__ u,
                                                    uint8_t* __restrict__ codes, float* __restrict__ scales) {
  __shared__ double part[4];
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int groups = H / 128;
  const T* xr = x + row * H;
  double ss = 0.0;
  for (int gi = wave; gi < groups; gi += 4) {
    float a, b;
    load2(xr + gi * 128 + 2 * lane, a, b);
    ss += static_cast<double>(a) * a;
    ss += static_cast<double>(b) * b;
  }
  ss = wave_sum_f64(ss);
  if (lane == 0) part[wave] = ss;
  __syncthreads();
  const double total = ((part[0] + part[1]) + part[2]) + part[3];
  const double rms = sqrt(total / H + eps);
  for (int gi = wave; gi < groups; gi += 4) {
    const int c = gi * 128 + 2 * lane;
    float a, b, ga, gb, ra, rb;
    load2(xr + c, a, b);
    load2(g + c, ga, gb);
    store2(u + row * H + c, a / rms * ga, b / rms * gb, ra, rb);
    if (QUANT) {
      float s;
      *reinterpret_cast<uint16_t*>(codes + row * H + c) = quant_pair(ra, rb, s);
      if (lane == 0) scales[row * groups + gi] = s;
    }
  }
}

hipError_t launch_rmsnorm(const void* x, const void* g, double eps, int64_t T, int H, bool bf16, void* u,
                          uint8_t* codes, float* scales, hipStream_t st) {
  if (bf16) {
    const uint16_t* xs = static_cast<const uint16_t*>(x);
    const uint16_t* gs = static_cast<const uint16_t*>(g);
    uint16_t* us = static_cast<uint16_t*>(u);
    if (codes) hipLaunchKernelGGL((rmsnorm_rows<uint16_t, true>), dim3(T), dim3(256), 0, st, xs, gs, eps, H, us, codes, scales);
    else hipLaunchKernelGGL((rmsnorm_rows<uint16_t, false>), dim3(T), dim3(256), 0, st, xs, gs, eps, H, us, codes, scales);
  } else {
    hipLaunchKernelGGL((rmsnorm_rows<float, false>), dim3(T), dim3(256), 0, st, static_cast<const float*>(x),
                       static_cast<const float*>(g), eps, H, static_cast<float*>(u), codes, scales);
  }
  return hipGetLastError();
}

}  // namespace moe
