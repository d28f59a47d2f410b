// Measurement kernels for the benchmark's measured ceilings (libmoe_probe.so,
// not part of libmoe): what one MI355X sustains, against which the layer's
// kernels are also reported.
//  * read: HBM read rate of the access form the weight streams use -- every
//    wave instruction covers whole 128-byte lines (64 lanes x 16 bytes), with
//    the nontemporal hint, 8 loads in flight per lane, each block over one
//    contiguous chunk of the buffer;
//  * mfma: back-to-back MFMAs on register operands (no memory traffic) in the
//    two forms the expert GEMMs issue: bf16 32x32x16 and the block-scaled
//    fp8 32x32x64 with unit scales.  Four independent accumulators per wave,
//    one wave per SIMD: the rate the MFMA pipes reach at the clock the chip
//    holds under that load.
// Every kernel folds what it computed into one value per block, stored, so
// nothing is optimised away.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

constexpr int kInFlight = 8;

// block b reads bytes [b * chunk, (b + 1) * chunk) (chunk a multiple of
// 256 threads x 16 B x kInFlight)
__global__ __launch_bounds__(256) void probe_read(const uint4* __restrict__ buf, int64_t chunk_vec,
                                                  uint4* __restrict__ sink) {
  const uint4* p = buf + static_cast<int64_t>(blockIdx.x) * chunk_vec + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t i = 0; i < chunk_vec; i += 256 * kInFlight) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u)
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + i + 256 * u));
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u];
  }
  __shared__ u32x4 red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    u32x4 s = red[0];
    for (int t = 1; t < 256; ++t) s ^= red[t];
    sink[blockIdx.x] = make_uint4(s.x, s.y, s.z, s.w);
  }
}

template <bool FP8>
__global__ __launch_bounds__(256) void probe_mfma(int iters, float* __restrict__ sink) {
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
  const int seed = static_cast<int>(threadIdx.x + blockIdx.x);
  i32x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x3c003c00 ^ (seed * (i + 1));   // finite bf16 pairs / e4m3 bytes
    b[i] = 0x38003800 ^ (seed * (i + 3));
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (FP8)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
      else
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, a, 0, 1, 2, 3)),
            __builtin_bit_cast(bf16x8, __builtin_shufflevector(b, b, 0, 1, 2, 3)), acc[c], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  if (s == 1.2345f) sink[blockIdx.x] = s;   // (practically never true; keeps the MFMAs live)
}

}  // namespace

extern "C" {

// Reads `bytes` of `buf` (a multiple of blocks * 256 * 16 * 8) with `blocks`
// blocks; sink holds blocks * 16 bytes.  Returns a hipError_t.
int moe_probe_read(const void* buf, int64_t bytes, int blocks, void* sink, void* stream) {
  const int64_t per = bytes / blocks / 16;
  if (bytes <= 0 || blocks <= 0 || per % (256 * kInFlight) != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(probe_read, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(buf), per, static_cast<uint4*>(sink));
  return hipGetLastError();
}

// blocks x 4 waves, each issuing iters x 4 MFMAs (fp8: 32x32x64 block-scaled
// form, else bf16 32x32x16); sink holds blocks floats.  Flops per launch:
// blocks * 4 * iters * 4 * 2 * 32 * 32 * (fp8 ? 64 : 16).
int moe_probe_mfma(int fp8, int blocks, int iters, void* sink, void* stream) {
  if (blocks <= 0 || iters <= 0) return hipErrorInvalidValue;
  if (fp8)
    hipLaunchKernelGGL(probe_mfma<true>, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters,
                       static_cast<float*>(sink));
  else
    hipLaunchKernelGGL(probe_mfma<false>, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters,
                       static_cast<float*>(sink));
  return hipGetLastError();
}

}  // extern "C"
