// Weighted combine fused with the shared-expert add:
//   out[t] = y_shared[t] + sum_j w[t][j] * y[inv[t*k + j]]
// (norm_topk_prob / routed_scaling_factor are already in w; the shared expert
// has weight 1 -- "Kimi K2 Base" raw config fields: n_shared_experts 1).
// With a residual (the sub-block around the layer) the sum starts from it:
//   out[t] = resid[t] + y_shared[t] + sum_j w[t][j] * y[inv[t*k + j]].
// fp32 accumulation in that order, one rounding at the end; one block per
// token, 16-byte vectors (a wave reads 1 KB of a row per instruction; the
// routed and shared rows, read once, with the nontemporal hint).  A slot whose
// inverse index lies outside [0, T*k) -- a pair the grouping did not place,
// inverse index -1 -- contributes nothing.  Up to 32 slots per token.
#include "kernels.h"

namespace moe {

template <bool BF16>
__global__ __launch_bounds__(256) void combine_rows(CombineArgs a) {
  __shared__ float ws[32];
  __shared__ int64_t rs[32];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < a.k) {
    const int64_t r = a.inv[t * a.k + threadIdx.x];
    ws[threadIdx.x] = a.w[t * a.k + threadIdx.x];
    rs[threadIdx.x] = r >= 0 && r < static_cast<int64_t>(a.T) * a.k ? r : -1;
  }
  __syncthreads();
  constexpr int VEC = BF16 ? 8 : 4;
  // columns split over gridDim.y blocks per token (few tokens: more blocks)
  const int nv = a.H / VEC, per = (nv + gridDim.y - 1) / gridDim.y;
  const int c1 = min(nv, static_cast<int>(blockIdx.y + 1) * per);
  for (int c = blockIdx.y * per + threadIdx.x; c < c1; c += blockDim.x) {
    float acc[VEC];
    if (BF16) {
      const uint16_t* ysh = static_cast<const uint16_t*>(a.y_sh);
      const uint16_t* y = static_cast<const uint16_t*>(a.y);
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
      const uint16_t* res = static_cast<const uint16_t*>(a.resid);
      if (res) {
        uint4 v = reinterpret_cast<const uint4*>(res + t * a.H)[c];
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = bf16_to_f32(static_cast<uint16_t>(w4[i] & 0xffffu));
          acc[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(w4[i] >> 16));
        }
      }
      if (ysh) {
        uint4 v = load_nt(reinterpret_cast<const uint4*>(ysh + t * a.H) + c);
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += bf16_to_f32(static_cast<uint16_t>(w4[i] & 0xffffu));
          acc[2 * i + 1] += bf16_to_f32(static_cast<uint16_t>(w4[i] >> 16));
        }
      }
      // up to 8 routed rows' loads in flight per thread, then the sums in
      // slot order; the rows are read once (nontemporal)
      for (int j0 = 0; j0 < a.k; j0 += 8) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (j0 + u < a.k && rs[j0 + u] >= 0) v[u] = load_nt(reinterpret_cast<const uint4*>(y + rs[j0 + u] * a.H) + c);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (j0 + u >= a.k) break;
          if (rs[j0 + u] < 0) continue;
          const uint32_t w4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
          const float wj = ws[j0 + u];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] = fmaf(wj, bf16_to_f32(static_cast<uint16_t>(w4[i] & 0xffffu)), acc[2 * i]);
            acc[2 * i + 1] = fmaf(wj, bf16_to_f32(static_cast<uint16_t>(w4[i] >> 16)), acc[2 * i + 1]);
          }
        }
      }
      uint4 o;
      uint32_t* op = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        op[i] = static_cast<uint32_t>(f32_to_bf16(acc[2 * i])) |
                (static_cast<uint32_t>(f32_to_bf16(acc[2 * i + 1])) << 16);
      reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + t * a.H)[c] = o;
    } else {
      const float* ysh = static_cast<const float*>(a.y_sh);
      const float* y = static_cast<const float*>(a.y);
      const float* res = static_cast<const float*>(a.resid);
      float4 r = res ? reinterpret_cast<const float4*>(res + t * a.H)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
      acc[0] = r.x; acc[1] = r.y; acc[2] = r.z; acc[3] = r.w;
      if (ysh) {
        float4 s = reinterpret_cast<const float4*>(ysh + t * a.H)[c];
        acc[0] += s.x; acc[1] += s.y; acc[2] += s.z; acc[3] += s.w;
      }
      for (int j = 0; j < a.k; ++j) {
        if (rs[j] < 0) continue;
        float4 v = reinterpret_cast<const float4*>(y + rs[j] * a.H)[c];
        const float wj = ws[j];
        acc[0] = fmaf(wj, v.x, acc[0]); acc[1] = fmaf(wj, v.y, acc[1]);
        acc[2] = fmaf(wj, v.z, acc[2]); acc[3] = fmaf(wj, v.w, acc[3]);
      }
      reinterpret_cast<float4*>(static_cast<float*>(a.out) + t * a.H)[c] =
          make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
  }
}

hipError_t launch_combine(const CombineArgs& a, bool bf16, hipStream_t st) {
  const int threads = 256;
  // below 256 tokens, one block per token and 256 vectors of columns
  const int nv = a.H / (bf16 ? 8 : 4);
  const int split = a.T < 256 ? (nv + threads - 1) / threads : 1;
  const dim3 grid(a.T, split);
  if (bf16) hipLaunchKernelGGL(combine_rows<true>, grid, dim3(threads), 0, st, a);
  else hipLaunchKernelGGL(combine_rows<false>, grid, dim3(threads), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
