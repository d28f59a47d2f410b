// Router: logits = x W_r^T (fp32 accumulate), then per token sigmoid scores,
// correction-bias selection (noaux_tc), optional group restriction, top-k and
// renormalised, scaled weights.  Config fields from the "Kimi K2 Base" /
// "Kimi K2 0905" raw config tables (scoring_func sigmoid, topk_method
// noaux_tc, n_group, topk_group, num_experts_per_tok, norm_topk_prob,
// routed_scaling_factor).
#include "kernels.h"

namespace moe {

// K parts of the small-batch logits kernel (partial sums added by top-k)
constexpr int kMaxParts = 8;

// ---------------------------------------------------------------------------
// logits, bf16: one block = 16 tokens x 16 experts, 4 waves split the K loop
// (K steps of 128 taken round-robin), reduced through LDS in a fixed order.
// MFMA 16x16x32 bf16 with A = router rows (experts), B = token rows.  Each
// lane streams 64 contiguous bytes of its row per K step; the K order inside
// a step is permuted identically for A and B, which a dot product allows.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_logits_bf16(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wr,
                                                          int T, int E, int H,
                                                          float* __restrict__ logits) {
  __shared__ f32x4 red[3][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int e0 = blockIdx.x * 16, t0 = blockIdx.y * 16;
  const int tok = min(t0 + r, T - 1);
  const uint16_t* pa = wr + static_cast<int64_t>(min(e0 + r, E - 1)) * H + q * 32;
  const uint16_t* pb = x + static_cast<int64_t>(tok) * H + q * 32;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // K part blockIdx.z of gridDim.z: steps [s0, s1) of 128; its partial sums
  // go to logits + part * T * E
  const int steps = H / 128, per = (steps + gridDim.z - 1) / gridDim.z;
  const int s0 = blockIdx.z * per, s1 = min(s0 + per, steps);
  logits += static_cast<int64_t>(blockIdx.z) * T * E;
  // steps s0 + wave, s0 + wave + 4, ...; the next step's loads are issued
  // before the current step's MFMAs
  auto load = [&](int s, uint4 (&a)[4], uint4 (&b)[4]) {
    const uint4* a4 = reinterpret_cast<const uint4*>(pa + s * 128);
    const uint4* b4 = reinterpret_cast<const uint4*>(pb + s * 128);
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] = a4[i]; b[i] = b4[i]; }
  };
  uint4 a[4], b[4], an[4], bn[4];
  int s = s0 + wave;
  if (s < s1) load(s, a, b);
#pragma unroll 1
  while (s < s1) {
    const int sn = s + 4;
    if (sn < s1) load(sn, an, bn);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[i]),
                                                    __builtin_bit_cast(bf16x8, b[i]), acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] = an[i]; b[i] = bn[i]; }
    s = sn;
  }
  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < 3; ++w) acc += red[w][lane];
    // lane holds experts e0 + 4q + i (i = 0..3) of token t0 + r
    if (t0 + r < T) {
      float* dst = logits + static_cast<int64_t>(t0 + r) * E;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (e0 + 4 * q + i < E) dst[e0 + 4 * q + i] = acc[i];
    }
  }
}

// ---------------------------------------------------------------------------
// logits, bf16, many tokens: one block = 128 tokens x 64 experts, both staged
// through LDS (144-byte padded rows, conflict-free 128-bit reads) one K step
// of 64 ahead in registers; wave w owns tokens 32w..32w+31 x all 64 experts
// (two 32x32x16 MFMA tiles, C[expert][token]).  Every router row is read
// once per 128 tokens instead of once per 16.  K part blockIdx.z of gridDim.z
// covers steps [s0, s1) and writes its partial sums to logits + part * T * E
// (added in part order by the top-k kernel).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_logits_bf16_tile(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ wr,
                                                               int T, int E, int H,
                                                               float* __restrict__ logits) {
  constexpr int kTok = 128, kExp = 64, kLd = 72;   // LDS row stride, bf16 elements
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][(kTok + kExp) * kLd];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r32 = lane & 31, kh = lane >> 5;
  const int t0 = blockIdx.x * kTok, e0 = blockIdx.y * kExp;
  // staging: 192 rows x 8 chunks of 16 B = 1536 chunks, 6 per thread
  const uint16_t* src[6];
  int ldo[6];
#pragma unroll
  for (int c = 0; c < 6; ++c) {
    const int idx = tid + 256 * c, row = idx >> 3, cc = idx & 7;
    src[c] = row < kTok ? x + static_cast<int64_t>(min(t0 + row, T - 1)) * H + cc * 8
                        : wr + static_cast<int64_t>(e0 + row - kTok) * H + cc * 8;
    ldo[c] = row * kLd + cc * 8;
  }
  f32x16 acc[2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[m][i] = 0.f;
  const int steps = H / 64, per = (steps + gridDim.z - 1) / gridDim.z;
  const int s0 = blockIdx.z * per, s1 = min(s0 + per, steps);
  logits += static_cast<int64_t>(blockIdx.z) * T * E;
  uint4 st[6];
  if (s0 < s1) {
#pragma unroll
    for (int c = 0; c < 6; ++c) st[c] = *reinterpret_cast<const uint4*>(src[c] + s0 * 64);
#pragma unroll
    for (int c = 0; c < 6; ++c) *reinterpret_cast<uint4*>(&lds[0][ldo[c]]) = st[c];
  }
  __syncthreads();
  for (int s = s0; s < s1; ++s) {
    const int buf = (s - s0) & 1;
    const int ko = min(s + 1, s1 - 1) * 64;
#pragma unroll
    for (int c = 0; c < 6; ++c) st[c] = *reinterpret_cast<const uint4*>(src[c] + ko);
    const uint16_t* bt = &lds[buf][(32 * wave + r32) * kLd + kh * 32];
    const uint16_t* at = &lds[buf][(kTok + r32) * kLd + kh * 32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 b = *reinterpret_cast<const uint4*>(bt + 8 * i);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint4 av = *reinterpret_cast<const uint4*>(at + 32 * m * kLd + 8 * i);
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                         __builtin_bit_cast(bf16x8, b), acc[m], 0, 0, 0);
      }
    }
#pragma unroll
    for (int c = 0; c < 6; ++c) *reinterpret_cast<uint4*>(&lds[buf ^ 1][ldo[c]]) = st[c];
    __syncthreads();
  }
  // lane holds experts e0 + 32m + 8(i/4) + 4kh + (i%4) of token t0 + 32w + r32
  const int t = t0 + 32 * wave + r32;
  if (t >= T) return;
  float* dst = logits + static_cast<int64_t>(t) * E + e0 + 4 * kh;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float4*>(dst + 32 * m + 8 * g) =
          make_float4(acc[m][4 * g], acc[m][4 * g + 1], acc[m][4 * g + 2], acc[m][4 * g + 3]);
}

// fp32 logits: one thread per (token, expert), plain fp32 FMA over H.
__global__ __launch_bounds__(256) void router_logits_f32(const float* __restrict__ x,
                                                         const float* __restrict__ wr, int T, int E,
                                                         int H, float* __restrict__ logits) {
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(T) * E) return;
  int t = static_cast<int>(i / E), e = static_cast<int>(i % E);
  const float4* a = reinterpret_cast<const float4*>(x + static_cast<int64_t>(t) * H);
  const float4* b = reinterpret_cast<const float4*>(wr + static_cast<int64_t>(e) * H);
  float s = 0.f;
  for (int h = 0; h < H / 4; ++h) {
    float4 u = a[h], v = b[h];
    s = fmaf(u.x, v.x, s); s = fmaf(u.y, v.y, s); s = fmaf(u.z, v.z, s); s = fmaf(u.w, v.w, s);
  }
  logits[i] = s;
}

// ---------------------------------------------------------------------------
// top-k: one wave per token, 4 tokens per block.  Lane l holds experts
// l*V .. l*V+V-1.  The selection scores become order-preserving 32-bit keys
// (NaN as -inf, -0 as +0; experts past E key 0, below every score), and the
// k-th largest key is found bit by bit, 32 steps of "how many keys are >=
// this", each a compare and a ballot popcount per slot -- scalar work, no
// cross-lane shuffle chain.  The chosen experts are the keys above it plus
// the lowest ids among the keys equal to it (ties: lower expert id), and a
// prefix popcount puts each chosen id at its ascending position.  So a token
// always gets k distinct ids in [0, E) (k <= E): experts of groups that were
// not kept, or with a -inf bias, score -inf and are taken, lowest id first,
// only when fewer than k finite eligible scores remain.
// With fp8 expert weights the same launch quantises x: blocks from
// `topk_blocks` on are activation-quant blocks (quant_groups).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);   // (-0 + 0 = +0)
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int V>
__global__ __launch_bounds__(256) void router_topk(const float* __restrict__ logits, int kparts,
                                                   const float* __restrict__ bias, int T, int E,
                                                   int k, int n_group, int topk_group, int norm,
                                                   float scale, int32_t* __restrict__ ids_out,
                                                   float* __restrict__ w_out, int topk_blocks,
                                                   QuantSeg<uint16_t> xq) {
  if (static_cast<int>(blockIdx.x) >= topk_blocks) {   // block-uniform: x's fp8 codes
    quant_groups<uint16_t, 4>(xq, QuantSeg<uint16_t>{xq.src, 0, xq.C, xq.codes, xq.scales},
                              blockIdx.x - topk_blocks);
    return;
  }
  __shared__ float sel_lds[4][64 * V];
  __shared__ float gsc_lds[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  const bool valid = t < T;
  const int tt = valid ? t : T - 1;
  float s[V], sel[V];
  // partial logits of the K parts (at most kMaxParts), all loaded at once
  // (every load unconditional: a part past kparts re-reads part 0 and is not
  // added), then added in part order
  float zp[kMaxParts][V];
#pragma unroll
  for (int p = 0; p < kMaxParts; ++p)
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int e = min(lane * V + i, E - 1);
      zp[p][i] = logits[(static_cast<int64_t>(p < kparts ? p : 0) * T + tt) * E + e];
    }
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = lane * V + i;
    if (e < E) {
      float z = zp[0][i];
#pragma unroll
      for (int p = 1; p < kMaxParts; ++p)
        if (p < kparts) z += zp[p][i];
      s[i] = 1.0f / (1.0f + expf(-z));
      const float v = s[i] + bias[e];
      sel[i] = v == v ? v : -INFINITY;
    } else {
      s[i] = 0.f;
      sel[i] = -INFINITY;
    }
  }
  if (n_group > 1) {  // block-uniform branch
    const int gsz = E / n_group;
#pragma unroll
    for (int i = 0; i < V; ++i) sel_lds[wave][lane * V + i] = sel[i];
    __syncthreads();
    float gscore = -INFINITY;
    if (lane < n_group) {
      float b1 = -INFINITY, b2 = -INFINITY;
      for (int j = 0; j < gsz; ++j) {
        const float v = sel_lds[wave][lane * gsz + j];
        if (v > b1) { b2 = b1; b1 = v; } else if (v > b2) { b2 = v; }
      }
      gscore = gsz > 1 ? b1 + b2 : b1;
      if (!(gscore == gscore)) gscore = -INFINITY;   // +inf + -inf
      gsc_lds[wave][lane] = gscore;
    }
    __syncthreads();
    int keep = 0;
    if (lane < n_group) {
      int rank = 0;
      for (int g = 0; g < n_group; ++g) {
        const float o = gsc_lds[wave][g];
        rank += (o > gscore) || (o == gscore && g < lane);
      }
      keep = rank < topk_group;
    }
    __syncthreads();
    if (lane < n_group) gsc_lds[wave][lane] = keep ? 1.f : 0.f;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int e = lane * V + i;
      if (e < E && gsc_lds[wave][e / gsz] == 0.f) sel[i] = -INFINITY;
    }
  }
  uint32_t key[V];
#pragma unroll
  for (int i = 0; i < V; ++i) key[i] = lane * V + i < E ? order_key(sel[i]) : 0u;
  auto count = [&](auto pred) {   // wave-wide number of keys satisfying pred
    int c = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) c += __popcll(__ballot(pred(key[i])));
    return c;
  };
  // the k-th largest key: the largest thr with at least k keys >= thr
  uint32_t thr = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = thr | (1u << b);
    if (count([c](uint32_t x) { return x >= c; }) >= k) thr = c;
  }
  const int need = k - count([thr](uint32_t x) { return x > thr; });   // >= 1 keys equal to thr
  const uint64_t below = (1ull << lane) - 1ull;   // lanes holding lower ids
  int eq_rank = 0;                                // equal keys at lower ids
#pragma unroll
  for (int i = 0; i < V; ++i) eq_rank += __popcll(__ballot(key[i] == thr) & below);
  bool chosen[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const bool eq = key[i] == thr;
    chosen[i] = key[i] > thr || (eq && eq_rank < need);
    eq_rank += eq;
  }
  int pos = 0;   // chosen experts at lower ids: this lane's first output slot
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    pos += __popcll(__ballot(chosen[i]) & below);
    if (chosen[i]) part += s[i];
  }
  const float sum = wave_sum(part);
  if (valid) {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      if (!chosen[i]) continue;
      const float w = norm ? (s[i] / sum) * scale : s[i] * scale;
      ids_out[static_cast<int64_t>(t) * k + pos] = lane * V + i;
      w_out[static_cast<int64_t>(t) * k + pos] = w;
      ++pos;
    }
  }
}

// K parts of the 16x16 logits kernel: few tokens give few blocks (24 for one
// token and 384 experts), so the K loop is split over up to 8 blocks per tile
// until the grid has ~512 blocks; the top-k kernel adds the parts in order
// K parts of the logits kernels: doubled while the grid has fewer than 512
// blocks and every part keeps at least 4 K steps of 128 (16 x 16 kernel: one
// per wave) or 8 of 64 (the 128 x 64 LDS-tiled kernel, whose blocks
// otherwise walk all of H one latency-bound step at a time: at 512 tokens
// and 384 experts its 24 blocks took 0.11 ms).
bool router_tiled(int64_t T, int E, bool bf16) { return bf16 && T >= 512 && E % 64 == 0; }

int router_kparts(int64_t T, int E, int H, bool bf16) {
  if (!bf16) return 1;
  const bool tiled = router_tiled(T, E, bf16);
  const int64_t blocks = tiled ? ((T + 127) / 128) * (E / 64) : static_cast<int64_t>((E + 15) / 16) * ((T + 15) / 16);
  const int ksteps = tiled ? H / 64 : H / 128, min_steps = tiled ? 8 : 4;
  int kp = 1;
  while (kp < kMaxParts && blocks * kp < 512 && ksteps >= 2 * kp * min_steps) kp *= 2;
  return kp;
}

hipError_t launch_router(const RouterArgs& a, hipStream_t st) {
  if (router_tiled(a.T, a.E, a.bf16)) {
    dim3 grid((a.T + 127) / 128, a.E / 64, router_kparts(a.T, a.E, a.H, a.bf16));
    hipLaunchKernelGGL(router_logits_bf16_tile, grid, dim3(256), 0, st,
                       static_cast<const uint16_t*>(a.x), static_cast<const uint16_t*>(a.wr), a.T,
                       a.E, a.H, a.logits);
  } else if (a.bf16) {
    dim3 grid((a.E + 15) / 16, (a.T + 15) / 16, router_kparts(a.T, a.E, a.H, a.bf16));
    hipLaunchKernelGGL(router_logits_bf16, grid, dim3(256), 0, st,
                       static_cast<const uint16_t*>(a.x), static_cast<const uint16_t*>(a.wr), a.T,
                       a.E, a.H, a.logits);
  } else {
    const int64_t n = static_cast<int64_t>(a.T) * a.E;
    hipLaunchKernelGGL(router_logits_f32, dim3((n + 255) / 256), dim3(256), 0, st,
                       static_cast<const float*>(a.x), static_cast<const float*>(a.wr), a.T, a.E,
                       a.H, a.logits);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return hipSuccess;
}

hipError_t launch_topk(const RouterArgs& a, hipStream_t st) {
  const int topk_blocks = (a.T + 3) / 4;
  // with x's fp8 codes: one quant block per 16 groups of 128 channels
  const QuantSeg<uint16_t> xq{static_cast<const uint16_t*>(a.x), a.xq_codes ? a.T : 0, a.H, a.xq_codes,
                              a.xq_scales};
  const int64_t qblocks = (xq.R * (a.H / 128) + 15) / 16;
  dim3 grid(static_cast<unsigned>(topk_blocks + qblocks)), block(256);
  const int V = (a.E + 63) / 64;
#define MOE_TOPK(VV)                                                                         \
  hipLaunchKernelGGL(router_topk<VV>, grid, block, 0, st, a.logits, router_kparts(a.T, a.E, a.H, a.bf16), \
                     a.bias, a.T, a.E, a.k, a.n_group, a.topk_group, a.norm, a.scale, a.ids, a.w,            \
                     topk_blocks, xq)
  if (V <= 1) MOE_TOPK(1);
  else if (V <= 2) MOE_TOPK(2);
  else if (V <= 4) MOE_TOPK(4);
  else if (V <= 6) MOE_TOPK(6);
  else if (V <= 8) MOE_TOPK(8);
  else MOE_TOPK(16);
#undef MOE_TOPK
  return hipGetLastError();
}

}  // namespace moe
