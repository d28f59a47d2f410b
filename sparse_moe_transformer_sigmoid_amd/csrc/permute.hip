// Grouping of (token, slot) pairs by expert: per-chunk histograms (LDS
// atomics), a per-expert scan over chunks plus an exclusive scan over experts,
// and a stable scatter.  Stability comes from 64-bit token masks: for a run
// of 64 tokens every pair ORs its token bit into its expert's LDS mask (OR is
// order-independent), and its row is the expert's running base plus the
// number of lower token bits set -- no dependence on atomic arrival order, so
// the result is the same bit for bit on every run.
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void perm_count(const int32_t* __restrict__ ids, int T, int k,
                                                  int E, int32_t* __restrict__ chunk_counts) {
  extern __shared__ int32_t cnt[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kPermChunk;
  const int64_t n = min(static_cast<int64_t>(kPermChunk), T - t0) * k;
  const int32_t* p = ids + t0 * k;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) atomicAdd(&cnt[p[i]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    chunk_counts[static_cast<int64_t>(blockIdx.x) * E + e] = cnt[e];
}

// exclusive block scan of one value per thread (blockDim.x <= 1024)
__device__ int block_exclusive_scan(int v, int* total) {
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  int inc = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(inc, o, 64);
    if (lane >= o) inc += u;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int base = 0, all = 0;
  for (int w = 0; w < nw; ++w) {
    const int s = wsum[w];
    if (w < wave) base += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return base + inc - v;
}

// one block of 1024 threads; thread e owns expert e (E <= 1024)
__global__ __launch_bounds__(1024) void perm_scan(const int32_t* __restrict__ chunk_counts,
                                                  int nchunk, int E, int64_t total_rows,
                                                  int32_t* __restrict__ chunk_base,
                                                  int32_t* __restrict__ offsets) {
  const int e = threadIdx.x;
  int run = 0;
  if (e < E)
    for (int c = 0; c < nchunk; ++c) {
      const int64_t i = static_cast<int64_t>(c) * E + e;
      const int v = chunk_counts[i];
      chunk_base[i] = run;
      run += v;
    }
  int all;
  const int off = block_exclusive_scan(e < E ? run : 0, &all);
  if (e < E) {
    offsets[e] = off;
    for (int c = 0; c < nchunk; ++c) chunk_base[static_cast<int64_t>(c) * E + e] += off;
  }
  if (e == 0) offsets[E] = static_cast<int32_t>(total_rows);
}

__global__ __launch_bounds__(256) void perm_scatter(const int32_t* __restrict__ ids, int T, int k,
                                                    int E, const int32_t* __restrict__ chunk_base,
                                                    int32_t* __restrict__ sorted,
                                                    int32_t* __restrict__ inv, int identity_tail) {
  extern __shared__ unsigned long long smem[];
  unsigned long long* mask = smem;                            // [E]
  int32_t* run = reinterpret_cast<int32_t*>(smem + E);        // [E]
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    run[e] = chunk_base[static_cast<int64_t>(blockIdx.x) * E + e];
  const int t_begin = blockIdx.x * kPermChunk;
  const int t_end = min(t_begin + kPermChunk, T);
  for (int g0 = t_begin; g0 < t_end; g0 += 64) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) mask[e] = 0ull;
    __syncthreads();
    const int n = min(64, t_end - g0) * k;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const int tl = i / k;
      const int e = ids[static_cast<int64_t>(g0) * k + i];
      atomicOr(&mask[e], 1ull << tl);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const int tl = i / k;
      const int64_t flat = static_cast<int64_t>(g0) * k + i;
      const int e = ids[flat];
      const int pos = run[e] + __popcll(mask[e] & ((1ull << tl) - 1ull));
      sorted[pos] = g0 + tl;
      inv[flat] = pos;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) run[e] += __popcll(mask[e]);
    __syncthreads();
  }
  if (identity_tail)
    for (int t = t_begin + threadIdx.x; t < t_end; t += blockDim.x)
      sorted[static_cast<int64_t>(T) * k + t] = t;
}

// The whole grouping for T <= kPermChunk in one block of 1024 threads: the
// histogram (LDS atomics), the exclusive scan over experts (thread e owns
// expert e), the stable scatter with the same 64-bit token masks as
// perm_scatter and, optionally, the work list of build_tiles.  Small batches
// (decode) are bound by launch latency, so one launch instead of four.
__global__ __launch_bounds__(1024) void perm_single(PermArgs a) {
  extern __shared__ unsigned long long smem[];
  unsigned long long* mask = smem;                               // [E]
  int32_t* run = reinterpret_cast<int32_t*>(smem + a.E);         // [E]
  const int E = a.E, T = a.T, k = a.k, tid = threadIdx.x;
  const int n_all = T * k;
  for (int e = tid; e < E; e += blockDim.x) run[e] = 0;
  __syncthreads();
  for (int i = tid; i < n_all; i += blockDim.x) atomicAdd(&run[a.ids[i]], 1);
  __syncthreads();
  const int cnt = tid < E ? run[tid] : 0;
  int all;
  const int off = block_exclusive_scan(cnt, &all);
  if (tid < E) {
    a.offsets[tid] = off;
    run[tid] = off;
  }
  if (tid == 0) a.offsets[E] = n_all;
  __syncthreads();
  for (int g0 = 0; g0 < T; g0 += 64) {
    for (int e = tid; e < E; e += blockDim.x) mask[e] = 0ull;
    __syncthreads();
    const int n = min(64, T - g0) * k;
    for (int i = tid; i < n; i += blockDim.x) atomicOr(&mask[a.ids[g0 * k + i]], 1ull << (i / k));
    __syncthreads();
    for (int i = tid; i < n; i += blockDim.x) {
      const int tl = i / k, flat = g0 * k + i, e = a.ids[flat];
      const int pos = run[e] + __popcll(mask[e] & ((1ull << tl) - 1ull));
      a.sorted[pos] = g0 + tl;
      a.inv[flat] = pos;
    }
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) run[e] += __popcll(mask[e]);
    __syncthreads();
  }
  if (a.identity_tail)
    for (int t = tid; t < T; t += blockDim.x) a.sorted[n_all + t] = t;
  if (a.tiles == nullptr) return;
  // work list: group g < E = expert g (cnt rows from off), group E = shared
  int n = 0, base = 0;
  if (tid < E) {
    n = cnt;
    base = off;
  } else if (tid == E && a.shared) {
    n = T;
    base = n_all;
  }
  const int nt = (n + a.bm - 1) / a.bm;
  int tiles_all;
  const int start = block_exclusive_scan(nt, &tiles_all);
  for (int i = 0; i < nt && start + i < a.cap; ++i) {
    Tile t;
    t.group = tid;
    t.row0 = base + i * a.bm;
    t.rows = min(a.bm, n - i * a.bm);
    t.pad = 0;
    a.tiles[start + i] = t;
  }
  if (tid == 0) *a.tile_count = static_cast<int32_t>(min(static_cast<int64_t>(tiles_all), a.cap));
}

hipError_t launch_permute(const PermArgs& a, hipStream_t st, bool* tiles_built) {
  if (tiles_built) *tiles_built = false;
  if (a.T <= kPermChunk) {
    hipLaunchKernelGGL(perm_single, dim3(1), dim3(1024), a.E * (sizeof(unsigned long long) + 4), st, a);
    if (tiles_built) *tiles_built = a.tiles != nullptr;
    return hipGetLastError();
  }
  const int nchunk = (a.T + kPermChunk - 1) / kPermChunk;
  hipLaunchKernelGGL(perm_count, dim3(nchunk), dim3(256), a.E * sizeof(int32_t), st, a.ids, a.T,
                     a.k, a.E, a.chunk_counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(perm_scan, dim3(1), dim3(1024), 0, st, a.chunk_counts, nchunk, a.E,
                     static_cast<int64_t>(a.T) * a.k, a.chunk_base, a.offsets);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(perm_scatter, dim3(nchunk), dim3(256), a.E * (sizeof(unsigned long long) + 4),
                     st, a.ids, a.T, a.k, a.E, a.chunk_base, a.sorted, a.inv,
                     a.identity_tail ? 1 : 0);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// work list of the grouped GEMMs: group g (expert, or the shared expert as
// group E) contributes ceil(n_g / bm) tiles of consecutive grouped rows.
// ---------------------------------------------------------------------------
int64_t max_tiles(int64_t T, int k, int E, bool shared, int bm) {
  const int64_t rows = T * k;
  return rows / bm + std::min<int64_t>(E, rows) + (shared ? (T + bm - 1) / bm : 0);
}

// Work list of the grouped GEMMs: group g < E covers the rows of expert g,
// group E the shared expert's T rows after the T*k routed ones.  Offsets come
// from the caller of moe_expert_ffn, so each segment is clamped into
// [0, T*k] and at most `cap` tiles are written: any offsets array yields
// tiles inside the row buffers.
__global__ __launch_bounds__(1024) void build_tiles(const int32_t* __restrict__ offsets, int T,
                                                    int k, int E, int bm, int shared, int cap,
                                                    Tile* __restrict__ tiles,
                                                    int32_t* __restrict__ tile_count) {
  const int g = threadIdx.x;  // groups 0..E (E <= 1023)
  const int TK = T * k;
  int n = 0, base = 0;
  if (g < E) {
    base = min(max(offsets[g], 0), TK);
    n = min(max(offsets[g + 1], base), TK) - base;
  } else if (g == E && shared) {
    base = TK;
    n = T;
  }
  const int nt = (n + bm - 1) / bm;
  int all;
  const int start = block_exclusive_scan(nt, &all);
  for (int i = 0; i < nt && start + i < cap; ++i) {
    Tile t;
    t.group = g;
    t.row0 = base + i * bm;
    t.rows = min(bm, n - i * bm);
    t.pad = 0;
    tiles[start + i] = t;
  }
  if (g == 0) *tile_count = min(all, cap);
}

hipError_t launch_build_tiles(const TileArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(build_tiles, dim3(1), dim3(1024), 0, st, a.offsets, a.T, a.k, a.E, a.bm,
                     a.shared ? 1 : 0, static_cast<int>(a.cap), a.tiles, a.tile_count);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// row gather (16-byte vectors), one block per 4 rows
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gather_rows(const uint4* __restrict__ src,
                                                   const int32_t* __restrict__ rows, int64_t n,
                                                   int64_t vec_per_row, uint4* __restrict__ dst) {
  const int64_t p = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (p >= n) return;
  const uint4* s = src + static_cast<int64_t>(rows[p]) * vec_per_row;
  uint4* d = dst + p * vec_per_row;
  for (int64_t i = threadIdx.x & 63; i < vec_per_row; i += 64) d[i] = s[i];
}

hipError_t launch_gather(const void* src, const int32_t* rows, int64_t n, int64_t row_bytes,
                         void* dst, hipStream_t st) {
  hipLaunchKernelGGL(gather_rows, dim3((n + 3) / 4), dim3(256), 0, st,
                     static_cast<const uint4*>(src), rows, n, row_bytes / 16,
                     static_cast<uint4*>(dst));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// dynamic activation quantisation ("Kimi K2 . Down projection", config.json
// quantization_config: fmt e4m3, activation_scheme dynamic): per row and 128
// channels s = amax / 448 (1 when the group is all zero), code = e4m3(v / s).
// One wave per group of 128: two values per lane.
// ---------------------------------------------------------------------------
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

// Dynamic activation quantisation, per row and 128-channel group: s = amax /
// 448 (1 for an all-zero group), codes e4m3(v / s) with the division in fp32.
// 16 lanes hold one group (8 values each), so a wave covers 4 groups per
// load and GPW groups in all, every load issued before the arithmetic.
template <typename In, int GPW>
__global__ __launch_bounds__(256) void act_quant_rows(const In* __restrict__ src, int64_t R, int C,
                                                      uint8_t* __restrict__ codes,
                                                      float* __restrict__ scales) {
  const int lane = threadIdx.x & 63, sub = lane & 15;
  const int groups = C / 128;
  const int64_t total = R * groups;
  const int64_t g0 = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * GPW + (lane >> 4);
  float v[GPW / 4][8];
#pragma unroll
  for (int i = 0; i < GPW / 4; ++i) {
    const int64_t gi = g0 + 4 * i;
    if (gi < total) {
      const int64_t row = gi / groups;
      load8(src + row * C + (gi - row * groups) * 128 + 8 * sub, v[i]);
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
    const int64_t row = gi / groups;
    const int64_t off = row * C + (gi - row * groups) * 128 + 8 * sub;
    *reinterpret_cast<uint2*>(codes + off) = make_uint2(lo, hi);
    if (sub == 0) scales[gi] = sc;
  }
}

hipError_t launch_act_quant(const uint16_t* src, int64_t R, int C, uint8_t* codes, float* scales,
                            hipStream_t st) {
  const int64_t groups = R * (C / 128);
  // 8 groups per wave on large inputs (two loads in flight per lane), 4 on
  // small ones, where the grid would be too small to fill the chip
  if (groups >= (1 << 16))
    hipLaunchKernelGGL((act_quant_rows<uint16_t, 8>), dim3((groups + 31) / 32), dim3(256), 0, st, src, R, C,
                       codes, scales);
  else
    hipLaunchKernelGGL((act_quant_rows<uint16_t, 4>), dim3((groups + 15) / 16), dim3(256), 0, st, src, R, C,
                       codes, scales);
  return hipGetLastError();
}

hipError_t launch_act_quant_f32(const float* src, int64_t R, int C, uint8_t* codes, float* scales,
                                hipStream_t st) {
  const int64_t groups = R * (C / 128);
  if (groups == 0) return hipSuccess;
  if (groups >= (1 << 16))
    hipLaunchKernelGGL((act_quant_rows<float, 8>), dim3((groups + 31) / 32), dim3(256), 0, st, src, R, C,
                       codes, scales);
  else
    hipLaunchKernelGGL((act_quant_rows<float, 4>), dim3((groups + 15) / 16), dim3(256), 0, st, src, R, C,
                       codes, scales);
  return hipGetLastError();
}

}  // namespace moe
