// Grouping of (token, slot) pairs by expert: per-chunk histograms (LDS
// atomics), a per-expert scan over chunks plus an exclusive scan over experts,
// and a stable scatter.  Stability comes from 64-bit masks: for a run of 64
// tokens every pair ORs its token bit into its expert's LDS mask (OR is
// order-independent), and its row is the expert's running base plus the
// number of lower token bits set -- no dependence on atomic arrival order, so
// the result is the same bit for bit on every run.
//
// Ids come from the caller of moe_permute as well as from the router, so any
// int32 values are handled: a pair whose id lies outside [0, E) is not
// grouped (not counted, inverse map -1), and a token that names one expert in
// several slots -- which the token masks cannot tell apart -- sends its run
// of 64 tokens down a slower path with one mask bit per (token, slot) pair,
// in flat order t * k + j.  Either way the grouped order is the stable sort of
// the valid pairs by expert.
#include "kernels.h"

namespace moe {

__device__ __forceinline__ bool valid_id(int e, int E) {
  return static_cast<unsigned>(e) < static_cast<unsigned>(E);
}

__global__ __launch_bounds__(256) void perm_count(const int32_t* __restrict__ ids, int T, int k,
                                                  int E, int32_t* __restrict__ chunk_counts) {
  extern __shared__ int32_t cnt[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kPermChunk;
  const int64_t n = min(static_cast<int64_t>(kPermChunk), T - t0) * k;
  const int32_t* p = ids + t0 * k;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const int e = p[i];
    if (valid_id(e, E)) atomicAdd(&cnt[e], 1);
  }
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
                                                  int nchunk, int E,
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
  if (e == 0) offsets[E] = all;   // the grouped (valid) pairs
}

// Stable scatter of the pairs of tokens [g0, g0 + ntok), ntok <= 64, whose
// experts' rows start at run[e] (advanced past them on return).  Every thread
// of the block calls it; `mask` [E] and `flag` are LDS scratch.
__device__ void scatter_run(const int32_t* __restrict__ ids, int g0, int ntok, int k, int E,
                            unsigned long long* mask, int32_t* run, int* flag,
                            int32_t* __restrict__ sorted, int32_t* __restrict__ inv) {
  const int n = ntok * k, tid = threadIdx.x, nt = blockDim.x;
  const int64_t base = static_cast<int64_t>(g0) * k;
  for (int e = tid; e < E; e += nt) mask[e] = 0ull;
  if (tid == 0) *flag = 0;
  __syncthreads();
  for (int i = tid; i < n; i += nt) {
    const int e = ids[base + i];
    if (!valid_id(e, E)) continue;
    const unsigned long long bit = 1ull << (i / k);
    if (atomicOr(&mask[e], bit) & bit) atomicOr(flag, 1);   // expert repeated by a token
  }
  __syncthreads();
  if (*flag == 0) {
    // token masks: a pair's row is its expert's base + the lower tokens
    // routed to it
    for (int i = tid; i < n; i += nt) {
      const int tl = i / k, e = ids[base + i];
      int pos = -1;
      if (valid_id(e, E)) {
        pos = run[e] + __popcll(mask[e] & ((1ull << tl) - 1ull));
        sorted[pos] = g0 + tl;
      }
      inv[base + i] = pos;
    }
    __syncthreads();
    for (int e = tid; e < E; e += nt) run[e] += __popcll(mask[e]);
    __syncthreads();
    return;
  }
  // a repeated expert: one bit per pair, 64 flat pairs at a time
  for (int q0 = 0; q0 < n; q0 += 64) {
    const int m = min(64, n - q0);
    for (int e = tid; e < E; e += nt) mask[e] = 0ull;
    __syncthreads();
    for (int i = tid; i < m; i += nt) {
      const int e = ids[base + q0 + i];
      if (valid_id(e, E)) atomicOr(&mask[e], 1ull << i);
    }
    __syncthreads();
    for (int i = tid; i < m; i += nt) {
      const int e = ids[base + q0 + i];
      int pos = -1;
      if (valid_id(e, E)) {
        pos = run[e] + __popcll(mask[e] & ((1ull << i) - 1ull));
        sorted[pos] = g0 + (q0 + i) / k;
      }
      inv[base + q0 + i] = pos;
    }
    __syncthreads();
    for (int e = tid; e < E; e += nt) run[e] += __popcll(mask[e]);
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void perm_scatter(const int32_t* __restrict__ ids, int T, int k,
                                                    int E, const int32_t* __restrict__ chunk_base,
                                                    int32_t* __restrict__ sorted,
                                                    int32_t* __restrict__ inv, int identity_tail) {
  extern __shared__ unsigned long long smem[];
  __shared__ int flag;
  unsigned long long* mask = smem;                            // [E]
  int32_t* run = reinterpret_cast<int32_t*>(smem + E);        // [E]
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    run[e] = chunk_base[static_cast<int64_t>(blockIdx.x) * E + e];
  const int t_begin = blockIdx.x * kPermChunk;
  const int t_end = min(t_begin + kPermChunk, T);
  // (scatter_run's first barrier orders these run[] writes before their use)
  for (int g0 = t_begin; g0 < t_end; g0 += 64)
    scatter_run(ids, g0, min(64, t_end - g0), k, E, mask, run, &flag, sorted, inv);
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
  __shared__ int flag;
  unsigned long long* mask = smem;                               // [E]
  int32_t* run = reinterpret_cast<int32_t*>(smem + a.E);         // [E]
  const int E = a.E, T = a.T, k = a.k, tid = threadIdx.x;
  const int n_all = T * k;
  for (int e = tid; e < E; e += blockDim.x) run[e] = 0;
  __syncthreads();
  for (int i = tid; i < n_all; i += blockDim.x) {
    const int e = a.ids[i];
    if (valid_id(e, E)) atomicAdd(&run[e], 1);
  }
  __syncthreads();
  const int cnt = tid < E ? run[tid] : 0;
  int all;
  const int off = block_exclusive_scan(cnt, &all);
  if (tid < E) {
    a.offsets[tid] = off;
    run[tid] = off;
  }
  if (tid == 0) a.offsets[E] = all;   // the grouped (valid) pairs
  // (scatter_run's first barrier orders these run[] writes before their use)
  for (int g0 = 0; g0 < T; g0 += 64)
    scatter_run(a.ids, g0, min(64, T - g0), k, E, mask, run, &flag, a.sorted, a.inv);
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
  hipLaunchKernelGGL(perm_scan, dim3(1), dim3(1024), 0, st, a.chunk_counts, nchunk, a.E, a.chunk_base,
                     a.offsets);
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
// row gather (16-byte vectors), one block per 4 rows; rows [*n_rows, n) (pairs
// that were not grouped) are left alone
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gather_rows(const uint4* __restrict__ src,
                                                   const int32_t* __restrict__ rows, int64_t n,
                                                   const int32_t* __restrict__ n_rows,
                                                   int64_t vec_per_row, uint4* __restrict__ dst) {
  const int64_t p = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (p >= n || p >= *n_rows) return;
  const uint4* s = src + static_cast<int64_t>(rows[p]) * vec_per_row;
  uint4* d = dst + p * vec_per_row;
  for (int64_t i = threadIdx.x & 63; i < vec_per_row; i += 64) d[i] = s[i];
}

hipError_t launch_gather(const void* src, const int32_t* rows, int64_t n, const int32_t* n_rows,
                         int64_t row_bytes, void* dst, hipStream_t st) {
  hipLaunchKernelGGL(gather_rows, dim3((n + 3) / 4), dim3(256), 0, st,
                     static_cast<const uint4*>(src), rows, n, n_rows, row_bytes / 16,
                     static_cast<uint4*>(dst));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// dynamic activation quantisation ("Kimi K2 . Down projection", config.json
// quantization_config: fmt e4m3, activation_scheme dynamic), the body in
// common.h (quant_groups), one block per 16 or 32 groups
// ---------------------------------------------------------------------------
template <typename In, int GPW>
__global__ __launch_bounds__(256) void act_quant_rows(QuantSeg<In> s0, QuantSeg<In> s1) {
  quant_groups<In, GPW>(s0, s1, blockIdx.x);
}

template <typename In>
static hipError_t launch_quant(QuantSeg<In> s0, QuantSeg<In> s1, hipStream_t st) {
  const int64_t groups = s0.R * (s0.C / 128) + s1.R * (s1.C / 128);
  if (groups == 0) return hipSuccess;
  // 8 groups per wave on large inputs (two loads in flight per lane), 4 on
  // small ones, where the grid would be too small to fill the chip
  if (groups >= (1 << 16))
    hipLaunchKernelGGL((act_quant_rows<In, 8>), dim3((groups + 31) / 32), dim3(256), 0, st, s0, s1);
  else
    hipLaunchKernelGGL((act_quant_rows<In, 4>), dim3((groups + 15) / 16), dim3(256), 0, st, s0, s1);
  return hipGetLastError();
}

hipError_t launch_act_quant(const uint16_t* src, int64_t R, int C, uint8_t* codes, float* scales,
                            hipStream_t st) {
  return launch_quant(QuantSeg<uint16_t>{src, R, C, codes, scales}, QuantSeg<uint16_t>{src, 0, C, codes, scales},
                      st);
}

hipError_t launch_act_quant_f32(const float* src, int64_t R, int C, uint8_t* codes, float* scales,
                                const float* src2, int64_t R2, int C2, uint8_t* codes2, float* scales2,
                                hipStream_t st) {
  return launch_quant(QuantSeg<float>{src, R, C, codes, scales}, QuantSeg<float>{src2, R2, C2, codes2, scales2},
                      st);
}

}  // namespace moe
