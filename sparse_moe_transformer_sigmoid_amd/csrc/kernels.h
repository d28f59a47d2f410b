// Launch interfaces of the libmoe kernels (host side of each .hip file).
#pragma once
#include "common.h"

namespace moe {

constexpr int kPermChunk = 256;  // tokens per block in the grouping kernels

struct RouterArgs {
  const void* x;
  const void* wr;
  const float* bias;
  int T, E, H, k, n_group, topk_group, norm;
  float scale;
  bool bf16;
  float* logits;  // [T][E] scratch
  int32_t* ids;   // [T][k]
  float* w;       // [T][k]
  // optional (fp8 expert weights): the top-k launch also quantises x (bf16)
  // per token and 128 channels into codes [T][H] and scales [T][H/128]
  uint8_t* xq_codes = nullptr;
  float* xq_scales = nullptr;
};
hipError_t launch_router(const RouterArgs& a, hipStream_t st);
// K parts of the router logits (partial sums [kparts][T][E] in the logits scratch)
int router_kparts(int64_t T, int E, int H, bool bf16);
hipError_t launch_topk(const RouterArgs& a, hipStream_t st);

struct PermArgs {
  const int32_t* ids;  // [T][k]
  int T, k, E;
  int32_t* chunk_counts;  // [nchunk][E] scratch
  int32_t* chunk_base;    // [nchunk][E] scratch
  int32_t* offsets;       // [E+1]
  int32_t* sorted;        // [T*k] (+T identity rows when identity_tail)
  int32_t* inv;           // [T*k]
  bool identity_tail;
  // optional (tiles != nullptr, T <= kPermChunk): also build the work list of
  // the grouped GEMMs in the same single-block launch (see TileArgs)
  Tile* tiles;
  int32_t* tile_count;
  int bm, shared;
  int64_t cap;
};
// T <= kPermChunk: one single-block kernel (count, scan, stable scatter and,
// with `tiles`, the work list); else three kernels.  Returns whether the work
// list was built.
hipError_t launch_permute(const PermArgs& a, hipStream_t st, bool* tiles_built = nullptr);

struct TileArgs {
  const int32_t* offsets;  // [E+1]
  int T, k, E, bm;
  bool shared;             // append the shared group (rows T*k + t)
  int64_t cap;             // capacity of `tiles`
  Tile* tiles;
  int32_t* tile_count;
};
// upper bound on the number of tiles for T tokens (grid size of the GEMMs)
int64_t max_tiles(int64_t T, int k, int E, bool shared, int bm);
hipError_t launch_build_tiles(const TileArgs& a, hipStream_t st);

// gather rows: dst[p] = src[rows[p]] for p < min(n, *n_rows) (n_rows a device
// int), row_bytes per row (multiple of 16)
hipError_t launch_gather(const void* src, const int32_t* rows, int64_t n, const int32_t* n_rows,
                         int64_t row_bytes, void* dst, hipStream_t st);

// dynamic fp8 quantisation of bf16 / fp32 rows: codes [R][C] e4m3, scales [R][C/128]
hipError_t launch_act_quant(const uint16_t* src, int64_t R, int C, uint8_t* codes, float* scales,
                            hipStream_t st);
// the same for fp32 rows, in one launch over two row sets (R2 may be 0)
hipError_t launch_act_quant_f32(const float* src, int64_t R, int C, uint8_t* codes, float* scales,
                                const float* src2, int64_t R2, int C2, uint8_t* codes2, float* scales2,
                                hipStream_t st);

// grouped expert FFN
struct FfnArgs {
  int T, k, E, H, F, Fs;
  const Tile* tiles;
  const int32_t* tile_count;
  int64_t tile_bound;  // grid size along tiles
  int bm;              // rows per tile used to build `tiles`
  int kind;            // FfnPlan::Kind of the kernels to launch
  int ks_gu, ks_dn;    // K parts of the tiled gate_up / down (1: no split)
  bool w_once;         // tiled bf16: each expert expected in one tile (its weights read once)
  float* part;         // fp32 partial sums [ks][T*k + T][width] when a K part count > 1
  const int32_t* offsets;  // [E+1] (simple fp32 kernels)
  // weights (dtype per mode); routed [E][F][H] / [E][H][F], shared [Fs][H] / [H][Fs]
  const void *w_gate, *w_up, *w_down, *sh_gate, *sh_up, *sh_down;
  const float *s_gate, *s_up, *s_down, *sh_s_gate, *sh_s_up, *sh_s_down;
  // gate/up input rows: routed grouped row p reads xr[xr_rows ? xr_rows[p] : p],
  // shared row T*k+t reads xs[t]; fp8 carries per-128 scales alongside
  const void* xr;
  const float* xr_scales;
  const int32_t* xr_rows;
  const void* xs;
  const float* xs_scales;
  // fp8 tiled gate_up: workspace for the row scales of all grouped rows in
  // K-block-major order [H/128][T*k + T] (gathered by the gate_up launch), or
  // null
  float* xrs_t;
  // SwiGLU output: routed [T*k][F], shared [T][Fs] (act dtype; fp32 for fp8
  // weights, then quantised into hq / hq_sh codes with per-128 scales)
  void* h;
  void* h_sh;
  void* hq;            // fp8: [T*k][F] e4m3
  void* hq_sh;         // fp8: [T][Fs] e4m3
  float* h_scales;     // fp8: [T*k][F/128]
  float* h_sh_scales;  // fp8: [T][Fs/128]
  // down output: routed [T*k][H], shared [T][H] (act dtype)
  void* y;
  void* y_sh;
};
hipError_t launch_gate_up(const FfnArgs& a, int act_dtype, int weight_dtype, hipStream_t st);
hipError_t launch_down(const FfnArgs& a, int act_dtype, int weight_dtype, hipStream_t st);
struct FfnPlan {
  enum Kind { kSimple = 0, kStream = 1, kTiled = 2 };
  int bm;    // rows per work-list tile
  int kind;
  int ks_gu = 1, ks_dn = 1;  // K parts of the tiled bf16 kernels
  bool w_once = false;      // tiled bf16: nontemporal weight DMA (weights expected read once)
  // bytes of fp32 partial sums the K parts need (0 without a split)
  int64_t part_bytes(int64_t T, int k, int H, int F, int Fs) const {
    const int64_t R = T * k + T, Fm = F > Fs ? F : Fs;
    const int64_t a = ks_gu > 1 ? ks_gu * R * 2 * Fm : 0, b = ks_dn > 1 ? ks_dn * R * H : 0;
    return 4 * (a > b ? a : b);
  }
};
FfnPlan ffn_plan(const FfnArgs& a, int weight_dtype, int act_dtype);
bool tile_shapes_ok(int64_t T, int H, int F, int Fs);
// per-kernel-family launchers (ffn_stream.hip, ffn_fp8.hip)
hipError_t launch_gate_up_stream(const FfnArgs& a, hipStream_t st);
hipError_t launch_down_stream(const FfnArgs& a, hipStream_t st);
hipError_t launch_simple_f32(const FfnArgs& a, bool gate_up, hipStream_t st);
hipError_t launch_gate_up_fp8(const FfnArgs& a, hipStream_t st);
hipError_t launch_down_fp8(const FfnArgs& a, hipStream_t st);
hipError_t launch_gate_up_tile(const FfnArgs& a, hipStream_t st);  // ffn_tile.hip
hipError_t launch_down_tile(const FfnArgs& a, hipStream_t st);
int tile_rows();
int tile_ksplit(int64_t blocks, int K1, int K2, int max_ks, int target, bool one_round);

// pre-MoE RMSNorm, fp64, rounded once to the activation dtype into u [T][H];
// with `codes` (bf16 only) also the fp8 quantisation of u (codes [T][H],
// scales [T][H/128]); H a multiple of 128
hipError_t launch_rmsnorm(const void* x, const void* g, double eps, int64_t T, int H, bool bf16, void* u,
                          uint8_t* codes, float* scales, hipStream_t st);

struct CombineArgs {
  const void* y;
  const void* y_sh;
  const float* w;
  const int32_t* inv;
  int T, k, H;
  void* out;
  const void* resid;   // nullable: residual stream added first (act dtype)
};
hipError_t launch_combine(const CombineArgs& a, bool bf16, hipStream_t st);

}  // namespace moe

namespace moe {
// ffn_tile_fp8.hip
hipError_t launch_gate_up_tile_fp8(const FfnArgs& a, hipStream_t st);
hipError_t launch_down_tile_fp8(const FfnArgs& a, hipStream_t st);
int tile_fp8_rows();
bool tile_fp8_shapes_ok(int64_t T, int k, int H, int F, int Fs);
}  // namespace moe
