// Grouped expert FFN, tiled schedule for many rows per expert (the
// compute-bound prefill regime: "prefill is compute-bound" -- "Behind
// Kimi-K2's Config", section 2.1, Prefill bullet).
//
// Expert form ("Kimi K2 . Down projection"): y = W_down (silu(W_gate a) *
// (W_up a)), weights [out][in].
//
// Work item = up to 128 grouped rows of one expert (a tile of the work list)
// x one slab of 512 weight rows, computed transposed (C[weight row][row])
// with 32x32x16 bf16 MFMA.  Each wave owns 128 weight rows x all 128 rows,
// its 128 x 128 accumulator tile filling the AGPR file:
//  * gate_up: a wave's 128 weight rows are 64 gate + 64 up rows of the same
//    64 features, so SiLU * up is applied on matching accumulators;
//  * down: a wave owns 128 output rows.
// Both operands go global -> LDS by DMA (global_load_lds_dwordx4, no VGPR
// staging, issued from inline asm with explicit waits), 64 K-elements (128 B
// per row) per step, in two stages that fill the whole 160 KB LDS: per stage
// the 512 weight rows as 16 m-tiles of 32 rows (4 per wave: each wave DMAs
// and reads only its own 128 weight rows) and the 128 grouped rows.  Each DMA
// source is a wave-uniform base in scalar registers plus a 32-bit lane
// offset (the instruction's SADDR form).  Rows are unpadded; 16-byte slot =
// chunk ^ ((row >> 1) & 7), because with 128-byte rows the 64 banks give bank
// group 8*(row%2) + slot and a 128-bit read serves 16 lanes per cycle, so any
// 16 consecutive rows land in distinct groups.  The grouped rows are gathered
// by the DMA itself through the row -> token map.
// A K step consumes the weights m-tile by m-tile (4 sub-steps of 16 K each,
// the step's token fragments read during m-tile 0 and kept in registers),
// and each freed m-tile slot takes the data of step s + 2 at once, so a
// weight batch has 1.25 - 1.75 steps to land instead of under one; the token
// stage of step s + 2 is refilled after the one barrier per step (after
// m-tile 0, when every wave has read its token fragments).  Measured on the
// prefill's routing (136 experts, 65,536 rows, standalone gate_up): 890 -
// 897 TFLOP/s against 835 - 845 with both operands refilled a step ahead
// (the dense 8192 x 4096 x 7168 shape, whose operands stay in L2, went from
// 992 - 999 to 937 - 946).
//
// XCD-aware order: workgroups are dealt round-robin to the 8 XCDs.  The
// (slab, tile) pairs are numbered slab-major and cut into 8 contiguous
// ranges, range i going to the blocks that land on XCD i, so the tiles that
// share a weight slab run on one XCD and reuse its L2, for any slab count.
#include <type_traits>

#include "kernels.h"

namespace moe {

namespace {

constexpr int kBM = 128;                      // grouped rows per work item
constexpr int kBW = 512;                      // weight rows per slab
constexpr int kBK = 64;                       // K elements per step
constexpr int kRowB = 128;                    // bytes per LDS row (kBK bf16)
constexpr int kXcd = 8;

__device__ __forceinline__ f32x16 mma32(const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}
}  // namespace

// MODE 0: gate_up (K = H, slab = 256 features = 256 gate + 256 up rows)
// MODE 1: down    (K = F or Fs, slab = 512 output rows)
// `ks` > 1 splits the K loop over ks blocks (few work items): each writes its
// fp32 partial sums to a.part, and ffn_split_finish adds them up in part
// order and applies the epilogue.
// The body of one block's work item (K part kp of slab `slab` of tile tl).
// WNT: the weight DMA carries the nontemporal hint.  The LDS stages are the
// kernel's (one allocation for both copies of this body that it inlines).
template <int MODE, bool WNT>
__device__ __forceinline__ void tile_bf16_body(const FfnArgs& a, int ks, int kp, int slab, const Tile& tl,
                                               uint8_t (&wst)[2][4][4 * 32 * kRowB],
                                               uint8_t (&tst)[2][kBM * kRowB]) {
  const bool sh = tl.group == a.E;
  const int Fg = sh ? a.Fs : a.F;
  const int64_t TK = static_cast<int64_t>(a.T) * a.k;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, kh = lane >> 5;
  // DMA lane geometry: one wave instruction fills 8 LDS rows (1 KB); lane ->
  // row (lane >> 3) of that group, slot (lane & 7), which must hold global
  // chunk slot ^ f(row); f changes by 4 between even and odd 8-row groups
  const int drow = lane >> 3;
  const int dch[2] = {(lane & 7) ^ ((drow >> 1) & 7), (lane & 7) ^ ((4 + (drow >> 1)) & 7)};
  // DMA sources: wave-uniform bases plus 32-bit lane byte offsets

  // ---- weight rows of this wave: two 64-row halves ----
  int K, o0;
  const uint8_t* wsb[2];
  if (MODE == 0) {
    K = a.H;
    o0 = slab * (kBW / 2);
    if (o0 >= Fg) return;
    const int64_t wofs = sh ? 0 : static_cast<int64_t>(tl.group) * a.F * a.H;
    const uint16_t* wg = static_cast<const uint16_t*>(sh ? a.sh_gate : a.w_gate) + wofs;
    const uint16_t* wu = static_cast<const uint16_t*>(sh ? a.sh_up : a.w_up) + wofs;
    const int64_t f = o0 + 64 * wave;
    wsb[0] = reinterpret_cast<const uint8_t*>(wg + f * K);
    wsb[1] = reinterpret_cast<const uint8_t*>(wu + f * K);
  } else {
    K = Fg;
    o0 = slab * kBW;
    const int64_t wofs = sh ? 0 : static_cast<int64_t>(tl.group) * a.H * a.F;
    const uint16_t* wd = static_cast<const uint16_t*>(sh ? a.sh_down : a.w_down) + wofs;
    const int64_t r = o0 + 128 * wave;
    wsb[0] = reinterpret_cast<const uint8_t*>(wd + r * K);
    wsb[1] = reinterpret_cast<const uint8_t*>(wd + (r + 64) * K);
  }
  uint32_t woff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) woff[i] = static_cast<uint32_t>((8 * i + drow) * K * 2 + dch[i & 1] * 16);
  // ---- grouped rows of this wave's 4 DMA instructions (LDS rows 32w + 8i + drow) ----
  // contiguous rows (shared rows, ungathered routed rows, h) are offsets from
  // the tile's first row; gathered rows are offsets token * H * 2 from x
  // (under 2^32 bytes: tile_shapes_ok)
  const bool gather = MODE == 0 && !sh && a.xr_rows != nullptr;
  const int ld = MODE == 0 ? a.H : Fg;                          // row length, elements
  const int64_t row0 = sh ? tl.row0 - TK : tl.row0;
  const uint16_t* xbase = MODE == 0 ? static_cast<const uint16_t*>(sh ? a.xs : a.xr)
                                    : static_cast<const uint16_t*>(sh ? a.h_sh : a.h);
  const uint8_t* xsb = reinterpret_cast<const uint8_t*>(gather ? xbase : xbase + row0 * ld);
  uint32_t xoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tr = min(32 * wave + 8 * i + drow, tl.rows - 1);
    const int64_t r = gather ? a.xr_rows[tl.row0 + tr] : tr;
    xoff[i] = static_cast<uint32_t>(r) * static_cast<uint32_t>(ld * 2) + dch[i & 1] * 16;
  }

  // DMA from inline asm (the compiler neither tracks it nor waits for it:
  // every wait is an explicit s_waitcnt below), SADDR form: wave-uniform
  // 64-bit base in SGPRs + 32-bit lane offset; LDS destinations as byte
  // addresses from the two LDS bases (taken once)
  const uint32_t wlds = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)(&wst[0][0][0])));
  const uint32_t tlds = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)(&tst[0][0])));
  // (readfirstlane returns int: each half goes through uint32_t, or the low
  // word would sign-extend into the high one)
  auto sbase = [](const uint8_t* base) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32)));
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b)));
    return (static_cast<uint64_t>(hi) << 32) | lo;
  };
  const uint64_t wsb_s[2] = {sbase(wsb[0]), sbase(wsb[1])};
  const uint64_t xsb_s = sbase(xsb);
  auto dma_asm = [&](uint64_t bu, uint32_t voff, uint32_t lds, auto nt_tag) {
    const uint32_t m0v = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(lds));
    if (decltype(nt_tag)::value)
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(m0v), "v"(voff), "s"(bu) : "memory", "m0");
    else
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0v), "v"(voff), "s"(bu) : "memory", "m0");
  };
  // weight m-tile m (this wave's rows 32 m + [0, 32): 4 instructions of 8
  // rows) of K step s into stage stg: wst[stg][m] starts at (4 stg + m) * 16 KB
  auto dma_w = [&](int m, int s, int stg) {
    const uint32_t ko = static_cast<uint32_t>(s) * kRowB;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dma_asm(wsb_s[m >> 1], woff[4 * (m & 1) + j] + ko,
              wlds + (4 * stg + m) * (4 * 32 * kRowB) + (32 * wave + 8 * j) * kRowB,
              std::integral_constant<bool, WNT>{});
  };
  // this wave's 32 of the 128 token rows of K step s into stage stg
  auto dma_t = [&](int s, int stg) {
    const uint32_t ko = static_cast<uint32_t>(s) * kRowB;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dma_asm(xsb_s, xoff[i] + ko, tlds + stg * (kBM * kRowB) + (32 * wave + 8 * i) * kRowB,
              std::integral_constant<bool, false>{});
  };

  // this block's K steps [s0, s0 + steps): part kp of ks parts of `kper`
  // steps (even), the last part shorter; every part is non-empty
  // (tile_ksplit) and even, since K / 64 is even
  const int ksteps = K / kBK, kper = ((ksteps + ks - 1) / ks + 1) & ~1;
  const int s0 = kp * kper, steps = min(kper, ksteps - s0);
  const int sw = (r32 >> 1) & 7;                       // row swizzle of this lane's rows
  const int arow = (32 * wave + r32) * kRowB;        // in wst[stg][m]
  const int brow = r32 * kRowB;                      // in tst[stg]

  // The K loop and the epilogue for NN active 32-row groups of grouped rows
  // (NN = ceil(rows / 32)): a work list's last tile of an expert is usually
  // partly filled, and its MFMAs and fragment reads on groups past the last
  // row are skipped (block-uniform: every wave covers all the tile's rows).
  auto run = [&](auto nn_tag) {
    constexpr int NN = decltype(nn_tag)::value;
    f32x16 acc[4][NN];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < NN; ++n)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[m][n][i] = 0.f;

    auto slot = [&](int i) { return ((kh * 4 + i) ^ sw) * 16; };
    // One K step s on stage STG.  Per wave, DMAs go out in the order T(s+2),
    // W(s+2, 0..3) (tokens, then weight m-tiles) every step, so the waits are
    // constants.  Weights are consumed m-tile by m-tile and each freed m-tile
    // slot takes the data of step s + 2 at once; the step's token fragments
    // are read during m-tile 0 and kept in registers.  The first fragments
    // of step s + 1 (tokens, landed at this step's barrier; m-tile 0, which
    // has 28 later DMAs at that point) are read during m-tile 3.
    uint4 nb[NN], na;   // step s's first fragments, read during step s - 1
    auto step = [&](auto stg_tag, int s) {
      constexpr int STG = decltype(stg_tag)::value;
      const int sn = s0 + min(s + 2, steps - 1);   // past the end: re-load the last step (never read)
      const uint8_t* tk = tst[STG];
      uint4 bf[4][NN], af[2];
#pragma unroll
      for (int n = 0; n < NN; ++n) bf[0][n] = nb[n];
      af[0] = na;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < 3) {
#pragma unroll
          for (int n = 0; n < NN; ++n)
            bf[i + 1][n] = *reinterpret_cast<const uint4*>(tk + brow + 32 * n * kRowB + slot(i + 1));
          af[(i + 1) & 1] = *reinterpret_cast<const uint4*>(wst[STG][0] + arow + slot(i + 1));
        }
#pragma unroll
        for (int n = 0; n < NN; ++n) acc[0][n] = mma32(af[i & 1], bf[i][n], acc[0][n]);
      }
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      dma_t(sn, STG);
      dma_w(0, sn, STG);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 1; m < 4; ++m) {
        if (m == 3) {
          // next step's first fragments: its tokens landed at the barrier
          // above; its m-tile 0 (W(s+1, 0)) has W(s+1, 1..3), T(s+2) and
          // W(s+2, 0..2) after it
          asm volatile("s_waitcnt vmcnt(28)" ::: "memory");
#pragma unroll
          for (int n = 0; n < NN; ++n)
            nb[n] = *reinterpret_cast<const uint4*>(tst[STG ^ 1] + brow + 32 * n * kRowB + slot(0));
          na = *reinterpret_cast<const uint4*>(wst[STG ^ 1][0] + arow + slot(0));
        }
        af[0] = *reinterpret_cast<const uint4*>(wst[STG][m] + arow + slot(0));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i < 3) af[(i + 1) & 1] = *reinterpret_cast<const uint4*>(wst[STG][m] + arow + slot(i + 1));
#pragma unroll
          for (int n = 0; n < NN; ++n) acc[m][n] = mma32(af[i & 1], bf[i][n], acc[m][n]);
        }
        // this wave's reads of m-tile m are done before its slot is refilled
        // (fenced, so no later fragment read is hoisted above the wait)
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        dma_w(m, sn, STG);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // prologue: steps 0 and 1 into stages 0 and 1 (order T, W0..W3 each),
    // then every wave's T(0) landed (36 later DMAs)
    dma_t(s0, 0);
#pragma unroll
    for (int m = 0; m < 4; ++m) dma_w(m, s0, 0);
    dma_t(s0 + min(1, steps - 1), 1);
#pragma unroll
    for (int m = 0; m < 4; ++m) dma_w(m, s0 + min(1, steps - 1), 1);
    asm volatile("s_waitcnt vmcnt(36)\n\ts_barrier" ::: "memory");
    // step 0's first fragments (W(0, 0) has 32 later DMAs)
    asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
#pragma unroll
    for (int n = 0; n < NN; ++n) nb[n] = *reinterpret_cast<const uint4*>(tst[0] + brow + 32 * n * kRowB + slot(0));
    na = *reinterpret_cast<const uint4*>(wst[0][0] + arow + slot(0));
    for (int s = 0; s < steps; s += 2) {
      step(std::integral_constant<int, 0>{}, s);
      step(std::integral_constant<int, 1>{}, s + 1);
    }
    // no DMA may still be writing LDS when the workgroup ends
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (ks > 1) {
      // ---- partial sums: row p of part kp holds gate | up (gate_up, width
      // 2 * max(F, Fs)) or the output row (down, width H), fp32 ----
      const int64_t R = TK + a.T;
      const int width = MODE == 0 ? 2 * max(a.F, a.Fs) : a.H;
#pragma unroll
      for (int n = 0; n < NN; ++n) {
        const int tr = 32 * n + r32;
        if (tr >= tl.rows) continue;
        float* dst = a.part + (static_cast<int64_t>(kp) * R + tl.row0 + tr) * width;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          // gate_up: m = 0, 1 gate features, 2, 3 the same features' up rows
          const int col = MODE == 0 ? (m >> 1) * (width / 2) + o0 + 64 * wave + 32 * (m & 1)
                                    : o0 + 128 * wave + 32 * m;
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<float4*>(dst + col + 8 * g + 4 * kh) =
                make_float4(acc[m][n][4 * g], acc[m][n][4 * g + 1], acc[m][n][4 * g + 2], acc[m][n][4 * g + 3]);
        }
      }
      return;
    }

    // ---- epilogue: lane holds rows 8*(i/4) + 4*kh + (i%4) of each 32-row
    // weight sub-tile, for grouped row 32*n + r32 ----
#pragma unroll
    for (int n = 0; n < NN; ++n) {
      const int tr = 32 * n + r32;
      if (tr >= tl.rows) continue;
      const int64_t p = tl.row0 + tr;
      if (MODE == 0) {
        uint16_t* dst = sh ? static_cast<uint16_t*>(a.h_sh) + (p - TK) * a.Fs
                           : static_cast<uint16_t*>(a.h) + p * a.F;
        dst += o0 + 64 * wave + 4 * kh;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = silu(acc[m][n][4 * g + e]) * acc[m + 2][n][4 * g + e];
            uint2 v2;
            v2.x = pack_bf16(h[0], h[1]);
            v2.y = pack_bf16(h[2], h[3]);
            *reinterpret_cast<uint2*>(dst + 32 * m + 8 * g) = v2;
          }
      } else {
        uint16_t* dst = sh ? static_cast<uint16_t*>(a.y_sh) + (p - TK) * a.H
                           : static_cast<uint16_t*>(a.y) + p * a.H;
        dst += o0 + 128 * wave + 4 * kh;
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            uint2 v2;
            v2.x = pack_bf16(acc[m][n][4 * g + 0], acc[m][n][4 * g + 1]);
            v2.y = pack_bf16(acc[m][n][4 * g + 2], acc[m][n][4 * g + 3]);
            *reinterpret_cast<uint2*>(dst + 32 * m + 8 * g) = v2;
          }
      }
    }
  };

  const int nn = (tl.rows + 31) >> 5;
  if (nn >= 4) run(std::integral_constant<int, 4>{});
  else if (nn == 3) run(std::integral_constant<int, 3>{});
  else if (nn == 2) run(std::integral_constant<int, 2>{});
  else run(std::integral_constant<int, 1>{});
}

// WNT: the weight DMA of routed tiles carries the nontemporal hint (each
// routed weight slab is expected to be read by one tile only); never that
// of the shared expert, whose slabs every token tile reads.  The block
// branches once, on its tile, between two inlined copies of the body.
template <int MODE, bool WNT>
__global__ __launch_bounds__(256) void ffn_tile_bf16(FfnArgs a, int slabs, int ks) {
  // two stages as separate objects: the compiler then knows that a DMA into
  // one stage does not alias LDS reads of the other
  // weights: [stage][m-tile][wave's 32 rows x 128 B]; tokens: [stage][128 rows x 128 B]
  __shared__ __attribute__((aligned(16))) uint8_t wst[2][4][4 * 32 * kRowB];
  __shared__ __attribute__((aligned(16))) uint8_t tst[2][kBM * kRowB];
  // ---- XCD-chunked mapping of this block to (K part, slab, tile) ----
  const int ntile = *a.tile_count;
  const int total = slabs * ntile * ks;
  const int per = (total + kXcd - 1) / kXcd;
  const int j = blockIdx.x / kXcd;
  const int v0 = (blockIdx.x % kXcd) * per + j;
  if (j >= per || v0 >= total) return;
  const int kp = v0 / (slabs * ntile);
  const int v = v0 - kp * (slabs * ntile);
  const int slab = v / ntile;
  const Tile tl = a.tiles[v - slab * ntile];
  // (without the hint one copy serves every tile)
  if (WNT && tl.group != a.E)
    tile_bf16_body<MODE, WNT>(a, ks, kp, slab, tl, wst, tst);
  else
    tile_bf16_body<MODE, false>(a, ks, kp, slab, tl, wst, tst);
}

// Sum of the K-part partials of each grouped row in part order, then the
// epilogue: SiLU(gate) * up to h (gate_up) or the output row to y (down).
// Block (x, y) = grouped row x, output columns [1024 y, 1024 (y + 1)) (one
// float4 per thread), so that the few rows of a split launch still give the
// chip many blocks; routed rows past offsets[E] (unused capacity) and rows of
// no group are skipped.
template <int MODE>
__global__ __launch_bounds__(256) void ffn_split_finish(FfnArgs a, int ks) {
  const int64_t p = blockIdx.x;
  const int64_t TK = static_cast<int64_t>(a.T) * a.k, R = TK + a.T;
  const bool sh = p >= TK;
  if (sh ? a.Fs == 0 : p >= a.offsets[a.E]) return;
  const int Fg = sh ? a.Fs : a.F;
  const int width = MODE == 0 ? 2 * max(a.F, a.Fs) : a.H;
  const int n4 = (MODE == 0 ? Fg : a.H) / 4;
  const int c = blockIdx.y * blockDim.x + threadIdx.x;
  if (c < n4) {
    float4 g = make_float4(0.f, 0.f, 0.f, 0.f), u = g;
    for (int kp = 0; kp < ks; ++kp) {
      const float* src = a.part + (static_cast<int64_t>(kp) * R + p) * width;
      const float4 x = reinterpret_cast<const float4*>(src)[c];
      g.x += x.x; g.y += x.y; g.z += x.z; g.w += x.w;
      if (MODE == 0) {
        const float4 y = reinterpret_cast<const float4*>(src + width / 2)[c];
        u.x += y.x; u.y += y.y; u.z += y.z; u.w += y.w;
      }
    }
    uint2 v2;
    if (MODE == 0) {
      v2.x = pack_bf16(silu(g.x) * u.x, silu(g.y) * u.y);
      v2.y = pack_bf16(silu(g.z) * u.z, silu(g.w) * u.w);
      uint16_t* dst = sh ? static_cast<uint16_t*>(a.h_sh) + (p - TK) * a.Fs : static_cast<uint16_t*>(a.h) + p * a.F;
      reinterpret_cast<uint2*>(dst)[c] = v2;
    } else {
      v2.x = pack_bf16(g.x, g.y);
      v2.y = pack_bf16(g.z, g.w);
      uint16_t* dst = sh ? static_cast<uint16_t*>(a.y_sh) + (p - TK) * a.H : static_cast<uint16_t*>(a.y) + p * a.H;
      reinterpret_cast<uint2*>(dst)[c] = v2;
    }
  }
}

int tile_rows() { return kBM; }

// K parts of the tiled kernels for a grid of `blocks` (slabs x work items).
// The kernel holds a whole CU's LDS, so 256 blocks make one round of the
// chip.
//  * one_round (gate_up), for a grid under one round of `target` blocks:
//    the fewest parts (any count: parts of an even number of 64-wide steps,
//    the last one shorter) for which the grid's last round is at least 80 %
//    full.  A half-empty last round costs a whole round; more parts cost
//    partial sums and shorter blocks.  Measured: one expert-parallel rank's
//    3 experts (80 blocks): 0.158 ms with 4 parts, 0.142 with 2, 0.120 with
//    3.  Grids past one round are not split: for 48 experts (392 blocks,
//    1.5 rounds) 3 parts gained nothing (0.578 ms against 0.581).
//  * otherwise (down, fp32 partial sums 7168 wide): doubled while the grid
//    has fewer than `target` blocks and every part keeps a multiple of 4
//    steps of both K1 and K2: the dense layer's 14 blocks gain up to 16 parts
//    (0.10 ms against 0.154 with 4), while at 140 blocks the extra pass cost
//    more than the split gained.
int tile_ksplit(int64_t blocks, int K1, int K2, int max_ks, int target, bool one_round) {
  if (one_round) {
    if (blocks >= target) return 1;
    // every part non-empty: (ks - 1) parts of per = ceil_even(steps / ks)
    // steps leave at least one step for the last
    auto valid = [](int K, int ks) {
      const int n = K / kBK, per = ((n + ks - 1) / ks + 1) & ~1;
      return (ks - 1) * per < n;
    };
    int best = 1;
    double best_fill = 0.0;
    for (int ks = 1; ks <= max_ks; ++ks) {
      if (!(valid(K1, ks) && valid(K2, ks))) break;
      const int64_t n = blocks * ks, rounds = (n + target - 1) / target;
      const double fill = static_cast<double>(n) / static_cast<double>(rounds * target);
      if (fill >= 0.8) return ks;
      if (fill > best_fill) {
        best_fill = fill;
        best = ks;
      }
    }
    return best;
  }
  int ks = 1;
  while (ks < max_ks && blocks * ks < target && (K1 / kBK) % (4 * ks) == 0 && (K2 / kBK) % (4 * ks) == 0) ks *= 2;
  return ks;
}

// slabs must divide the weight dimensions: F, Fs by 256, H by 512; the
// token-row DMA offsets (token * H * 2 bytes) must fit in 32 bits
bool tile_shapes_ok(int64_t T, int H, int F, int Fs) {
  return F % (kBW / 2) == 0 && Fs % (kBW / 2) == 0 && H % kBW == 0 && T * H * 2 <= 0xffffffffLL;
}

template <int MODE>
static hipError_t launch_tile(const FfnArgs& a, int slabs, int ks, hipStream_t st) {
  // a multiple of 8: block b serves item (b % 8) * per + b / 8 with
  // per = ceil(items / 8), which needs 8 * per blocks to reach every item
  const int64_t blocks = (static_cast<int64_t>(slabs) * a.tile_bound * ks + kXcd - 1) / kXcd * kXcd;
  if (a.w_once)
    hipLaunchKernelGGL((ffn_tile_bf16<MODE, true>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, a,
                       slabs, ks);
  else
    hipLaunchKernelGGL((ffn_tile_bf16<MODE, false>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, a,
                       slabs, ks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ks == 1) return e;
  const int64_t rows = static_cast<int64_t>(a.T) * a.k + a.T;
  const int cols4 = (MODE == 0 ? std::max(a.F, a.Fs) : a.H) / 4;
  hipLaunchKernelGGL((ffn_split_finish<MODE>), dim3(static_cast<unsigned>(rows), (cols4 + 255) / 256), dim3(256), 0,
                     st, a, ks);
  return hipGetLastError();
}

hipError_t launch_gate_up_tile(const FfnArgs& a, hipStream_t st) {
  return launch_tile<0>(a, std::max(a.F, a.Fs) / (kBW / 2), a.ks_gu, st);
}

hipError_t launch_down_tile(const FfnArgs& a, hipStream_t st) {
  return launch_tile<1>(a, a.H / kBW, a.ks_dn, st);
}

}  // namespace moe
