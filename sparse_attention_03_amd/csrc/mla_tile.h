// mla_tile.h -- the latent-row tiles of the sparse MLA kernels (gfx950):
// sizes, the line-block LDS layout and the HBM -> LDS gather of one tile of
// 32 selected latent rows.  Shared by the attention (sparse_mla.hip) and its
// backward (mla_backward.hip).
#pragma once
#include "dsa_common.h"

namespace dsa {
namespace mla {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRowBytes = kDqk * 2;        // 1152
constexpr int kChunksPerRow = kRowBytes / 16;  // 72
constexpr int kTile = 32;                  // selected entries per tile
constexpr int kTileBytes = kTile * kRowBytes;  // 36864
constexpr int kNumBuf = 4;                 // LDS tile buffers (147456 bytes)
constexpr int kMaxSel = 2048;              // selected entries staged in LDS per row
constexpr int kQkAhead = 3;                // K fragment steps read ahead of their MFMAs
constexpr int kPvAhead = 8;                // V^T fragments read ahead of their MFMAs
constexpr int kQkSteps = kDqk / 32;        // 18
constexpr int kDvTiles = kDv / 16;         // 32
constexpr int kMaxSplits = 256;            // key splits of one row (the merge's weight buffer)
constexpr float kSumLimit = 0x1p60f;       // per-lane row sums beyond this trigger the recompute

// Tile layout in LDS: line blocks.  The tile (32 rows x 72 chunks of 16 bytes)
// is 36 blocks of 1 KB; block 4 s + rg holds segment s (chunks 8 s .. 8 s + 7,
// one 128-byte line of each latent row) of tile rows 8 rg .. 8 rg + 7.  Rows 2k
// and 2k + 1 of a block share its 256-byte bank row k, and chunk 8 s + x of row
// r sits in 16-byte slot 8 (r & 1) + (x ^ tile_swz(r)) of it.  Properties:
//   * every 8 lanes of a copy instruction read one whole 128-byte line of one
//     latent row (a row's chunks permuted inside the line), so the gather
//     touches each line of a tile once;
//   * a lane copies from one latent row for the whole tile (one address per
//     lane and row group, immediate offsets after);
//   * a transposed V read (8 rows x 2 chunks per 32 lanes) covers each bank
//     once;
//   * the 16 rows of one chunk in a K fragment read sit in 16 different
//     slots, but lane groups 0 and 1 (2 and 3) read different chunks of the
//     same rows, which the LDS serves in two passes.  Line-sized gathers are
//     worth far more than that pass.
constexpr int kSegments = kChunksPerRow / 8;  // 9 lines per latent row
__device__ __forceinline__ int tile_swz(int r) { return 2 * ((r >> 1) & 3) + ((r >> 3) & 1); }
__device__ __forceinline__ int tile_off(int r, int ch) {
  return ((ch >> 3) * 4 + (r >> 3)) * 1024 + ((r & 7) >> 1) * 256 + (8 * (r & 1) + ((ch & 7) ^ tile_swz(r))) * 16;
}

__device__ __forceinline__ uint16_t to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;  // round to nearest even
  return __builtin_bit_cast(uint16_t, b);
}

// Issue the HBM -> LDS copy of tile t (the latent rows of selected entries
// 32 t .. 32 t + 31): 36 lane-contiguous 1-KB copy instructions, one per block.
// Wave w copies the row groups rg = w, w + NW, ... (all nine segments of each);
// lane l copies tile row 8 rg + l / 8.  Invalid entries (-1) copy row 0 of the
// sequence, always in bounds, and are masked later.
template <int NW>
constexpr int row_groups_per_wave() { return 4 / NW; }

// Tile row copied by this lane for its k-th row group.
__device__ __forceinline__ int gather_row(int wave, int NW, int k, int lane) { return 8 * (wave + NW * k) + (lane >> 3); }

// Lines [SG0, SG1) of each latent row of the tile (a kernel that reads only
// some columns fetches only their lines; the layout is the whole tile's).
// p[k]: selected position of this lane's tile row for row group k.
template <int NW, int SG0, int SG1>
__device__ __forceinline__ void gather_lines(const uint8_t* kv, int32_t kbase, const int32_t (&p)[4 / NW],
                                             uint8_t* buf) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < row_groups_per_wave<NW>(); ++k) {
    const int rg = wave + NW * k;
    const int x = (lane & 7) ^ tile_swz(8 * rg + (lane >> 3));  // chunk of the line this lane copies
    const int32_t pk = p[k] < 0 ? 0 : p[k];
    const uint8_t* src = kv + ((int64_t)(kbase + pk) * kChunksPerRow + x) * 16;
#pragma unroll
    for (int sg = SG0; sg < SG1; ++sg)
      copy16_to_lds(src + 128 * sg, (DSA_LDS uint8_t*)buf + 1024 * (4 * sg + rg));
  }
}

// The whole tile: every line of every row.
template <int NW>
__device__ __forceinline__ void gather_tile(const uint8_t* kv, int32_t kbase, const int32_t (&p)[4 / NW],
                                            uint8_t* buf) {
  gather_lines<NW, 0, kSegments>(kv, kbase, p, buf);
}

// The row's selected positions in LDS, -1 padded to whole tiles
// (sel[0 .. 32 ntiles)), and per tile the mask of its valid entries
// (tmask[t] bit j: entry 32 t + j is >= 0).  Every load of the wave is issued
// before the first is used (range-checked buffer loads: entries past k read
// nothing and become -1), so staging the row costs one load latency rather
// than one per 64 entries.
template <int NW>
__device__ __forceinline__ void stage_selection(const int32_t* idx_row, int32_t k, int ntiles, DSA_LDS int32_t* sel,
                                                DSA_LDS uint32_t* tmask) {
  constexpr int kIters = kMaxSel / (NW * 64);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const auto rs = __builtin_amdgcn_make_buffer_rsrc((void*)idx_row, 0, (uint32_t)k * 4u, 0x00020000);
  int32_t v[kIters];
#pragma unroll
  for (int it = 0; it < kIters; ++it)
    v[it] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)((it * NW + wave) * 64 + lane) * 4u, 0, 0);
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int base = (it * NW + wave) * 64;
    if (base < ntiles * kTile) {
      const int e = base + lane;
      const bool in = e < ntiles * kTile;
      const int32_t x = e < k ? v[it] : -1;
      if (in) sel[e] = x;
      const uint64_t m = __ballot(in && x >= 0);
      if (lane == 0) {
        tmask[base / kTile] = (uint32_t)m;
        tmask[base / kTile + 1] = (uint32_t)(m >> 32);
      }
    }
  }
}

}  // namespace mla
}  // namespace dsa
