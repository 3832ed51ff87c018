// Paged latent-cache tile loader (bhfrc.com/news/60867 S3: a page is 64 consecutive tokens
// stored contiguously; a token row is [c_KV | k_R] in bf16).
//
// A tile is ROWS consecutive token rows of one page (ROWS divides 64), so it is one contiguous
// block of ROWS*ROWB bytes in global memory. It is copied to LDS with direct global->LDS loads:
// one wave instruction moves 64 lanes x 16 bytes into one contiguous KiB of LDS, and each lane
// picks its own global source, which is how the LDS copy gets its layout:
//   LDS byte offset of 16-byte chunk ch of row r = r*ROWB + 16*swz(r, ch),
//   swz(r, ch) = ch ^ (r & 7) for ch < SWZ (the whole groups of 8 chunks), ch otherwise.
// The XOR spreads the same chunk of eight consecutive rows over eight different bank groups,
// so column reads down a tile (the score MFMA operand) and 4-row transposing reads (the value
// MFMA operand) do not pile onto one bank.
// Rows at or past `valid` (cache slots past the end of the sequence) are loaded from row
// valid-1 instead: they hold finite data and their softmax weight is forced to zero.
#pragma once
#include "device.h"

namespace mla {

template <int ROWS, int ROWB>
struct PagedTile {
  static constexpr int NCH = ROWB / 16;   // 16-byte chunks per token row
  static constexpr int SWZ = NCH & ~7;    // chunks inside the XOR swizzle
  static constexpr int BYTES = ROWS * ROWB;
  static constexpr int INSTR = BYTES / 1024;
  static_assert(ROWB % 16 == 0 && BYTES % 1024 == 0, "tile must be whole KiB of 16B chunks");
  static_assert(kPage % ROWS == 0, "tile rows must divide the page");

  __device__ static __forceinline__ uint32_t lds_off(int r, int ch) {
    const int s = ch < SWZ ? (ch ^ (r & 7)) : ch;
    return (uint32_t)(r * ROWB + s * 16);
  }

  // Global address of the tile holding logical sub-tile j (ROWS tokens) of a sequence.
  __device__ static __forceinline__ const char* tile_base(const char* kv,
                                                          const int32_t* page_row, int j,
                                                          int num_pages) {
    constexpr int TPP = kPage / ROWS;  // tiles per page
    int page = ld_uniform(page_row + j / TPP);
    page = page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
    return kv + (size_t)page * (kPage * ROWB) + (size_t)(j % TPP) * BYTES;
  }

  // Issue this wave's share of the tile: instructions i0 + k*STEP for k < INSTR/STEP.
  template <int STEP>
  __device__ static __forceinline__ void issue(const char* base, int valid, MLA_LDS char* lds,
                                               int i0, int lane) {
    static_assert(INSTR % STEP == 0, "instructions must split evenly");
#pragma unroll
    for (int k = 0; k < INSTR / STEP; ++k) {
      const int i = i0 + k * STEP;
      const int q = i * 64 + lane;
      const int r = q / NCH, s = q - r * NCH;
      const int ch = s < SWZ ? (s ^ (r & 7)) : s;  // logical chunk kept at LDS position s
      const int rr = r < valid ? r : valid - 1;
      load_lds_16(base + rr * ROWB + ch * 16, lds + i * 1024);
    }
  }
};

}  // namespace mla
