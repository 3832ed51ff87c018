// Paged latent-cache tile loader (bhfrc.com/news/60867 S3: a page is 64 consecutive tokens
// stored contiguously; a token row is [c_KV | k_R] in bf16).
//
// A tile is ROWS consecutive token rows of one page (ROWS divides 64), so it is one contiguous
// block of ROWS*ROWB bytes in global memory. It is copied to LDS with direct global->LDS loads:
// one wave instruction moves 64 lanes x 16 bytes into one contiguous KiB of LDS, and each lane
// picks its own global source, which is how the LDS copy gets its layout:
//   LDS byte offset of 16-byte chunk ch of row r = r*ROWB + 16*s,
//   s = (ch & ~7) | ((ch & 7) ^ swz(r)) inside the whole groups of 8 chunks, s = ch past them.
// The row swizzle swz(r) is chosen per row width from measured LDS costs on gfx950:
//   1152-byte rows (DeepSeek widths): swz(r) = (r >> 1) & 7. Both reads of the attention
//     kernel run at the conflict-free rate with it: the score operand of 16x16x32 MFMA
//     (rows 16t..16t+15 x 4 consecutive chunks, 16 bytes per lane) and the transposing 8-byte
//     reads of the value operand.
//   other widths: m = (r >> 1) & 7, swz = ((m & 3) << 1) | (m >> 2).
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

  __device__ static __forceinline__ int swz(int r) {
    const int m = (r >> 1) & 7;
    if constexpr (ROWB == 1152) return m;
    else return ((m & 3) << 1) | (m >> 2);
  }
  // Position of logical chunk ch of row r (and, the XOR being an involution, the logical chunk
  // kept at position ch).
  __device__ static __forceinline__ int chunk_pos(int r, int ch) {
    return ch < SWZ ? (ch ^ swz(r)) : ch;
  }
  __device__ static __forceinline__ uint32_t lds_off(int r, int ch) {
    return (uint32_t)(r * ROWB + chunk_pos(r, ch) * 16);
  }

  static constexpr int TPP = kPage / ROWS;  // tiles per page

  // Page-table entry of logical sub-tile j (ROWS tokens) of a sequence (a scalar load; callers
  // that read it ahead of use hide its latency).
  __device__ static __forceinline__ int page_of(const int32_t* page_row, int j) {
    return ld_uniform(page_row + j / TPP);
  }
  // Global address of sub-tile j given its page-table entry, clamped into the pool.
  __device__ static __forceinline__ const char* base_of(const char* kv, int page, int j,
                                                        int num_pages) {
    page = page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
    return kv + (size_t)page * (kPage * ROWB) + (size_t)(j % TPP) * BYTES;
  }
  __device__ static __forceinline__ const char* tile_base(const char* kv,
                                                          const int32_t* page_row, int j,
                                                          int num_pages) {
    return base_of(kv, page_of(page_row, j), j, num_pages);
  }

  // Byte offset inside the tile that lane `lane` of load instruction i fetches.
  __device__ static __forceinline__ uint32_t src_off(int i, int lane, int valid) {
    const int q = i * 64 + lane;
    const int r = q / NCH, s = q - r * NCH;
    const int rr = r < valid ? r : valid - 1;
    return (uint32_t)(rr * ROWB + chunk_pos(r, s) * 16);
  }

  // Issue part of this wave's share of the tile: instructions i0 + k*STEP for KB <= k < KE.
  // Full tiles use the precomputed lane offsets `offs`; a tile with fewer valid rows computes
  // them.
  template <int STEP, int KB, int KE>
  __device__ static __forceinline__ void issue_part(const char* base, int valid,
                                                    const uint32_t* offs, MLA_LDS char* lds,
                                                    int i0, int lane) {
    static_assert(INSTR % STEP == 0 && 0 <= KB && KB <= KE && KE <= INSTR / STEP, "range");
    if (valid >= ROWS) {
#pragma unroll
      for (int k = KB; k < KE; ++k) load_lds_16(base, offs[k], lds + (i0 + k * STEP) * 1024);
    } else {
#pragma unroll
      for (int k = KB; k < KE; ++k)
        load_lds_16(base, src_off(i0 + k * STEP, lane, valid), lds + (i0 + k * STEP) * 1024);
    }
  }
  // Issue this wave's whole share of the tile: instructions i0 + k*STEP for k < INSTR/STEP.
  template <int STEP>
  __device__ static __forceinline__ void issue(const char* base, int valid, const uint32_t* offs,
                                               MLA_LDS char* lds, int i0, int lane) {
    issue_part<STEP, 0, INSTR / STEP>(base, valid, offs, lds, i0, lane);
  }
};

}  // namespace mla
