// Logical copy of the paged cache through the attention kernels' own tile loader: each work
// group stages one tile with PagedTile::issue (page-table lookup, clamping, direct
// global->LDS loads, swizzled layout), then reads it back with PagedTile::lds_off and writes
// dst[b][t] = token t of sequence b (zero for t >= S_b). A bit-exact check of the page loads.
#include "device.h"
#include "kernels.h"
#include "paged_tile.h"

namespace mla {

template <int ROWS, int ROWB>
__global__ void __launch_bounds__(64)
gather_kernel(const char* __restrict__ kv, const int32_t* __restrict__ page_table,
              const int32_t* __restrict__ seq_lens, int B, int max_pages, int num_pages,
              int S_max, char* __restrict__ dst) {
  using Tile = PagedTile<ROWS, ROWB>;
  __shared__ __attribute__((aligned(1024))) char lds[Tile::BYTES];
  MLA_LDS char* tl = (MLA_LDS char*)lds;
  const int lane = threadIdx.x;
  const int tiles = (S_max + ROWS - 1) / ROWS;
  const int b = blockIdx.x / tiles, j = blockIdx.x % tiles;
  const int S = clamp_len(seq_lens[b], max_pages);
  const int valid = min(ROWS, S - j * ROWS);
  if (valid > 0) {
    const char* base = Tile::tile_base(kv, page_table + (size_t)b * max_pages, j, num_pages);
    uint32_t offs[Tile::INSTR];
#pragma unroll
    for (int k = 0; k < Tile::INSTR; ++k) offs[k] = Tile::src_off(k, lane, ROWS);
    Tile::template issue<1>(base, valid, offs, tl, 0, lane);
    wait_vmcnt<0>();
  }
  __syncthreads();
  for (int q = lane; q < ROWS * Tile::NCH; q += 64) {
    const int r = q / Tile::NCH, ch = q % Tile::NCH;
    const int t = j * ROWS + r;
    if (t >= S_max) continue;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < valid) v = *reinterpret_cast<const MLA_LDS u32x4*>(tl + Tile::lds_off(r, ch));
    *reinterpret_cast<u32x4*>(dst + ((size_t)b * S_max + t) * ROWB + ch * 16) = v;
  }
}

hipError_t launch_gather(int d_latent, int d_rope, const void* kv, const int32_t* page_table,
                         const int32_t* seq_lens, int B, int max_pages, int num_pages, int S_max,
                         void* dst, hipStream_t stream) {
  if (d_latent == 512 && d_rope == 64) {
    constexpr int ROWS = kSub;  // the DeepSeek attention tile
    const int tiles = (S_max + ROWS - 1) / ROWS;
    gather_kernel<ROWS, 1152><<<B * tiles, 64, 0, stream>>>(
        (const char*)kv, page_table, seq_lens, B, max_pages, num_pages, S_max, (char*)dst);
  } else {
    constexpr int ROWS = kPage;  // the MHA2MLA attention tile
    const int tiles = (S_max + ROWS - 1) / ROWS;
    gather_kernel<ROWS, 144><<<B * tiles, 64, 0, stream>>>(
        (const char*)kv, page_table, seq_lens, B, max_pages, num_pages, S_max, (char*)dst);
  }
  return hipGetLastError();
}

}  // namespace mla
