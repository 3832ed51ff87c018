// Cache append: the latent and the decoupled RoPE key of new tokens, written into their page
// slots (lpnh.cn/news/2494972 S2.1: c_kv = x W_dkv, and a RoPE key that is not decompressed;
// bhfrc.com/news/60867 S1 cache format [c_KV | k_R], S3 RoPE computed in fp32, 64-token pages).
//
// For every new token (sequence b, i-th of its T new tokens, position p = S_b + i):
//   c_KV[c] = sum_k x[k] W_DKV[c][k]                        (W_DKV [d_latent, hidden])
//   k[j]    = sum_k x[k] W_KR[j][k]                         (W_KR  [d_rope, hidden])
//   (k[j], k[j + d_rope/2]) rotated by p * base^(-2j/d_rope) (pairs of the two halves)
// rounded to bf16 and stored at slot p % 64 of page page_table[b][p / 64].
//
// One work group per block of 4 output columns (144 work groups at the DeepSeek widths) and
// eight waves; wave w sums the hidden slice [w * hidden/8, (w+1) * hidden/8) on 16x16x32 bf16
// MFMA (A = the block's weight rows, each repeated four times to fill the MFMA's 16 rows;
// B = up to 64 token rows in four blocks), four contraction steps' loads in flight at once.
// The waves' partial sums meet in LDS, and four waves finish 16 token rows each. The RoPE
// columns are grouped so that both elements of a rotated pair sit in one block and in one
// lane: block q of the RoPE part holds pairs j = 2q, 2q+1 as columns 0, 1 (first elements) and
// 2, 3 (second elements). The rotation angle is formed in fp64 (an fp32 product p * inv_freq
// would carry an error of up to 2^-8 rad at p near 65536); the rotation itself is fp32.
#include <math.h>

#include "device.h"
#include "kernels.h"

namespace mla {

namespace app {
constexpr int NW = 8;     // waves per work group
constexpr int CB = 4;     // output columns per work group
constexpr int ROWS = 64;  // token rows per pass (four MFMA blocks of 16)
constexpr int U = 4;      // contraction steps whose loads are issued together
}  // namespace app

__global__ void __launch_bounds__(64 * app::NW)
append_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ W_DKV,
              const uint16_t* __restrict__ W_KR, const int32_t* __restrict__ page_table,
              const int32_t* __restrict__ seq_lens, uint16_t* __restrict__ kv, int B, int T,
              int hidden, int d_c, int d_R, int max_pages, int num_pages, double log2_base) {
  using namespace app;
  __shared__ __attribute__((aligned(16))) float red[NW][4][4][64];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int R = B * T;
  const int W = d_c + d_R;              // elements per cached token
  const int lat_blocks = d_c / CB;
  const int cb = blockIdx.x;
  const bool rope = cb >= lat_blocks;
  const int q = cb - lat_blocks;        // RoPE block: pairs 2q, 2q+1
  // output column of local column c, and its weight row
  auto column = [&](int c) -> int {
    if (!rope) return CB * cb + c;
    return d_c + 2 * q + (c & 1) + (c >= 2 ? d_R / 2 : 0);
  };
  auto weight_row = [&](int c) -> const uint16_t* {
    const int col = column(c);
    return col < d_c ? W_DKV + (size_t)col * hidden : W_KR + (size_t)(col - d_c) * hidden;
  };
  const int G16 = lane >> 4, q16 = lane & 15;
  const uint16_t* wrow = weight_row(q16 % CB);  // A operand row (MFMA rows 4..15 repeat 0..3)
  const int ksw = hidden / 32 / NW;             // 32-wide steps per wave (a multiple of U)
  const int k0 = wave * ksw * 32 + 8 * G16;

  for (int r0 = 0; r0 < R; r0 += ROWS) {
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc[4] = {zero4, zero4, zero4, zero4};
    const uint16_t* xrow[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int r = r0 + 16 * m + q16;
      xrow[m] = x + (size_t)(r < R ? r : R - 1) * hidden;  // rows past R: a valid row, dropped
    }
    for (int s0 = 0; s0 < ksw; s0 += U) {
      bf16x8 a[U], bx[U][4];
#pragma unroll
      for (int u = 0; u < U; ++u) a[u] = *reinterpret_cast<const bf16x8*>(wrow + k0 + 32 * (s0 + u));
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          if (r0 + 16 * m < R)
            bx[u][m] = *reinterpret_cast<const bf16x8*>(xrow[m] + k0 + 32 * (s0 + u));
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          if (r0 + 16 * m < R) acc[m] = mfma_16x16x32(a[u], bx[u][m], acc[m]);
    }
    // partial sums of the waves meet in LDS; wave m < 4 finishes token rows 16m .. 16m+15
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[wave][m][e][lane] = acc[m][e];
    __syncthreads();
    if (wave < 4 && G16 == 0) {  // lanes 0..15 hold MFMA rows 0..3, the block's 4 columns
      const int m = wave;
      const int r = r0 + 16 * m + q16;  // token row of this lane
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) t += red[w][m][e][lane];
        v[e] = t;  // local column e
      }
      const int b = r < R ? r / T : 0, i = r < R ? r - (r / T) * T : 0;
      const int pos = clamp_len(seq_lens[b], max_pages) + i;
      if (rope) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {  // pair j = 2q + e: (v[e], v[e + 2])
          const int j = 2 * q + e;
          const double theta = (double)pos * exp2(-(2.0 * j / d_R) * log2_base);
          const float cs = (float)cos(theta), sn = (float)sin(theta);
          const float x1 = v[e], x2 = v[e + 2];
          v[e] = x1 * cs - x2 * sn;
          v[e + 2] = x1 * sn + x2 * cs;
        }
      }
      // a token whose position is past its page-table row, or whose page-table entry names
      // no pool page (say -1, a page not allocated yet), is not written: a clamped write would
      // overwrite another sequence's cached token
      const int page = r < R && pos < max_pages * kPage
                           ? page_table[(size_t)b * max_pages + pos / kPage]
                           : -1;
      if (page >= 0 && page < num_pages) {
        uint16_t* dst = kv + ((size_t)page * kPage + pos % kPage) * W;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[column(e)] = bf16_bits((__bf16)v[e]);
      }
    }
    __syncthreads();
  }
}

hipError_t launch_append(const void* x, const void* W_DKV, const void* W_KR,
                         const int32_t* page_table, const int32_t* seq_lens, void* kv, int B,
                         int T, int hidden, int d_c, int d_R, int max_pages, int num_pages,
                         double rope_base, hipStream_t stream) {
  const int blocks = d_c / app::CB + d_R / 4;
  return launch_kernel(append_kernel, dim3(blocks), dim3(64 * app::NW), Launch{stream},
                       (const uint16_t*)x, (const uint16_t*)W_DKV, (const uint16_t*)W_KR,
                       page_table, seq_lens, (uint16_t*)kv, B, T, hidden, d_c, d_R, max_pages,
                       num_pages, log2(rope_base));
}

}  // namespace mla
