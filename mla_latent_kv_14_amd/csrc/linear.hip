// Output projection with a merged weight (lpnh.cn/news/2494972 S2.2: W_uv and W_o merged into
// one matrix offline): out[r][n] = sum_k o_lat[r][k] W_UVO[n][k], where row r is one decoded
// (sequence, query token), k runs over (head, latent column) = H * d_latent, and n over the
// model width. The merged latent rows o_lat come from the combine kernel's latent-output mode.
//
// A weight-streaming product with few rows: one work group per 16 output columns, eight waves
// splitting the contraction, 16x16x32 bf16 MFMA (A = the 16 weight rows, B = up to 64 latent
// rows), four steps' loads in flight at once, the waves' partial sums reduced in LDS, bf16 out.
#include "device.h"
#include "kernels.h"

namespace mla {

namespace lin {
constexpr int NW = 8;     // waves per work group
constexpr int ROWS = 64;  // latent rows per pass (four MFMA blocks of 16)
constexpr int U = 4;      // contraction steps whose loads are issued together
}  // namespace lin

__global__ void __launch_bounds__(64 * lin::NW)
linear_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ W,
              uint16_t* __restrict__ out, int R, int K, int N) {
  using namespace lin;
  __shared__ __attribute__((aligned(16))) float red[NW][4][4][64];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cb = blockIdx.x;  // output columns 16cb .. 16cb+15
  const int G16 = lane >> 4, q16 = lane & 15;
  const uint16_t* wrow = W + (size_t)(16 * cb + q16) * K;  // A operand: weight row of column q16
  const int ksw = K / 32 / NW;                               // 32-wide steps per wave
  const int k0 = wave * ksw * 32 + 8 * G16;

  for (int r0 = 0; r0 < R; r0 += ROWS) {
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc[4] = {zero4, zero4, zero4, zero4};
    const uint16_t* xrow[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int r = r0 + 16 * m + q16;
      xrow[m] = x + (size_t)(r < R ? r : R - 1) * K;  // rows past R: a valid row, dropped
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
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[wave][m][e][lane] = acc[m][e];
    __syncthreads();
    if (wave < 4) {  // wave m writes rows 16m .. 16m+15; lane: row q16, columns 4 G16 .. +3
      const int m = wave;
      const int r = r0 + 16 * m + q16;
      bf16x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) t += red[w][m][e][lane];
        o[e] = (__bf16)t;
      }
      if (r < R) *reinterpret_cast<bf16x4*>(out + (size_t)r * N + 16 * cb + 4 * G16) = o;
    }
    __syncthreads();
  }
}

hipError_t launch_linear(const void* x, const void* W, void* out, int R, int K, int N,
                         const Launch& L) {
  return launch_kernel(linear_kernel, dim3(N / 16), dim3(64 * lin::NW), L, (const uint16_t*)x,
                       (const uint16_t*)W, (uint16_t*)out, R, K, N);
}

}  // namespace mla
