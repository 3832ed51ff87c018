// Cache append: the latent and the decoupled RoPE key of new tokens, written into their page
// slots (lpnh.cn/news/2494972 S2.1: c_kv = x W_dkv, and a RoPE key that is not decompressed;
// bhfrc.com/news/60867 S1 cache format [c_KV | k_R], S3 RoPE computed in fp32, 64-token pages).
//
// For every new token (sequence b, i-th of its T new tokens, position p = S_b + i):
//   c_KV[c] = sum_k x[k] W_DKV[c][k]                        (W_DKV [d_latent, hidden])
//   k[j]    = sum_k x[k] W_KR[j][k]                         (W_KR  [d_rope, hidden])
//   (k[j], k[j + d_rope/2]) rotated by p * base^(-2j/d_rope) (pairs of the two halves)
// stored at slot p % 64 of page page_table[b][p / 64]: as bf16, or (FP8 cache) c_KV as E4M3
// codes with a power-of-two scale per token and k_R as bf16, or (MXFP4 cache, the OCP
// Microscaling format) c_KV as E2M1 codes with an E8M0 scale per block of 32 elements and k_R
// as bf16.
//
// The product is a skinny GEMM (B*T token rows against d_latent + d_rope weight rows over the
// model width) bound by reading the weights once. It runs split over the contraction:
//   partial: one work group per (32 output columns, slice of the width, 16, 32 or 64 token
//     rows): four waves, each a quarter of every 256-wide step of the slice, 16x16x32 bf16
//     MFMA (A = the weight rows, B = the token rows); all loads of a step in flight at once
//     and the next step's issued before the current one's MFMAs. The waves' sums meet in LDS
//     and the work group's fp32 partial goes to the workspace [slice][token][column].
//   finish: one work group of 1024 threads per token: up to 8 threads per 16-byte column quad,
//     each summing up to 8 slices in registers (all loads in flight at once), the threads' sums
//     added in a fixed order through LDS, the RoPE pairs rotated (angle in fp64: an fp32
//     product p * inv_freq would carry an error of up to 2^-8 rad at p near 65536; rotation in
//     fp32), and the row written. For the FP8 cache the
//     token's scale is the smallest power of two 2^e with max|c_KV| <= 448 * 2^e (448: the
//     largest E4M3 value), and each element is c_KV / 2^e rounded to nearest even E4M3. For
//     the MXFP4 cache each block's scale is 2^X, X = floor(log2 max|c_KV|) - 2 over the block,
//     and each element is c_KV / 2^X rounded to nearest even E2M1, saturating at 6.
#include <math.h>

#include <algorithm>

#include "device.h"
#include "kernels.h"

namespace mla {

namespace app {
constexpr int NT = 256;    // threads per work group
constexpr int CB = 32;     // partial: output columns per work group
constexpr int STEP = 256;  // partial: contraction per step (64 per wave)
constexpr int FT = 1024;   // finish: threads per work group
constexpr int FG = 8;      // finish: most threads that sum one column quad
constexpr int FK = 8;      // finish: most slices one thread sums
constexpr float kFp8Max = 448.f;
}  // namespace app

// W rows of the output columns: c < d_c from W_DKV, then W_KR.
__device__ __forceinline__ const uint16_t* append_wrow(const uint16_t* W_DKV,
                                                       const uint16_t* W_KR, int c, int d_c,
                                                       int hidden) {
  return c < d_c ? W_DKV + (size_t)c * hidden : W_KR + (size_t)(c - d_c) * hidden;
}

// Grid: x = 32-column block, y = contraction slice, z = block of 16 * RB token rows (each wave
// carries all RB 16-row blocks, so a weight fragment loaded once serves 16 * RB tokens).
template <int RB>
__global__ void __launch_bounds__(app::NT)
append_partial_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ W_DKV,
                      const uint16_t* __restrict__ W_KR, float* __restrict__ part, int R,
                      int hidden, int d_c, int d_R, int slice) {
  using namespace app;
  __shared__ float red[4][2][RB][4][64];  // [wave][column block][row block][element][lane]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = d_c + d_R;
  const int c0 = CB * blockIdx.x, ks = blockIdx.y, r0 = 16 * RB * blockIdx.z;
  const int q16 = lane & 15, G16 = lane >> 4;
  // A operand rows (two 16-column blocks) and B operand rows (RB 16-row blocks), clamped into
  // range (results of clamped rows and columns are dropped)
  const uint16_t* wr[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int c = min(c0 + 16 * cb + q16, N - 1);
    wr[cb] = append_wrow(W_DKV, W_KR, c, d_c, hidden);
  }
  const uint16_t* xr[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) xr[rb] = x + (size_t)min(r0 + 16 * rb + q16, R - 1) * hidden;
  const int kbase = ks * slice + 64 * wave + 8 * G16;
  const int nstep = slice / STEP;
  bf16x8 a[2][2], b[2][RB];  // [k half][column block], [k half][row block]
  auto load = [&](int s) {
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int k = kbase + STEP * s + 32 * kh;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) a[kh][cb] = *reinterpret_cast<const bf16x8*>(wr[cb] + k);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) b[kh][rb] = *reinterpret_cast<const bf16x8*>(xr[rb] + k);
    }
  };
  f32x4 acc[2][RB];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[cb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  load(0);
  for (int s = 0; s < nstep; ++s) {
    bf16x8 ca[2][2], cx[2][RB];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      ca[kh][0] = a[kh][0];
      ca[kh][1] = a[kh][1];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) cx[kh][rb] = b[kh][rb];
    }
    if (s + 1 < nstep) load(s + 1);  // the next step's loads fly during these MFMAs
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          acc[cb][rb] = mfma_16x16x32(ca[kh][cb], cx[kh][rb], acc[cb][rb]);
  }
  // lane holds tokens r0 + 16rb + q16 and columns c0 + 16cb + 4G16 + e
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[wave][cb][rb][e][lane] = acc[cb][rb][e];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2 * RB; ++j) {
    const int v = tid + NT * j;           // (token t, column c) of the work group's 16RB x 32
    const int t = v >> 5, c = v & 31;
    const int rb = t >> 4, tl = t & 15;   // row block and row inside it
    const int cb = c >> 4, cl = c & 15;   // column block and column inside it
    const int ln = (cl >> 2) * 16 + tl, e = cl & 3;
    const float sum = red[0][cb][rb][e][ln] + red[1][cb][rb][e][ln] + red[2][cb][rb][e][ln] +
                      red[3][cb][rb][e][ln];
    if (r0 + t < R && c0 + c < N) part[((size_t)ks * R + r0 + t) * N + c0 + c] = sum;
  }
}

// One work group per token row r (sequence r / T, new token r % T).
template <int FMT>
__global__ void __launch_bounds__(app::FT)
append_finish_kernel(const float* __restrict__ part, int nslice,
                     const int32_t* __restrict__ page_table,
                     const int32_t* __restrict__ seq_lens, char* __restrict__ kv,
                     void* __restrict__ kv_scales, int R, int T, int d_c, int d_R,
                     int max_pages, int num_pages, double log2_base) {
  using namespace app;
  constexpr bool FP8 = FMT == kKvFp8, MX = FMT == kKvMxfp4;
  __shared__ __attribute__((aligned(16))) float red[4 * FT];  // [group][column]
  __shared__ float wmax[FT / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.x;
  const int N = d_c + d_R, NQ = N >> 2;
  // thread (group g, quad q) sums the 16-byte column quad q (N is a multiple of 4) over slices
  // g, g + G, g + 2G, ... (at most FK of them). Every load is issued before the first is used:
  // loads past the thread's slices, or of a thread with no task, are clamped onto a valid
  // address and their values dropped by a select (predicated loads come out as one branch and
  // one wait each).
  const int G = min(FG, FT / NQ);
  const int g = tid / NQ, q = tid - g * NQ;
  const bool task = g < G;
  const float4* src = reinterpret_cast<const float4*>(part);
  float4 ld[FK];
#pragma unroll
  for (int j = 0; j < FK; ++j) {
    const int k = g + G * j;
    const int kk = task && k < nslice ? k : nslice - 1;
    ld[j] = src[((size_t)kk * R + r) * NQ + (task ? q : 0)];
  }
  // the token's slot (looked up while the loads are in flight)
  const int b = r / T, i = r - b * T;
  const int pos = clamp_len(seq_lens[b], max_pages) + i;
  // a token whose position is past its page-table row, or whose page-table entry names no pool
  // page (say -1, a page not allocated yet), is not written: a clamped write would overwrite
  // another sequence's cached token
  const int page = pos < max_pages * kPage ? page_table[(size_t)b * max_pages + pos / kPage] : -1;
  const bool write = page >= 0 && page < num_pages;  // the same for the whole work group
  const size_t slot = (size_t)(write ? page : 0) * kPage + pos % kPage;
  // the angle of the RoPE pair this thread rotates if tid < d_R/2 (also while the loads are in
  // flight): p * base^(-2j/d_R) in fp64 (an fp32 product would carry an error of up to 2^-8
  // rad at p near 65536), its cosine and sine rounded to fp32
  const int h = d_R / 2;
  float cs = 0.f, sn = 0.f;
  if (tid < h) {
    const double theta = (double)pos * exp2(-(2.0 * tid / d_R) * log2_base);
    double sd, cd;
    sincos(theta, &sd, &cd);
    cs = (float)cd;
    sn = (float)sd;
  }
  float4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < FK; ++j) {
    const bool in = g + G * j < nslice;
    acc.x += in ? ld[j].x : 0.f;
    acc.y += in ? ld[j].y : 0.f;
    acc.z += in ? ld[j].z : 0.f;
    acc.w += in ? ld[j].w : 0.f;
  }
  if (task) reinterpret_cast<float4*>(red)[g * NQ + q] = acc;  // red[g][4q .. 4q + 3]
  __syncthreads();
  // column c's sum: the groups' sums in group order (colsum2: columns c, c + 1, c even)
  auto colsum = [&](int c) {
    float s = 0.f;
#pragma unroll
    for (int gg = 0; gg < FG; ++gg) {
      const float u = red[min(gg, G - 1) * N + c];  // read unconditionally, dropped by a select
      s += gg < G ? u : 0.f;
    }
    return s;
  };
  auto colsum2 = [&](int c) {
    float2 s = {0.f, 0.f};
#pragma unroll
    for (int gg = 0; gg < FG; ++gg) {
      const float2 u = *reinterpret_cast<const float2*>(red + min(gg, G - 1) * N + c);
      s.x += gg < G ? u.x : 0.f;
      s.y += gg < G ? u.y : 0.f;
    }
    return s;
  };
  // RoPE pairs: thread j < d_R/2 rotates (k[j], k[j + d_R/2]) in fp32
  if (tid < h) {
    const float k1 = colsum(d_c + tid), k2 = colsum(d_c + tid + h);
    const float o1 = k1 * cs - k2 * sn, o2 = k1 * sn + k2 * cs;
    if (write) {
      uint16_t* kr = FP8  ? reinterpret_cast<uint16_t*>(kv + slot * (d_c + 2 * d_R) + d_c)
                     : MX ? reinterpret_cast<uint16_t*>(kv + slot * (d_c / 2 + 2 * d_R) + d_c / 2)
                          : reinterpret_cast<uint16_t*>(kv) + slot * N + d_c;
      kr[tid] = bf16_bits((__bf16)o1);
      kr[tid + h] = bf16_bits((__bf16)o2);
    }
  }
  // latent: thread t < d_latent/2 holds columns 2t, 2t + 1
  const int c = 2 * tid;
  const bool mine = c < d_c;
  const float2 vv = colsum2(mine ? c : 0);
  const float v0 = mine ? vv.x : 0.f, v1 = mine ? vv.y : 0.f;
  if constexpr (MX) {
    // OCP MX, per block of 32 latent elements (16 consecutive lanes): the shared exponent
    // X = floor(log2 amax) - 2 (2: the exponent of E2M1's largest value, 6), within -127 .. 127,
    // 0 for an all-zero block; with amax = m * 2^k (0.5 <= m < 1), floor(log2 amax) = k - 1
    float amax = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
    int X = 0;
    if (amax > 0.f) {
      int k;
      frexpf(amax, &k);
      X = k - 3;
      X = X < -127 ? -127 : (X > 127 ? 127 : X);
    }
    const float inv = ldexpf(1.f, -X);  // exact: c_KV / 2^X (X <= 125 for a finite fp32 amax)
    // E2M1 code of c_KV / 2^X: the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6, ties to the even
    // code (a midpoint goes up exactly when the upper neighbour's mantissa bit is 0), above 6
    // saturating; the sign in bit 3 unless the magnitude rounds to 0
    auto code = [inv](float v) -> uint32_t {
      const float a = fabsf(v) * inv;
      const uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                         (uint32_t)(a > 5.f);
      return m | (v < 0.f && m != 0u ? 8u : 0u);
    };
    if (write && mine) {
      unsigned char* row = reinterpret_cast<unsigned char*>(kv + slot * (d_c / 2 + 2 * d_R));
      row[tid] = (unsigned char)(code(v0) | (code(v1) << 4));  // columns 2 tid, 2 tid + 1
      if ((c & 31) == 0)
        reinterpret_cast<unsigned char*>(kv_scales)[slot * (d_c / 32) + c / 32] =
            (unsigned char)(X + 127);
    }
  } else if constexpr (!FP8) {
    if (write && mine)
      *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(kv) + slot * N + c) =
          pack_bf16x2(v0, v1);
  } else {
    // the token's amax, then its scale 2^e: the smallest e with amax <= 448 * 2^e. With
    // amax = m * 2^k (0.5 <= m < 1) and 448 = 0.875 * 2^9, that is e = k - 9 if m <= 0.875,
    // else k - 8 (exact, no rounding), kept within the normal powers of two 2^-126 .. 2^127
    float amax = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
    if (lane == 0) wmax[wave] = amax;
    __syncthreads();
    amax = 0.f;
#pragma unroll
    for (int w = 0; w < FT / 64; ++w) amax = fmaxf(amax, wmax[w]);
    int e = 0;
    if (amax > 0.f) {
      int k;
      const float m = frexpf(amax, &k);
      e = m <= 0.875f ? k - 9 : k - 8;
      e = e < -126 ? -126 : (e > 127 ? 127 : e);
    }
    const float inv = ldexpf(1.f, -e);  // exact: c_KV / 2^e
    if (write) {
      unsigned char* row = reinterpret_cast<unsigned char*>(kv + slot * (d_c + 2 * d_R));
      if (mine) {
        // round to nearest even E4M3 (|value| <= 448 by the choice of e)
        const int w = __builtin_amdgcn_cvt_pk_fp8_f32(v0 * inv, v1 * inv, 0, false);
        *reinterpret_cast<uint16_t*>(row + c) = (uint16_t)(w & 0xFFFF);
      }
      if (tid == 0) reinterpret_cast<float*>(kv_scales)[slot] = ldexpf(1.f, e);
    }
  }
}

// 16-row token blocks per partial work group: one up to 64 token rows (where the grid needs
// the work groups more than fewer weight reads), then more rows per block as the token count
// grows, so that the weights are read fewer times
static int append_row_blocks(int R) { return R <= 64 ? 1 : (R <= 128 ? 2 : 4); }

int append_slices(int R, int hidden, int d_c, int d_R) {
  // as many contraction slices (a divisor of hidden / 256) as keep the partial grid within
  // 1024 work groups and within what the finishing work group sums (G threads per column
  // quad, FK slices each); at least one (d_latent + d_rope <= 1536: N / 4 <= FT)
  const int steps = hidden / app::STEP;
  const int N = d_c + d_R;
  const int G = std::min(app::FG, app::FT / (N / 4));
  const int TB = 16 * append_row_blocks(R);
  const int blocks = ((N + app::CB - 1) / app::CB) * ((R + TB - 1) / TB);
  int best = 1;
  for (int s = 1; s <= steps; ++s)
    if (steps % s == 0 && (long long)blocks * s <= 1024 && s <= G * app::FK) best = s;
  return best;
}

size_t append_workspace_bytes(int R, int hidden, int d_c, int d_R) {
  return (size_t)append_slices(R, hidden, d_c, d_R) * R * (d_c + d_R) * sizeof(float);
}

hipError_t launch_append(const void* x, const void* W_DKV, const void* W_KR,
                         const int32_t* page_table, const int32_t* seq_lens, void* kv,
                         void* kv_scales, int kv_format, void* workspace, int B, int T,
                         int hidden, int d_c, int d_R, int max_pages, int num_pages,
                         double rope_base, hipStream_t stream) {
  const int R = B * T;
  const int S = append_slices(R, hidden, d_c, d_R);
  const int N = d_c + d_R;
  float* part = (float*)workspace;
  const int RB = append_row_blocks(R);
  auto partial = [&](auto kernel) {
    return launch_kernel(kernel,
                         dim3((N + app::CB - 1) / app::CB, S, (R + 16 * RB - 1) / (16 * RB)),
                         dim3(app::NT), Launch{stream}, (const uint16_t*)x,
                         (const uint16_t*)W_DKV, (const uint16_t*)W_KR, part, R, hidden, d_c,
                         d_R, hidden / S);
  };
  hipError_t e = RB == 1   ? partial(append_partial_kernel<1>)
                 : RB == 2 ? partial(append_partial_kernel<2>)
                           : partial(append_partial_kernel<4>);
  if (e != hipSuccess) return e;
  auto fin = [&](auto kernel) {
    return launch_kernel(kernel, dim3(R), dim3(app::FT), Launch{stream}, (const float*)part, S,
                         page_table, seq_lens, (char*)kv, kv_scales, R, T, d_c, d_R, max_pages,
                         num_pages, log2(rope_base));
  };
  if (kv_format == kKvFp8) return fin(append_finish_kernel<kKvFp8>);
  if (kv_format == kKvMxfp4) return fin(append_finish_kernel<kKvMxfp4>);
  return fin(append_finish_kernel<kKvBf16>);
}

}  // namespace mla
