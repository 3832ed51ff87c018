// K3: merge the split partials of each sequence and up-project through W_UV.
//
//   lse_b      = ln sum_s exp(lse_s)                       over the segments s of sequence b
//   o_lat[c]   = sum_s exp(lse_s - lse_b) * o_s[c]         (fp32; o_s are normalised partials)
//   out[b,h,e] = sum_c o_lat[c] * W_UV[h,c,e]              (lpnh.cn/news/2494972 S2.1, v = c_kv W_uv)
//
// One work group per (head h, block of EB output columns). The W_UV block [d_latent x EB] is
// staged in LDS by direct loads (32-byte units XOR-swizzled by row); the merged latent rows of
// 16 sequences at a time go to LDS as bf16; then out^T[e, b] = W^T[e, c] * o_lat^T[c, b] runs on
// 16x16x32 bf16 MFMA with transposing reads for the W operand. A sequence with no tokens gets
// out = 0 and lse = -inf.
#include "device.h"
#include "kernels.h"

namespace mla {

template <int H, int DC, int DV, int EB>
__global__ void __launch_bounds__(256)
combine_kernel(const uint16_t* __restrict__ part_o, const float* __restrict__ part_lse,
               const Plan* __restrict__ plan, const int32_t* __restrict__ seq_lens,
               const uint16_t* __restrict__ W_UV, uint16_t* __restrict__ out,
               float* __restrict__ lse_out, int B, int max_pages) {
  constexpr int ROWB = EB * 2;        // LDS bytes per W row
  constexpr int UNITS = ROWB / 32;    // swizzle period (32-byte units per row)
  constexpr int NCHUNK = DC * ROWB / 16;
  constexpr int OPITCH = DC * 2 + 16; // bytes per merged latent row in LDS
  static_assert(NCHUNK % 64 == 0 && DC % 32 == 0 && EB == 64, "shape");
  __shared__ __attribute__((aligned(16))) char lds_w[DC * ROWB];
  __shared__ __attribute__((aligned(16))) char lds_o[16 * OPITCH];
  __shared__ float lds_lse[16];
  __shared__ int lds_first[16], lds_count[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nblk = DV / EB;
  const int h = blockIdx.x / nblk, eblk = blockIdx.x % nblk;
  MLA_LDS char* wl = (MLA_LDS char*)lds_w;
  MLA_LDS char* ol = (MLA_LDS char*)lds_o;

  // ---- stage W_UV[h][:, eblk*EB : +EB]
  const char* Wg = reinterpret_cast<const char*>(W_UV + (size_t)h * DC * DV + (size_t)eblk * EB);
  for (int k = wave; k < NCHUNK / 64; k += 4) {
    const int q = k * 64 + lane;
    const int row = q / (ROWB / 16), p = q % (ROWB / 16);
    const int lunit = (p >> 1) ^ (row % UNITS);
    load_lds_16(Wg, (uint32_t)(row * DV * 2 + lunit * 32 + (p & 1) * 16), wl + k * 1024);
  }

  const int total = plan->total, per = plan->per;
  const int32_t* off = plan_off(plan);
  const int G16 = lane >> 4, q16 = lane & 15;

  for (int b0 = 0; b0 < B; b0 += 16) {
    // ---- per-sequence slot range and merged lse
    if (tid < 16) {
      const int b = b0 + tid;
      int first = 0, count = 0;
      float L = -INFINITY;
      if (b < B) {
        const int nt = (b + 1 < B ? off[b + 1] : total) - off[b];
        if (nt > 0) {
          const int g0 = off[b] / per, g1 = (off[b] + nt - 1) / per;
          first = g0 + b;
          count = g1 - g0 + 1;
          float m = -INFINITY;
          for (int s = 0; s < count; ++s) m = fmaxf(m, part_lse[(size_t)(first + s) * H + h]);
          float z = 0.f;
          for (int s = 0; s < count; ++s) z += __expf(part_lse[(size_t)(first + s) * H + h] - m);
          L = m + __logf(z);
        }
      }
      lds_first[tid] = first;
      lds_count[tid] = count;
      lds_lse[tid] = L;
      if (b < B && eblk == 0 && lse_out) lse_out[(size_t)b * H + h] = L;
    }
    __syncthreads();
    // ---- merged latent rows, 8 columns per thread-item
    for (int item = tid; item < 16 * (DC / 8); item += 256) {
      const int bi = item / (DC / 8), c0 = (item % (DC / 8)) * 8;
      float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      const int count = lds_count[bi], first = lds_first[bi];
      const float L = lds_lse[bi];
      for (int s = 0; s < count; ++s) {
        const size_t slot = (size_t)(first + s);
        const float w = __expf(part_lse[slot * H + h] - L);
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(part_o + (slot * H + h) * DC + c0);
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] += w * (float)v[e];
      }
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (__bf16)a[e];
      *reinterpret_cast<MLA_LDS bf16x8*>(ol + bi * OPITCH + c0 * 2) = o;
    }
    wait_vmcnt<0>();  // W block (first pass only; later passes have nothing outstanding)
    __syncthreads();
    // ---- out^T[e][b] for this wave's 16 columns e
    {
      const int mb = wave;  // EB / 16 == 4 blocks of e
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int ks = 0; ks < DC / 32; ++ks) {
        const int row0 = ks * 32 + 8 * G16 + (q16 >> 2), row1 = row0 + 4;
        const bf16x4 a0 = lds_read_tr16(
            wl, row0 * ROWB + ((mb ^ (row0 % UNITS)) * 32) + 8 * (q16 & 3));
        const bf16x4 a1 = lds_read_tr16(
            wl, row1 * ROWB + ((mb ^ (row1 % UNITS)) * 32) + 8 * (q16 & 3));
        const bf16x8 bo = lds_read_b128(ol, q16 * OPITCH + (ks * 32 + 8 * G16) * 2);
        acc = mfma_16x16x32(cat4(a0, a1), bo, acc);
      }
      const int b = b0 + q16;
      if (b < B) {
        const int e0 = eblk * EB + mb * 16 + 4 * G16;
        bf16x4 o = {(__bf16)acc[0], (__bf16)acc[1], (__bf16)acc[2], (__bf16)acc[3]};
        *reinterpret_cast<bf16x4*>(out + ((size_t)b * H + h) * DV + e0) = o;
      }
    }
    __syncthreads();
  }
  (void)max_pages;
  (void)seq_lens;
}

hipError_t launch_combine(int shape, const void* part_o, const float* part_lse, const void* plan,
                          const int32_t* seq_lens, const void* W_UV, void* out, float* lse_out,
                          int B, int H, int max_pages, hipStream_t stream) {
  if (shape == kShapeDeepSeek) {
    combine_kernel<128, 512, 128, 64><<<H * 2, 256, 0, stream>>>(
        (const uint16_t*)part_o, part_lse, (const Plan*)plan, seq_lens, (const uint16_t*)W_UV,
        (uint16_t*)out, lse_out, B, max_pages);
  } else {
    combine_kernel<32, 64, 128, 64><<<H * 2, 256, 0, stream>>>(
        (const uint16_t*)part_o, part_lse, (const Plan*)plan, seq_lens, (const uint16_t*)W_UV,
        (uint16_t*)out, lse_out, B, max_pages);
  }
  return hipGetLastError();
}

}  // namespace mla
