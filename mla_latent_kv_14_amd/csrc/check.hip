// Validation of the device-resident inputs, run before the decode when MLA_CHECK=1 is set:
// every S_b must lie in [0, max_len] and every page-table entry that the sequence uses
// (logical pages j < ceil(S_b / 64)) must name a pool page in [0, num_pages); with an FP8 cache
// the scale of every slot a sequence uses (tokens t < S_b) must be a positive normal power of
// two, and with an MXFP4 cache none of its block scale bytes may be 255 (E8M0's NaN).
// Violations set bits of *flag (1: a length, 2: a page id, 4: a scale); the fast path itself
// only clamps lengths and page ids.
#include "device.h"
#include "kernels.h"

namespace mla {

__global__ void check_clear_kernel(int* flag) { *flag = 0; }

__global__ void __launch_bounds__(256)
check_inputs_kernel(const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ page_table,
                    int B, int max_pages, int num_pages, int max_len,
                    const void* __restrict__ kv_scales, int kv_format, int mx_blocks,
                    int* flag) {
  for (int b = blockIdx.x; b < B; b += gridDim.x) {
    const int S = seq_lens[b];
    if (S < 0 || S > max_len) {
      if (threadIdx.x == 0) atomicOr(flag, 1);
      continue;
    }
    const int np = (S + kPage - 1) / kPage;  // <= max_pages, as max_len <= max_pages * 64
    for (int j = threadIdx.x; j < np; j += blockDim.x) {
      const int p = page_table[(size_t)b * max_pages + j];
      if (p < 0 || p >= num_pages) atomicOr(flag, 2);
    }
    if (kv_format == kKvFp8) {
      // a positive normal power of two: sign and mantissa bits clear, exponent in 1..254
      const float* sc = reinterpret_cast<const float*>(kv_scales);
      for (int t = threadIdx.x; t < S; t += blockDim.x) {
        const int p = page_table[(size_t)b * max_pages + t / kPage];
        if (p < 0 || p >= num_pages) continue;  // reported above
        const uint32_t u = __builtin_bit_cast(uint32_t, sc[(size_t)p * kPage + t % kPage]);
        const uint32_t e = (u >> 23) & 0xFFu;
        if ((u & 0x807FFFFFu) != 0 || e == 0 || e == 0xFFu) atomicOr(flag, 4);
      }
    } else if (kv_format == kKvMxfp4) {
      const unsigned char* sc = reinterpret_cast<const unsigned char*>(kv_scales);
      for (int t = threadIdx.x; t < S; t += blockDim.x) {
        const int p = page_table[(size_t)b * max_pages + t / kPage];
        if (p < 0 || p >= num_pages) continue;  // reported above
        const unsigned char* row = sc + ((size_t)p * kPage + t % kPage) * mx_blocks;
        for (int k = 0; k < mx_blocks; ++k)
          if (row[k] == 0xFFu) atomicOr(flag, 4);
      }
    }
  }
}

hipError_t launch_check(const int32_t* seq_lens, const int32_t* page_table, int B, int max_pages,
                        int num_pages, int max_len, const void* kv_scales, int kv_format,
                        int mx_blocks, int* flag, hipStream_t stream) {
  check_clear_kernel<<<1, 1, 0, stream>>>(flag);
  const int blocks = B < 1024 ? B : 1024;
  check_inputs_kernel<<<blocks, 256, 0, stream>>>(seq_lens, page_table, B, max_pages, num_pages,
                                                   max_len, kv_scales, kv_format, mx_blocks,
                                                   flag);
  return hipGetLastError();
}

}  // namespace mla
