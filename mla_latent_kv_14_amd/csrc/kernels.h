// Host-side launch entry points of the gfx950 kernels (implemented in the .hip files).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Where a kernel goes: the stream, and optionally two events that the runtime binds to the
// kernel's own start and end (hipExtLaunchKernel), so that their elapsed time is the kernel's
// execution alone, without the launch gap before it.
struct Launch {
  hipStream_t stream;
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

template <typename F, typename... Args>
hipError_t launch_kernel(F kernel, dim3 grid, dim3 block, const Launch& L, Args... args) {
  if (L.start || L.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, L.stream, L.start, L.stop, 0, args...);
  else
    kernel<<<grid, block, 0, L.stream>>>(args...);
  return hipGetLastError();
}

// The two head/width families the kernels are built for.
enum Shape : int {
  kShapeDeepSeek = 0,  // H=128, d_nope=128, d_latent=512, d_rope=64, d_v=128
  kShapeMha2Mla = 1,   // H=32,  d_nope=120, d_latent=64,  d_rope=8,  d_v=128
};

// MHA2MLA attention: waves per work group; each wave is one plan unit. (DeepSeek widths: one
// plan unit is served by two work groups, one per half of the heads.)
constexpr int kAttnWavesMha2Mla = 4;
// FP8 cache (MHA2MLA widths): ring depth of the attention kernel, and its work groups per CU
// (the same for the MXFP4 cache)
constexpr int kRingFp8 = 3;
constexpr int kGroupsPerCuFp8 = 2;

// Latent-cache formats: bf16 rows; FP8 E4M3 c_KV with an fp32 power-of-two scale per token;
// MXFP4 c_KV (E2M1 codes, two per byte) with an E8M0 scale byte per token and 32-element block.
enum KvFormat : int { kKvBf16 = 0, kKvFp8 = 1, kKvMxfp4 = 2 };

// B counts virtual sequences (sequences x query tokens, q_len per sequence) in the three
// decode launches; seq_lens and page_table stay per sequence.
hipError_t launch_absorb(int shape, const void* q_nope, const void* W_UK, void* q_abs, int B,
                         int H, const int32_t* seq_lens, const int32_t* page_table, int max_pages,
                         int q_len, int G, void* plan, const Launch& L);

hipError_t launch_attention(int shape, const void* q_abs, const void* q_rope, const void* kv,
                            const int32_t* page_table, const int32_t* seq_lens, int B,
                            int max_pages, int q_len, int num_pages, const void* plan, int G,
                            float scale_log2, void* part_o, float* part_lse,
                            const void* kv_scales, int kv_format, const Launch& L);

// The decompressed branch for T query tokens per sequence at or above the prefill threshold:
// W_UV transposed into W_UVt [H][d_v][d_c], then per group of `group` sequences the
// decompression of their cached tokens into kbuf [group][smax][H][d_nope] and vbuf
// [group][smax][H][d_v], and causal attention over them into out [B][T][H][d_v] and lse.
hipError_t launch_prefill(int shape, const void* q_nope, const void* q_rope, const void* W_UK,
                          const void* W_UV, const void* kv, const int32_t* page_table,
                          const int32_t* seq_lens, int B, int T, int max_pages, int num_pages,
                          int smax, int group, float scale_log2, void* W_UVt, void* kbuf,
                          void* vbuf, void* out, float* lse_out, const Launch& L);

hipError_t launch_combine(int shape, const void* part_o, const float* part_lse, const void* plan,
                          const int32_t* seq_lens, const void* W_UV, void* out, float* lse_out,
                          int B, int H, int max_pages, const Launch& L);

// The combine kernel's latent-output mode: merged latent rows o_lat bf16 [B][H][d_latent]
// (B virtual sequences), no up-projection.
hipError_t launch_combine_latent(int shape, const void* part_o, const float* part_lse,
                                 const void* plan, void* o_lat, float* lse_out, int B, int H,
                                 const Launch& L);

// out bf16 [R][N] = x bf16 [R][K] * W bf16 [N][K]^T. Needs K % 1024 == 0 and N % 16 == 0.
hipError_t launch_linear(const void* x, const void* W, void* out, int R, int K, int N,
                         const Launch& L);

// Sets bits of *flag (cleared first) for out-of-range lengths (1), used page ids (2) or used
// scales outside the format's contract (4): with an FP8 cache a scale that is not a positive
// normal power of two, with an MXFP4 cache a scale byte of 255 (E8M0's NaN); mx_blocks is
// d_latent / 32.
hipError_t launch_check(const int32_t* seq_lens, const int32_t* page_table, int B, int max_pages,
                        int num_pages, int max_len, const void* kv_scales, int kv_format,
                        int mx_blocks, int* flag, hipStream_t stream);

// Writes [c_KV | RoPE(k_R)] of B*T new tokens (token i of sequence b at position
// seq_lens[b] + i) in the cache format kv_format: bf16 rows; an FP8 cache (E4M3 c_KV, bf16
// k_R, an fp32 power-of-two scale per token); or an MXFP4 cache (E2M1 c_KV two per byte, bf16
// k_R, an E8M0 scale byte per token and block of 32, d_c a multiple of 32). Needs d_c even and
// at most 1024, d_R even and at most 512, hidden % 256 == 0, and a workspace of
// append_workspace_bytes.
hipError_t launch_append(const void* x, const void* W_DKV, const void* W_KR,
                         const int32_t* page_table, const int32_t* seq_lens, void* kv,
                         void* kv_scales, int kv_format, void* workspace, int B, int T,
                         int hidden, int d_c, int d_R, int max_pages, int num_pages,
                         double rope_base, hipStream_t stream);
// Workspace of launch_append: fp32 partial rows of the split contraction.
size_t append_workspace_bytes(int R, int hidden, int d_c, int d_R);

hipError_t launch_gather(int d_latent, int d_rope, const void* kv, const int32_t* page_table,
                         const int32_t* seq_lens, int B, int max_pages, int num_pages, int S_max,
                         void* dst, hipStream_t stream);

}  // namespace mla
