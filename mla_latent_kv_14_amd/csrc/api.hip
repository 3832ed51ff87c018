// C ABI of libmla_decode.so: argument checks, workspace layout, work plan size and the
// launches on the caller's stream: absorb -> attention -> combine for the absorbed branch, or
// transpose -> (decompress -> attention) per group of sequences for the decompressed one. No
// allocation, no sync.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "mla_decode.h"
#include "device.h"
#include "kernels.h"

namespace {

constexpr int kMaxQLen = 65536;         // query tokens per sequence
constexpr int kPrefillThreshold = 256;  // DeepSeek widths, default: decompressed from here on
// Bytes of decompressed keys and values the decompressed branch keeps for one group of
// sequences (at least one sequence, whatever its size). Measured at B = 16, S = 4096, T = 256
// (DeepSeek widths): one sequence per group (256 MiB) took 9.1 ms, four (1 GiB) 6.8 ms; the
// attention grid of a group needs several sequences to fill the chip.
constexpr size_t kPrefillGroupBytes = (size_t)1024 << 20;

thread_local char g_hip_err[256] = "";

struct ShapeInfo {
  int shape, H, DN, DC, DR, DV, TT;  // TT: tokens per plan tile
};

bool shape_of(const mla_dims_t* d, ShapeInfo* s) {
  if (d->num_heads == 128 && d->d_nope == 128 && d->d_latent == 512 && d->d_rope == 64 &&
      d->d_v == 128) {
    *s = {mla::kShapeDeepSeek, 128, 128, 512, 64, 128, mla::kSub};
    return true;
  }
  if (d->num_heads == 32 && d->d_nope == 120 && d->d_latent == 64 && d->d_rope == 8 &&
      d->d_v == 128) {
    *s = {mla::kShapeMha2Mla, 32, 120, 64, 8, 128, mla::kPage};
    return true;
  }
  return false;
}

// Validates the sizes; fills the shape on success.
mla_status_t check_dims(const mla_dims_t* d, ShapeInfo* s) {
  if (!d) return MLA_ERR_NULL_ARG;
  if (d->batch < 1 || d->batch > (1 << 20) || d->max_pages_per_seq < 1 || d->num_pages < 1 ||
      d->num_units < 0 || d->num_units > 65536 || d->num_heads < 1 || d->d_nope < 1 ||
      d->d_latent < 1 || d->d_rope < 1 || d->d_v < 1 || d->page_size < 1 || d->q_len < 0 ||
      d->q_len > kMaxQLen || (int64_t)d->batch * (d->q_len > 1 ? d->q_len : 1) > (1 << 20))
    return MLA_ERR_BAD_DIMS;
  if ((int64_t)d->batch * d->max_pages_per_seq > (int64_t)1 << 29) return MLA_ERR_BAD_DIMS;
  if ((int64_t)d->max_seq_len > (int64_t)d->max_pages_per_seq * d->page_size)
    return MLA_ERR_BAD_DIMS;
  if (d->page_size != mla::kPage) return MLA_ERR_UNSUPPORTED;
  if (d->prefill_threshold < 0) return MLA_ERR_BAD_DIMS;
  if (!shape_of(d, s)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

// The decompressed branch serves the call: query tokens per sequence at or above the
// threshold. By default 256 at the DeepSeek widths; never at the MHA2MLA widths, whose latent
// (64) is narrower than a head's key (d_nope + d_rope = 128), so that expanding the cache per
// head costs more work at every T than scoring in the latent space.
bool decompressed(const mla_dims_t* d) {
  const int T = d->q_len > 1 ? d->q_len : 1;
  if (d->prefill_threshold > 0) return T >= d->prefill_threshold;
  return d->num_heads == 128 && T >= kPrefillThreshold;
}

// Query tokens per sequence (0 in the dims means 1).
int q_len(const mla_dims_t* d) { return d->q_len > 1 ? d->q_len : 1; }

// Decoded rows: one per (sequence, query token), the kernels' virtual sequences.
int rows(const mla_dims_t* d) { return d->batch * q_len(d); }

int max_len(const mla_dims_t* d) {
  return d->max_seq_len > 0 ? d->max_seq_len : d->max_pages_per_seq * d->page_size;
}

// Plan units sharing the cache stream: tile streams served by two work groups (DeepSeek
// widths) or single waves (MHA2MLA). The automatic count fills 256 compute units (with the FP8
// cache two work groups fit on one); it is capped by the tiles that can exist so that no unit
// is sure to be idle.
int plan_units(const mla_dims_t* d, const ShapeInfo& s, bool fp8) {
  const int64_t upper = (int64_t)rows(d) * ((max_len(d) + s.TT - 1) / s.TT);
  int64_t g = d->num_units;
  if (g == 0)
    g = s.shape == mla::kShapeDeepSeek
            ? 128
            : 256 * mla::kAttnWavesMha2Mla * (fp8 ? mla::kGroupsPerCuFp8 : 1);
  if (g > upper) g = upper;
  return g < 1 ? 1 : (int)g;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// MLA_CHECK=1 in the environment: validate device-resident inputs before each decode.
bool check_mode() {
  const char* e = getenv("MLA_CHECK");
  return e && e[0] == '1' && e[1] == 0;
}

// MLA_LOG=1 in the environment: print each decode's work plan on stderr.
bool log_mode() {
  const char* e = getenv("MLA_LOG");
  return e && e[0] == '1' && e[1] == 0;
}

const char* format_name(int kv_format) {
  return kv_format == mla::kKvFp8 ? "fp8" : (kv_format == mla::kKvMxfp4 ? "mxfp4" : "bf16");
}


struct Layout {
  size_t plan, q_abs, part_lse, part_o, total;
};

// Workspace of the decompressed branch: the MLA_CHECK flag, W_UV transposed, and the
// decompressed keys and values of one group of sequences.
struct PrefillLayout {
  size_t flag, wuvt, kbuf, vbuf, total;
  int group;
};

PrefillLayout prefill_layout(const mla_dims_t* d, const ShapeInfo& s) {
  const size_t smax = (size_t)max_len(d);
  const size_t per_seq = smax * s.H * (s.DN + s.DV) * 2;
  size_t g = per_seq > 0 ? kPrefillGroupBytes / per_seq : 1;
  g = g < 1 ? 1 : (g > (size_t)d->batch ? (size_t)d->batch : g);
  PrefillLayout L;
  L.group = (int)g;
  L.flag = 0;
  L.wuvt = 256;
  L.kbuf = L.wuvt + align256((size_t)s.H * s.DV * s.DC * 2);
  L.vbuf = L.kbuf + align256(g * smax * s.H * s.DN * 2);
  L.total = L.vbuf + align256(g * smax * s.H * s.DV * 2);
  return L;
}

Layout layout(const mla_dims_t* d, const ShapeInfo& s, bool fp8) {
  const size_t B = (size_t)rows(d), slots = (size_t)plan_units(d, s, fp8) + B;
  Layout L;
  L.plan = 0;
  L.q_abs = align256(mla::plan_bytes((int)B, plan_units(d, s, fp8)));
  L.part_lse = L.q_abs + align256(B * s.H * s.DC * 2);
  L.part_o = L.part_lse + align256(slots * s.H * 4);
  L.total = L.part_o + align256(slots * s.H * s.DC * 2);
  return L;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

mla_status_t hip_status(hipError_t e) {
  if (e == hipSuccess) return MLA_OK;
  snprintf(g_hip_err, sizeof g_hip_err, "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
  return MLA_ERR_HIP;
}

// The plan the absorb kernel wrote into the workspace, copied back (the stream is synchronised)
// and printed: the tile stream, each (virtual) sequence's first tile, and every unit's start.
mla_status_t log_plan(const char* plan, int R, int T, int G, int TT, int kv_format,
                      hipStream_t hs) {
  std::vector<char> host(mla::plan_bytes(R, G));
  mla_status_t st = hip_status(hipMemcpyAsync(host.data(), plan, host.size(),
                                              hipMemcpyDeviceToHost, hs));
  if (st == MLA_OK) st = hip_status(hipStreamSynchronize(hs));
  if (st != MLA_OK) return st;
  const mla::Plan* p = reinterpret_cast<const mla::Plan*>(host.data());
  const int32_t* off = reinterpret_cast<const int32_t*>(p + 1);
  const mla::UnitStart* u =
      reinterpret_cast<const mla::UnitStart*>(host.data() + mla::plan_units_offset(R));
  fprintf(stderr,
          "mla_decode plan: %d sequences x %d query tokens, %d tiles of %d tokens, %d units "
          "of up to %d tiles, %s cache\n",
          R / T, T, p->total, TT, p->groups, p->per, format_name(kv_format));
  for (int v = 0; v < R; ++v)
    fprintf(stderr, "  row %d: tiles %d..%d\n", v, off[v], (v + 1 < R ? off[v + 1] : p->total) - 1);
  for (int g = 0; g < G; ++g)
    fprintf(stderr, "  unit %d: row %d tile %d of %d (length %d, page %d), %d tiles\n", g, u[g].b,
            u[g].j, u[g].nj, u[g].S, u[g].page, u[g].n);
  return MLA_OK;
}

}  // namespace

extern "C" {

size_t mla_decode_workspace_bytes(const mla_dims_t* dims) {
  ShapeInfo s;
  if (check_dims(dims, &s) != MLA_OK) return 0;
  if (decompressed(dims)) return prefill_layout(dims, s).total;
  // enough for either cache format (the FP8 one may use more plan units)
  const size_t a = layout(dims, s, false).total;
  if (s.shape != mla::kShapeMha2Mla) return a;
  const size_t b = layout(dims, s, true).total;
  return a > b ? a : b;
}

}  // extern "C"

namespace {

// The decode. hidden == 0: W_up is W_UV and out is [rows][H][d_v]. hidden > 0: W_up is the
// merged W_UVO [hidden][H * d_latent] and out is [rows][hidden] (the combine writes the merged
// latent rows into the query region of the workspace, dead by then, and a product with W_UVO
// follows).
// kv_format (mla::KvFormat) and kv_scales: NULL for the bf16 cache, the fp32 per-token
// scales of an FP8 cache, or the E8M0 block scale bytes of an MXFP4 cache.
mla_status_t decode_call(const mla_dims_t* dims, int hidden, const void* q_nope,
                         const void* q_rope, const void* W_UK, const void* W_UV,
                         const void* kv_pages, int kv_format, const void* kv_scales,
                         const int32_t* page_table, const int32_t* seq_lens, void* out,
                         float* lse_out, void* workspace, size_t workspace_bytes, void* stream,
                         void* const* stage_events) {
  ShapeInfo s;
  mla_status_t st = check_dims(dims, &s);
  if (st != MLA_OK) return st;
  if (kv_scales && !aligned16(kv_scales)) return MLA_ERR_MISALIGNED;
  if (hidden < 0 || hidden > (1 << 20)) return MLA_ERR_BAD_DIMS;
  if (hidden > 0 && (hidden % 16 != 0 || (s.H * s.DC) % 1024 != 0)) return MLA_ERR_UNSUPPORTED;
  if (!q_nope || !q_rope || !W_UK || !W_UV || !kv_pages || !page_table || !seq_lens || !out)
    return MLA_ERR_NULL_ARG;
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(W_UK) || !aligned16(W_UV) ||
      !aligned16(kv_pages) || !aligned16(page_table) || !aligned16(seq_lens) ||
      !aligned16(out) || (lse_out && !aligned16(lse_out)) ||
      (workspace && ((uintptr_t)workspace & 255) != 0))
    return MLA_ERR_MISALIGNED;
  if ((kv_format != mla::kKvBf16) != (kv_scales != nullptr)) return MLA_ERR_NULL_ARG;
  const bool fp8 = kv_format != mla::kKvBf16;  // a quantised cache: FP8 or MXFP4
  // the MXFP4 cache is read at the MHA2MLA widths only
  if (kv_format == mla::kKvMxfp4 && s.shape != mla::kShapeMha2Mla) return MLA_ERR_UNSUPPORTED;
  const bool prefill = decompressed(dims);
  // the decompressed branch reads a bf16 cache and writes the per-head output
  if (prefill && (fp8 || hidden > 0)) return MLA_ERR_UNSUPPORTED;
  const Layout L = prefill ? Layout{} : layout(dims, s, fp8);
  const PrefillLayout PL = prefill ? prefill_layout(dims, s) : PrefillLayout{};
  if (!workspace || workspace_bytes < (prefill ? PL.total : L.total)) return MLA_ERR_WORKSPACE;

  const hipStream_t hs = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int B = dims->batch, mp = dims->max_pages_per_seq, T = q_len(dims), R = B * T;
  if (check_mode()) {
    // validate the device-resident inputs first; the flag lives in a region the decode
    // overwrites afterwards (the queries, or the branch's own flag word)
    int* flag = (int*)(ws + (prefill ? PL.flag : L.q_abs));
    int host_flag = 0;
    st = hip_status(mla::launch_check(seq_lens, page_table, B, mp, dims->num_pages,
                                      max_len(dims), kv_scales, kv_format, s.DC / 32, flag,
                                      hs));
    if (st != MLA_OK) return st;
    st = hip_status(hipMemcpyAsync(&host_flag, flag, sizeof(int), hipMemcpyDeviceToHost, hs));
    if (st != MLA_OK) return st;
    if ((st = hip_status(hipStreamSynchronize(hs))) != MLA_OK) return st;
    if (host_flag != 0) return MLA_ERR_DEVICE_CHECK;
  }
  const float scale = dims->softmax_scale > 0.f ? dims->softmax_scale
                                                : 1.0f / sqrtf((float)(s.DN + s.DR));
  const float scale_log2 = scale * mla::kLog2e;
  if (prefill) {
    if (log_mode())
      fprintf(stderr,
              "mla_decode: decompressed branch, %d sequences x %d query tokens, groups of %d "
              "sequences\n", B, T, PL.group);
    // stage events: 0/1 and 4/5 mark one point each (no absorb or combine kernel), 2/3 bracket
    // the branch's kernels
    auto record = [&](int k) -> mla_status_t {
      if (!stage_events || !stage_events[k]) return MLA_OK;
      return hip_status(hipEventRecord((hipEvent_t)stage_events[k], hs));
    };
    for (int k = 0; k < 3; ++k)
      if ((st = record(k)) != MLA_OK) return st;
    st = hip_status(mla::launch_prefill(s.shape, q_nope, q_rope, W_UK, W_UV, kv_pages,
                                        page_table, seq_lens, B, T, mp, dims->num_pages,
                                        max_len(dims), PL.group, scale_log2, ws + PL.wuvt,
                                        ws + PL.kbuf, ws + PL.vbuf, out, lse_out,
                                        mla::Launch{hs}));
    if (st != MLA_OK) return st;
    for (int k = 3; k < 6; ++k)
      if ((st = record(k)) != MLA_OK) return st;
    return MLA_OK;
  }
  const int G = plan_units(dims, s, fp8);
  // stage_events: start and end of each kernel's own execution (bound to the kernels)
  auto ctx = [&](int k) {
    mla::Launch L{hs};
    if (stage_events) {
      L.start = (hipEvent_t)stage_events[2 * k];
      L.stop = (hipEvent_t)stage_events[2 * k + 1];
    }
    return L;
  };
  st = hip_status(mla::launch_absorb(s.shape, q_nope, W_UK, ws + L.q_abs, R, s.H, seq_lens,
                                     page_table, mp, T, G, ws + L.plan, ctx(0)));
  if (st != MLA_OK) return st;
  if (log_mode() && (st = log_plan(ws + L.plan, R, T, G, s.TT, kv_format, hs)) != MLA_OK)
    return st;
  st = hip_status(mla::launch_attention(s.shape, ws + L.q_abs, q_rope, kv_pages, page_table,
                                        seq_lens, R, mp, T, dims->num_pages, ws + L.plan, G,
                                        scale_log2, ws + L.part_o, (float*)(ws + L.part_lse),
                                        kv_scales, kv_format, ctx(1)));
  if (st != MLA_OK) return st;
  if (hidden == 0)
    return hip_status(mla::launch_combine(s.shape, ws + L.part_o,
                                          (const float*)(ws + L.part_lse), ws + L.plan, seq_lens,
                                          W_UV, out, lse_out, R, s.H, mp, ctx(2)));
  st = hip_status(mla::launch_combine_latent(s.shape, ws + L.part_o,
                                             (const float*)(ws + L.part_lse), ws + L.plan,
                                             ws + L.q_abs, lse_out, R, s.H, ctx(2)));
  if (st != MLA_OK) return st;
  return hip_status(mla::launch_linear(ws + L.q_abs, W_UV, out, R, s.H * s.DC, hidden,
                                       mla::Launch{hs}));
}

}  // namespace

namespace {

// Scratch of mla_decode_noalloc: one array per GPU in the code object, sized for every
// supported call whose mla_decode_workspace_bytes is at most kNoAllocScratchBytes (the five
// benchmark workloads need 2.4 to 33.7 MB). Host code never uses the array's name as an
// address: the device address comes from hipGetSymbolAddress, once per device, with that
// device current.
constexpr size_t kNoAllocScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on the first call on that device).
mla_status_t scratch_for_current_device(void** ptr) {
  int dev = 0;
  mla_status_t st = hip_status(hipGetDevice(&dev));
  if (st != MLA_OK) return st;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    st = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (st != MLA_OK) return st;
    if (!p || ((uintptr_t)p & 255) != 0) return MLA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status_t mla_decode_timed(const mla_dims_t* dims, const void* q_nope, const void* q_rope,
                              const void* W_UK, const void* W_UV, const void* kv_pages,
                              const int32_t* page_table, const int32_t* seq_lens, void* out,
                              float* lse_out, void* workspace, size_t workspace_bytes,
                              void* stream, void* const* stage_events) {
  return decode_call(dims, 0, q_nope, q_rope, W_UK, W_UV, kv_pages, mla::kKvBf16, nullptr,
                     page_table, seq_lens, out, lse_out, workspace, workspace_bytes, stream,
                     stage_events);
}

mla_status_t mla_decode_fp8(const mla_dims_t* dims, const void* q_nope, const void* q_rope,
                            const void* W_UK, const void* W_UV, const void* kv_pages,
                            const float* kv_scales, const int32_t* page_table,
                            const int32_t* seq_lens, void* out, float* lse_out, void* workspace,
                            size_t workspace_bytes, void* stream, void* const* stage_events) {
  if (!kv_scales) return MLA_ERR_NULL_ARG;
  return decode_call(dims, 0, q_nope, q_rope, W_UK, W_UV, kv_pages, mla::kKvFp8, kv_scales,
                     page_table, seq_lens, out, lse_out, workspace, workspace_bytes, stream,
                     stage_events);
}

mla_status_t mla_decode_mxfp4(const mla_dims_t* dims, const void* q_nope, const void* q_rope,
                              const void* W_UK, const void* W_UV, const void* kv_pages,
                              const uint8_t* kv_scales, const int32_t* page_table,
                              const int32_t* seq_lens, void* out, float* lse_out,
                              void* workspace, size_t workspace_bytes, void* stream,
                              void* const* stage_events) {
  if (!kv_scales) return MLA_ERR_NULL_ARG;
  return decode_call(dims, 0, q_nope, q_rope, W_UK, W_UV, kv_pages, mla::kKvMxfp4, kv_scales,
                     page_table, seq_lens, out, lse_out, workspace, workspace_bytes, stream,
                     stage_events);
}

mla_status_t mla_decode_out(const mla_dims_t* dims, int32_t hidden, const void* q_nope,
                            const void* q_rope, const void* W_UK, const void* W_UVO,
                            const void* kv_pages, const int32_t* page_table,
                            const int32_t* seq_lens, void* out_hidden, float* lse_out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (hidden < 1) return MLA_ERR_BAD_DIMS;
  return decode_call(dims, hidden, q_nope, q_rope, W_UK, W_UVO, kv_pages, mla::kKvBf16, nullptr,
                     page_table, seq_lens, out_hidden, lse_out, workspace, workspace_bytes,
                     stream, nullptr);
}

mla_status_t mla_decode(const mla_dims_t* dims, const void* q_nope, const void* q_rope,
                        const void* W_UK, const void* W_UV, const void* kv_pages,
                        const int32_t* page_table, const int32_t* seq_lens, void* out,
                        float* lse_out, void* workspace, size_t workspace_bytes, void* stream) {
  return mla_decode_timed(dims, q_nope, q_rope, W_UK, W_UV, kv_pages, page_table, seq_lens, out,
                          lse_out, workspace, workspace_bytes, stream, nullptr);
}

mla_status_t mla_decode_noalloc(const mla_dims_t* dims, const void* q_nope, const void* q_rope,
                                const void* W_UK, const void* W_UV, const void* kv_pages,
                                const int32_t* page_table, const int32_t* seq_lens, void* out,
                                float* lse_out, void* stream) {
  ShapeInfo s;
  const mla_status_t st0 = check_dims(dims, &s);
  if (st0 != MLA_OK) return st0;
  const size_t need = mla_decode_workspace_bytes(dims);
  if (need == 0 || need > kNoAllocScratchBytes) return MLA_ERR_WORKSPACE;
  void* ws = nullptr;
  const mla_status_t st = scratch_for_current_device(&ws);
  if (st != MLA_OK) return st;
  return decode_call(dims, 0, q_nope, q_rope, W_UK, W_UV, kv_pages, mla::kKvBf16, nullptr,
                     page_table, seq_lens, out, lse_out, ws, kNoAllocScratchBytes, stream,
                     nullptr);
}

mla_status_t mla_gather_pages(const mla_dims_t* dims, const void* kv_pages,
                              const int32_t* page_table, const int32_t* seq_lens, void* dst,
                              void* stream) {
  if (!dims) return MLA_ERR_NULL_ARG;
  if (dims->batch < 1 || dims->max_pages_per_seq < 1 || dims->num_pages < 1 ||
      (int64_t)dims->batch * dims->max_pages_per_seq > (int64_t)1 << 29 ||
      (int64_t)dims->max_seq_len > (int64_t)dims->max_pages_per_seq * dims->page_size)
    return MLA_ERR_BAD_DIMS;
  if (dims->page_size != mla::kPage) return MLA_ERR_UNSUPPORTED;
  if (!((dims->d_latent == 512 && dims->d_rope == 64) ||
        (dims->d_latent == 64 && dims->d_rope == 8)))
    return MLA_ERR_UNSUPPORTED;
  if (!kv_pages || !page_table || !seq_lens || !dst) return MLA_ERR_NULL_ARG;
  if (!aligned16(kv_pages) || !aligned16(page_table) || !aligned16(seq_lens) || !aligned16(dst))
    return MLA_ERR_MISALIGNED;
  return hip_status(mla::launch_gather(dims->d_latent, dims->d_rope, kv_pages, page_table,
                                       seq_lens, dims->batch, dims->max_pages_per_seq,
                                       dims->num_pages, max_len(dims), dst,
                                       (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Checks of the append's dims; fills T.
mla_status_t check_append_dims(const mla_append_dims_t* d, int* T_out) {
  if (!d) return MLA_ERR_NULL_ARG;
  const int T = d->q_len > 1 ? d->q_len : 1;
  if (d->batch < 1 || d->q_len < 0 || (int64_t)d->batch * T > (1 << 20) || d->hidden < 1 ||
      d->d_latent < 1 || d->d_rope < 1 || d->max_pages_per_seq < 1 || d->num_pages < 1 ||
      (int64_t)d->batch * d->max_pages_per_seq > (int64_t)1 << 29 || d->page_size < 1)
    return MLA_ERR_BAD_DIMS;
  if (d->page_size != mla::kPage || d->hidden % 1024 != 0 || d->hidden > (1 << 20) ||
      d->d_latent % 4 != 0 || d->d_rope % 4 != 0 || d->d_latent > 1024 || d->d_rope > 512)
    return MLA_ERR_UNSUPPORTED;
  *T_out = T;
  return MLA_OK;
}

mla_status_t append_call(const mla_append_dims_t* d, const void* x, const void* W_DKV,
                         const void* W_KR, const int32_t* page_table, const int32_t* seq_lens,
                         void* kv_pages, int kv_format, void* kv_scales, void* workspace,
                         size_t workspace_bytes, void* stream) {
  int T = 1;
  mla_status_t st = check_append_dims(d, &T);
  if (st != MLA_OK) return st;
  if (kv_format == mla::kKvMxfp4 && d->d_latent % 32 != 0) return MLA_ERR_UNSUPPORTED;
  if (!x || !W_DKV || !W_KR || !page_table || !seq_lens || !kv_pages) return MLA_ERR_NULL_ARG;
  if (!aligned16(x) || !aligned16(W_DKV) || !aligned16(W_KR) || !aligned16(page_table) ||
      !aligned16(seq_lens) || !aligned16(kv_pages) || (kv_scales && !aligned16(kv_scales)) ||
      (workspace && ((uintptr_t)workspace & 255) != 0))
    return MLA_ERR_MISALIGNED;
  const size_t need = mla::append_workspace_bytes(d->batch * T, d->hidden, d->d_latent, d->d_rope);
  if (!workspace || workspace_bytes < need) return MLA_ERR_WORKSPACE;
  const hipStream_t hs = (hipStream_t)stream;
  if (check_mode()) {
    // validate on the host: every S_b in [0, max_pages_per_seq * 64], and the page-table
    // entry of every new token that falls inside its row in [0, num_pages)
    const int B = d->batch, mp = d->max_pages_per_seq;
    std::vector<int32_t> lens(B), table((size_t)B * mp);
    st = hip_status(hipMemcpyAsync(lens.data(), seq_lens, sizeof(int32_t) * B,
                                   hipMemcpyDeviceToHost, hs));
    if (st == MLA_OK)
      st = hip_status(hipMemcpyAsync(table.data(), page_table, sizeof(int32_t) * table.size(),
                                     hipMemcpyDeviceToHost, hs));
    if (st == MLA_OK) st = hip_status(hipStreamSynchronize(hs));
    if (st != MLA_OK) return st;
    for (int b = 0; b < B; ++b) {
      if (lens[b] < 0 || (int64_t)lens[b] > (int64_t)mp * mla::kPage) return MLA_ERR_DEVICE_CHECK;
      for (int i = 0; i < T; ++i) {
        const int64_t pos = (int64_t)lens[b] + i;
        if (pos >= (int64_t)mp * mla::kPage) break;
        const int32_t page = table[(size_t)b * mp + pos / mla::kPage];
        if (page < 0 || page >= d->num_pages) return MLA_ERR_DEVICE_CHECK;
      }
    }
  }
  const double base = d->rope_base > 0.f ? (double)d->rope_base : 10000.0;
  return hip_status(mla::launch_append(x, W_DKV, W_KR, page_table, seq_lens, kv_pages, kv_scales,
                                       kv_format, workspace, d->batch, T, d->hidden, d->d_latent,
                                       d->d_rope, d->max_pages_per_seq, d->num_pages, base, hs));
}

}  // namespace

extern "C" {

size_t mla_cache_append_workspace_bytes(const mla_append_dims_t* d) {
  int T = 1;
  if (check_append_dims(d, &T) != MLA_OK) return 0;
  return mla::append_workspace_bytes(d->batch * T, d->hidden, d->d_latent, d->d_rope);
}

mla_status_t mla_cache_append(const mla_append_dims_t* d, const void* x, const void* W_DKV,
                              const void* W_KR, const int32_t* page_table,
                              const int32_t* seq_lens, void* kv_pages, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return append_call(d, x, W_DKV, W_KR, page_table, seq_lens, kv_pages, mla::kKvBf16, nullptr,
                     workspace, workspace_bytes, stream);
}

mla_status_t mla_cache_append_fp8(const mla_append_dims_t* d, const void* x, const void* W_DKV,
                                  const void* W_KR, const int32_t* page_table,
                                  const int32_t* seq_lens, void* kv_pages, float* kv_scales,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (!kv_scales) return MLA_ERR_NULL_ARG;
  return append_call(d, x, W_DKV, W_KR, page_table, seq_lens, kv_pages, mla::kKvFp8, kv_scales,
                     workspace, workspace_bytes, stream);
}

mla_status_t mla_cache_append_mxfp4(const mla_append_dims_t* d, const void* x,
                                    const void* W_DKV, const void* W_KR,
                                    const int32_t* page_table, const int32_t* seq_lens,
                                    void* kv_pages, uint8_t* kv_scales, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (!kv_scales) return MLA_ERR_NULL_ARG;
  return append_call(d, x, W_DKV, W_KR, page_table, seq_lens, kv_pages, mla::kKvMxfp4,
                     kv_scales, workspace, workspace_bytes, stream);
}

const char* mla_status_str(mla_status_t s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL_ARG: return "a required pointer is NULL";
    case MLA_ERR_BAD_DIMS: return "sizes out of range or inconsistent";
    case MLA_ERR_MISALIGNED: return "a tensor pointer is not 16-byte aligned (workspace: 256)";
    case MLA_ERR_WORKSPACE: return "workspace missing or smaller than mla_decode_workspace_bytes";
    case MLA_ERR_UNSUPPORTED: return "head/width combination or page size not supported";
    case MLA_ERR_HIP: return "HIP runtime error while enqueueing";
    case MLA_ERR_DEVICE_CHECK:
      return "MLA_CHECK: a sequence length or a used page-table entry is out of range";
  }
  return "unknown status";
}

const char* mla_last_hip_error(void) { return g_hip_err; }

}  // extern "C"
