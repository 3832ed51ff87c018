/*
 * mla_decode.h -- C ABI of the MI355X (gfx950) absorbed MLA decode library, libmla_decode.so.
 *
 * The operation (one query token per sequence, one layer):
 *   For every sequence b and head h, with the sequence's S_b cached tokens t, each stored once
 *   as [c_KV (d_latent) | k_R (d_rope)] in 64-token pages
 *     (bhfrc.com/news/60867 S1 cache format, S3 page size 64),
 *     q_abs[c]   = sum_d q_nope[b,h,d] * W_UK[h,d,c]                    (absorbed query,
 *                  lpnh.cn/news/2494972 S2.1; bhfrc.com/news/60867 S4 path B)
 *     s_t        = scale * (q_abs . c_KV[t] + q_rope[b,h] . k_R[t])      (NoPE + RoPE logits)
 *     p_t        = softmax_t(s_t),  lse = ln sum_t exp(s_t)
 *     o_lat[c]   = sum_t p_t * c_KV[t][c]                               (values in latent space)
 *     out[b,h,e] = sum_c o_lat[c] * W_UV[h,c,e]                         (up-projection,
 *                  lpnh.cn/news/2494972 S2.1 v = c_kv W_uv)
 *   K and V are never decompressed. k_R is shared by all heads; q_rope and k_R arrive already
 *   rotated. The default scale is 1/sqrt(d_nope + d_rope) (bhfrc.com/news/60867 S4).
 *
 * Supported shapes: (num_heads, d_nope, d_latent, d_rope, d_v) = (128, 128, 512, 64, 128),
 * the DeepSeek-V2/V3 widths (bhfrc.com/news/60867 S3), and (32, 120, 64, 8, 128), the MHA2MLA
 * Llama-2-7B attention config (lpnh.cn/news/2494972 S3.2). page_size must be 64. The cache is
 * bf16 (mla_decode, mla_decode_timed, mla_decode_out), FP8 E4M3 with a power-of-two scale
 * per token (mla_decode_fp8), or MXFP4 with an E8M0 scale per token and block of 32 latent
 * elements (mla_decode_mxfp4, MHA2MLA widths).
 *
 * Conventions for every entry point:
 *   - tensors are dense row-major, in device memory, 16-byte aligned; bf16 is stored as its
 *     16-bit pattern; int32 is native.
 *   - the caller allocates and owns every buffer, including the workspace. The library
 *     allocates no device memory, keeps no per-call state, and does not synchronise the
 *     stream (except in the MLA_CHECK mode below).
 *     Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and the call
 *     returns; results are valid once the stream reaches that point.
 *   - argument errors are reported by the return value before anything is enqueued; a HIP
 *     launch failure returns MLA_ERR_HIP (details: mla_last_hip_error()).
 *   - device-resident values are clamped, never trusted: seq_lens[b] is clamped to
 *     [0, max_pages_per_seq * 64] and page ids to [0, num_pages - 1], so a bad table gives
 *     wrong numbers, not a memory fault. A sequence with S_b <= 0 gets out = 0, lse = -inf.
 *   - with MLA_CHECK=1 in the environment, every decode entry point first validates
 *     seq_lens, the page-table entries the sequences use and (FP8 or MXFP4 cache) the scales
 *     of the slots they use on the device, synchronises the stream, and returns
 *     MLA_ERR_DEVICE_CHECK (with nothing else enqueued) when one is out of range.
 *   - with MLA_LOG=1 in the environment, every decode entry point prints its work plan on
 *     stderr: the split of the tile stream over plan units, copied back from the workspace
 *     right after the plan is built (the stream is synchronised there), or, for the
 *     decompressed branch, its grouping of sequences. These two debugging modes are the only
 *     cases in which the library synchronises.
 *   - page-table entries at or past ceil(S_b / 64) and cache slots at or past S_b are never
 *     read into the result (they may hold anything, including NaN).
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MLA_OK = 0,
    MLA_ERR_NULL_ARG = 1,    /* a required pointer is NULL                                */
    MLA_ERR_BAD_DIMS = 2,    /* a size is out of range or sizes disagree with each other  */
    MLA_ERR_MISALIGNED = 3,  /* a tensor pointer is not 16-byte aligned                   */
    MLA_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than mla_decode_workspace_bytes */
    MLA_ERR_UNSUPPORTED = 5, /* head/width combination or page size not built             */
    MLA_ERR_HIP = 6,         /* the HIP runtime reported an error while enqueueing        */
    MLA_ERR_DEVICE_CHECK = 7 /* MLA_CHECK=1 only: a seq_lens value is outside
                                [0, max_seq_len], a page-table entry that its sequence uses
                                is outside [0, num_pages), or (FP8 cache) the scale of a slot
                                a sequence uses is not a positive normal power of two;
                                nothing else was enqueued                                   */
} mla_status_t;

typedef struct {
    int32_t batch;             /* B >= 1 sequences, one query token each                    */
    int32_t num_heads;         /* H                                                        */
    int32_t d_nope;            /* d_n: NoPE width of a query head                          */
    int32_t d_latent;          /* d_c: latent width of the cache (c_KV)                    */
    int32_t d_rope;            /* d_R: decoupled RoPE width (k_R shared by all heads)      */
    int32_t d_v;               /* value width of a head after W_UV                         */
    int32_t page_size;         /* tokens per cache page; must be 64                        */
    int32_t max_pages_per_seq; /* row stride of page_table (>= 1)                          */
    int32_t num_pages;         /* pages in the kv_pages pool (>= 1)                        */
    int32_t max_seq_len;       /* host-side bound on every S_b, used to size the work plan;
                                  <= 0 means max_pages_per_seq * 64                         */
    float softmax_scale;       /* <= 0 means 1/sqrt(d_nope + d_rope)                        */
    int32_t num_units;         /* independent streams over the cache (the split plan): the
                                  tiles of all sequences are dealt to this many units in
                                  order. 0 = automatic (fills the 256 compute units: 128 for
                                  the DeepSeek widths, one unit = two work groups; 1024 for
                                  MHA2MLA, one unit = one wave; 2048 for MHA2MLA with the
                                  FP8 cache, two work groups to a CU). At most 65536.      */
    int32_t q_len;             /* T: query tokens per sequence, 0 or 1 = one (plain decode),
                                  at most 65536, B*T at most 2^20. With T > 1 the T query
                                  tokens of sequence b are its T newest tokens, whose
                                  [c_KV | k_R] are already in the cache (multi-token decode,
                                  or the prompt of a prefill): query token i sits at
                                  position S_b - T + i and attends to tokens
                                  0 .. S_b - T + i, itself included. A query token with no
                                  token to attend to (S_b - T + i < 0) gets out = 0,
                                  lse = -inf.                                              */
    int32_t prefill_threshold; /* T from which the call takes the decompressed branch
                                  (bhfrc.com/news/60867 S3 and S6: the absorb/decompress split
                                  threshold on query rows, tuned there at 128/256/512): keys
                                  and values are expanded per head from c_KV (K_nope =
                                  W_UK c_KV, V = W_UV^T c_KV) and attention runs at the head
                                  widths. 0 = the default: 256 at the DeepSeek widths, never
                                  at the MHA2MLA widths (their latent is narrower than a
                                  head's key, so expanding never saves work). Below it the
                                  absorbed branch serves the call. The decompressed branch
                                  reads a bf16 cache and writes out [B][T][H][d_v]
                                  (mla_decode, mla_decode_timed, mla_decode_noalloc);
                                  mla_decode_out, mla_decode_fp8 and mla_decode_mxfp4
                                  return MLA_ERR_UNSUPPORTED for it. Both branches compute
                                  the same result up to rounding.                           */
} mla_dims_t;

/* Bytes of scratch a call with these dims needs (pure function of the dims, host only), for
 * every cache format (mla_decode, mla_decode_fp8 and mla_decode_mxfp4). Returns 0 when the
 * dims are invalid or unsupported. */
size_t mla_decode_workspace_bytes(const mla_dims_t* dims);

/*
 * Absorbed MLA decode (the operation above). T = q_len (1 when dims->q_len is 0 or 1).
 *   q_nope     bf16 [B, T, H, d_nope]                    ([B, H, d_nope] when T = 1)
 *   q_rope     bf16 [B, T, H, d_rope]                    already rotated
 *   W_UK       bf16 [H, d_nope, d_latent]
 *   W_UV       bf16 [H, d_latent, d_v]
 *   kv_pages   bf16 [num_pages, 64, d_latent + d_rope]   token = [c_KV | k_R]
 *   page_table int32 [B, max_pages_per_seq]              logical page j of b -> pool page
 *   seq_lens   int32 [B]                                 S_b, 1 <= S_b <= max_seq_len
 *   out        bf16 [B, T, H, d_v]                       written
 *   lse_out    fp32 [B, T, H] natural-log LSE of the logits, or NULL
 *   workspace  device scratch, 256-byte aligned, of at least mla_decode_workspace_bytes(dims)
 *              bytes; its contents need no initialisation and are garbage afterwards
 * Inputs are read only; out, lse_out and workspace are the only memory written. Calls that
 * share a workspace must be ordered on one stream.
 */
mla_status_t mla_decode(const mla_dims_t* dims, const void* q_nope, const void* q_rope,
                        const void* W_UK, const void* W_UV, const void* kv_pages,
                        const int32_t* page_table, const int32_t* seq_lens, void* out,
                        float* lse_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same operation, arguments and
 * results, without the workspace. Its scratch is an array built into the library, one per
 * GPU, of MLA_NOALLOC_SCRATCH_BYTES; each GPU that calls it holds that memory until the
 * process ends. The call allocates nothing and calls no allocating routine; its first call on
 * a device looks the array's address up once (hipGetSymbolAddress).
 *   - Uses the array of the current device; `stream` must belong to that device.
 *   - Returns MLA_ERR_WORKSPACE when the dims need more scratch than the array holds
 *     (mla_decode_workspace_bytes(dims) > MLA_NOALLOC_SCRATCH_BYTES), before enqueueing.
 *   - Every call on a GPU shares that GPU's array, which keeps the last call's contents:
 *     calls that overlap on one GPU (on different streams, or from several threads without
 *     ordering) race and give wrong results. Order them on one stream.
 * Everything else (dims, layouts, MLA_CHECK, errors) is as for mla_decode.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)
mla_status_t mla_decode_noalloc(const mla_dims_t* dims, const void* q_nope, const void* q_rope,
                                const void* W_UK, const void* W_UV, const void* kv_pages,
                                const int32_t* page_table, const int32_t* seq_lens, void* out,
                                float* lse_out, void* stream);

/*
 * mla_decode with kernel timing: identical work and results, and, when stage_events is not
 * NULL, binds six caller-owned events (hipEvent_t, each may be NULL) to the kernels it enqueues
 * on `stream`: stage_events[2k] to the start and stage_events[2k+1] to the end of kernel k's
 * execution, k = 0 absorb, 1 attention, 2 combine (hipExtLaunchKernel semantics). The elapsed
 * time of a pair is that kernel's execution alone, without the launch gap before it, which is
 * what the benchmark's roofline measurement divides by. The events must have been created
 * with timing enabled.
 */
mla_status_t mla_decode_timed(const mla_dims_t* dims, const void* q_nope, const void* q_rope,
                              const void* W_UK, const void* W_UV, const void* kv_pages,
                              const int32_t* page_table, const int32_t* seq_lens, void* out,
                              float* lse_out, void* workspace, size_t workspace_bytes,
                              void* stream, void* const* stage_events);

/*
 * The decode over a quantised latent cache: c_KV stored as 8-bit floats with a scale per token
 * (bhfrc.com/news/60867 S1 and S5 quantise the latent cache that the decode gathers; this is
 * the FP8 form of that cache), at both supported widths: a token takes d_latent + 2*d_rope
 * bytes plus its 4-byte scale (644 bytes at the DeepSeek widths, against 1152 in bf16).
 *   kv_pages   uint8 [num_pages, 64, d_latent + 2*d_rope]  token row = [c_KV as d_latent
 *              FP8 E4M3 bytes (OCP format: 4 exponent bits, bias 7, 3 mantissa bits, no
 *              infinities, S.1111.111 = NaN) | k_R as d_rope bf16 values]
 *   kv_scales  fp32 [num_pages, 64]                      the scale of the token in each slot:
 *              c_KV[c] = value(byte c) * kv_scales[page][slot]. Precondition: the scale of
 *              every slot a sequence uses is a positive normal power of two, 2^e with
 *              -126 <= e <= 127 (exponent-only, as in the microscaling formats). Other values
 *              are not reinterpreted: the result is then unspecified, and the MLA_CHECK mode
 *              reports them (MLA_ERR_DEVICE_CHECK). Slots no sequence uses may hold anything.
 * Each dequantised c_KV element (an E4M3 value times a power of two) is a bf16 value. At the
 * MHA2MLA widths the decode forms those values exactly and runs as in mla_decode: the result
 * is that of mla_decode on the bf16 cache holding them, bit for bit. At the DeepSeek widths the
 * latent part of each score is taken by the block-scaled FP8 matrix instruction straight from
 * the bytes, with the token's scale as the block scale and the absorbed query split exactly
 * into two E4M3 parts; that instruction's sum differs from an fp32 sum by up to about 1e-4 of
 * the sum of |products|, so the result is mla_decode's on those values up to that rounding
 * (within 1e-3 relative on the tested workloads), not bit for bit. Slots at or past S_b (bytes
 * and scales) are never read
 * into the result. kv_scales must be 16-byte aligned and non-NULL; everything else, including
 * q_len, the workspace size and stage_events (NULL or six events, as for mla_decode_timed),
 * is as for mla_decode_timed.
 */
mla_status_t mla_decode_fp8(const mla_dims_t* dims, const void* q_nope, const void* q_rope,
                            const void* W_UK, const void* W_UV, const void* kv_pages,
                            const float* kv_scales, const int32_t* page_table,
                            const int32_t* seq_lens, void* out, float* lse_out, void* workspace,
                            size_t workspace_bytes, void* stream, void* const* stage_events);

/*
 * The decode over a 4-bit quantised latent cache (bhfrc.com/news/60867 S1 and S5 quantise the
 * latent cache the decode gathers; this is its microscaled 4-bit form, the OCP Microscaling
 * (MX) v1.0 MXFP4 format): c_KV in blocks of 32 elements, each element a 4-bit float, each
 * block sharing one power-of-two scale. MHA2MLA widths only (MLA_ERR_UNSUPPORTED at the
 * DeepSeek widths): a token takes d_latent/2 + 2*d_rope bytes plus d_latent/32 scale bytes
 * (48 + 2 = 50 bytes, against 144 in bf16 and 84 in FP8).
 *   kv_pages   uint8 [num_pages, 64, d_latent/2 + 2*d_rope]  token row = [c_KV as d_latent
 *              E2M1 codes, two per byte, element 2k in the low nibble of byte k (E2M1: sign,
 *              2 exponent bits with bias 1, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3,
 *              4, 6) | k_R as d_rope bf16 values]
 *   kv_scales  uint8 [num_pages, 64, d_latent/32]  E8M0 scale bytes of each slot's blocks:
 *              c_KV[c] = value(code c) * 2^(kv_scales[page][slot][c/32] - 127).
 *              Precondition: no slot a sequence uses holds 255 (E8M0's NaN); the MLA_CHECK
 *              mode reports one (MLA_ERR_DEVICE_CHECK). Slots no sequence uses may hold
 *              anything.
 * Each dequantised c_KV element is a bf16 value, formed exactly, and the decode then runs as in
 * mla_decode: the result is that of mla_decode on the bf16 cache holding those values. Slots at
 * or past S_b are never read into the result. kv_scales must be 16-byte aligned and non-NULL;
 * everything else, including q_len, the workspace size and stage_events, is as for
 * mla_decode_timed.
 */
mla_status_t mla_decode_mxfp4(const mla_dims_t* dims, const void* q_nope, const void* q_rope,
                              const void* W_UK, const void* W_UV, const void* kv_pages,
                              const uint8_t* kv_scales, const int32_t* page_table,
                              const int32_t* seq_lens, void* out, float* lse_out,
                              void* workspace, size_t workspace_bytes, void* stream,
                              void* const* stage_events);

/*
 * The decode with the output projection merged into the up-projection (lpnh.cn/news/2494972
 * S2.2: W_uv and W_o are merged into one matrix offline): instead of out[b,h,:] = o_lat W_UV[h]
 * it returns
 *   out_hidden[b, n] = sum_h sum_c o_lat[b,h,c] * W_UVO[n, h*d_latent + c]
 * where the caller has formed W_UVO[n, h*d_latent + c] = sum_e W_UV[h,c,e] W_O[h*d_v + e, n].
 *   W_UVO      bf16 [hidden, H * d_latent]            (replaces W_UV)
 *   out_hidden bf16 [B, T, hidden]                     written
 * Every other argument, the workspace size (mla_decode_workspace_bytes) and the conventions
 * are those of mla_decode. Needs hidden a multiple of 16 (at most 2^20) and H * d_latent a
 * multiple of 1024 (both supported shapes are). Returns MLA_ERR_BAD_DIMS for hidden < 1.
 */
mla_status_t mla_decode_out(const mla_dims_t* dims, int32_t hidden, const void* q_nope,
                            const void* q_rope, const void* W_UK, const void* W_UVO,
                            const void* kv_pages, const int32_t* page_table,
                            const int32_t* seq_lens, void* out_hidden, float* lse_out,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Cache append (the step before the decode): the latent and the decoupled RoPE key of new
 * tokens, written into their page slots (lpnh.cn/news/2494972 S2.1: c_kv = x W_dkv and a
 * RoPE key taken from the hidden state; bhfrc.com/news/60867 S1 [c_KV | k_R] format, S3
 * RoPE computed in fp32 and 64-token pages).
 * For token i of sequence b (i < T), at position p = seq_lens[b] + i:
 *   c_KV[c] = sum_k x[b,i,k] W_DKV[c,k]
 *   k[j]    = sum_k x[b,i,k] W_KR[j,k]
 *   (k[j], k[j + d_rope/2]) <- (k[j] cos a - k[j + d_rope/2] sin a,
 *                               k[j] sin a + k[j + d_rope/2] cos a),  a = p * base^(-2j/d_rope)
 * (fp32 sums and rotation, the angle formed in fp64), rounded to bf16 and stored at slot
 * p % 64 of page page_table[b][p / 64]: kv_pages[page][slot] = [c_KV | k].
 *   x          bf16 [B, T, hidden]
 *   W_DKV      bf16 [d_latent, hidden]    (a linear layer's weight: out x in)
 *   W_KR       bf16 [d_rope, hidden]
 *   page_table int32 [B, max_pages_per_seq], seq_lens int32 [B]: tokens already cached
 *   kv_pages   bf16 [num_pages, 64, d_latent + d_rope], written at the new tokens' slots only
 * seq_lens is not updated (the caller adds T after the call). A token whose position falls
 * outside its page-table row (p >= max_pages_per_seq * 64), or whose page-table entry is not
 * a pool page (outside [0, num_pages), e.g. -1 for a page not allocated yet), is not written:
 * no other slot changes. With MLA_CHECK=1 the call first copies seq_lens and the page table to
 * the host, synchronises the stream, and returns MLA_ERR_DEVICE_CHECK (writing nothing) when
 * an S_b is outside [0, max_pages_per_seq * 64] or such an entry of a new token is outside
 * the pool. Sizes: hidden a multiple of 1024, d_latent and d_rope multiples of 4, B*T at most
 * 2^20, d_latent at most 1024, d_rope at most 512. The workspace (256-byte aligned, at least
 * mla_cache_append_workspace_bytes) holds fp32 partial sums; the caller owns it and may reuse
 * it between calls. Same conventions as above otherwise (enqueued on `stream`, no allocation,
 * argument errors before anything is enqueued). The decode's q_rope must be rotated with the
 * same pairing and base.
 */
typedef struct {
    int32_t batch;             /* B sequences                                               */
    int32_t q_len;             /* T new tokens per sequence; 0 means 1                      */
    int32_t hidden;            /* width of x                                                */
    int32_t d_latent;          /* d_c                                                       */
    int32_t d_rope;            /* d_R                                                       */
    int32_t page_size;         /* must be 64                                                */
    int32_t max_pages_per_seq; /* row stride of page_table                                  */
    int32_t num_pages;         /* pages in the pool                                         */
    float rope_base;           /* RoPE base; <= 0 means 10000                               */
} mla_append_dims_t;

/* Bytes of scratch mla_cache_append, mla_cache_append_fp8 and mla_cache_append_mxfp4 need for
 * these dims (fp32 partial rows of the contraction, split over the model width); 0 if the dims
 * are invalid. */
size_t mla_cache_append_workspace_bytes(const mla_append_dims_t* dims);

mla_status_t mla_cache_append(const mla_append_dims_t* dims, const void* x, const void* W_DKV,
                              const void* W_KR, const int32_t* page_table,
                              const int32_t* seq_lens, void* kv_pages, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * The same append into an FP8 cache (the layout mla_decode_fp8 reads): kv_pages uint8
 * [num_pages, 64, d_latent + 2*d_rope] with rows [c_KV as E4M3 bytes | k_R as bf16], and
 * kv_scales fp32 [num_pages, 64]. For each new token the scale is the smallest power of two
 * 2^e with max_c |c_KV[c]| <= 448 * 2^e (448 is the largest E4M3 value; e kept within
 * -126 .. 127, 1 for an all-zero row), and byte c is c_KV[c] / 2^e rounded to the nearest E4M3
 * value, ties to even (c_KV as fp32 sums, not rounded to bf16 first). k_R is rotated and
 * rounded to bf16 as above. Everything else is as for mla_cache_append; kv_scales must be
 * non-NULL and 16-byte aligned.
 */
mla_status_t mla_cache_append_fp8(const mla_append_dims_t* dims, const void* x,
                                  const void* W_DKV, const void* W_KR,
                                  const int32_t* page_table, const int32_t* seq_lens,
                                  void* kv_pages, float* kv_scales, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * The same append into an MXFP4 cache (the layout mla_decode_mxfp4 reads): kv_pages uint8
 * [num_pages, 64, d_latent/2 + 2*d_rope] with rows [c_KV as E2M1 codes, two per byte |
 * k_R as bf16], and kv_scales uint8 [num_pages, 64, d_latent/32]. For each new token and
 * block of 32 latent elements (the OCP MX conversion): the shared exponent is
 * X = floor(log2(max |c_KV[c]|)) - 2 over the block (2 is the exponent of E2M1's largest
 * value, 6), kept within -127 .. 127, and 0 for an all-zero block; the scale byte is X + 127;
 * element c is c_KV[c] / 2^X rounded to the nearest E2M1 value, ties to the even code,
 * magnitudes above 6 saturating to 6, zero stored as +0 (c_KV as fp32 sums, not rounded to
 * bf16 first). k_R is rotated and rounded to bf16 as above. d_latent must be a multiple of
 * 32. Everything else is as for mla_cache_append; kv_scales must be non-NULL and 16-byte
 * aligned.
 */
mla_status_t mla_cache_append_mxfp4(const mla_append_dims_t* dims, const void* x,
                                    const void* W_DKV, const void* W_KR,
                                    const int32_t* page_table, const int32_t* seq_lens,
                                    void* kv_pages, uint8_t* kv_scales, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * Logical copy of the paged cache, through the same page addressing and LDS staging the
 * attention kernel uses (a bit-exact test of the page loads).
 *   dst bf16 [B, S_max, d_latent + d_rope]; row t of sequence b is token t for t < S_b and
 *   zero for S_b <= t < S_max, where S_max = max_seq_len (or max_pages_per_seq * 64).
 * Only batch, d_latent, d_rope, page_size, max_pages_per_seq, num_pages and max_seq_len of
 * dims are used.
 */
mla_status_t mla_gather_pages(const mla_dims_t* dims, const void* kv_pages,
                              const int32_t* page_table, const int32_t* seq_lens, void* dst,
                              void* stream);

/* Static description of a status code. */
const char* mla_status_str(mla_status_t status);

/* Text of the last HIP error this library saw on the calling thread ("" if none). */
const char* mla_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
